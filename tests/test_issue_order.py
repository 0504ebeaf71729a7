"""The decode main kernel's counted waits rely on its K loop issuing each
stage's row loads before the next stage's W loads; these tests pin the
checker on hand-made listings and run it on the kernel as compiled for gfx950
(device code only; no GPU needed)."""

import os
import shutil

import pytest

from lora_normal_form_amd import build, issue_order

HEAD = "_ZN5scute13k_decode_mainILi5ELi8EEEvNS_8MainArgsE:\n"
END = ".Lfunc_end0:\n"


def _listing(*steps):
    body = []
    for ops in steps:
        body += ["\t" + o + " v[0:1], off" for o in ops] + ["\ts_barrier"]
    return HEAD + "\n".join(body) + "\n" + END


def test_checker_accepts_rows_then_w():
    asm = _listing(["buffer_load_dwordx4", "global_load_lds_dwordx4"],
                   ["global_load_lds_dwordx4"] * 4 + ["buffer_load_dwordx4"] * 2,
                   ["global_load_lds_dwordx4"] * 4 + ["buffer_load_dwordx4"] * 2)
    assert issue_order.violations(asm) == []
    assert len(issue_order.kernel_steps(asm)) == 1


def test_checker_flags_a_w_load_moved_above_a_row_load():
    asm = _listing(["buffer_load_dwordx4"],
                   ["global_load_lds_dwordx4"] * 3 + ["buffer_load_dwordx4", "global_load_lds_dwordx4"])
    assert issue_order.violations(asm) == [("_ZN5scute13k_decode_mainILi5ELi8EEEvNS_8MainArgsE", 1)]


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not installed")
def test_compiled_kernel_keeps_the_issue_order():
    assert issue_order.main() == 0


def test_phase_stamps_apply_to_the_decode_kernel():
    # the phase-timestamp tool instruments k_decode_main at fixed anchors;
    # every anchor must still be found exactly once
    from lora_normal_form_amd import phases
    src = open(os.path.join(build.CSRC, "decode.hip")).read()
    out = phases._patch(src)
    assert out.count("phase_stamp(") == 9  # the helper plus eight boundaries
    assert "scute_phase_read" in out
