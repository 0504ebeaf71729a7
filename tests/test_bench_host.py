"""Host-side checks of bench.py (no GPU): the matched all-LoRA comparison
batch, and the refusal of more than one GPU."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import make_config  # noqa: E402


def test_matched_lora_keeps_the_batch_and_replaces_every_adapter():
    wl = make_config(2)
    m = bench.matched_lora(wl)
    assert (m.n, m.d_in, m.d_out, m.dtype) == (wl.n, wl.d_in, wl.d_out, wl.dtype)
    assert np.array_equal(m.token_adapter, wl.token_adapter)
    assert np.array_equal(m.x, wl.x) and np.array_equal(m.W, wl.W)
    assert len(m.adapters) == len(wl.adapters)
    assert all(a.method == "lora" and a.rank == 16 for a in m.adapters)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_sources_hash_ignores_comments_only():
    from lora_normal_form_amd.profsum import strip_comments
    code = 'int a = 1;  // one\n/* block\n   comment */\nconst char* s = "x // y /* z */";\nchar q = \'"\';\n'
    recommented = 'int a = 1;  // first\n// added line\nconst char* s = "x // y /* z */";\n/* another */ char q = \'"\';\n'
    assert strip_comments(code) == strip_comments(recommented)
    # literals that look like comments stay, and a change of code is seen
    assert '"x // y /* z */"' in strip_comments(code)
    assert strip_comments(code) != strip_comments(code.replace("a = 1", "a = 2"))


def test_cpu_baseline_is_median_of_three_runs():
    import bench
    from synth import make_config
    wl = make_config(0)
    cb = bench.cpu_baseline(wl, 0.3)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert len(cb["runs"]) == 3
    assert cb["value"] == sorted(cb["runs"])[1] or abs(cb["value"] - sorted(cb["runs"])[1]) < 1e-3
    assert cb["cores"] >= 1 and cb["host_cpu_count"] == __import__("os").cpu_count()
