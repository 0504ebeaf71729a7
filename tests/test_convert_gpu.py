"""GPU: LoRA conversions (truncated SVD of each adapter's weight change,
optionally zero-padded to the pool's largest rank) run on the MFMA decode
path and match the oracle's evaluation of the converted LoRA adapters at the
bf16 bars: max|y - ref| <= 1e-2 max|ref| and mean effect error <= 1%."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

SPECS = [AdapterSpec("lora", rank=16, bias=True), AdapterSpec("dora", rank=16),
         AdapterSpec("ia3"), AdapterSpec("vera", bias=True), AdapterSpec("oft", blk=32)]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("pad", [0, 128])
def test_converted_workload_matches_oracle(pad):
    _need_gpu()
    from lora_normal_form_amd import conversion
    from lora_normal_form_amd import workload as glue
    ta = np.random.default_rng(81).integers(-1, len(SPECS), size=96)
    wl = make_workload(WorkloadSpec("conv_src", "bf16", 512, 384, len(ta), SPECS, vera_rank=64,
                                    assign="explicit", token_adapter=ta, seed=81))
    cw, errs = conversion.converted(wl, {"dora": 64, "ia3": 64, "oft": 64, "vera": 64}, pad_to=pad)
    assert errs["vera"][0] < 1e-9  # the VeRA term has rank <= r_v = 64: exact
    assert all(a.method == "lora" for a in cw.adapters)
    print(f"\n[gpu] {cw.name} n={cw.n} pad={pad}", flush=True)
    ld = glue.load(cw, device=0)
    assert ld.batch.info()["path"] == 1, ld.batch.info()
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    y = ld.y.cpu().numpy().astype(np.float64)
    ref = oracle.forward(cw)
    ok, rep = oracle.check(y, ref, cw.x @ cw.W.T, cw.token_adapter, cw.dtype)
    print(f"[gpu] {rep}", flush=True)
    assert ok, rep
