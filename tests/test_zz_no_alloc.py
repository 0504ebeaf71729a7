"""GPU: the no-allocation forward (scute_layer_forward_noalloc, static
device scratch, batch in token order) against the planned forward
(scute_layer_forward) on the same layer and inputs, and against the fp64
oracle, at the parity bars: fp32 max|y - ref| <= 1e-4 max|ref|; bf16
max|y - ref| <= 1e-2 max|ref| plus every adapter's mean effect error <= 1%.

Two calls in a row share the scratch: the second, smaller batch must not
see anything the first left there.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

ADS = [AdapterSpec("lora", rank=16, c=2.0, bias=True), AdapterSpec("dora", rank=16),
       AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=32),
       AdapterSpec("lora", rank=8), AdapterSpec("oft", blk=16),
       AdapterSpec("nf", rank=16, blk=16, c=0.5, nf_R=True, nf_s=True, nf_b=True, nf_term=True,
                   nf_vera=True)]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _wl(dtype, n, seed, d_in=512, d_out=384):
    rng = np.random.default_rng(seed)
    ta = rng.integers(0, len(ADS), size=n)
    ta[rng.random(n) < 0.1] = -1
    return make_workload(WorkloadSpec(f"noalloc_{dtype}_n{n}", dtype, d_in, d_out, n, ADS,
                                      vera_rank=64, assign="explicit", token_adapter=ta,
                                      seed=seed))


def _sub(wl, m):
    """The first m tokens of a workload (same layer, adapters and weights)."""
    import dataclasses
    return dataclasses.replace(wl, name=f"{wl.name}_first{m}", n=m, x=wl.x[:m],
                               token_adapter=wl.token_adapter[:m])


def _bar(wl, y, ref):
    assert np.all(np.isfinite(y))
    ok, rep = oracle.check(y, ref, wl.x @ wl.W.T, wl.token_adapter, wl.dtype)
    print(f"[gpu] {wl.name}: {rep}", flush=True)
    assert ok, rep


def _both(ld, wl, m):
    """Planned and no-allocation forwards of the first m tokens."""
    L = ld.layer
    ta = wl.token_adapter[:m]
    x = ld.x[:m]
    B = L.plan(ta)
    y_plan = torch.full((m, wl.d_out), float("nan"), dtype=torch.float32, device=ld.y.device)
    L.forward(B, x, ld.W, y_plan)
    ta_dev = torch.tensor(ta, dtype=torch.int32, device=ld.y.device)
    y_na = torch.full((m, wl.d_out), float("nan"), dtype=torch.float32, device=ld.y.device)
    print(f"[gpu] noalloc forward n={m} d_in={wl.d_in} d_out={wl.d_out} {wl.dtype}", flush=True)
    L.forward_noalloc(ta_dev, x, ld.W, y_na)
    torch.cuda.synchronize()
    B.close()
    return (y_plan.cpu().numpy().astype(np.float64), y_na.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_planned_forward_twice(dtype):
    _need_gpu()
    from lora_normal_form_amd import workload as glue
    wl = _wl(dtype, 77, seed=3)
    ld = glue.load(wl, device=0, plan=False)
    tol = 1e-4 if dtype == "f32" else 1e-2
    for m in (77, 33):  # the second call is smaller
        w = _sub(wl, m) if m < wl.n else wl
        ref = oracle.forward(w)
        y_plan, y_na = _both(ld, w, m)
        _bar(w, y_plan, ref)
        _bar(w, y_na, ref)
        assert np.max(np.abs(y_na - y_plan)) <= tol * np.max(np.abs(ref))
    ld.layer.close()


def test_noalloc_bad_ids_give_nan_rows():
    # ids are checked on the device: an unloaded or out-of-range id makes
    # its row NaN and leaves the other rows exact
    _need_gpu()
    from lora_normal_form_amd import workload as glue
    wl = _wl("bf16", 40, seed=4)
    ld = glue.load(wl, device=0, plan=False, max_adapters=len(ADS) + 2)
    ta = wl.token_adapter.copy()
    ta[5] = len(ADS)        # in range, never loaded
    ta[9] = len(ADS) + 7    # out of range
    ta_dev = torch.tensor(ta, dtype=torch.int32, device=ld.y.device)
    y = torch.zeros((wl.n, wl.d_out), dtype=torch.float32, device=ld.y.device)
    ld.layer.forward_noalloc(ta_dev, ld.x, ld.W, y)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(y[[5, 9]]))
    good = np.setdiff1d(np.arange(wl.n), [5, 9])
    ref = oracle.forward(wl)
    assert np.all(np.isfinite(y[good]))
    assert np.max(np.abs(y[good] - ref[good])) <= 1e-2 * np.max(np.abs(ref))
    ld.layer.close()


def test_noalloc_rejects_batches_beyond_the_scratch():
    _need_gpu()
    from lora_normal_form_amd import scute
    from lora_normal_form_amd import workload as glue
    wl = _wl("f32", 8, seed=5, d_in=4096, d_out=64)
    ld = glue.load(wl, device=0, plan=False)
    # 1100 rotated fp32 rows of 4096 need 1100 * 16 KB > 16 MB of scratch
    n = 1100
    x = torch.zeros((n, wl.d_in), dtype=torch.float32, device=ld.y.device)
    y = torch.zeros((n, wl.d_out), dtype=torch.float32, device=ld.y.device)
    ta = torch.zeros(n, dtype=torch.int32, device=ld.y.device)
    with pytest.raises(scute.ScuteError) as ei:
        ld.layer.forward_noalloc(ta, x, ld.W, y)
    assert ei.value.code == scute.E_SHAPE and "scratch" in str(ei.value)
    ld.layer.close()
