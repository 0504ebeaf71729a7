"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bars (in every test): fp32 workloads max|y - ref| <= 1e-4 max|ref|;
bf16-in / fp32-accumulate workloads max|y - ref| <= 1e-2 max|ref| and, for
every adapter with tokens, mean adapter-effect error <= 1% of its effect.
The five named workloads run at full size and are compared element by
element (the oracle finishes each in seconds).
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_config, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

_cache = {}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(wl, loaded=None):
    from lora_normal_form_amd import workload as glue
    print(f"\n[gpu] {wl.name} dtype={wl.dtype} n={wl.n} d_in={wl.d_in} d_out={wl.d_out} "
          f"seed={wl.seed}", flush=True)
    ld = loaded or glue.load(wl, device=0)
    ld.y.fill_(float("nan"))
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    return ld, ld.y.cpu().numpy().astype(np.float64)


def _assert_parity(wl, y, ref=None):
    ref = oracle.forward(wl) if ref is None else ref
    assert np.all(np.isfinite(y)), "non-finite output"
    ok, rep = oracle.check(y, ref, wl.x @ wl.W.T, wl.token_adapter, wl.dtype)
    print(f"[gpu] {wl.name}: {rep}", flush=True)
    assert ok, rep
    return rep


def _config(idx):
    if idx not in _cache:
        wl = make_config(idx)
        _cache[idx] = (wl, oracle.forward(wl))
    return _cache[idx]


# kernels each named workload must run on: 0 generic (fp32), 1 MFMA decode,
# 2 MFMA prefill; a planner change that sent one of them elsewhere fails here
NAMED_PATH = {0: 0, 1: 1, 2: 1, 3: 1, 4: 2}


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_named_workload_full_size(idx):
    _need_gpu()
    wl, ref = _config(idx)
    ld, y = _run(wl)
    assert ld.batch.info()["path"] == NAMED_PATH[idx], ld.batch.info()
    _assert_parity(wl, y, ref)


@pytest.mark.parametrize("idx", [1, 2, 3])
@pytest.mark.parametrize("mode", [1, 2], ids=["fused", "two_launch"])
def test_named_decode_workload_each_path(idx, mode):
    # the decode workloads on each MFMA decode path by name (SCUTE_DECODE)
    _need_gpu()
    from lora_normal_form_amd import workload as glue
    wl, ref = _config(idx)
    old = os.environ.get("SCUTE_DECODE")
    os.environ["SCUTE_DECODE"] = str(mode)
    try:
        ld = glue.load(wl, device=0)
    finally:
        if old is None:
            del os.environ["SCUTE_DECODE"]
        else:
            os.environ["SCUTE_DECODE"] = old
    ld, y = _run(wl, ld)
    assert ld.batch.info()["path"] == 1, ld.batch.info()
    _assert_parity(wl, y, ref)


def _small(dtype, adapters, ta, d_in=96, d_out=72, vera_rank=8, seed=0, **kw):
    return make_workload(WorkloadSpec(f"edge_{dtype}", dtype, d_in, d_out, len(ta), adapters,
                                      vera_rank=vera_rank, assign="explicit", token_adapter=ta,
                                      seed=seed, **kw))


ALL_METHODS = [AdapterSpec("lora", rank=4, c=2.0, bias=True), AdapterSpec("dora", rank=3),
               AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=8),
               AdapterSpec("nf", rank=2, blk=4, c=0.5, nf_R=True, nf_s=True, nf_b=True,
                           nf_term=True, nf_vera=True)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("aid", range(6))
def test_single_token_each_method(dtype, aid):
    _need_gpu()
    wl = _small(dtype, ALL_METHODS, [aid], seed=aid)
    _, y = _run(wl)
    _assert_parity(wl, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_tokens_and_columns(dtype):
    # 77 tokens (not a tile multiple), d_out 72 (ragged column tile), some
    # tokens without adapter, adapter 6 loaded but never used
    _need_gpu()
    rng = np.random.default_rng(1)
    ta = rng.integers(-1, 6, size=77)
    wl = _small(dtype, ALL_METHODS + [AdapterSpec("lora", rank=2)], ta, seed=3)
    _, y = _run(wl)
    _assert_parity(wl, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_tokens_unassigned(dtype):
    _need_gpu()
    wl = _small(dtype, ALL_METHODS, [-1] * 40, seed=4)
    _, y = _run(wl)
    _assert_parity(wl, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rank_one_and_block_two(dtype):
    _need_gpu()
    ads = [AdapterSpec("lora", rank=1), AdapterSpec("oft", blk=2), AdapterSpec("dora", rank=1)]
    wl = _small(dtype, ads, [0, 1, 2, 1, 0, 2, 1] * 5, seed=5, sigma_q=0.2)
    _, y = _run(wl)
    _assert_parity(wl, y)


def test_far_from_identity_vectors():
    # the pages' accuracy protocol pushes vectors off identity (e.g. s = 1 + 0.3 N)
    _need_gpu()
    rng = np.random.default_rng(6)
    wl = _small("bf16", ALL_METHODS, rng.integers(0, 6, size=64), d_in=256, d_out=128,
                vera_rank=16, seed=6, sigma_l=0.3, sigma_m=0.3, sigma_vd=0.3, sigma_ve=0.3,
                sigma_q=0.05)
    _, y = _run(wl)
    _assert_parity(wl, y)


def test_repeat_runs_and_plan_reuse():
    # the MFMA decode path adds K-slice partials with float atomics, so
    # repeated runs agree to rounding, not bit for bit; the generic kernels
    # are deterministic
    _need_gpu()
    wl, ref = _config(2)
    ld, y1 = _run(wl)
    _, y2 = _run(wl, loaded=ld)
    assert np.max(np.abs(y1 - y2)) <= 1e-5 * np.max(np.abs(ref))
    import os
    from lora_normal_form_amd import workload as glue
    os.environ["SCUTE_DECODE"] = "0"
    os.environ["SCUTE_PREFILL"] = "0"
    try:
        ldg = glue.load(wl, device=0)
    finally:
        del os.environ["SCUTE_DECODE"]
        del os.environ["SCUTE_PREFILL"]
    assert ldg.batch.info()["path"] == 0
    _, g1 = _run(wl, loaded=ldg)
    _, g2 = _run(wl, loaded=ldg)
    np.testing.assert_array_equal(g1, g2)
    _assert_parity(wl, g1, ref)
    # same plan, new activations
    from lora_normal_form_amd import workload as glue
    rng = np.random.default_rng(8)
    from synth import round_bf16
    wl.x = round_bf16(rng.normal(size=wl.x.shape))
    ld.x.copy_(glue.to_device(wl.x, "bf16", torch.device("cuda", 0)))
    _, y3 = _run(wl, loaded=ld)
    _assert_parity(wl, y3)


def test_empty_batch_and_errors_on_device():
    _need_gpu()
    from lora_normal_form_amd import scute
    from lora_normal_form_amd import workload as glue
    wl = _small("bf16", ALL_METHODS, [0, 1, 2], seed=7)
    ld = glue.load(wl, device=0)
    b0 = ld.layer.plan(np.zeros(0, np.int32))
    ld.layer.forward(b0, ld.x, ld.W, ld.y)          # n = 0: nothing to do
    with pytest.raises(scute.ScuteError) as e:
        scute.scute_layer_forward(ld.layer.h, ld.batch.h, ld.x.data_ptr() + 2, ld.W, ld.y)
    assert e.value.code == scute.E_INVALID
    ld.layer.unload(2)
    with pytest.raises(scute.ScuteError) as e:
        ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    assert e.value.code == scute.E_STATE
    torch.cuda.synchronize()


def test_plan_freed_after_its_layer():
    # the plan records its device: freeing it after the layer touches no
    # freed layer memory and leaves no HIP error behind for the next launch
    _need_gpu()
    from lora_normal_form_amd import workload as glue
    wl = _small("bf16", ALL_METHODS, [0, 1, 2], seed=8)
    ld = glue.load(wl, device=0)
    ld.layer.close()
    ld.batch.close()
    t = torch.zeros(1024, device="cuda:0")
    t.fill_(1.0)
    torch.cuda.synchronize()
    assert float(t.sum()) == 1024.0


def test_trace_logs_one_line_per_forward():
    # SCUTE_TRACE=1 (read once per process): the path, shape and launch count
    # of every forward on stderr; run in a child process so the setting is
    # fresh
    _need_gpu()
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import torch\nfrom synth import make_config\nfrom lora_normal_form_amd import workload as glue\n"
            "wl = make_config(0)\nld = glue.load(wl, device=0)\n"
            "for _ in range(2):\n    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)\n"
            "torch.cuda.synchronize()\n")
    env = dict(os.environ, SCUTE_TRACE="1", PYTHONPATH=root)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("scute: forward")]
    assert len(lines) == 2, r.stderr[-2000:]
    assert "path=generic" in lines[0] and "n=16" in lines[0] and "status=0" in lines[0]
