"""GPU parity of the decode path's route variants (plan flags
SCUTE_PLAN_ROUTE_*: the expand step, the separate s pass, the VeRA term and
the OFT rotation as passes of their own) against the fp64 oracle and against
the default fused route, at the bf16 bars: max|y - ref| <= 1e-2 max|ref| and
every adapter's mean effect error <= 1% of its effect.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_config, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

E, S, V, R = 2, 4, 8, 16
ROUTES = {"expand_pass": E, "separate_s": E | S, "vera_pass": V, "rotate_pass": R,
          "expand_vera_rotate": E | V | R, "all": E | S | V | R}

MIX32 = [AdapterSpec("lora", rank=16, c=2.0, bias=True), AdapterSpec("dora", rank=16),
         AdapterSpec("ia3"), AdapterSpec("vera", bias=True), AdapterSpec("oft", blk=32),
         AdapterSpec("lora", rank=8), AdapterSpec("dora", rank=72),
         AdapterSpec("nf", rank=16, blk=32, c=0.5, nf_R=True, nf_s=True, nf_b=True, nf_term=True,
                     nf_vera=True)]
MIXB = MIX32[:4] + [AdapterSpec("oft", blk=16), AdapterSpec("oft", blk=64)]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _wl(n, seed, adapters, d_in=512, d_out=384):
    rng = np.random.default_rng(seed)
    ta = rng.integers(0, len(adapters), size=n)
    ta[rng.random(n) < 0.1] = -1
    return make_workload(WorkloadSpec(f"route_n{n}_s{seed}", "bf16", d_in, d_out, n, adapters,
                                      vera_rank=64, assign="explicit", token_adapter=ta, seed=seed))


def _expected_launches(flags, info):
    nl = 2
    if flags & R and info["n_rot_rows"] > 0:
        nl += 1
    if flags & S:
        nl += 2
    if flags & E:
        nl += 1  # every workload here has rows with s, b or an own term
    if flags & (E | V) and info["n_vera_rows"] > 0:
        nl += 1
    return nl


def _run(wl, flags):
    from lora_normal_form_amd import workload as glue
    print(f"\n[gpu] {wl.name} n={wl.n} d_in={wl.d_in} d_out={wl.d_out} flags={flags}", flush=True)
    ld = glue.load(wl, device=0, flags=flags)
    info = ld.batch.info()
    assert info["path"] == 1, info
    if flags:
        assert ld.layer.cost(ld.batch)["launches"] == _expected_launches(flags, info)
    ld.y.fill_(float("nan"))
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    y = ld.y.cpu().numpy().astype(np.float64)
    ld.batch.close()
    ld.layer.close()
    return y


def _check(wl, y, ref):
    assert np.all(np.isfinite(y))
    ok, rep = oracle.check(y, ref, wl.x @ wl.W.T, wl.token_adapter, wl.dtype)
    print(f"[gpu] {rep}", flush=True)
    assert ok, rep


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("case", ["blk32", "mixed_blocks"])
def test_route_matches_oracle_and_default(route, case):
    _need_gpu()
    wl = _wl(77, seed=31, adapters=MIX32) if case == "blk32" else _wl(90, seed=32, adapters=MIXB)
    ref = oracle.forward(wl)
    y = _run(wl, ROUTES[route])
    _check(wl, y, ref)
    y0 = _run(wl, 0)
    assert np.max(np.abs(y - y0)) <= 1e-2 * np.max(np.abs(ref))


@pytest.mark.parametrize("route", ["separate_s", "all"])
@pytest.mark.parametrize("idx", [1, 2])
def test_route_named_workload(route, idx):
    # the all-LoRA and mixed decode workloads at full size
    _need_gpu()
    wl = make_config(idx)
    _check(wl, _run(wl, ROUTES[route]), oracle.forward(wl))


def test_route_refuses_batches_off_the_decode_path():
    _need_gpu()
    from lora_normal_form_amd import scute
    from lora_normal_form_amd import workload as glue
    wl = make_config(0)  # fp32: the generic kernels only
    ld = glue.load(wl, device=0, plan=False)
    with pytest.raises(scute.ScuteError) as ei:
        ld.layer.plan(wl.token_adapter, flags=E)
    assert ei.value.code == scute.E_UNSUPPORTED
    ld.layer.close()
