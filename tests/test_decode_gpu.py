"""GPU parity of the MFMA decode paths (bf16, up to 256 rows) against the
fp64 oracle, plus agreement with the generic kernels on the same inputs. Every
test runs on both decode paths: the fused single-kernel one (SCUTE_DECODE=1)
and the two-launch one (SCUTE_DECODE=2).

Bars as in test_parity_gpu: max|y - ref| <= 1e-2 max|ref| and every touched
adapter's mean effect error <= 1% of its effect.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class _env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        for k, v in self.kv.items():
            os.environ[k] = str(v)

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.fixture(autouse=True, params=[1, 2], ids=["fused", "two_launch"])
def decode_mode(request):
    with _env(SCUTE_DECODE=request.param):
        yield request.param


def _forward(wl, expect_path=None, **env):
    from lora_normal_form_amd import workload as glue
    with _env(**env):
        print(f"\n[gpu] {wl.name} n={wl.n} d_in={wl.d_in} d_out={wl.d_out} env={env}", flush=True)
        ld = glue.load(wl, device=0)
    info = ld.batch.info()
    if expect_path is not None:
        assert info["path"] == expect_path, info
    ld.y.fill_(float("nan"))
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    return ld, ld.y.cpu().numpy().astype(np.float64)


def _check(wl, y, ref=None):
    ref = oracle.forward(wl) if ref is None else ref
    assert np.all(np.isfinite(y))
    ok, rep = oracle.check(y, ref, wl.x @ wl.W.T, wl.token_adapter, wl.dtype)
    print(f"[gpu] {rep}", flush=True)
    if not ok:
        eff = oracle.effect_errors(y, ref, wl.x @ wl.W.T, wl.token_adapter)
        meth = {a.id: a.method for a in wl.adapters}
        bad = {f"{aid}:{meth[aid]}": round(e, 4) for aid, e in eff.items() if e > 0.01}
        print(f"[gpu] adapters over 1%: {bad}", flush=True)
    assert ok, rep
    return ref


MIX = [AdapterSpec("lora", rank=16, c=2.0, bias=True), AdapterSpec("dora", rank=16),
       AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=32),
       AdapterSpec("lora", rank=8), AdapterSpec("dora", rank=24, bias=True),
       AdapterSpec("oft", blk=64), AdapterSpec("vera", bias=True),
       AdapterSpec("nf", rank=16, blk=16, c=0.5, nf_R=True, nf_s=True, nf_b=True, nf_term=True,
                   nf_vera=True),
       AdapterSpec("nf", rank=8, nf_s=True, nf_term=True),
       AdapterSpec("lora", rank=64)]


def _wl(n, seed, d_in=512, d_out=384, vera_rank=64, none_frac=0.1, adapters=MIX, **kw):
    rng = np.random.default_rng(seed)
    ta = rng.integers(0, len(adapters), size=n)
    ta[rng.random(n) < none_frac] = -1
    return make_workload(WorkloadSpec(f"decode_n{n}_s{seed}", "bf16", d_in, d_out, n, adapters,
                                      vera_rank=vera_rank, assign="explicit", token_adapter=ta,
                                      seed=seed, **kw))


@pytest.mark.parametrize("n", [1, 5, 33, 77, 128, 200, 256])
def test_decode_path_mixed(n, decode_mode):
    # the MFMA paths stage ceil(n / 32) row groups plus one per 32 rotated
    # rows, at most 8 (fused) or 9 (two-launch); larger batches run the
    # generic kernels
    _need_gpu()
    wl = _wl(n, seed=n)
    ld, y = _forward(wl)
    info = ld.batch.info()
    groups = -(-n // 32) + -(-info["n_rot_rows"] // 32)
    assert info["path"] == (1 if groups <= (8 if decode_mode == 1 else 9) else 0), info
    _check(wl, y)


def test_decode_path_256_rows_few_rotated():
    _need_gpu()
    wl = _wl(256, seed=21, adapters=MIX[:4] + MIX[5:7] + MIX[8:9] + MIX[10:])
    _, y = _forward(wl, expect_path=1)
    _check(wl, y)


@pytest.mark.parametrize("splitk", [1, 2])
def test_decode_long_k_slices_with_w_through_lds(splitk):
    # d_in 4096 in one slice (32 stages of 64 k per K half, the loop unrolled
    # at compile time) or two (16 stages, the runtime loop), with at most 5
    # staged row groups, where W passes through each wave's LDS block
    _need_gpu()
    wl = _wl(100, seed=61, d_in=4096, d_out=1024)
    ld, y = _forward(wl, expect_path=1, SCUTE_DECODE_SPLITK=splitk, SCUTE_FD_SPLITK=splitk)
    info = ld.batch.info()
    assert -(-wl.n // 32) + -(-info["n_rot_rows"] // 32) <= 5, info
    _check(wl, y)


@pytest.mark.parametrize("splitk", [1, 2, 4])
def test_decode_path_split_k(splitk):
    # S = 1 stores y directly; S > 1 combines the slices' partial products
    _need_gpu()
    wl = _wl(96, seed=11, d_in=1024)
    _, y = _forward(wl, expect_path=1, SCUTE_DECODE_SPLITK=splitk, SCUTE_FD_SPLITK=splitk)
    _check(wl, y)


@pytest.mark.parametrize("case", ["d_in_8192", "r_v_32", "r_v_96_dense", "r_v_96_steps", "oft_blk4",
                                  "oft_blk8", "oft_blk16"])
def test_decode_edge_shapes(case, decode_mode):
    # the largest d_in the decode paths take (16 pieces per lane in the
    # gather), VeRA pairs whose rank is not a multiple of 64 (dense product
    # forced on and off), and rotation blocks below 32 (the rotation's
    # 8-wide and scalar branches)
    _need_gpu()
    ads = MIX
    kw = dict(d_in=512, d_out=384, vera_rank=64)
    env = {}
    if case == "d_in_8192":
        kw.update(d_in=8192, d_out=512)
    elif case == "r_v_32":
        kw.update(vera_rank=32)
    elif case.startswith("r_v_96"):
        kw.update(vera_rank=96)
        ads = [AdapterSpec("vera"), AdapterSpec("vera", bias=True), AdapterSpec("lora", rank=8),
               AdapterSpec("ia3")]
        env["SCUTE_DECODE_DENSE_VERA"] = 1 if case.endswith("dense") else 0
    else:
        blk = int(case[len("oft_blk"):])
        ads = [AdapterSpec("oft", blk=blk), AdapterSpec("lora", rank=16), AdapterSpec("vera"),
               AdapterSpec("oft", blk=blk, bias=True)]
    wl = _wl(120, seed=400 + len(case), adapters=ads, **kw)
    _, y = _forward(wl, expect_path=1, **env)
    _check(wl, y)


@pytest.mark.parametrize("kind", ["ia3_vera_256", "lora_256", "ia3_vera_128"])
def test_decode_path_choice_when_unset(kind, decode_mode):
    # with SCUTE_DECODE unset the planner takes the fused path for batches of
    # 7 or more staged row groups with no own low-rank term, the two-launch
    # path otherwise; the kernels a forward runs show which
    if decode_mode != 2:
        pytest.skip("one run per case: the choice does not depend on the fixture's mode")
    _need_gpu()
    from lora_normal_form_amd import scute
    n = 128 if kind.endswith("128") else 256
    ads = ([AdapterSpec("ia3"), AdapterSpec("vera")] * 4 if kind.startswith("ia3")
           else [AdapterSpec("lora", rank=16)] * 8)
    wl = _wl(n, seed=500 + n, adapters=ads, none_frac=0.0, d_in=1024, d_out=512)
    saved = os.environ.pop("SCUTE_DECODE", None)
    try:
        from lora_normal_form_amd import workload as glue
        ld = glue.load(wl, device=0)
    finally:
        if saved is not None:
            os.environ["SCUTE_DECODE"] = saved
    assert ld.batch.info()["path"] == 1
    scute.scute_profile_enable(ld.layer.h, True)
    ld.y.fill_(float("nan"))
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    names = set(scute.scute_profile_read(ld.layer.h))
    scute.scute_profile_enable(ld.layer.h, False)
    fused = kind == "ia3_vera_256"
    assert ("fd_main" in names) == fused and ("decode_main" in names) == (not fused), names
    _check(wl, ld.y.cpu().numpy().astype(np.float64))


def test_decode_matches_generic_kernels():
    _need_gpu()
    wl = _wl(150, seed=12)
    ref = oracle.forward(wl)
    _, y_fast = _forward(wl, expect_path=1)
    _, y_gen = _forward(wl, expect_path=0, SCUTE_DECODE=0)
    _check(wl, y_fast, ref)
    _check(wl, y_gen, ref)
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(y_fast - y_gen)) <= 1e-2 * scale


def test_decode_far_from_identity():
    _need_gpu()
    wl = _wl(100, seed=13, sigma_l=0.3, sigma_m=0.3, sigma_vd=0.3, sigma_ve=0.3, sigma_q=0.05)
    _, y = _forward(wl, expect_path=1)
    _check(wl, y)


def test_decode_all_unassigned_and_only_vera():
    _need_gpu()
    wl = _wl(64, seed=14, none_frac=1.0)
    _, y = _forward(wl, expect_path=1)
    _check(wl, y)
    wl2 = _wl(64, seed=15, adapters=[AdapterSpec("vera"), AdapterSpec("vera")], none_frac=0.0)
    _, y2 = _forward(wl2, expect_path=1)
    _check(wl2, y2)


def test_decode_falls_back_when_rows_exceed_lds():
    # 256 rows all rotated need 16 staged row groups (> 10): generic kernels
    _need_gpu()
    wl = _wl(256, seed=16, adapters=[AdapterSpec("oft", blk=32)], none_frac=0.0)
    _, y = _forward(wl, expect_path=0)
    _check(wl, y)


def test_decode_repeated_forwards_reuse_counters():
    # the VeRA shrink's arrival counters return to zero after every forward
    _need_gpu()
    wl = _wl(120, seed=17)
    ref = oracle.forward(wl)
    ld, y0 = _forward(wl, expect_path=1)
    _check(wl, y0, ref)
    for _ in range(3):
        ld.y.fill_(float("nan"))
        ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
        torch.cuda.synchronize()
        _check(wl, ld.y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("shape", [(200, 512, 384, 64), (256, 512, 14336, 256)])
def test_decode_dense_vera_matches_steps(shape):
    # the VeRA term as a dense product over LDS-staged sums (one split of the
    # ranks per K slice; one slice over all 256 ranks for the wide layer)
    # against the same term as expand steps
    _need_gpu()
    n, d_in, d_out, r_v = shape
    ads = [AdapterSpec("vera"), AdapterSpec("ia3"), AdapterSpec("vera", bias=True),
           AdapterSpec("lora", rank=16)]
    wl = _wl(n, seed=41, d_in=d_in, d_out=d_out, vera_rank=r_v, none_frac=0.05, adapters=ads)
    ref = oracle.forward(wl)
    _, yd = _forward(wl, expect_path=1, SCUTE_DECODE_DENSE_VERA=1)
    _check(wl, yd, ref)
    _, ys = _forward(wl, expect_path=1, SCUTE_DECODE_DENSE_VERA=0)
    _check(wl, ys, ref)
    assert np.max(np.abs(yd - ys)) <= 1e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("d_out", [1024, 14336])
def test_decode_many_expand_steps_per_row_group(d_out):
    # every row its own adapter: 40 LoRA and 8 DoRA of rank 64 (4 expand steps
    # of 16 ranks each) and 16 VeRA rows (r_v 256: 16 steps per row group), so
    # a row group's step list in one K slice holds ~70 (two slices, 1024
    # columns) to ~150 (one slice, 14336 columns) steps: several operand
    # batches per wave and, at 14336 columns, a second descriptor window
    _need_gpu()
    ads = ([AdapterSpec("lora", rank=64) for _ in range(40)] +
           [AdapterSpec("dora", rank=64) for _ in range(8)] +
           [AdapterSpec("vera") for _ in range(16)])
    n = 64
    ta = np.arange(n) % len(ads)
    wl = make_workload(WorkloadSpec(f"decode_many_steps_{d_out}", "bf16", 512, d_out, n, ads,
                                    vera_rank=256, assign="explicit", token_adapter=ta, seed=51))
    _, y = _forward(wl, expect_path=1)
    _check(wl, y)


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_deterministic_plan_is_bit_repeatable(idx, decode_mode):
    # a plan built with SCUTE_PLAN_DETERMINISTIC runs the fused decode path
    # (K slices and shrink slices added in a fixed order, no float atomics),
    # whatever path the environment prefers, and gives the same bits on
    # every forward, also after other work ran on the device in between
    _need_gpu()
    from lora_normal_form_amd import workload as glue
    from synth import make_config
    wl = make_config(idx)
    print(f"\n[gpu] deterministic {wl.name}", flush=True)
    ld = glue.load(wl, device=0, deterministic=True)
    assert ld.batch.info()["path"] == 1, ld.batch.info()
    outs = []
    for i in range(4):
        ld.y.fill_(float("nan"))
        ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
        torch.cuda.synchronize()
        outs.append(ld.y.cpu().numpy().copy())
        if i == 1:
            other = glue.load(_wl(64, seed=99), device=0)
            other.layer.forward(other.batch, other.x, other.W, other.y)
            torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    _check(wl, outs[0].astype(np.float64))


def test_decode_ranks_not_multiple_of_8():
    # ranks 4 and 12 (stored at 8 and 16 with zero rows / columns) run on the
    # MFMA decode path
    _need_gpu()
    ads = [AdapterSpec("lora", rank=4), AdapterSpec("lora", rank=12, c=2.0),
           AdapterSpec("dora", rank=12), AdapterSpec("nf", rank=4, nf_s=True, nf_term=True),
           AdapterSpec("vera")]
    wl = _wl(100, seed=71, adapters=ads)
    _, y = _forward(wl, expect_path=1)
    _check(wl, y)


def test_decode_overflow_rows_take_the_prefill_path():
    # 256 rows with 64 rotated rows need 10 staged row groups, more than the
    # decode paths stage: the batch runs on the MFMA prefill path
    _need_gpu()
    n = 256
    ta = np.r_[np.zeros(64, dtype=np.int64), 1 + np.arange(n - 64) % 3]
    ads = [AdapterSpec("oft", blk=32), AdapterSpec("lora", rank=16), AdapterSpec("ia3"),
           AdapterSpec("vera")]
    wl = make_workload(WorkloadSpec("decode_overflow", "bf16", 512, 512, n, ads, vera_rank=64,
                                    assign="explicit", token_adapter=ta, seed=72))
    _, y = _forward(wl, expect_path=2)
    _check(wl, y)


def test_fused_wait_failures_are_reported(decode_mode):
    # the fused path's cross-work-group waits are bounded: a plan whose waits
    # the host makes fail (SCUTE_FD_FORCE_WAIT_FAIL: they look for a forward
    # no arrival reaches and give up after a few polls) reports the failure
    # after its forward, and every wave still finishes; a normal plan of the
    # same batch reports none and matches the oracle
    _need_gpu()
    if decode_mode != 1:
        pytest.skip("only the fused path waits across work-groups")
    wl = make_workload(WorkloadSpec("waits", "bf16", 1024, 1024, 96,
                                    [AdapterSpec("lora", rank=16), AdapterSpec("vera"), AdapterSpec("ia3")],
                                    vera_rank=64, seed=61))
    ld, y = _forward(wl, expect_path=1)
    assert ld.batch.wait_failures() == 0
    _check(wl, y)
    bad, _ = _forward(wl, expect_path=1, SCUTE_FD_FORCE_WAIT_FAIL=1)
    assert bad.batch.wait_failures() == 1
    assert bad.batch.wait_failures(reset=True) == 1
    assert bad.batch.wait_failures() == 0
