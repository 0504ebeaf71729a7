"""GPU parity of the MFMA prefill path (bf16, d_in % 64 == 0 (% 256 with a
rotation or a low-rank term), d_out % 256 == 0, batches the decode paths do
not take) against the fp64 oracle, plus agreement with the generic kernels on
the same inputs.

Bars as in test_parity_gpu: max|y - ref| <= 1e-2 max|ref| and every touched
adapter's mean effect error <= 1% of its effect.
"""

import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

PREFILL = 2


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


def _load(wl, **env):
    from lora_normal_form_amd import workload as glue
    with _env(**env):
        print(f"\n[gpu] {wl.name} n={wl.n} d_in={wl.d_in} d_out={wl.d_out} env={env}", flush=True)
        return glue.load(wl, device=0)


def _forward(ld):
    ld.y.fill_(float("nan"))
    ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
    torch.cuda.synchronize()
    return ld.y.cpu().numpy().astype(np.float64)


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


MIX = [AdapterSpec("lora", rank=64, c=2.0, bias=True), AdapterSpec("dora", rank=64),
       AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=64),
       AdapterSpec("lora", rank=8), AdapterSpec("dora", rank=24, bias=True),
       AdapterSpec("oft", blk=32), AdapterSpec("vera", bias=True),
       AdapterSpec("nf", rank=16, blk=16, c=0.5, nf_R=True, nf_s=True, nf_b=True, nf_term=True,
                   nf_vera=True),
       AdapterSpec("nf", rank=40, nf_s=True, nf_term=True),
       AdapterSpec("lora", rank=128)]


def _segments(lengths, ids):
    ta = []
    for ln, a in zip(lengths, ids):
        ta += [a] * ln
    return np.array(ta, dtype=np.int64)


def _wl(name, ta, adapters=MIX, d_out=512, vera_rank=128, seed=0, d_in=4096, **kw):
    return make_workload(WorkloadSpec(name, "bf16", d_in, d_out, len(ta), adapters,
                                      vera_rank=vera_rank, assign="explicit", token_adapter=ta,
                                      seed=seed, **kw))


def test_prefill_ragged_segments():
    # segment lengths around the chunk sizes (64 with rotation, 128 without),
    # every method, ranks over one and several 64-rank pieces, a tail of
    # tokens without an adapter
    _need_gpu()
    lengths = [1, 63, 64, 65, 127, 128, 129, 200, 31, 97, 130, 70, 45]
    ids = [0, 4, 7, 1, 2, 3, 9, 11, 8, 6, 10, 5, -1]
    wl = _wl("prefill_ragged", _segments(lengths, ids), seed=31)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL, ld.batch.info()
    _check(wl, _forward(ld))


def test_prefill_random_order_tokens():
    # tokens drawn uniformly: the kernel gathers every chunk's rows by token
    _need_gpu()
    rng = np.random.default_rng(32)
    ta = rng.integers(-1, len(MIX), size=700)
    wl = _wl("prefill_random", ta, seed=32, d_out=768)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    _check(wl, _forward(ld))


def test_prefill_matches_generic_and_repeats():
    # no atomics on this path: consecutive forwards of one plan agree bit for
    # bit; the generic kernels agree to rounding
    _need_gpu()
    rng = np.random.default_rng(33)
    ta = rng.permutation(_segments([300, 150, 80, 290], [0, 4, 3, 9]))
    wl = _wl("prefill_vs_generic", ta, seed=33, d_out=256)
    ref = oracle.forward(wl)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    y1 = _forward(ld)
    _check(wl, y1, ref)
    for _ in range(3):
        y = _forward(ld)
        np.testing.assert_array_equal(y, y1)
    lg = _load(wl, SCUTE_PREFILL=0)
    assert lg.batch.info()["path"] == 0
    yg = _forward(lg)
    _check(wl, yg, ref)
    assert np.max(np.abs(y1 - yg)) <= 1e-2 * np.max(np.abs(ref))


def test_prefill_only_vera_and_only_unassigned():
    _need_gpu()
    wl = _wl("prefill_vera", _segments([333, 190], [0, 1]),
             adapters=[AdapterSpec("vera"), AdapterSpec("vera", bias=True)], vera_rank=256,
             seed=34, d_out=256)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    _check(wl, _forward(ld))
    wl2 = _wl("prefill_none", np.full(300, -1), seed=35, d_out=256)
    ld2 = _load(wl2)
    assert ld2.batch.info()["path"] == PREFILL
    _check(wl2, _forward(ld2))


def test_prefill_far_from_identity():
    _need_gpu()
    rng = np.random.default_rng(36)
    ta = rng.integers(0, len(MIX), size=400)
    wl = _wl("prefill_far", ta, seed=36, d_out=256, sigma_l=0.3, sigma_m=0.3, sigma_vd=0.3,
             sigma_ve=0.3, sigma_q=0.05)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    _check(wl, _forward(ld))


@pytest.mark.parametrize("parts", [1, 2, 4])
def test_prefill_split_k_parts(parts):
    # tiles left over after the whole-K rounds run as 2 or 4 K parts that add
    # their partial tiles in part order; each plan repeats bit for bit
    _need_gpu()
    rng = np.random.default_rng(37)
    ta = rng.permutation(_segments([600, 300, 260, 300, 100], [0, 4, 3, 9, 2]))
    wl = _wl("prefill_parts", ta, seed=37, d_out=1024)
    ref = oracle.forward(wl)
    ld = _load(wl, SCUTE_PREFILL_PARTS=parts)
    assert ld.batch.info()["path"] == PREFILL
    y = _forward(ld)
    _check(wl, y, ref)
    np.testing.assert_array_equal(_forward(ld), y)


@pytest.mark.parametrize("xscale", [2.0 ** -20, 2.0 ** 12])
def test_prefill_input_scale(xscale):
    # the shrink sums of the K parts are fp32 partial tiles added in part
    # order, so the result holds at any input scale fp32 represents: x
    # scaled by a power of two (exact in bf16), every method, repeat bit for
    # bit
    _need_gpu()
    rng = np.random.default_rng(38)
    ta = rng.permutation(_segments([200, 150, 130, 170, 90, 60], [0, 1, 3, 4, 9, 10]))
    wl = _wl("prefill_scale", ta, seed=38, d_out=256)
    wl.x = wl.x * xscale
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    y = _forward(ld)
    _check(wl, y)
    np.testing.assert_array_equal(_forward(ld), y)


@pytest.mark.parametrize("d_in", [5120, 2304])
def test_prefill_other_input_widths(d_in):
    # the K loop's stage count at run time (80 and 36 stages), K parts of the
    # shrinks with a short last part (5 x 1024; 2 x 1024 + 256), the split
    # into K parts of a tile where the stage count allows it
    _need_gpu()
    rng = np.random.default_rng(d_in)
    ta = rng.integers(-1, len(MIX), size=600)
    wl = _wl(f"prefill_din{d_in}", ta, seed=33, d_in=d_in, d_out=768)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL, ld.batch.info()
    _check(wl, _forward(ld))


def test_prefill_input_width_multiple_of_64_without_prologue():
    # d_in 4160 (65 stages): only slots applied in the epilogue ((IA)^3 s,
    # a b) run on the prefill path; with a low-rank term the batch falls to
    # the generic kernels
    _need_gpu()
    ads = [AdapterSpec("ia3"), AdapterSpec("nf", nf_s=True, nf_b=True)]
    ta = np.random.default_rng(34).integers(-1, 2, size=300)
    wl = _wl("prefill_din4160", ta, adapters=ads, seed=34, d_in=4160, d_out=512)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL, ld.batch.info()
    _check(wl, _forward(ld))
    wl2 = _wl("prefill_din4160_lora", ta, adapters=[AdapterSpec("lora", rank=16)] * 2, seed=35,
              d_in=4160, d_out=512)
    assert _load(wl2).batch.info()["path"] == 0


def test_prefill_ranks_not_multiple_of_8():
    # ranks 4, 12 and 20 run on the MFMA path at the stored rank (rounded
    # up to 8 with zero rows / columns)
    _need_gpu()
    ads = [AdapterSpec("lora", rank=4), AdapterSpec("lora", rank=12, c=2.0),
           AdapterSpec("dora", rank=20), AdapterSpec("nf", rank=12, nf_s=True, nf_term=True)]
    ta = _segments([130, 70, 200, 90, 20], [0, 1, 2, 3, -1])
    wl = _wl("prefill_odd_ranks", ta, adapters=ads, seed=36)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL, ld.batch.info()
    _check(wl, _forward(ld))


def test_prefill_long_batch_sampled_rows():
    # 16384 tokens at 4096 -> 4096 (eight times the prefill workload's
    # batch): every method in ragged segments, tokens in random order. The
    # oracle checks 1024 rows sampled across the batch (each row's output
    # depends only on its own x and adapter).
    _need_gpu()
    rng = np.random.default_rng(41)
    ta = rng.integers(-1, len(MIX), size=16384)
    wl = _wl("prefill_long", ta, seed=41, d_out=4096)
    ld = _load(wl)
    assert ld.batch.info()["path"] == PREFILL
    y = _forward(ld)
    idx = np.sort(rng.choice(wl.n, size=1024, replace=False))
    sub = dataclasses.replace(wl, name="prefill_long_sample", n=len(idx), x=wl.x[idx],
                              token_adapter=wl.token_adapter[idx])
    _check(sub, y[idx])
