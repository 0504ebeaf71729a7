"""Host logic of libscute.so, without a GPU (host-only layers, device = -1).

  * the library loads and exports every function include/scute.h declares
  * the load-time fold matches the oracle's fold (fp64 then one rounding)
  * the planner: stable sort, row classes, segments, unassigned rows last
  * the cost model: hand-computed bytes / FLOPs, the pages' time-model example
  * error paths return their status and leave the layer usable
"""

import os
import re

import numpy as np
import pytest

import oracle
from oracle import layer as OL
from synth import AdapterSpec, WorkloadSpec, make_config, make_workload, round_bf16

from lora_normal_form_amd import costmodel, scute
from lora_normal_form_amd import workload as glue

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "scute.h")).read()
    declared = set(re.findall(r"\b(scute_[a-z_]+)\s*\(", hdr))
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(scute.lib, name), name
        assert name in scute.SIGNATURES, name


def test_version():
    assert "gfx950" in scute.scute_version()


# --------------------------------------------------------------------------
# fold
# --------------------------------------------------------------------------

def _rounding_tol(ref, dtype):
    # one rounding of an fp64 value to the storage type, plus fp64 noise
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    return ulp * np.abs(ref) + 1e-12 * (np.max(np.abs(ref)) + 1e-300)


def _check_stored(got, ref, dtype):
    assert got.shape == ref.shape
    assert np.all(np.abs(got - ref) <= _rounding_tol(ref, dtype)), np.max(np.abs(got - ref))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fold_matches_oracle_fold(dtype):
    ads = [AdapterSpec("lora", rank=3, c=2.0, bias=True), AdapterSpec("dora", rank=4, c=2.0),
           AdapterSpec("ia3"), AdapterSpec("vera"), AdapterSpec("oft", blk=8),
           AdapterSpec("nf", rank=2, blk=4, c=0.5, nf_R=True, nf_s=True, nf_b=True,
                       nf_term=True, nf_vera=True)]
    wl = make_workload(WorkloadSpec("fold", dtype, 32, 24, 12, ads, vera_rank=5, seed=4,
                                    sigma_q=0.2))
    ld = glue.load(wl, device=-1)
    L = ld.layer
    sdt = "bf16" if dtype == "bf16" else np.float32
    for a in wl.adapters:
        fl = OL.fold_slots(OL.nf_slots(wl, a))
        info = L.info(a.id)
        assert info["loaded"] == 1
        own = [t for t in fl["terms"] if not t["shared"]]
        shared = [t for t in fl["terms"] if t["shared"]]
        assert info["has_term"] == bool(own) and info["has_vera"] == bool(shared)
        assert info["has_R"] == (fl["R"] is not None)
        assert info["has_s"] == (fl["s"] is not None)
        assert info["has_b"] == (fl["b"] is not None)
        if own:
            t = own[0]
            r = t["A"].shape[1]
            # A' stored [rank8][d_in] = (c A diag d)^T ; B' stored [d_out][rank8] = (B diag e)^T,
            # rank8 = r rounded up to 8 with zero padding
            r8 = -(-r // 8) * 8
            assert info["rank"] == r8
            Ap = L.read_slot(a.id, scute.SLOT_A, (r8, wl.d_in), sdt)
            Bp = L.read_slot(a.id, scute.SLOT_B, (wl.d_out, r8), sdt)
            _check_stored(Ap[:r], t["A"].T, dtype)
            _check_stored(Bp[:, :r], t["B"].T, dtype)
            assert not np.any(Ap[r:]) and not np.any(Bp[:, r:])
        if fl["s"] is not None:
            _check_stored(L.read_slot(a.id, scute.SLOT_S, (wl.d_out,), np.float32), fl["s"], "f32")
        if fl["b"] is not None:
            _check_stored(L.read_slot(a.id, scute.SLOT_BIAS, (wl.d_out,), np.float32), fl["b"],
                          "f32")
        if shared:
            t = shared[0]
            _check_stored(L.read_slot(a.id, scute.SLOT_VD, (wl.vera_rank,), np.float32), t["d"],
                          "f32")
            _check_stored(L.read_slot(a.id, scute.SLOT_VE, (wl.d_out,), np.float32), t["e"], "f32")
        if fl["R"] is not None:
            blk = a.blk
            P = L.read_slot(a.id, scute.SLOT_P, (wl.d_in // blk, blk, blk), sdt)
            for kb in range(wl.d_in // blk):
                blkR = fl["R"][kb * blk:(kb + 1) * blk, kb * blk:(kb + 1) * blk]
                _check_stored(P[kb], blkR - np.eye(blk), dtype)


def test_dora_fold_lengths_and_e_equals_s():
    wl = make_workload(WorkloadSpec("d", "f32", 64, 40, 4, [AdapterSpec("dora", rank=4)],
                                    seed=9, sigma_m=0.3))
    ld = glue.load(wl, device=-1)
    a = wl.adapters[0]
    s = ld.layer.read_slot(0, scute.SLOT_S, (wl.d_out,), np.float32)
    WD = oracle.dora_weight(wl.W.T, a.A.T, a.B.T, a.c, a.m)
    # s = m / colnorm(W + cAB): the folded base path W diag(s) plus the folded
    # low-rank path reproduces W_D, whose column lengths are m
    r8 = -(-a.rank // 8) * 8  # stored rank (zero-padded to a multiple of 8)
    Bp = ld.layer.read_slot(0, scute.SLOT_B, (wl.d_out, r8), np.float32)
    Ap = ld.layer.read_slot(0, scute.SLOT_A, (r8, wl.d_in), np.float32)
    WD_lib = wl.W.T * s[None, :] + Ap.T @ Bp.T
    np.testing.assert_allclose(WD_lib, WD, rtol=0, atol=2e-6 * np.max(np.abs(WD)))
    np.testing.assert_allclose(np.sqrt(np.sum(WD_lib ** 2, axis=0)), a.m, rtol=2e-6)


def test_oft_fold_p_is_cayley_minus_identity():
    wl = make_workload(WorkloadSpec("o", "f32", 64, 8, 2, [AdapterSpec("oft", blk=16)], seed=2,
                                    sigma_q=0.3))
    ld = glue.load(wl, device=-1)
    P = ld.layer.read_slot(0, scute.SLOT_P, (4, 16, 16), np.float32)
    for kb in range(4):
        R = P[kb] + np.eye(16)
        assert np.max(np.abs(R.T @ R - np.eye(16))) < 1e-6
        np.testing.assert_allclose(R, oracle.cayley(wl.adapters[0].Q[kb]), atol=1e-7)


# --------------------------------------------------------------------------
# planner
# --------------------------------------------------------------------------

def _mixed(n=40, seed=5, none_frac=0.2):
    ads = [AdapterSpec("lora", rank=2), AdapterSpec("oft", blk=4), AdapterSpec("vera"),
           AdapterSpec("ia3"), AdapterSpec("dora", rank=2), AdapterSpec("oft", blk=8),
           AdapterSpec("vera")]
    rng = np.random.default_rng(seed)
    ta = rng.integers(0, len(ads), size=n)
    ta[rng.random(n) < none_frac] = -1
    return make_workload(WorkloadSpec("p", "f32", 16, 8, n, ads, vera_rank=3, assign="explicit",
                                      token_adapter=ta, seed=seed))


def test_plan_stable_sort_and_classes():
    wl = _mixed()
    ld = glue.load(wl, device=-1)
    perm, seg = ld.batch.read()
    ta = wl.token_adapter
    assert sorted(perm.tolist()) == list(range(wl.n))          # a permutation
    meth = {a.id: a.method for a in wl.adapters}
    cls = [3 if ta[t] < 0 else (0 if meth[ta[t]] == "oft" else 1 if meth[ta[t]] == "vera" else 2)
           for t in perm]
    keys = [(c, ta[t] if ta[t] >= 0 else 0, t) for c, t in zip(cls, perm)]
    assert keys == sorted(keys)                                 # stable by (class, id)
    info = ld.batch.info()
    assert info["n_rot_rows"] == sum(1 for c in cls if c == 0)
    assert info["n_vera_rows"] == sum(1 for c in cls if c == 1)
    # segments: maximal runs of one adapter covering every adapted row once
    covered = []
    for a, start, ln in seg:
        assert ln >= 1
        assert all(ta[perm[p]] == a for p in range(start, start + ln))
        covered.extend(range(start, start + ln))
    assert covered == [p for p in range(wl.n) if ta[perm[p]] >= 0]
    for (a0, s0, l0), (a1, s1, l1) in zip(seg[:-1], seg[1:]):
        assert a0 != a1 or s0 + l0 != s1
    assert info["max_rank"] == 8  # stored ranks are padded to a multiple of 8


def test_plan_empty_and_all_unassigned():
    wl = _mixed(n=6, none_frac=1.0)
    ld = glue.load(wl, device=-1)
    assert ld.batch.info()["n_segments"] == 0
    b0 = ld.layer.plan(np.zeros(0, np.int32))
    assert b0.info()["n"] == 0
    assert ld.layer.cost(b0)["bytes"] == 0.0


def test_plan_c1_segments_are_the_composition():
    wl = make_config(1)
    ld = glue.load(wl, device=-1)
    perm, seg = ld.batch.read()
    np.testing.assert_array_equal(perm, np.arange(128))
    np.testing.assert_array_equal(seg[:, 0], np.arange(64))
    np.testing.assert_array_equal(seg[:, 2], np.bincount(wl.token_adapter, minlength=64))


# --------------------------------------------------------------------------
# cost model
# --------------------------------------------------------------------------

def test_cost_model_c1_hand_count():
    wl = make_config(1)
    ld = glue.load(wl, device=-1)
    c = ld.layer.cost(ld.batch)
    W = 4096 * 4096 * 2
    adapters = 64 * (16 * 4096 * 2 + 4096 * 16 * 2)
    x, y = 128 * 4096 * 2, 128 * 4096 * 4
    assert c["bytes"] == W + adapters + x + y == 53_477_376
    assert c["adapter_bytes"] == adapters
    assert c["flops"] == 2 * 128 * 4096 * 4096 + 128 * 2 * (4096 * 16 + 16 * 4096)
    assert c["n_touched"] == 64 and c["n_segments"] == 64


def test_cost_model_counts_shared_vera_once_and_touched_only():
    ads = [AdapterSpec("vera"), AdapterSpec("vera"), AdapterSpec("lora", rank=4)]
    wl = make_workload(WorkloadSpec("v", "bf16", 64, 32, 6, ads, vera_rank=8, assign="explicit",
                                    token_adapter=[0, 1, 0, 1, -1, 0], seed=1))
    ld = glue.load(wl, device=-1)
    c = ld.layer.cost(ld.batch)
    vera_vec = 8 * 4 + 32 * 4                     # d fp32 + e fp32 per touched adapter
    shared = 8 * (64 + 32) * 2                    # A_sh + B_sh bf16, once
    assert c["adapter_bytes"] == 2 * vera_vec + shared   # the LoRA adapter has no token
    assert c["n_vera_rows"] == 5 and c["n_touched"] == 2


def test_time_model_example_from_the_pages():
    # 1.34 GB of adapter bytes at 680 GB/s copy bandwidth is about 1.97 ms
    t = costmodel.added_time(1.34e9, 680e9)
    assert abs(t - 1.97e-3) < 0.005e-3
    assert costmodel.added_time(0.0, 1.0, 3, 0.96e-6) == pytest.approx(2.88e-6)


# --------------------------------------------------------------------------
# error paths
# --------------------------------------------------------------------------

def _err(fn, *args, **kw):
    with pytest.raises(scute.ScuteError) as e:
        fn(*args, **kw)
    return e.value.code


def test_error_paths_leave_layer_usable():
    L = scute.Layer(32, 16, "f32", max_adapters=4, device=-1)
    A, B = np.ones((2, 32)), np.ones((16, 2))
    assert _err(scute.scute_layer_create, -1, 33, 16, scute.F32, 4) == scute.E_SHAPE
    assert _err(scute.scute_layer_create, -1, 32, 16, 7, 4) == scute.E_INVALID
    assert _err(L.load, 9, "lora", rank=2, A=A, B=B) == scute.E_INVALID        # id range
    assert _err(L.load, 0, "lora", rank=0, A=A, B=B) == scute.E_SHAPE          # rank 0
    assert _err(L.load, 0, "lora", rank=2, A=A) == scute.E_INVALID             # missing B
    assert _err(L.load, 0, "dora", rank=2, A=A, B=B, m=np.ones(16)) == scute.E_INVALID  # no W
    assert _err(L.load, 0, "oft", blk=5, Q=np.zeros((6, 5, 5))) == scute.E_SHAPE  # blk | d_in
    assert _err(L.load, 0, "vera", vd=np.ones(3), ve=np.ones(16)) == scute.E_STATE  # no pair
    L.load(0, "lora", rank=2, A=A, B=B)
    assert _err(L.load, 0, "ia3", l=np.ones(16)) == scute.E_STATE              # occupied
    assert _err(L.plan, [0, 1]) == scute.E_STATE                               # 1 not loaded
    assert _err(L.plan, [0, 7]) == scute.E_INVALID                             # out of range
    b = L.plan([0, -1, 0])
    L.load(1, "ia3", l=np.ones(16))
    assert _err(L.cost, b) == scute.E_STATE                                    # stale plan
    assert _err(L.forward, b, 16, 16, 16) == scute.E_STATE
    b2 = L.plan([1, 0])
    assert _err(L.forward, b2, 16, 16, 16) == scute.E_UNSUPPORTED              # host-only
    assert b2.wait_failures() == 0                                             # no fused path
    assert _err(scute.scute_batch_wait_failures, 0) == scute.E_INVALID
    L2 = scute.Layer(32, 16, "f32", max_adapters=4, device=-1)
    assert _err(scute.scute_cost_model, L2.h, b2.h) == scute.E_STATE           # other layer
    assert _err(L.unload, 3) == scute.E_STATE
    L.unload(1)
    assert L.info(1)["loaded"] == 0
    L.load(1, "ia3", l=np.ones(16))                                            # still usable
    assert L.info(1)["loaded"] == 1 and L.info(1)["has_s"] == 1
    assert _err(L.read_slot, 1, scute.SLOT_A, (2, 32), np.float32) == scute.E_STATE
    assert _err(scute.scute_read_slot, L.h, 1, scute.SLOT_S, 3) == scute.E_SHAPE
    assert _err(scute.scute_set_vera_shared, L.h, 16, 32, 0) == scute.E_SHAPE
    assert _err(scute.scute_set_vera_shared, L.h, 17, 32, 3) == scute.E_INVALID  # misaligned


def test_plan_outlives_its_layer():
    # a plan may be freed after its layer (finalisers of objects caught in a
    # reference cycle run in any order); a layer created afterwards, possibly
    # at the same address, rejects the old plan instead of using it
    for _ in range(8):
        L1 = scute.Layer(32, 16, "f32", max_adapters=2, device=-1)
        L1.load(0, "lora", rank=2, A=np.ones((2, 32)), B=np.ones((16, 2)))
        b = L1.plan([0, -1, 0])
        L1.close()
        L2 = scute.Layer(32, 16, "f32", max_adapters=2, device=-1)
        L2.load(0, "lora", rank=2, A=np.ones((2, 32)), B=np.ones((16, 2)))
        assert _err(scute.scute_cost_model, L2.h, b.h) == scute.E_STATE
        b.close()
        assert L2.cost(L2.plan([0, 0]))["bytes"] > 0
        L2.close()


def test_plan_flags_are_validated():
    # unknown bits, SEPARATE_S without EXPAND_PASS and DETERMINISTIC with a
    # route bit are refused; route variants need a device layer
    wl = make_config(0)
    ld = glue.load(wl, device=-1, plan=False)
    ta = wl.token_adapter
    bad = [(1 << 9, scute.E_INVALID),
           (scute.PLAN_ROUTE_SEPARATE_S, scute.E_INVALID),
           (scute.PLAN_DETERMINISTIC | scute.PLAN_ROUTE_VERA_PASS, scute.E_INVALID),
           (scute.PLAN_ROUTE_ROTATE_PASS, scute.E_UNSUPPORTED)]
    for flags, code in bad:
        with pytest.raises(scute.ScuteError) as ei:
            ld.layer.plan(ta, flags=flags)
        assert ei.value.code == code, (flags, ei.value)
    b = ld.layer.plan(ta, flags=scute.PLAN_DETERMINISTIC)  # host plan: fine
    b.close()


def test_route_extra_bytes_by_hand():
    # 128 rows of 4096 fp32 outputs: one pass over y is 2 x 128 x 16 KB
    row = 4 * 4096
    b, l = costmodel.route_extra("expand_pass", n=128, d_out=4096, exp_rows=100, vera_rows=20)
    assert (b, l) == (2 * row * 120, 2)
    b, l = costmodel.route_extra("expand_pass", n=128, d_out=4096, exp_rows=0, vera_rows=20)
    assert (b, l) == (2 * row * 20, 1)
    # copy: 40 rows read s, all 128 rows write S; multiply: y, S read and y
    # written for 128 rows; 5 chunks no longer read s in the expand
    b, l = costmodel.route_extra("separate_s", n=128, d_out=4096, s_rows=40, s_chunks=5)
    assert (b, l) == (row * (40 + 128 + 3 * 128 - 5), 2)
    assert costmodel.route_extra("vera_pass", n=128, d_out=4096, vera_rows=0) == (0.0, 0)
    assert costmodel.route_extra("rotate_pass", n=128, d_out=4096, rot_rows=26) == (0.0, 1)
    with pytest.raises(ValueError):
        costmodel.route_extra("nope", n=1, d_out=1)


def test_sanitizer_build_instruments_host_code_only():
    # every -fsanitize= of the sanitized build follows -Xarch_host, so hipcc
    # instruments only the host side (no sanitized device code)
    from lora_normal_form_amd import build as B
    for flags in (B.SAN_FLAGS,):
        for i, f in enumerate(flags):
            if f.startswith("-fsanitize") or f.startswith("-fno-sanitize"):
                assert i > 0 and flags[i - 1] == "-Xarch_host", flags
    assert B.LIB_SAN != B.LIB and B.BUILD_SAN != B.BUILD


# --------------------------------------------------------------------------
# projections: one rotation per output column range
# --------------------------------------------------------------------------

def _rot_blocks(rng, nb, blk):
    out = []
    for _ in range(nb):
        q = rng.normal(0.0, 0.3, size=(blk, blk))
        out.append(oracle.cayley(q - q.T))
    return np.stack(out)


def test_projections_state_and_per_projection_fold():
    rng = np.random.default_rng(21)
    L = scute.Layer(32, 192, "f32", max_adapters=4, device=-1)
    R0, R2 = _rot_blocks(rng, 4, 8), _rot_blocks(rng, 4, 8)
    s = rng.normal(1.0, 0.1, size=192)
    # no projections yet
    assert _err(L.load_proj, 0, [R0, None, R2], 8, s=s) == scute.E_STATE
    # ends: increasing, all but the last multiples of 64, the last d_out, at most 4
    assert _err(L.set_projections, [100, 192]) == scute.E_SHAPE
    assert _err(L.set_projections, [128, 64, 192]) == scute.E_SHAPE
    assert _err(L.set_projections, [64, 128]) == scute.E_SHAPE
    assert _err(L.set_projections, [64, 128, 192, 192]) == scute.E_SHAPE
    assert _err(L.set_projections, [64] * 5) == scute.E_SHAPE
    L.set_projections([64, 128, 192])
    # only normal-form descriptors without their own R, whole blocks
    desc, keep = scute.make_desc("lora", 2, 8, 1.0, A=np.ones((2, 32)), B=np.ones((192, 2)))
    assert _err(scute.scute_load_adapter_proj, L.h, 0, desc, [R0, None, R2]) == scute.E_INVALID
    desc, keep = scute.make_desc("nf", 0, 8, 1.0, R=R0)
    assert _err(scute.scute_load_adapter_proj, L.h, 0, desc, [R0, None, R2]) == scute.E_INVALID
    assert _err(L.load_proj, 0, [R0, None, R2], 5) == scute.E_SHAPE
    del keep
    L.load_proj(0, [R0, None, R2], 8, s=s)
    L.load(1, "lora", rank=2, A=np.ones((2, 32)), B=np.ones((192, 2)))
    info = L.info(0)
    assert info["has_R"] == 1 and info["has_s"] == 1 and info["blk"] == 8
    P = L.read_slot(0, scute.SLOT_P, (3, 4, 8, 8), np.float32)
    for pj, R in enumerate([R0, None, R2]):
        want = np.zeros((4, 8, 8)) if R is None else R - np.eye(8)[None]
        _check_stored(P[pj].astype(np.float64), want, "f32")
    # projections change only while no adapter is loaded
    assert _err(L.set_projections, [128, 192]) == scute.E_STATE
    # cost: x R_p for each of the three projections
    b = L.plan([0, 1, 0, -1])
    c = L.cost(b)
    assert c["n_rot_rows"] == 2
    base = 2.0 * 4 * 32 * 192
    r = L.info(1)["rank"]  # (stored rank, padded at load)
    lora = 2.0 * (32 * r + r * 192)
    assert np.isclose(c["flops"], base + lora + 2 * 3 * 2.0 * 32 * 8)
    L.unload(0)
    L.unload(1)
    L.set_projections([192])  # one projection again
    assert _err(L.load_proj, 0, [R0], 8) == scute.E_STATE
