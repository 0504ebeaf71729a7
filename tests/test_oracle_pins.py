"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test would fail on a plausible mistake in the oracle: a dropped term, a
wrong sign or index, a transposed operand, a slot applied on the wrong side.

  * closed form: the 2x2 Cayley block (tests/golden/cayley_2x2.txt)
  * invariants: orthogonality and det of OFT blocks, DoRA's column lengths
  * identity reductions: unused slots hold the identity ("The big picture")
  * fold identities ("Which slots can be merged at load?")
  * the (IA)^3 reorder through the FFN gate ("The big picture")
  * two evaluators: method definitions vs the normal form (exactness claim)
  * brute force: scalar loops over buffer indices on tiny non-square shapes
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import layer as L
from synth import AdapterSpec, WorkloadSpec, make_config, make_workload

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# --------------------------------------------------------------------------
# OFT rotation
# --------------------------------------------------------------------------

def test_cayley_2x2_closed_form():
    rows = np.loadtxt(os.path.join(HERE, "golden", "cayley_2x2.txt"), comments="#")
    for q, r00, r01, r10, r11 in rows:
        R = oracle.cayley(np.array([[0.0, q], [-q, 0.0]]))
        np.testing.assert_allclose(R, [[r00, r01], [r10, r11]], atol=1e-15)


@pytest.mark.parametrize("blk", [2, 4, 32, 64])
def test_cayley_orthogonal_det_one_norm_preserving(blk):
    rng = np.random.default_rng(blk)
    for sigma in (0.01, 0.3):
        A = rng.normal(0.0, sigma, size=(blk, blk))
        Q = np.triu(A, 1) - np.triu(A, 1).T
        R = oracle.cayley(Q)
        assert np.max(np.abs(R.T @ R - np.eye(blk))) <= 1e-13
        assert abs(np.linalg.det(R) - 1.0) <= 1e-12
        v = rng.normal(size=blk)
        assert abs(np.linalg.norm(v @ R) - np.linalg.norm(v)) <= 1e-13 * np.linalg.norm(v)


def test_cayley_direction_first_order():
    # R = (I+Q)(I-Q)^-1 = I + 2Q + O(Q^2): the convention, not its transpose
    Q = np.array([[0.0, 1e-6], [-1e-6, 0.0]])
    R = oracle.cayley(Q)
    np.testing.assert_allclose(R - np.eye(2), 2 * Q, atol=1e-11)


def test_oft_rotation_block_placement():
    rng = np.random.default_rng(3)
    Qb = np.stack([np.triu(m, 1) - np.triu(m, 1).T for m in rng.normal(size=(3, 4, 4))])
    R = oracle.oft_rotation(Qb)
    assert R.shape == (12, 12)
    for kb in range(3):
        np.testing.assert_allclose(R[4 * kb:4 * kb + 4, 4 * kb:4 * kb + 4], oracle.cayley(Qb[kb]))
    mask = np.kron(np.eye(3), np.ones((4, 4)))
    assert np.all(R[mask == 0] == 0.0)


# --------------------------------------------------------------------------
# DoRA
# --------------------------------------------------------------------------

def test_dora_columns_have_length_m():
    rng = np.random.default_rng(5)
    Wf = rng.normal(size=(7, 5))
    Af, Bf = rng.normal(size=(7, 2)), rng.normal(size=(2, 5))
    m = rng.uniform(0.5, 2.0, size=5)
    WD = oracle.dora_weight(Wf, Af, Bf, 1.7, m)
    np.testing.assert_allclose(np.sqrt(np.sum(WD * WD, axis=0)), m, rtol=1e-14)
    # each column is parallel to the column of W + cAB
    Wp = Wf + 1.7 * Af @ Bf
    for j in range(5):
        cosv = WD[:, j] @ Wp[:, j] / (np.linalg.norm(WD[:, j]) * np.linalg.norm(Wp[:, j]))
        assert abs(cosv - 1.0) <= 1e-14


# --------------------------------------------------------------------------
# identity reductions: an unused slot holds the identity
# --------------------------------------------------------------------------

def _tiny(adapters, n=9, d_in=16, d_out=12, vera_rank=4, seed=11, dtype="f32"):
    ta = [i % len(adapters) for i in range(n)]
    return make_workload(WorkloadSpec("tiny", dtype, d_in, d_out, n, adapters,
                                      vera_rank=vera_rank, assign="explicit",
                                      token_adapter=ta, seed=seed))


def test_dora_with_m_equal_colnorm_is_lora():
    wl = _tiny([AdapterSpec("dora", rank=3, c=2.0)])
    a = wl.adapters[0]
    Wp = wl.W.T + a.c * a.A.T @ a.B.T
    a.m = np.sqrt(np.sum(Wp * Wp, axis=0))
    y = oracle.forward(wl)
    a.method = "lora"
    np.testing.assert_allclose(y, oracle.forward(wl), rtol=0, atol=1e-12)


def test_ia3_with_unit_l_is_base():
    wl = _tiny([AdapterSpec("ia3")])
    wl.adapters[0].l = np.ones(wl.d_out)
    np.testing.assert_allclose(oracle.forward(wl), wl.x @ wl.W.T, atol=1e-13)


def test_vera_with_unit_vectors_is_lora_on_shared_pair():
    wl = _tiny([AdapterSpec("vera")])
    a = wl.adapters[0]
    a.vd, a.ve = np.ones(wl.vera_rank), np.ones(wl.d_out)
    y = oracle.forward(wl)
    a.method, a.A, a.B, a.c = "lora", wl.A_sh, wl.B_sh, 1.0
    np.testing.assert_allclose(y, oracle.forward(wl), atol=1e-13)


def test_oft_with_zero_q_is_base():
    wl = _tiny([AdapterSpec("oft", blk=4)])
    wl.adapters[0].Q = np.zeros_like(wl.adapters[0].Q)
    np.testing.assert_allclose(oracle.forward(wl), wl.x @ wl.W.T, atol=1e-13)


def test_lora_with_zero_b_is_base():
    wl = _tiny([AdapterSpec("lora", rank=3)])
    wl.adapters[0].B = np.zeros_like(wl.adapters[0].B)
    np.testing.assert_allclose(oracle.forward(wl), wl.x @ wl.W.T, atol=1e-13)


def test_unassigned_tokens_take_base_path():
    wl = _tiny([AdapterSpec("lora", rank=3)])
    wl.token_adapter[:] = -1
    np.testing.assert_allclose(oracle.forward(wl), wl.x @ wl.W.T, atol=0)


def test_each_method_changes_output():
    # guards against a slot silently dropped: every method has a nonzero effect
    wl = make_config(0)
    y, h = oracle.forward(wl), wl.x @ wl.W.T
    for a in wl.adapters:
        rows = wl.token_adapter == a.id
        assert np.max(np.abs(y[rows] - h[rows])) > 1e-3 * np.max(np.abs(h[rows])), a.method


# --------------------------------------------------------------------------
# fold identities and the normal form
# --------------------------------------------------------------------------

def test_fold_identity_d_into_A_and_e_into_B():
    rng = np.random.default_rng(7)
    x, A, B = rng.normal(size=(5, 9)), rng.normal(size=(9, 3)), rng.normal(size=(3, 6))
    d, e, c = rng.normal(size=3), rng.normal(size=6), 1.3
    lhs = c * (((x @ A) * d) @ B) * e
    rhs = x @ (c * A @ np.diag(d)) @ (B @ np.diag(e))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)
    sl = {"R": None, "s": None, "b": None,
          "terms": [dict(A=A, B=B, c=c, d=d, e=e, shared=False)]}
    fl = L.fold_slots(sl)
    assert fl["terms"][0]["d"] is None and fl["terms"][0]["e"] is None
    np.testing.assert_allclose(L.normal_form_output(x, np.zeros((9, 6)), fl), lhs, rtol=1e-12)


def test_fold_keeps_shared_vera_slots_live():
    wl = _tiny([AdapterSpec("vera")])
    sl = L.fold_slots(L.nf_slots(wl, wl.adapters[0]))
    t = sl["terms"][0]
    assert t["A"] is not None and np.array_equal(t["A"], wl.A_sh.T)
    assert np.array_equal(t["B"], wl.B_sh.T)
    np.testing.assert_array_equal(t["d"], wl.adapters[0].vd)


@pytest.mark.parametrize("cfg", [0])
def test_method_definitions_equal_normal_form(cfg):
    wl = make_config(cfg)
    y_def = oracle.forward(wl)
    y_nf = oracle.forward_normal_form(wl, fold=False)
    y_fold = oracle.forward_normal_form(wl, fold=True)
    assert rel(y_nf, y_def) <= 1e-12
    assert rel(y_fold, y_def) <= 1e-12


def test_method_definitions_equal_normal_form_random_shapes():
    for seed in range(4):
        rng = np.random.default_rng(seed)
        d_in = int(rng.choice([8, 12, 24]))
        d_out = int(rng.choice([5, 8, 20]))
        ads = [AdapterSpec("lora", rank=2, bias=True), AdapterSpec("dora", rank=3),
               AdapterSpec("ia3", bias=True), AdapterSpec("vera"),
               AdapterSpec("oft", blk=4), AdapterSpec("oft", blk=2, bias=True),
               AdapterSpec("nf", rank=2, blk=4, nf_R=True, nf_s=True, nf_b=True,
                           nf_term=True, nf_vera=True)]
        wl = make_workload(WorkloadSpec("r", "f32", d_in, d_out, 30, ads, vera_rank=3,
                                        assign="uniform", seed=seed))
        y_def = oracle.forward(wl)
        assert rel(oracle.forward_normal_form(wl), y_def) <= 1e-12
        assert rel(oracle.forward_normal_form(wl, fold=True), y_def) <= 1e-12


def test_ia3_reorder_through_gate():
    # sigma(x W_g) (.) (x W_u) (.) l  ==  sigma(x W_g) (.) ((x W_u) (.) l):
    # the oracle's (IA)^3 output, fed through a gate, equals scaling the gated
    # activation by l. A version scaling the input by l (x (.) l) W would fail.
    wl = _tiny([AdapterSpec("ia3")], d_in=12, d_out=12)
    rng = np.random.default_rng(2)
    Wg = rng.normal(size=(12, 12))
    gate = 1.0 / (1.0 + np.exp(-(wl.x @ Wg)))
    up = oracle.forward(wl)
    lhs = gate * (wl.x @ wl.W.T) * wl.adapters[0].l[None, :]
    np.testing.assert_allclose(gate * up, lhs, rtol=1e-13)
    wrong = gate * ((wl.x * wl.adapters[0].l[None, :]) @ wl.W.T)
    assert rel(wrong, lhs) > 1e-3


# --------------------------------------------------------------------------
# brute force: scalar loops on buffer indices, tiny non-square shapes
# --------------------------------------------------------------------------

def _solve_py(M, Rhs):
    """Gauss-Jordan with partial pivoting on Python lists: returns M^-1 Rhs."""
    n = len(M)
    a = [list(map(float, M[i])) + list(map(float, Rhs[i])) for i in range(n)]
    for col in range(n):
        piv = max(range(col, n), key=lambda r: abs(a[r][col]))
        a[col], a[piv] = a[piv], a[col]
        p = a[col][col]
        a[col] = [v / p for v in a[col]]
        for r in range(n):
            if r != col and a[r][col] != 0.0:
                f = a[r][col]
                a[r] = [v - f * w for v, w in zip(a[r], a[col])]
    return [row[n:] for row in a]


def _brute_force(wl):
    n, d_in, d_out = wl.n, wl.d_in, wl.d_out
    x, W = wl.x.tolist(), wl.W.tolist()          # W[j][i]: output j, input i
    Ash = wl.A_sh.tolist() if wl.A_sh is not None else None   # [k][i]
    Bsh = wl.B_sh.tolist() if wl.B_sh is not None else None   # [j][k]
    ads = wl.adapter_by_id()
    out = []
    for t in range(n):
        xt = x[t]
        aid = int(wl.token_adapter[t])
        a = ads.get(aid)
        b = [0.0] * d_out if a is None or a.b is None else list(a.b)
        h = [sum(xt[i] * W[j][i] for i in range(d_in)) for j in range(d_out)]
        if a is None:
            out.append(h)
            continue
        m_ = a.method
        if m_ == "lora":
            r = a.rank
            u = [sum(xt[i] * a.A[k][i] for i in range(d_in)) for k in range(r)]
            y = [h[j] + b[j] + a.c * sum(u[k] * a.B[j][k] for k in range(r)) for j in range(d_out)]
        elif m_ == "dora":
            r = a.rank
            y = []
            for j in range(d_out):
                col = [W[j][i] + a.c * sum(a.B[j][k] * a.A[k][i] for k in range(r))
                       for i in range(d_in)]
                norm = math.sqrt(sum(v * v for v in col))
                y.append(sum(xt[i] * col[i] for i in range(d_in)) * a.m[j] / norm + b[j])
        elif m_ == "ia3":
            y = [h[j] * a.l[j] + b[j] for j in range(d_out)]
        elif m_ == "vera":
            rv = len(Ash)
            u = [sum(xt[i] * Ash[k][i] for i in range(d_in)) * a.vd[k] for k in range(rv)]
            y = [h[j] + b[j] + a.ve[j] * sum(u[k] * Bsh[j][k] for k in range(rv))
                 for j in range(d_out)]
        elif m_ in ("oft", "nf"):
            blk = a.blk
            xr = list(xt)
            if m_ == "oft" or a.R is not None:
                xr = [0.0] * d_in
                for kb in range(d_in // blk):
                    if m_ == "oft":
                        Q = a.Q[kb]
                        Im = [[(1.0 if p == q else 0.0) - Q[p][q] for q in range(blk)] for p in range(blk)]
                        Ip = [[(1.0 if p == q else 0.0) + Q[p][q] for q in range(blk)] for p in range(blk)]
                        R = _solve_py(Im, Ip)
                    else:
                        R = a.R[kb]
                    for jj in range(blk):
                        xr[kb * blk + jj] = sum(xt[kb * blk + ii] * R[ii][jj] for ii in range(blk))
            y = [sum(xr[i] * W[j][i] for i in range(d_in)) for j in range(d_out)]
            if m_ == "nf":
                if a.s is not None:
                    y = [y[j] * a.s[j] for j in range(d_out)]
                if a.A is not None:
                    r = a.rank
                    u = [sum(xt[i] * a.A[k][i] for i in range(d_in)) * a.d[k] for k in range(r)]
                    y = [y[j] + a.c * sum(u[k] * a.B[j][k] for k in range(r)) * a.e[j]
                         for j in range(d_out)]
                if a.vd is not None:
                    rv = len(Ash)
                    u = [sum(xt[i] * Ash[k][i] for i in range(d_in)) * a.vd[k] for k in range(rv)]
                    y = [y[j] + a.ve[j] * sum(u[k] * Bsh[j][k] for k in range(rv))
                         for j in range(d_out)]
            y = [y[j] + b[j] for j in range(d_out)]
        else:
            raise AssertionError(m_)
        out.append(y)
    return np.array(out)


def _brute_workload(seed, sigma_scale=1.0):
    ads = [AdapterSpec("lora", rank=2, c=2.0, bias=True), AdapterSpec("dora", rank=2, c=2.0),
           AdapterSpec("ia3"), AdapterSpec("vera", bias=True), AdapterSpec("oft", blk=4),
           AdapterSpec("nf", rank=2, blk=4, c=0.7, nf_R=True, nf_s=True, nf_b=True,
                       nf_term=True, nf_vera=True)]
    ta = [0, 1, 2, 3, 4, 5, -1, 5, 3, 0, 4]
    return make_workload(WorkloadSpec("bf", "f32", 8, 6, len(ta), ads, vera_rank=3,
                                      assign="explicit", token_adapter=ta, seed=seed,
                                      sigma_q=0.3 * sigma_scale, sigma_l=0.3,
                                      sigma_m=0.3, sigma_vd=0.5, sigma_ve=0.5))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    wl = _brute_workload(seed)
    y_bf = _brute_force(wl)
    assert rel(oracle.forward(wl), y_bf) <= 1e-12
    assert rel(oracle.forward_normal_form(wl, fold=True), y_bf) <= 1e-12


def test_brute_force_catches_planted_mistakes():
    # the pins are sharp: small planted errors in method parameters move the
    # output far beyond the 1e-12 agreement bound
    wl = _brute_workload(0)
    y_bf = _brute_force(wl)
    for mutate in (lambda a: setattr(a, "c", a.c * 1.001),
                   lambda a: setattr(a, "B", a.B * 1.001)):
        wl2 = _brute_workload(0)
        mutate(wl2.adapters[0])
        assert rel(oracle.forward(wl2), y_bf) > 1e-6
    wl3 = _brute_workload(0)
    wl3.adapters[4].Q = -wl3.adapters[4].Q     # transposed rotation R^T
    assert rel(oracle.forward(wl3), y_bf) > 1e-4


# --------------------------------------------------------------------------
# the comparison criteria
# --------------------------------------------------------------------------

def test_effect_error_hand_example():
    ref = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    base = np.array([[0.0, 2.0], [3.0, 3.0], [5.0, 6.0]])
    y = np.array([[1.1, 2.0], [3.0, 4.0], [5.0, 6.5]])
    e = oracle.effect_errors(y, ref, base, np.array([0, 0, -1]))
    assert e == {0: pytest.approx(0.1 / 2.0)}
    ok, err, scale = oracle.max_error_ok(y, ref, 0.1)
    assert ok and err == pytest.approx(0.5) and scale == 6.0


def _grid(n=4, d=5):
    # a reference with max |ref| = 10 exactly (one entry), base = ref minus a
    # known per-row effect
    ref = np.full((n, d), 2.0)
    ref[0, 0] = 10.0
    base = ref.copy()
    base[:, 1] -= 1.0          # every row's effect: 1.0 in column 1, so sum = d-independent
    return ref, base


def test_check_fp32_threshold_is_1e4_of_max():
    ref, base = _grid()
    ta = np.array([0, 0, 1, 1])
    y = ref.copy()
    y[2, 3] += 1.5e-3          # 1.5e-4 * max|ref| (=10): fails the fp32 bar
    ok, rep = oracle.check(y, ref, base, ta, "f32")
    assert not ok and rep["tol"] == 1e-4 and rep["max_abs_ref"] == 10.0
    y[2, 3] = ref[2, 3] + 0.9e-3   # 0.9e-4 * max: passes
    ok, _ = oracle.check(y, ref, base, ta, "f32")
    assert ok
    y[2, 3] = ref[2, 3] + 1.0e-3   # exactly at the bar: passes (<=)
    ok, _ = oracle.check(y, ref, base, ta, "f32")
    assert ok


def test_check_bf16_max_error_threshold_is_1e2_of_max():
    ref, base = _grid()
    ta = np.array([-1, -1, -1, -1])    # no adapters: only the max criterion grades
    y = ref.copy()
    y[1, 4] += 0.09            # 0.9e-2 * max: passes
    ok, rep = oracle.check(y, ref, base, ta, "bf16")
    assert ok and rep["tol"] == 1e-2
    y[1, 4] = ref[1, 4] + 0.11     # 1.1e-2 * max: fails
    ok, _ = oracle.check(y, ref, base, ta, "bf16")
    assert not ok


def test_check_bf16_effect_threshold_is_one_percent():
    ref, base = _grid()
    ta = np.array([0, 0, 1, 1])
    # adapter 1's effect is sum |ref - base| over rows 2, 3 = 2.0; an absolute
    # error of 0.022 there is 1.1% of it (far below the max-error bar of 0.1)
    y = ref.copy()
    y[3, 2] += 0.022
    ok, rep = oracle.check(y, ref, base, ta, "bf16")
    assert rep["max_ok"] and not rep["effect_ok"] and not ok
    assert rep["worst_effect_err"] == pytest.approx(0.011)
    y[3, 2] = ref[3, 2] + 0.018    # 0.9% of its effect: passes
    ok, rep = oracle.check(y, ref, base, ta, "bf16")
    assert ok and rep["worst_effect_err"] == pytest.approx(0.009)


def test_check_zero_effect_adapter_is_reported_not_graded():
    # adapter 2 changes nothing (ref == base on its rows): its effect error
    # is undefined, so it is reported and left to the max-error criterion
    ref, base = _grid()
    base[3] = ref[3]
    ta = np.array([0, 0, 1, 2])
    y = ref.copy()
    y[3, 0] += 0.05            # inside the 1e-2 * max bar
    e = oracle.effect_errors(y, ref, base, ta)
    assert np.isnan(e[2]) and e[0] == 0.0 and e[1] == 0.0
    ok, rep = oracle.check(y, ref, base, ta, "bf16")
    assert ok and rep["zero_effect_adapters"] == [2] and rep["worst_effect_err"] == 0.0
    y[3, 0] = ref[3, 0] + 0.2  # beyond the max-error bar: fails through that criterion
    ok, rep = oracle.check(y, ref, base, ta, "bf16")
    assert not ok and not rep["max_ok"]
