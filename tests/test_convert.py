"""The LoRA-conversion baseline (lora_normal_form_amd.convert): the weight
change it reads off the loaded slots is pinned against the oracle's adapter
effect, and its truncation against the SVD's own properties (exactness at
full rank, the Eckart-Young error)."""

import numpy as np
import pytest

import oracle
from synth import AdapterSpec, WorkloadSpec, make_workload

from lora_normal_form_amd import convert
from lora_normal_form_amd import workload as glue

ADS = [AdapterSpec("lora", rank=3, c=2.0, bias=True), AdapterSpec("dora", rank=4, c=2.0),
       AdapterSpec("ia3"), AdapterSpec("vera", bias=True), AdapterSpec("oft", blk=8),
       AdapterSpec("nf", rank=2, blk=4, c=0.5, nf_R=True, nf_s=True, nf_b=True, nf_term=True,
                   nf_vera=True)]


def _wl():
    ta = np.arange(24) % len(ADS)
    return make_workload(WorkloadSpec("conv", "f32", 32, 24, len(ta), ADS, vera_rank=5,
                                      assign="explicit", token_adapter=ta, seed=8, sigma_q=0.2,
                                      sigma_l=0.3, sigma_m=0.3, sigma_vd=0.3, sigma_ve=0.3))


def test_weight_change_matches_oracle_effect():
    # every method: x dM (+ b) equals the oracle's output minus the base x W^T
    wl = _wl()
    ld = glue.load(wl, device=-1, plan=False)
    ref = oracle.forward(wl)
    base = wl.x @ wl.W.T
    for a in wl.adapters:
        sl = convert.slots(ld.layer, a.id, wl.d_in, wl.d_out, wl.vera_rank)
        dM = convert.weight_change(sl, wl.W, wl.A_sh, wl.B_sh)
        rows = np.where(wl.token_adapter == a.id)[0]
        b = sl["b"] if sl["b"] is not None else 0.0
        got = wl.x[rows] @ dM + b
        want = ref[rows] - base[rows]
        assert np.max(np.abs(got - want)) <= 1e-5 * np.max(np.abs(ref)), a.method


def test_lora_at_full_rank_is_exact():
    wl = _wl()
    ld = glue.load(wl, device=-1, plan=False)
    for a in wl.adapters:
        sl = convert.slots(ld.layer, a.id, wl.d_in, wl.d_out, wl.vera_rank)
        A, B, _, err = convert.to_lora(sl, wl.W, wl.A_sh, wl.B_sh, rank=min(wl.d_in, wl.d_out))
        assert A.shape[1] == wl.d_in and B.shape[0] == wl.d_out and A.shape[0] == B.shape[1]
        assert err < 1e-10, (a.method, err)
        dM = convert.weight_change(sl, wl.W, wl.A_sh, wl.B_sh)
        assert np.allclose(A.T @ B.T, dM, atol=1e-10 * max(1.0, np.abs(dM).max()))


def test_truncation_error_is_the_eckart_young_tail():
    # rank-r error^2 = sum of the discarded squared singular values
    rng = np.random.default_rng(3)
    M = rng.standard_normal((60, 40)) @ np.diag(0.8 ** np.arange(40)) @ rng.standard_normal((40, 50))
    sv = np.linalg.svd(M, compute_uv=False)
    for r in (1, 5, 17):
        US, V = convert.truncated_svd(M, r)
        err = np.linalg.norm(M - US @ V.T)
        assert err == pytest.approx(np.sqrt(np.sum(sv[r:] ** 2)), rel=1e-9)
        # the factors are U_r S_r and V_r: orthogonal columns, norms = singular values
        assert np.allclose(V.T @ V, np.eye(r), atol=1e-10)
        assert np.allclose(np.linalg.norm(US, axis=0), sv[:r], rtol=1e-9)


def test_randomized_truncation_is_near_optimal():
    # above the exact-SVD size the randomized range finder is used; on a
    # matrix with a decaying spectrum it reaches the optimal error closely,
    # and a matrix of rank <= r + oversample comes out exact
    rng = np.random.default_rng(4)
    n = 1600
    U, _ = np.linalg.qr(rng.standard_normal((n, 200)))
    V, _ = np.linalg.qr(rng.standard_normal((n, 200)))
    sv = 0.9 ** np.arange(200)
    M = (U * sv) @ V.T
    US, Vr = convert.truncated_svd(M, 64)
    opt = np.sqrt(np.sum(sv[64:] ** 2))
    assert np.linalg.norm(M - US @ Vr.T) <= 1.01 * opt
    low = (U[:, :70] * sv[:70]) @ V[:, :70].T
    US, Vr = convert.truncated_svd(low, 64)
    assert np.linalg.norm(low - US @ Vr.T) == pytest.approx(np.sqrt(np.sum(sv[64:70] ** 2)), rel=1e-6)


def test_factored_svd_matches_dense():
    rng = np.random.default_rng(5)
    P, Q = rng.standard_normal((50, 7)), rng.standard_normal((40, 7))
    US, V = convert.factored_svd(P, Q, 7)
    assert np.allclose(US @ V.T, P @ Q.T, atol=1e-10)
    US3, V3 = convert.factored_svd(P, Q, 3)
    sv = np.linalg.svd(P @ Q.T, compute_uv=False)
    assert np.linalg.norm(P @ Q.T - US3 @ V3.T) == pytest.approx(np.sqrt(np.sum(sv[3:] ** 2)), rel=1e-9)
