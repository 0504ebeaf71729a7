"""GPU parity of the multi-projection layers against the fp64 oracle, bf16
bars (max|y - ref| <= 1e-2 max|ref|; effect error <= 1% per adapter):
q / k / v fused over the stacked weights and split into three layers (with
OFT and VeRA tenants), and the FFN's gated up projection
h = silu(x W_g^T) (.) y_up with (IA)^3's l on the up projection's s."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from synth import AdapterSpec, WorkloadSpec, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu

L, Dr, I3 = AdapterSpec("lora", rank=16, bias=True), AdapterSpec("dora", rank=16), AdapterSpec("ia3")
O, V = AdapterSpec("oft", blk=32), AdapterSpec("vera")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(wl, y):
    ref = oracle.forward(wl)
    y = y.cpu().numpy().astype(np.float64)
    ok, rep = oracle.check(y, ref, wl.x @ wl.W.T, wl.token_adapter, wl.dtype)
    print(f"[gpu] {wl.name}: {rep}", flush=True)
    assert ok, rep
    return y


def test_qkv_fused_and_split_match_oracle():
    _need_gpu()
    from lora_normal_form_amd import multiproj
    ten = [(L, L, L), (Dr, Dr, Dr), (None, I3, I3), (L, None, Dr)] * 2
    wls, tt = multiproj.projection_workloads(ten, 100, 512, (512, 128, 256), seed=91, none_frac=0.1)
    print("\n[gpu] qkv fused", flush=True)
    fu = multiproj.QKVFused(wls, tt, len(ten))
    yf = fu.forward()
    torch.cuda.synchronize()
    assert fu.batch.info()["path"] == 1
    print("[gpu] qkv split", flush=True)
    sp = multiproj.QKVSplit(wls)
    ys = sp.forward()
    torch.cuda.synchronize()
    for (wl, _), a, b in zip(wls, yf, ys):
        fa = _check(wl, a)
        fb = _check(wl, b)
        assert np.max(np.abs(fa - fb)) <= 1e-2 * np.max(np.abs(fb))
    fu.close()
    sp.close()


@pytest.mark.parametrize("n, path", [(90, 1), (300, 2)])
def test_qkv_split_and_fused_with_rotation_and_vera(n, path):
    """OFT and VeRA tenants: the split layers, and the fused layer with a
    rotation per projection and the projections' VeRA pairs side by side
    (decode path at 90 rows, prefill path at 300), against the oracles."""
    _need_gpu()
    from lora_normal_form_amd import multiproj
    ten = [(L, L, L), (O, O, O), (V, V, V), (None, I3, I3), (O, None, L), (V, None, Dr)]
    wls, tt = multiproj.projection_workloads(ten, n, 512, (512, 256, 256), seed=92, vera_rank=64)
    print(f"\n[gpu] qkv split with OFT and VeRA, {n} rows", flush=True)
    sp = multiproj.QKVSplit(wls)
    ys = sp.forward()
    torch.cuda.synchronize()
    for (wl, _), y in zip(wls, ys):
        _check(wl, y)
    sp.close()
    print(f"[gpu] qkv fused with OFT and VeRA, {n} rows", flush=True)
    fu = multiproj.QKVFused(wls, tt, len(ten))
    assert fu.batch.info()["path"] == path
    yf = fu.forward()
    torch.cuda.synchronize()
    for (wl, _), y in zip(wls, yf):
        _check(wl, y)
    fu.close()


def test_gated_up_projection_with_ia3():
    _need_gpu()
    from lora_normal_form_amd import multiproj
    ta = np.random.default_rng(93).integers(-1, 4, size=120)
    up = make_workload(WorkloadSpec("ffn_up", "bf16", 512, 768, len(ta), [I3, I3, L, V], vera_rank=64,
                                    assign="explicit", token_adapter=ta, seed=93))
    Wg = np.random.default_rng(94).normal(0.0, 1.0 / np.sqrt(512), size=up.W.shape)
    print("\n[gpu] gated up projection", flush=True)
    gu = multiproj.GatedUp(up, Wg)
    h = gu.forward()
    torch.cuda.synchronize()
    g_ref = up.x @ Wg.T
    ref = g_ref / (1.0 + np.exp(-g_ref)) * oracle.forward(up)
    got = h.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    print(f"[gpu] gated max err / max|ref| = {err:.2e}", flush=True)
    assert err <= 1e-2
    # (IA)^3's l applied to the up output before the gate equals applying it
    # to the gated product: the reorder the s slot relies on
    gate = g_ref / (1.0 + np.exp(-g_ref))
    rows = np.where(ta == 0)[0]
    l0 = up.adapters[0].l
    base = up.x @ up.W.T
    assert np.allclose(gate[rows] * (base[rows] * l0), (gate[rows] * base[rows]) * l0)
    # silu_gate alone against its definition on awkward lengths
    from lora_normal_form_amd import scute
    for n in (1, 7, 1024 + 3):
        gg = torch.randn(n, device="cuda:0") * 4
        uu = torch.randn(n, device="cuda:0")
        hh = torch.empty_like(uu)
        scute.scute_silu_gate(gg, uu, hh)
        want = (gg.double() * torch.sigmoid(gg.double()) * uu.double()).cpu().numpy()
        assert np.allclose(hh.cpu().numpy(), want, rtol=1e-5, atol=1e-6)
    gu.close()


def test_qkv_fused_keeps_rotations_per_projection():
    """OFT tenants in the fused q / k / v layer: one rotation per projection.
    100 rows run the two-launch decode path (each 64-column tile stages its
    projection's delta rows); 300 rows run the prefill path when the
    projections end on its 256-column tiles, else the generic kernels (one
    delta block per projection). Each against the per-projection oracles and
    the split layers; at 100 rows also the no-allocation forward."""
    _need_gpu()
    from lora_normal_form_amd import multiproj, scute
    ten = [(L, L, L), (O, O, O), (None, I3, I3), (O, None, L), (Dr, O, None)] * 2
    cases = [(100, (512, 128, 256), 1, "decode_main"), (300, (512, 128, 256), 0, "gemm"),
             (300, (512, 256, 256), 2, "prefill_main")]
    for n, d_outs, path, kernel in cases:
        wls, tt = multiproj.projection_workloads(ten, n, 512, d_outs, seed=95 + n, none_frac=0.1)
        print(f"\n[gpu] qkv fused with OFT tenants, {n} rows, {d_outs}", flush=True)
        fu = multiproj.QKVFused(wls, tt, len(ten))
        assert fu.batch.info()["path"] == path
        scute.scute_profile_enable(fu.layer.h, True)
        yf = fu.forward()
        torch.cuda.synchronize()
        names = set(scute.scute_profile_read(fu.layer.h))
        scute.scute_profile_enable(fu.layer.h, False)
        assert kernel in names and "fd_main" not in names, names
        sp = multiproj.QKVSplit(wls)
        ys = sp.forward()
        torch.cuda.synchronize()
        for (wl, _), a, b in zip(wls, yf, ys):
            fa = _check(wl, a)
            fb = _check(wl, b)
            assert np.max(np.abs(fa - fb)) <= 1e-2 * np.max(np.abs(fb))
        if n == 100:
            # the no-allocation forward (token order, generic kernels, one
            # delta block per projection in its scratch)
            ta = torch.as_tensor(np.asarray(tt, dtype=np.int32), device="cuda:0")
            yn = torch.full_like(fu.y, float("nan"))
            fu.layer.forward_noalloc(ta, fu.x, fu.W, yn)
            torch.cuda.synchronize()
            offs = np.concatenate([[0], np.cumsum(d_outs)])
            for p, (wl, _) in enumerate(wls):
                _check(wl, yn[:, offs[p]:offs[p + 1]])
        sp.close()
        fu.close()


@pytest.mark.parametrize("n, path, kernel", [(128, 1, "decode_main"), (2048, 2, "prefill_main")])
def test_qkv_fused_with_rotations_full_size(n, path, kernel):
    """The q / k / v layer at its real shape, 4096 -> (4096, 1024, 1024), with
    20 tenants of which four rotate (OFT, blocks of 32) on every projection:
    128 decode tokens and 2048 prefill tokens, each projection against its
    oracle."""
    _need_gpu()
    from lora_normal_form_amd import multiproj, scute
    ten = multiproj.qkv_tenants(True)
    wls, tt = multiproj.projection_workloads(ten, n, 4096, (4096, 1024, 1024), seed=12)
    print(f"\n[gpu] qkv fused with OFT tenants, full size, {n} tokens", flush=True)
    fu = multiproj.QKVFused(wls, tt, len(ten))
    assert fu.batch.info()["path"] == path
    scute.scute_profile_enable(fu.layer.h, True)
    yf = fu.forward()
    torch.cuda.synchronize()
    names = set(scute.scute_profile_read(fu.layer.h))
    scute.scute_profile_enable(fu.layer.h, False)
    assert kernel in names, names
    for (wl, _), a in zip(wls, yf):
        _check(wl, a)
    fu.close()


def test_qkv_fused_rotations_deterministic_plan():
    """A deterministic plan of rows that rotate per projection: decode-size
    batches run the generic kernels (no float atomics), so two forwards give
    the same bits, and the output matches the oracles."""
    _need_gpu()
    from lora_normal_form_amd import multiproj, scute
    ten = [(L, L, L), (O, O, O), (None, I3, I3), (O, None, L)]
    wls, tt = multiproj.projection_workloads(ten, 64, 512, (512, 128, 256), seed=96)
    fu = multiproj.QKVFused(wls, tt, len(ten), flags=scute.PLAN_DETERMINISTIC)
    assert fu.batch.info()["path"] == 0
    y1 = [t.clone() for t in fu.forward()]
    y2 = fu.forward()
    torch.cuda.synchronize()
    for (wl, _), a, b in zip(wls, y1, y2):
        assert torch.equal(a, b)
        _check(wl, a)
    fu.close()


def test_four_projections_with_rotations():
    """Four projections (the most a layer takes), each tenant rotating some
    of them: decode path, against each projection's oracle."""
    _need_gpu()
    from lora_normal_form_amd import multiproj
    ten = [(O, O, None, O), (L, O, O, None), (I3, None, L, O), (Dr, Dr, Dr, Dr)]
    d_outs = (256, 128, 64, 192)
    wls, tt = multiproj.projection_workloads(ten, 80, 512, d_outs, seed=97, none_frac=0.1)
    fu = multiproj.QKVFused(wls, tt, len(ten))
    assert fu.layer.h and fu.batch.info()["path"] == 1
    ys = fu.forward()
    torch.cuda.synchronize()
    assert len(ys) == 4
    for (wl, _), y in zip(wls, ys):
        _check(wl, y)
    fu.close()


@pytest.mark.parametrize("n, d_outs, path", [(96, (256, 128, 128), 1), (320, (256, 128, 128), 0),
                                            (320, (256, 256, 256), 2)])
def test_single_and_per_projection_rotations_together(n, d_outs, path):
    """A layer with projections holding an adapter with one rotation per
    projection (scute_load_adapter_proj) and one with a single rotation for
    every column (scute_load_adapter, normal form with R): the single
    rotation serves each projection's delta block. Decode path at 96 rows;
    at 320 the prefill path when the projections end on 256-column tiles,
    else the generic kernels; each projection against the oracle."""
    _need_gpu()
    from synth import Adapter, Workload, round_bf16
    from lora_normal_form_amd import scute
    from lora_normal_form_amd import workload as glue
    rng = np.random.default_rng(98 + n + len(set(d_outs)))
    d_in, blk = 512, 32

    def rotation():
        q = rng.normal(0.0, 0.05, size=(d_in // blk, blk, blk))
        return np.stack([oracle.cayley(qq - qq.T) for qq in q])

    R_proj, R_one = [rotation() for _ in d_outs], rotation()
    x = round_bf16(rng.normal(0.0, 1.0, size=(n, d_in)))
    Ws = [round_bf16(rng.normal(0.0, 1.0 / np.sqrt(d_in), size=(d, d_in))) for d in d_outs]
    ta = rng.integers(-1, 2, size=n)
    L_ = scute.Layer(d_in, sum(d_outs), "bf16", max_adapters=2, device=0)
    L_.set_projections(np.cumsum(d_outs))
    L_.load_proj(0, R_proj, blk)
    L_.load(1, "nf", blk=blk, R=R_one)
    batch = L_.plan(ta)
    assert batch.info()["path"] == path
    dev = torch.device("cuda", 0)
    xd = glue.to_device(x, "bf16", dev)
    Wd = glue.to_device(np.concatenate(Ws, 0), "bf16", dev)
    y = torch.full((n, sum(d_outs)), float("nan"), dtype=torch.float32, device=dev)
    L_.forward(batch, xd, Wd, y)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(d_outs)])
    for p, (d, Wp) in enumerate(zip(d_outs, Ws)):
        wl = Workload(f"rot_mix_p{p}", "bf16", d_in, d, n, x, Wp,
                      [Adapter(0, "nf", blk=blk, R=R_proj[p]), Adapter(1, "nf", blk=blk, R=R_one)],
                      np.asarray(ta, dtype=np.int64))
        _check(wl, y[:, offs[p]:offs[p + 1]])
    batch.close()
    L_.close()
