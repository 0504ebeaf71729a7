"""Host checks of the multi-projection layers: the fused q / k / v adapter
assembled from the per-projection folds has, slice by slice, exactly the
weight change of each projection's own adapter."""

import numpy as np
import pytest

from synth import AdapterSpec

from lora_normal_form_amd import convert, multiproj, scute
from lora_normal_form_amd import workload as glue

L, Dr, I3 = AdapterSpec("lora", rank=4, bias=True), AdapterSpec("dora", rank=3), AdapterSpec("ia3")
TENANTS = [(L, L, L), (Dr, Dr, Dr), (None, I3, I3), (L, None, Dr)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_qkv_adapter_is_the_projections_side_by_side(dtype):
    d_outs = (24, 8, 16)
    wls, tt = multiproj.projection_workloads(TENANTS, 20, 32, d_outs, seed=3, dtype=dtype)
    fused = multiproj.fused_layer(wls, len(TENANTS), device=-1)
    W = np.concatenate([wl.W for wl, _ in wls], 0)
    offs = np.concatenate([[0], np.cumsum(d_outs)])
    for t in range(len(TENANTS)):
        sl = convert.slots(fused, t, 32, sum(d_outs))
        dM = convert.weight_change(sl, W)
        for p, (wl, ids) in enumerate(wls):
            blockp = dM[:, offs[p]:offs[p + 1]]
            if t not in ids:
                assert not np.any(blockp)
                continue
            h = glue.load(wl, device=-1, plan=False)
            want = convert.weight_change(convert.slots(h.layer, ids[t], wl.d_in, wl.d_out), wl.W)
            assert np.allclose(blockp, want, rtol=0, atol=1e-12 + 1e-6 * np.abs(want).max()), (t, p)
            h.layer.close()
        b = sl["b"] if sl["b"] is not None else np.zeros(sum(d_outs))
        for p, (wl, ids) in enumerate(wls):
            want_b = np.zeros(d_outs[p])
            if t in ids and wl.adapters[ids[t]].b is not None:
                want_b = wl.adapters[ids[t]].b
            assert np.allclose(b[offs[p]:offs[p + 1]], want_b, atol=1e-6)
    fused.close()


def test_fused_qkv_keeps_a_rotation_per_projection():
    """OFT tenants: the fused adapter holds each projection's own rotation
    (the identity where the tenant does not rotate), and its other slots are
    the projections' side by side."""
    O = AdapterSpec("oft", blk=8)
    ten = [(O, O, O), (O, None, L), (L, O, I3)]
    d_outs = (64, 64, 128)
    wls, _ = multiproj.projection_workloads(ten, 6, 32, d_outs, seed=4, dtype="f32")
    fused = multiproj.fused_layer(wls, len(ten), device=-1)
    offs = np.concatenate([[0], np.cumsum(d_outs)])
    for t, per in enumerate(ten):
        P = fused.read_slot(t, scute.SLOT_P, (3, 4, 8, 8), np.float32).astype(np.float64)
        for p, (wl, ids) in enumerate(wls):
            if per[p] is not None and per[p].method == "oft":
                h = glue.load(wl, device=-1, plan=False)
                want = convert.slots(h.layer, ids[t], wl.d_in, wl.d_out)["R_minus_I"]
                h.layer.close()
            else:
                want = np.zeros((4, 8, 8))
            assert np.allclose(P[p], want, rtol=0, atol=1e-6), (t, p)
        # b and s side by side, as without rotations
        info = fused.info(t)
        if info["has_s"]:
            s_f = fused.read_slot(t, scute.SLOT_S, (sum(d_outs),), np.float32)
            for p, (wl, ids) in enumerate(wls):
                if per[p] is not None and per[p].method == "ia3":
                    assert np.allclose(s_f[offs[p]:offs[p + 1]], wl.adapters[ids[t]].l, atol=1e-6)
    fused.close()
    # projections must end on multiples of 64 when a tenant rotates
    wls, _ = multiproj.projection_workloads([(O, O, O)], 4, 32, (48, 16, 64), seed=6, dtype="f32")
    with pytest.raises(ValueError):
        multiproj.fused_layer(wls, 1, device=-1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_qkv_vera_pairs_side_by_side(dtype):
    """VeRA tenants: the fused layer's shared pair is the projections' pairs
    side by side (A_sh stacked, B_sh block diagonal), and each tenant's fused
    adapter has, slice by slice, exactly the weight change of each
    projection's own adapter over that projection's pair."""
    V = AdapterSpec("vera")
    ten = [(V, V, V), (V, None, L), (I3, V, None), (L, L, L)]
    d_outs = (24, 8, 16)
    wls, _ = multiproj.projection_workloads(ten, 20, 32, d_outs, seed=7, dtype=dtype, vera_rank=4)
    fused = multiproj.fused_layer(wls, len(ten), device=-1)
    A_f, B_f, ranks = multiproj.fused_vera_pair(wls)
    assert ranks == [4, 4, 4] and A_f.shape == (12, 32) and B_f.shape == (48, 12)
    W = np.concatenate([wl.W for wl, _ in wls], 0)
    offs = np.concatenate([[0], np.cumsum(d_outs)])
    for t in range(len(ten)):
        dM = convert.weight_change(convert.slots(fused, t, 32, sum(d_outs), sum(ranks)), W, A_f, B_f)
        for p, (wl, ids) in enumerate(wls):
            blockp = dM[:, offs[p]:offs[p + 1]]
            if t not in ids:
                assert not np.any(blockp)
                continue
            h = glue.load(wl, device=-1, plan=False)
            want = convert.weight_change(convert.slots(h.layer, ids[t], wl.d_in, wl.d_out, wl.vera_rank), wl.W,
                                         wl.A_sh, wl.B_sh)
            h.layer.close()
            assert np.allclose(blockp, want, rtol=0, atol=1e-12 + 1e-6 * np.abs(want).max()), (t, p)
    fused.close()
