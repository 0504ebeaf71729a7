"""Host checks of the multi-projection layers: the fused q / k / v adapter
assembled from the per-projection folds has, slice by slice, exactly the
weight change of each projection's own adapter."""

import numpy as np
import pytest

from synth import AdapterSpec

from lora_normal_form_amd import convert, multiproj
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


def test_fused_qkv_refuses_rotation():
    O = AdapterSpec("oft", blk=8)
    wls, _ = multiproj.projection_workloads([(O, O, O)], 4, 32, (8, 8, 8), seed=4, dtype="f32")
    with pytest.raises(ValueError):
        multiproj.fused_layer(wls, 1, device=-1)
