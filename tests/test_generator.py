"""The seeded workload generator: structure, rounding, determinism."""

import numpy as np
import pytest

from synth import (CONFIG_NAMES, AdapterSpec, WorkloadSpec, bf16_bits, config_spec,
                   make_config, make_workload, round_bf16)


def test_round_bf16_known_values():
    # bf16 has 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    # and rounds to even (1.0); 1 + 3*2^-8 is a tie rounding up to 1 + 2^-6
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -3.14159265, 0.0])
    exp = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -3.140625, 0.0])
    np.testing.assert_array_equal(round_bf16(vals), exp)
    bits = bf16_bits(exp)
    assert bits[0] == 0x3F80 and bits[4] == 0xC049


def test_bf16_bits_rejects_unrounded():
    with pytest.raises(ValueError):
        bf16_bits(np.array([1.0 + 2 ** -10]))


def test_c0_structure():
    wl = make_config(0)
    assert (wl.n, wl.d_in, wl.d_out, wl.dtype) == (16, 256, 256, "f32")
    ta = wl.token_adapter
    # contiguous segments in adapter order, four of 3 tokens and one of 4
    assert np.all(np.diff(ta) >= 0)
    counts = np.bincount(ta, minlength=5)
    assert sorted(counts.tolist()) == [3, 3, 3, 3, 4]
    assert [a.method for a in wl.adapters] == ["lora", "dora", "ia3", "vera", "oft"]
    assert wl.A_sh.shape == (32, 256) and wl.B_sh.shape == (256, 32)
    Q = wl.adapters[4].Q
    assert Q.shape == (8, 32, 32)
    np.testing.assert_array_equal(Q, -np.transpose(Q, (0, 2, 1)))
    # fp32 workload: values exactly representable in fp32
    assert np.array_equal(wl.x, wl.x.astype(np.float32).astype(np.float64))


def test_c1_composition_positive_parts():
    wl = make_config(1)
    counts = np.bincount(wl.token_adapter, minlength=64)
    assert counts.sum() == 128 and np.all(counts >= 1)
    assert np.all(np.diff(wl.token_adapter) >= 0)
    assert all(a.rank == 16 and a.method == "lora" for a in wl.adapters)


def test_c2_to_c4_structure():
    s2 = config_spec(2)
    assert [a.method for a in s2.adapters].count("oft") == 8 and s2.vera_rank == 256
    s3 = config_spec(3)
    assert len(s3.adapters) == 2048 and s3.d_out == 14336 and s3.n == 256
    s4 = config_spec(4)
    meths = [a.method for a in s4.adapters]
    assert meths[:5] == ["lora", "dora", "ia3", "vera", "oft"] and len(meths) == 16
    assert meths.count("lora") == 4 and meths.count("oft") == 3


def test_bf16_workload_values_are_bf16():
    ads = [AdapterSpec("lora", rank=4), AdapterSpec("dora", rank=4), AdapterSpec("ia3"),
           AdapterSpec("vera"), AdapterSpec("oft", blk=8)]
    wl = make_workload(WorkloadSpec("t", "bf16", 32, 24, 20, ads, vera_rank=8, seed=3))
    for arr in [wl.x, wl.W, wl.A_sh, wl.B_sh] + [getattr(a, f) for a in wl.adapters
                                                  for f in ("A", "B", "m", "l", "vd", "ve", "Q")
                                                  if getattr(a, f) is not None]:
        bf16_bits(arr)  # raises if not exactly bf16


def test_deterministic_and_seed_sensitive():
    a, b = make_config(0), make_config(0)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.adapters[1].m, b.adapters[1].m)
    c = make_config(0, seed=7)
    assert not np.array_equal(a.x, c.x)


def test_dora_magnitude_near_column_norm():
    wl = make_config(0)
    a = wl.adapters[1]
    Wp = wl.W + a.c * (a.B @ a.A)
    ratio = a.m / np.sqrt(np.sum(Wp * Wp, axis=1))
    assert abs(np.mean(ratio) - 1.0) < 0.02 and 0.02 < np.std(ratio) < 0.08


def test_names():
    assert len(CONFIG_NAMES) == 5


@pytest.mark.parametrize("idx", range(5))
def test_generator_digests_pinned(idx):
    # every array of the five named workloads hashes to its committed digest
    # (tests/golden/generator_sha256.json, written by generator_digests.py)
    import json
    import os
    import sys
    golden = os.path.join(os.path.dirname(__file__), "golden")
    sys.path.insert(0, golden)
    try:
        import generator_digests as gd
    finally:
        sys.path.remove(golden)
    with open(os.path.join(golden, "generator_sha256.json")) as f:
        want = json.load(f)[str(idx)]
    got = gd.digests(idx)
    assert got == want


def test_digest_catches_draw_order_change():
    # swapping two draws (x drawn after W) changes the x digest: the pin is
    # sensitive to draw order, not only to the multiset of values
    import hashlib
    rng = np.random.default_rng(np.random.PCG64(1001))
    x1 = rng.standard_normal(16)
    rng = np.random.default_rng(np.random.PCG64(1001))
    rng.standard_normal(16)
    x2 = rng.standard_normal(16)
    h = lambda a: hashlib.sha256(a.astype("<f8").tobytes()).hexdigest()
    assert h(x1) != h(x2)
