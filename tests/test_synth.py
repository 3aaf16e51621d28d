"""Seeded input generators: determinism and the stated recipe (no GPU)."""
import numpy as np

import oracle
from mxfp4_block_scaled_02_amd import synth


def test_deterministic_and_seed_dependent():
    a = synth.workload("tiny", 0)
    b = synth.workload("tiny", 0)
    c = synth.workload("tiny", 1)
    assert np.array_equal(a["A"], b["A"]) and np.array_equal(a["B"], b["B"])
    assert not np.array_equal(a["A"], c["A"])
    assert a["A"].shape == (4, 512) and a["B"].shape == (256, 512)
    assert a["A"].dtype == np.uint16


def test_bf16_rounding_matches_oracle_rounding():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * np.exp2(g.integers(-30, 30, 100000))).astype(np.float32)
    assert np.array_equal(synth.f32_to_bf16_bits(x), oracle.f64_to_bf16_bits(x.astype(np.float64)))


def test_distributions():
    w = synth.workload("tiny", 3)
    a = oracle.bf16_bits_to_f64(w["A"])
    b = oracle.bf16_bits_to_f64(w["B"])
    assert abs(a.std() - 1.0) < 0.1
    assert abs(b.std() - 0.02) < 0.002


def test_stress_recipe():
    M, K = 64, 2048
    a = oracle.bf16_bits_to_f64(synth.make_stress_a(M, K, 2))
    groups = a.reshape(-1, 32)
    assert (np.abs(groups).max(1) == 0).sum() == round(0.02 * M * K / 32)
    assert (np.abs(a) > 12).sum() > 0.5 * 0.01 * M * K  # outliers present (x50 of N(0,1))
    b = oracle.bf16_bits_to_f64(synth.make_stress_b(128, K, 2))
    rms = np.sqrt((b ** 2).mean(1))
    assert rms.max() / rms.min() > 2.0 ** 8  # per-row 2^u, u in [-8, 8]


def test_group_sizes():
    for seed in range(5):
        ms = synth.group_sizes(seed)
        assert len(ms) == 8 and all(128 <= m <= 1024 and (m - 128) % 64 == 0 for m in ms)


def test_decode_group_sizes():
    for seed in range(5):
        ms = synth.decode_group_sizes(seed)
        assert len(ms) == 8 and all(8 <= m <= 64 and m % 8 == 0 for m in ms)
    w = synth.workload("grouped_decode", synth.default_seed("grouped_decode"))
    assert w["Ms"] == synth.decode_group_sizes(synth.default_seed("grouped_decode"))
    assert [a.shape for a in w["A"]] == [(m, 7168) for m in w["Ms"]] and all(b.shape == (4096, 7168) for b in w["B"])
    # existing workloads keep their seeds
    assert [synth.default_seed(n) for n in ("tiny", "skinny", "stress", "square", "grouped")] == [0, 1, 2, 3, 4]


def test_shard_is_a_slice_of_its_parent():
    a, b = synth.workload("skinny_shard8", synth.default_seed("skinny_shard8")), synth.workload("skinny", 1)
    assert synth.default_seed("skinny_shard8") == synth.default_seed("skinny")
    assert np.array_equal(a["A"], b["A"]) and np.array_equal(a["B"], b["B"][:264])
