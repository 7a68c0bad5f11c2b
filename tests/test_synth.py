"""The seeded input generator: determinism, shapes and the workload arithmetic."""
import numpy as np

import synth


def test_workload_derived_sizes():
    w = synth.WORKLOADS["tiny"]
    assert (w.n_clusters, w.n_retrieve, w.group) == (256, 6, 4)
    w = synth.WORKLOADS["llama128k"]
    assert (w.n_segments, w.clusters_per_segment, w.n_clusters, w.n_retrieve) == (16, 512, 8192, 148)
    assert synth.WORKLOADS["llama1m"].n_retrieve == 1180
    assert synth.WORKLOADS["llama122k_b8"].n_clusters == 7680
    assert synth.WORKLOADS["llama122k_b8"].n_retrieve == 139
    assert synth.WORKLOADS["qwen256k"].group == 7


def test_generation_is_deterministic_and_shaped():
    w = synth.WORKLOADS["tiny"].with_(context=512, segment_size=512, steps=3)
    a = synth.generate_layer(w, 0, threads=3)
    b = synth.generate_layer(w, 0, threads=1)
    assert a.k.shape == (1, 8, 515, 128) and a.q.shape == (3, 1, 32, 128)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v) and np.array_equal(a.q, b.q)
    c = synth.generate_layer(w, 1)
    assert not np.array_equal(a.k, c.k)
    kf = synth.bf16_bits_to_f32(a.k)
    assert np.all(np.isfinite(kf)) and 0.5 < kf.std() < 2.0


def test_bf16_helpers_round_trip():
    x = np.array([1.0, -2.5, 3.140625, 0.0], dtype=np.float32)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), x)
    # round to nearest even at the tie 1 + 2^-8
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], dtype=np.float32)
    assert synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(t)).tolist() == [1.0, 1 + 2 ** -6]
