"""Pins for the CPU oracle: closed forms, invariants, library routines and a worked example.

Each test names the property it pins and the page passage behind it. None of these compares
the oracle with itself: the expected values come from hand arithmetic, from a library routine
(torch's bf16 conversion, torch's scaled_dot_product_attention in fp64, Python's sort), from
mathematics (Jensen's inequality, spherical k-means monotonicity) or from brute force on
tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import wave_oracle as wo


def bits(x):
    """float values -> bf16 bit patterns via torch's own conversion (round to nearest even)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def vals(b):
    return torch.from_numpy(np.asarray(b, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def sdpa(q_bits, K_bits, V_bits, scale=None):
    """Exact attention by torch's library routine, in fp64 on the CPU."""
    q = torch.from_numpy(vals(q_bits))[None, :, None, :]          # [1, G, 1, d]
    K = torch.from_numpy(vals(K_bits))[None, None].expand(1, q.shape[1], -1, -1)
    V = torch.from_numpy(vals(V_bits))[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=scale)
    return o[0, :, 0].numpy()


def random_case(rng, L0=160, d=16, G=2, steps=3, spread=0.5, n_topics=5):
    """Small keys with topic structure (so clusters are meaningful) and random values."""
    L = L0 + steps
    topics = rng.standard_normal((n_topics, d))
    z = np.repeat(rng.integers(0, n_topics, size=L // 8 + 1), 8)[:L]
    K = bits(topics[z] + spread * rng.standard_normal((L, d)))
    V = bits(rng.standard_normal((L, d)))
    q = bits(rng.standard_normal((G, d)) + topics[rng.integers(0, n_topics)])
    return K, V, q


# ------------------------------------------------------------------------------------------
# bf16 rounding: pinned to torch's conversion (a library routine)
# ------------------------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_values(rng):
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, size=20000),
        # exact halfway cases: a bf16 value plus half a spacing, both parities
        (vals(bits(rng.standard_normal(2000))) *
         (1 + 2.0 ** -8 * np.sign(rng.standard_normal(2000)))),
        np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, 2.0 ** -130, 3.0e38, -3.0e38]),
    ]).astype(np.float32).astype(np.float64)
    assert np.array_equal(wo.round_bf16(x), bits(x))


def test_round_bf16_is_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 lies just above the halfway point between bf16 neighbours 1 and 1+2^-7:
    # a single rounding goes up, while rounding through fp32 first (which drops 2^-30) would
    # land exactly on the tie and go to the even neighbour, 1.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30])
    assert vals(wo.round_bf16(x))[0] == 1 + 2.0 ** -7
    assert vals(wo.round_bf16(np.array([1 + 2.0 ** -8])))[0] == 1.0      # exact tie -> even


# ------------------------------------------------------------------------------------------
# Hand-worked example (d = 4): inputs and every expected value, with the derivation, are in
# tests/golden/hand_worked_d4.json (derived by hand from the method's definitions; the pages
# print no numeric example).
# ------------------------------------------------------------------------------------------

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_d4.json")))
GOLD_K = np.array(GOLD["inputs"]["K"], dtype=np.float64)
GOLD_V = np.array(GOLD["inputs"]["V"], dtype=np.float64)
GX = GOLD["expected"]


def golden_index():
    i = GOLD["inputs"]
    L0 = i["L0"]
    return wo.build_head(bits(GOLD_K), bits(GOLD_V), L0=L0, S=i["S"], k_seg=i["k_seg"],
                         n_iters=i["n_iters"], n_sink=i["n_sink"], n_recent=i["n_recent"])


def test_golden_build():
    idx, K_out, V_out = golden_index()
    assert idx.labels.tolist() == GX["labels"]
    assert idx.size.tolist() == GX["size"]
    assert idx.offset.tolist() == GX["offset"]
    assert idx.perm.tolist() == GX["perm"]
    assert np.array_equal(vals(idx.centroid_mean), GX["centroid_mean"])
    assert np.array_equal(vals(idx.value_sum), GX["value_sum"])
    assert np.array_equal(vals(idx.last_centroids), GX["last_centroids"])
    assert idx.objective[0] == pytest.approx(GX["objective"], rel=1e-13)
    assert np.array_equal(K_out, bits(GOLD_K[GX["perm"]]))
    assert np.array_equal(V_out, bits(GOLD_V[GX["perm"]]))


def test_golden_decode():
    idx, K_out, V_out = golden_index()
    i = GOLD["inputs"]
    L0, dec = i["L0"], i["decode"]
    Kc = np.concatenate([K_out, bits(GOLD_K[L0:])])
    Vc = np.concatenate([V_out, bits(GOLD_V[L0:])])
    q = bits(dec["q"])
    r = wo.decode_group(q, Kc, Vc, idx, L0=L0, L=dec["L"], n_sink=i["n_sink"],
                        n_recent=i["n_recent"], n_retrieve=dec["n_retrieve"])
    assert r.selected.tolist() == GX["selected"]
    assert r.score[0].tolist() == GX["score"]
    assert r.out[0] == pytest.approx(GX["out"], rel=1e-13, abs=1e-13)
    assert r.lse[0] == pytest.approx(GX["lse"], rel=1e-13)
    full, lse_full = wo.full_attention(q, Kc, Vc, dec["L"])
    assert full[0, 0] == pytest.approx(GX["full_out_0"], rel=1e-13)
    assert lse_full[0] == pytest.approx(GX["full_lse"], rel=1e-13)


# ------------------------------------------------------------------------------------------
# Decode pins
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_retrieve_all_equals_full_attention(seed):
    """n_r >= number of non-empty clusters: every token is exact, so the tripartite result is
    plain softmax attention over all L tokens (torch SDPA, fp64)."""
    rng = np.random.default_rng(seed)
    K, V, q = random_case(rng, L0=200, d=16, G=4)
    L0, L = 200, 203
    idx, Ko, Vo = wo.build_head(K, V, L0, S=64, k_seg=8, n_iters=3, n_sink=3, n_recent=7)
    Kc, Vc = np.concatenate([Ko, K[L0:]]), np.concatenate([Vo, V[L0:]])
    r = wo.decode_group(q, Kc, Vc, idx, L0, L, 3, 7, n_retrieve=10 ** 6)
    assert len(r.selected) == int((idx.size > 0).sum())
    np.testing.assert_allclose(r.out, sdpa(q, K[:L], V[:L]), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_r", [0, 1, 5, 40])
def test_singleton_clusters_make_the_estimate_exact(n_r):
    """Cluster size 1 (k_seg = S): each point seeds and keeps its own cluster, its mean key is
    the key itself and its value sum the value, so the estimate is exact for any n_r."""
    rng = np.random.default_rng(7)
    L0, L = 96, 98
    K = bits(rng.standard_normal((L, 8)))
    V = bits(rng.standard_normal((L, 8)))
    q = bits(rng.standard_normal((2, 8)))
    idx, Ko, Vo = wo.build_head(K, V, L0, S=32, k_seg=32, n_iters=2, n_sink=2, n_recent=4)
    nonempty = idx.size > 0
    assert np.all(idx.size[nonempty] == 1) and nonempty.sum() == L0 - 6
    Kc, Vc = np.concatenate([Ko, K[L0:]]), np.concatenate([Vo, V[L0:]])
    r = wo.decode_group(q, Kc, Vc, idx, L0, L, 2, 4, n_retrieve=n_r)
    np.testing.assert_allclose(r.out, sdpa(q, K[:L], V[:L]), rtol=1e-12, atol=1e-12)


def test_clusters_of_identical_keys_make_the_estimate_exact():
    """Jensen's bound is tight when a cluster's member logits are equal (gist.science/zh §2A):
    blocks of identical keys form the clusters, so the estimate equals exact attention."""
    rng = np.random.default_rng(11)
    k_seg, block, d = 6, 5, 8
    dirs = rng.standard_normal((k_seg, d)) * 3
    seg = np.repeat(dirs, block, axis=0)                 # 30 points, 6 blocks of 5 copies
    K = bits(np.concatenate([rng.standard_normal((1, d)), seg, rng.standard_normal((2, d))]))
    # values on a 1/4 grid so that their bf16 sums are exact (value sums are stored in bf16)
    V = bits(rng.integers(-8, 8, size=(33, d)) / 4.0)
    q = bits(rng.standard_normal((3, d)))
    L0 = 33
    idx, Ko, Vo = wo.build_head(K, V, L0, S=64, k_seg=k_seg, n_iters=3, n_sink=1, n_recent=2)
    assert idx.size.tolist() == [block] * k_seg
    for n_r in range(0, k_seg + 1):
        r = wo.decode_group(q, Ko, Vo, idx, L0, L0, 1, 2, n_retrieve=n_r)
        np.testing.assert_allclose(r.out, sdpa(q, K, V), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [4, 5])
def test_jensen_lower_bound_on_the_denominator(seed):
    """Per cluster n_j exp(q.mean/sqrt d) <= sum_i exp(q.k_i/sqrt d) (convexity of exp), so
    the estimated softmax denominator never exceeds the exact one: lse_wave <= lse_full.
    The stored mean is bf16-rounded, which allows a slack of a few bf16 spacings in the logit."""
    rng = np.random.default_rng(seed)
    K, V, q = random_case(rng, L0=256, d=16, G=2, spread=1.0)
    L0, L = 256, 259
    idx, Ko, Vo = wo.build_head(K, V, L0, S=128, k_seg=16, n_iters=3, n_sink=2, n_recent=8)
    Kc, Vc = np.concatenate([Ko, K[L0:]]), np.concatenate([Vo, V[L0:]])
    _, lse_full = wo.full_attention(q, Kc, Vc, L)
    # per-cluster check in fp64 with unrounded means
    Kf, Q = vals(K), vals(q)
    for j in np.nonzero(idx.size)[0]:
        mem = np.nonzero(idx.labels == j)[0]
        mean = Kf[mem].mean(axis=0)
        for h in range(2):
            est = len(mem) * math.exp(Q[h] @ mean / 4.0)
            exact = np.exp(Kf[mem] @ Q[h] / 4.0).sum()
            assert est <= exact * (1 + 1e-12)
    for n_r in [0, 2, 8]:
        r = wo.decode_group(q, Kc, Vc, idx, L0, L, 2, 8, n_retrieve=n_r)
        assert np.all(r.lse <= lse_full + 0.02)


def test_zero_query_gives_the_mean_value():
    """q = 0: every logit is 0, so the result is the plain mean of all L values and
    lse = ln L, whatever the clustering -- this needs the n_j weight of each estimate."""
    rng = np.random.default_rng(3)
    K, _, _ = random_case(rng, L0=150, d=8)
    V = bits(rng.integers(-4, 4, size=(153, 8)) / 4.0)   # bf16 value sums stay exact
    L0, L = 150, 153
    idx, Ko, Vo = wo.build_head(K, V, L0, S=50, k_seg=7, n_iters=2, n_sink=1, n_recent=3)
    Kc, Vc = np.concatenate([Ko, K[L0:]]), np.concatenate([Vo, V[L0:]])
    for n_r in [0, 3]:
        r = wo.decode_group(bits(np.zeros((2, 8))), Kc, Vc, idx, L0, L, 1, 3, n_retrieve=n_r)
        np.testing.assert_allclose(r.out, np.tile(vals(V[:L]).mean(axis=0), (2, 1)),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r.lse, math.log(L), rtol=1e-13)


def test_top_k_is_a_stable_sort_by_score_then_id():
    """Retrieval set = the n_r best group scores, ties to the lower id, empty clusters never
    chosen; checked against Python's sort on (-score, id)."""
    rng = np.random.default_rng(9)
    C = 200
    score = np.round(rng.standard_normal(C), 1)           # many exact ties
    size = rng.integers(0, 3, size=C)
    for n_r in [0, 1, 7, 50, 150, 199, 400]:
        ref = sorted((-score[j], j) for j in range(C) if size[j] > 0)[:n_r]
        got = wo.select_clusters(score, size, n_r)
        assert got.tolist() == sorted(j for _, j in ref)


def test_group_of_one_is_multi_head_attention():
    """G = 1 (MHA): decoding the heads of a GQA group one by one with G = 1 gives the same
    retrieval-free parts; with n_r large both are exact attention per head."""
    rng = np.random.default_rng(21)
    K, V, q = random_case(rng, L0=120, d=8, G=3)
    L0, L = 120, 123
    idx, Ko, Vo = wo.build_head(K, V, L0, S=40, k_seg=5, n_iters=2, n_sink=1, n_recent=2)
    Kc, Vc = np.concatenate([Ko, K[L0:]]), np.concatenate([Vo, V[L0:]])
    grp = wo.decode_group(q, Kc, Vc, idx, L0, L, 1, 2, n_retrieve=4)
    for h in range(3):
        one = wo.decode_group(q[h:h + 1], Kc, Vc, idx, L0, L, 1, 2, n_retrieve=4,
                              selected=grp.selected)
        np.testing.assert_allclose(one.out[0], grp.out[h], rtol=1e-13, atol=1e-14)


def test_batch_elements_are_independent():
    rng = np.random.default_rng(5)
    K1, V1, q1 = random_case(rng, L0=100, d=8, G=2)
    K2, V2, q2 = random_case(rng, L0=100, d=8, G=2)
    K = np.stack([K1, K2])[:, None]
    V = np.stack([V1, V2])[:, None]
    q = np.stack([q1, q2])
    lay = wo.build_layer(K, V, 100, 50, 4, 2, 1, 2)
    Kc = np.concatenate([lay.k_out, K[:, :, 100:]], axis=2)
    Vc = np.concatenate([lay.v_out, V[:, :, 100:]], axis=2)
    out, lse, sel, _ = wo.decode_layer(q, Kc, Vc, lay, 100, 102, 1, 2, 3)
    lay1 = wo.build_layer(K[1:], V[1:], 100, 50, 4, 2, 1, 2)
    Kc1 = np.concatenate([lay1.k_out, K[1:, :, 100:]], axis=2)
    Vc1 = np.concatenate([lay1.v_out, V[1:, :, 100:]], axis=2)
    out1, lse1, _, _ = wo.decode_layer(q[1:], Kc1, Vc1, lay1, 100, 102, 1, 2, 3)
    assert np.array_equal(out[1], out1[0]) and np.array_equal(lse[1], lse1[0])


def gqa_case(rng, B=2, H=2, G=3, L0=150, steps=2, d=8):
    """Distinct keys / values per (b, kv-head) (so mixing heads changes every result)."""
    L = L0 + steps
    K = np.empty((B, H, L, d), np.uint16)
    V = np.empty((B, H, L, d), np.uint16)
    for b in range(B):
        for g in range(H):
            K[b, g], V[b, g], _ = random_case(rng, L0=L0, d=d, G=1, steps=steps)
    q = bits(rng.standard_normal((B, H * G, d)) * 1.5)
    return K, V, q


def gqa_reference(q, K, V, L):
    """torch's fp64 SDPA with its own grouped-query mapping (query head h reads KV head
    h // G), and the log-sum-exp of the same logits by torch.logsumexp."""
    Q = torch.from_numpy(vals(q))[:, :, None, :]                  # [B, Hq, 1, d]
    Kt = torch.from_numpy(vals(K[:, :, :L]))                      # [B, Hkv, L, d]
    Vt = torch.from_numpy(vals(V[:, :, :L]))
    o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, enable_gqa=True)
    G = q.shape[1] // K.shape[1]
    Ke = Kt.repeat_interleave(G, dim=1)
    logits = (Q @ Ke.transpose(-1, -2))[:, :, 0, :] / math.sqrt(q.shape[2])
    return o[:, :, 0].numpy(), torch.logsumexp(logits, dim=-1).numpy()


@pytest.mark.parametrize("mode", ["retrieve_all", "singletons"])
def test_layer_drivers_group_query_heads_by_kv_head(mode):
    """Whole-layer build and decode with B = 2, Hkv = 2, G = 3: query head h uses KV head
    h // G (the GQA convention; torch's SDPA with enable_gqa fixes it independently). With
    every cluster retrieved, or with singleton clusters (exact estimate) at budgets 0 and 3,
    the layer's output and lse equal exact grouped attention over the original cache."""
    rng = np.random.default_rng(31)
    B, H, G, L0, steps = 2, 2, 3, 150, 2
    K, V, q = gqa_case(rng, B, H, G, L0, steps)
    L = L0 + steps
    if mode == "retrieve_all":
        lay = wo.build_layer(K, V, L0, 64, 6, 3, 2, 5)
        budgets = [10 ** 6]
    else:
        lay = wo.build_layer(K, V, L0, 32, 32, 2, 2, 5)
        budgets = [0, 3]
    Kc = np.concatenate([lay.k_out, K[:, :, L0:]], axis=2)
    Vc = np.concatenate([lay.v_out, V[:, :, L0:]], axis=2)
    ref, ref_lse = gqa_reference(q, K, V, L)
    for n_r in budgets:
        out, lse, sel, shat = wo.decode_layer(q, Kc, Vc, lay, L0, L, 2, 5, n_r)
        assert out.shape == (B, H * G, 8) and shat.shape[:2] == (B, H)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    # each (b, kv-head)'s permuted cache holds exactly that head's own rows
    for b in range(B):
        for g in range(H):
            got = sorted(map(bytes, lay.k_out[b, g]))
            assert got == sorted(map(bytes, K[b, g, :L0]))
            assert lay.stacked("size")[b, g].sum() == L0 - 7


def test_layer_decode_ranks_by_each_groups_own_heads():
    """Swapping the two query-head groups of a layer swaps the retrieval sets of the two KV
    heads' decodes only through their own keys: decoding group 1's queries against KV head 0
    (a layer with the KV heads swapped) gives KV head 0's selection of the swapped layer."""
    rng = np.random.default_rng(37)
    B, H, G, L0 = 1, 2, 3, 150
    K, V, q = gqa_case(rng, B, H, G, L0, 1)
    lay = wo.build_layer(K, V, L0, 64, 8, 3, 2, 5)
    Kc = np.concatenate([lay.k_out, K[:, :, L0:]], axis=2)
    Vc = np.concatenate([lay.v_out, V[:, :, L0:]], axis=2)
    out, lse, sel, _ = wo.decode_layer(q, Kc, Vc, lay, L0, L0 + 1, 2, 5, 4)
    Ks, Vs = K[:, ::-1].copy(), V[:, ::-1].copy()
    qs = np.concatenate([q[:, G:], q[:, :G]], axis=1)
    lay_s = wo.build_layer(Ks, Vs, L0, 64, 8, 3, 2, 5)
    Kcs = np.concatenate([lay_s.k_out, Ks[:, :, L0:]], axis=2)
    Vcs = np.concatenate([lay_s.v_out, Vs[:, :, L0:]], axis=2)
    out_s, lse_s, sel_s, _ = wo.decode_layer(qs, Kcs, Vcs, lay_s, L0, L0 + 1, 2, 5, 4)
    assert np.array_equal(sel_s[0][0], sel[0][1]) and np.array_equal(sel_s[0][1], sel[0][0])
    assert np.array_equal(out_s[0, :G], out[0, G:]) and np.array_equal(lse_s[0, G:], lse[0, :G])


# ------------------------------------------------------------------------------------------
# Build pins
# ------------------------------------------------------------------------------------------

def test_build_invariants():
    """Sizes sum to the indexed count; each segment's slots are a permutation of its own
    positions; rows move byte-for-byte; sizes times means and the value sums add up to the
    column sums of the keys and values; steady slots stay in place."""
    rng = np.random.default_rng(13)
    K, V, _ = random_case(rng, L0=300, d=16, steps=0)
    L0, S, k_seg, ns, nr = 300, 64, 8, 5, 11
    idx, Ko, Vo = wo.build_head(K, V, L0, S, k_seg, 3, ns, nr)
    assert idx.size.sum() == L0 - ns - nr
    assert sorted(idx.perm.tolist()) == list(range(L0))
    assert idx.perm[:ns].tolist() == list(range(ns))
    assert idx.perm[L0 - nr:].tolist() == list(range(L0 - nr, L0))
    for s, (lo, hi) in enumerate(wo.segment_ranges(L0, S, ns, nr)):
        assert sorted(idx.perm[lo:hi].tolist()) == list(range(lo, hi))
        ids = np.arange(s * k_seg, (s + 1) * k_seg)
        assert idx.offset[ids[0]] == lo
        assert np.all(idx.labels[lo:hi] // k_seg == s)
        for j in ids:  # each cluster's slots hold exactly its members, in position order
            sl = idx.perm[idx.offset[j]:idx.offset[j] + idx.size[j]]
            assert sl.tolist() == np.nonzero(idx.labels == j)[0].tolist()
    assert np.array_equal(Ko, K[idx.perm]) and np.array_equal(Vo, V[idx.perm])
    Kf, Vf = vals(K), vals(V)
    ind = np.nonzero(idx.labels >= 0)[0]
    np.testing.assert_allclose((idx.size[:, None] * vals(idx.centroid_mean)).sum(0),
                               Kf[ind].sum(0), rtol=0, atol=2e-2 * len(ind) ** 0.5)
    np.testing.assert_allclose(vals(idx.value_sum).sum(0), Vf[ind].sum(0), rtol=0,
                               atol=2e-2 * len(ind) ** 0.5)
    assert np.all(vals(idx.centroid_mean)[idx.size == 0] == 0)


def test_single_cluster_closed_form():
    """k_seg = 1: all labels are 0, the centroid is the normalised sum of the unit points and
    J = ||sum of unit points||."""
    rng = np.random.default_rng(17)
    K = bits(rng.standard_normal((40, 8)))
    V = bits(rng.standard_normal((40, 8)))
    idx, _, _ = wo.build_head(K, V, 40, S=64, k_seg=1, n_iters=3, n_sink=0, n_recent=0)
    assert np.all(idx.labels == 0)
    X = vals(K)
    u = (X / np.linalg.norm(X, axis=1, keepdims=True)).sum(0)
    assert np.array_equal(idx.last_centroids[0], bits(u / np.linalg.norm(u)))
    assert idx.objective[0] == pytest.approx(np.linalg.norm(u), rel=1e-13)


def test_objective_never_decreases_across_passes():
    """Spherical k-means monotonicity: each assignment and each normalised-mean update can only
    raise J = sum_i cos(x_i, mu_{a_i}); bf16 rounding of mu allows a tiny slack."""
    rng = np.random.default_rng(19)
    K, V, _ = random_case(rng, L0=512, d=16, steps=0, spread=1.0, n_topics=12)
    prev = None
    for T in range(1, 8):
        idx, _, _ = wo.build_head(K, V, 512, 512, 16, T, 0, 0)
        J = idx.objective[0]
        if prev is not None:
            assert J >= prev * (1 - 1e-4)
        prev = J


def test_kmeans_brute_force_tiny():
    """Exhaustive recomputation on a tiny segment with pure-Python loops: every pass assigns
    each point to the lowest-index centroid of maximal cosine, and the next centroid is the
    bf16 (torch conversion) of the normalised member sum; seeds at stride floor(n/k)."""
    rng = np.random.default_rng(23)
    n, d, k, T = 23, 5, 4, 4
    K = bits(rng.standard_normal((n, d)))
    X = [list(map(float, row)) for row in vals(K)]
    unit = []
    for x in X:
        r = math.sqrt(sum(c * c for c in x))
        unit.append([c / r for c in x])
    cl = wo.cluster_segment(vals(K), k, T)
    stride = n // k
    mu = [list(vals(bits([unit[j * stride]]))[0]) for j in range(k)]
    assert np.array_equal(cl.history[0], bits(mu))
    for t in range(T):
        assert np.array_equal(cl.history[t], bits(mu))
        lab = []
        for x in unit:
            best, bj = -1e300, -1
            for j in range(k):
                c = sum(a * b for a, b in zip(x, mu[j]))
                if c > best:
                    best, bj = c, j
            lab.append(bj)
        if t == T - 1:
            assert cl.labels.tolist() == lab
            break
        for j in range(k):
            mem = [unit[i] for i in range(n) if lab[i] == j]
            if mem:
                u = [sum(col) for col in zip(*mem)]
                nu = math.sqrt(sum(c * c for c in u))
                mu[j] = list(vals(bits([[c / nu for c in u]]))[0])


def test_short_segment_leaves_clusters_empty():
    """A segment with fewer points than clusters seeds one cluster per point; the rest stay
    empty, have zero statistics and are never retrieved."""
    rng = np.random.default_rng(29)
    K = bits(rng.standard_normal((70, 8)))
    V = bits(rng.standard_normal((70, 8)))
    # segments [0,32) and [32,64) full, [64,70) has 70-2-64 = 4 indexed points (< 8 clusters)
    idx, Ko, Vo = wo.build_head(K, V, 70, S=32, k_seg=8, n_iters=2, n_sink=1, n_recent=2)
    last = idx.size[16:24]
    assert last.sum() == 4 and np.all(last[4:] == 0)
    q = bits(rng.standard_normal((1, 8)))
    r = wo.decode_group(q, Ko, Vo, idx, 70, 70, 1, 2, n_retrieve=100)
    assert len(r.selected) == int((idx.size > 0).sum())
    assert not set(r.selected.tolist()) & set(np.nonzero(idx.size == 0)[0].tolist())
    np.testing.assert_allclose(r.out, sdpa(q, K, V), rtol=1e-12, atol=1e-12)


def test_group_ranking_uses_the_mean_logit():
    """GQA (reading R6): one retrieval set per KV head, ranked by the group-mean logit.
    Hand-built index with two singleton clusters e1, e2 and scale 1/2:
    head 0 q = (6,4,0,0) -> logits (3, 2); head 1 q = (-6,2,0,0) -> logits (-3, 1).
    Means (0, 1.5) pick cluster 1 (a max over heads would pick cluster 0)."""
    cm = bits([[1, 0, 0, 0], [0, 1, 0, 0]])
    idx = wo.HeadIndex(centroid_mean=cm, value_sum=bits([[1, 0, 0, 0], [0, 1, 0, 0]]),
                       size=np.array([1, 1], np.int32), offset=np.array([1, 2], np.int32),
                       labels=np.array([-1, 0, 1, -1], np.int32),
                       perm=np.arange(4, dtype=np.int32), last_centroids=cm,
                       objective=np.zeros(1))
    K = bits([[0, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 0, 0]])
    V = bits([[0, 0, 0, 0], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 0, 0]])
    r = wo.decode_group(bits([[6, 4, 0, 0], [-6, 2, 0, 0]]), K, V, idx, L0=4, L=4, n_sink=1,
                        n_recent=1, n_retrieve=1)
    assert r.selected.tolist() == [1]
    assert r.group_score.tolist() == [0.0, 1.5]
