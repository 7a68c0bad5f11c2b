"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

All inputs come from the seeded generator (synth); every expected value comes from the oracle
run on the CPU. Tolerances follow the protocol in wave_testlib.
"""
import sys
import zlib

import numpy as np
import pytest

import kv_vector_index_amd as wi
import synth
from oracle import wave_oracle as wo
import wave_testlib as tl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS["tiny"]
    x = synth.generate_layer(w)
    layer = tl.Layer(x.k, x.v, w.context, w.segment_size, w.clusters_per_segment, w.n_iters,
                     w.n_sink, w.n_recent, w.n_q_heads)
    return w, x, layer


def test_tiny_build_is_stepwise_identical_to_the_oracle(tiny):
    """Every pass of every head: labels = oracle assignment from the GPU's own centroids
    (ties 1e-4); next centroids = oracle update of those labels (1 bf16 ulp); seeds = oracle
    seeds (1 ulp)."""
    w, x, layer = tiny
    K = wo.bf16_to_f64(x.k)
    mus, labs = [], []
    for t in range(1, w.n_iters + 1):
        say(f"[tiny build] n_iters={t}")
        idx = layer.build(T=t)
        mus.append(tl.to_np16(idx.last_centroids))     # mu^(t-1)
        labs.append(idx.labels.cpu().numpy())           # a^(t)
    nflip = 0
    for b in range(layer.B):
        for g in range(layer.H):
            for s, (lo, hi) in enumerate(tl.segment_ranges(layer)):
                k = layer.kseg
                Xhat = wo.normalise_rows(K[b, g, lo:hi])
                seeds, nv = wo.kmeans_seeds(Xhat, k)
                assert tl.bf16_close(mus[0][b, g, s * k:(s + 1) * k], seeds) <= 1
                for t in range(w.n_iters):
                    mu_prev = mus[t][b, g, s * k:(s + 1) * k]
                    got = labs[t][b, g, lo:hi] - s * k
                    nflip += tl.check_assignment(Xhat, mu_prev, nv, got)
                    if t + 1 < w.n_iters:
                        u = wo.kmeans_cluster_sums(Xhat, got, k)
                        ref = wo.kmeans_update(u, np.bincount(got, minlength=k), mu_prev)
                        d = tl.bf16_close(mus[t + 1][b, g, s * k:(s + 1) * k], ref)
                        assert d <= 1, (b, g, s, t, d)
    say(f"[tiny build] label differences resolved as ties: {nflip}")


def test_tiny_index_matches_the_oracle_given_the_gpu_labels(tiny):
    """Sizes, offsets, permutation and permuted rows bit-exact; means / value sums within
    1 bf16 ulp; objective within 1e-4 relative; build bitwise reproducible."""
    w, x, layer = tiny
    say("[tiny index] build")
    idx = layer.build()
    k_out1 = tl.to_np16(layer.k_out)
    again = layer.build()
    assert np.array_equal(tl.to_np16(layer.k_out), k_out1)
    for f in ("centroid_mean", "value_sum", "last_centroids"):
        assert np.array_equal(tl.to_np16(getattr(idx, f)), tl.to_np16(getattr(again, f))), f
    for f in ("cluster_size", "cluster_offset", "labels", "perm", "objective"):
        assert np.array_equal(getattr(idx, f).cpu().numpy(), getattr(again, f).cpu().numpy()), f
    labels = idx.labels.cpu().numpy()
    k_out, v_out = tl.to_np16(layer.k_out), tl.to_np16(layer.v_out)
    obj = idx.objective.cpu().numpy()
    for b in range(layer.B):
        for g in range(layer.H):
            ref, ko, vo = wo.build_head(x.k[b, g], x.v[b, g], layer.L0, layer.S, layer.kseg,
                                        w.n_iters, layer.n_sink, layer.n_recent,
                                        labels_override=labels[b, g])
            hi = tl.head_index(idx, b, g)
            assert np.array_equal(hi.size, ref.size)
            assert np.array_equal(hi.offset, ref.offset)
            assert np.array_equal(hi.perm, ref.perm)
            assert np.array_equal(hi.labels, ref.labels)
            assert np.array_equal(k_out[b, g, :layer.L0], ko)
            assert np.array_equal(v_out[b, g, :layer.L0], vo)
            assert tl.bf16_close(hi.centroid_mean, ref.centroid_mean) <= 1
            assert tl.bf16_close(hi.value_sum, ref.value_sum) <= 1
            assert obj[b, g] == pytest.approx(ref.objective.sum(), rel=1e-4)


def test_tiny_objective_close_to_the_oracle_run(tiny):
    """The GPU's k-means (its own trajectory) reaches the oracle's own objective within 1e-4."""
    w, x, layer = tiny
    idx = layer.build()
    obj = idx.objective.cpu().numpy()
    for g in range(layer.H):
        ref, _, _ = wo.build_head(x.k[0, g], x.v[0, g], layer.L0, layer.S, layer.kseg,
                                  w.n_iters, layer.n_sink, layer.n_recent)
        assert obj[0, g] == pytest.approx(ref.objective.sum(), rel=1e-4)


def test_tiny_decode_every_step(tiny):
    """16 decode steps, all heads: selection (ties 1e-4), outputs and lse within 2e-3."""
    import kv_vector_index_amd as wi
    w, x, layer = tiny
    idx = layer.build()
    worst = 0.0
    # one workspace for every step: each call must leave its control words cleared
    ws = wi.alloc_decode_workspace(layer.decode_params(layer.L0 + 1, w.n_retrieve))
    for s in range(w.steps):
        L = layer.L0 + s + 1
        say(f"[tiny decode] step {s} L={L} n_r={w.n_retrieve}")
        out, lse, sel = layer.decode(idx, x.q[s], L, w.n_retrieve, ws=ws)
        worst = max(worst, tl.oracle_decode_check(layer, idx, x.q[s], L, w.n_retrieve, out,
                                                  lse, sel))
    say(f"[tiny decode] worst row error {worst:.2e}")


def test_workspace_reuse_across_budgets(tiny):
    """One workspace, sized for the largest budget and never cleared, serves calls with other
    budgets and gives the same results as a fresh workspace each time."""
    import kv_vector_index_amd as wi
    w, x, layer = tiny
    idx = layer.build()
    L = layer.L0 + 2
    ws = wi.alloc_decode_workspace(layer.decode_params(L, 11))   # sized for the largest
    for n_r in (3, 11, 3, 0, 11):
        out, lse, sel = layer.decode(idx, x.q[1], L, n_r, ws=ws)
        out2, lse2, sel2 = layer.decode(idx, x.q[1], L, n_r)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
        assert np.array_equal(sel, sel2)


def test_decode_on_an_oracle_built_index(tiny):
    """The index layout is the contract: an index built by the oracle and uploaded gives the
    oracle's decode result on the GPU."""
    t = tl.torch()
    w, x, layer = tiny
    lay = wo.build_layer(x.k, x.v, layer.L0, layer.S, layer.kseg, 2, layer.n_sink,
                         layer.n_recent)
    idx = wi_index_from_oracle(lay)
    layer.k_out[:, :, :layer.L0] = tl.to_dev(lay.k_out)
    layer.v_out[:, :, :layer.L0] = tl.to_dev(lay.v_out)
    layer.k_out[:, :, layer.L0:] = layer.k[:, :, layer.L0:]
    layer.v_out[:, :, layer.L0:] = layer.v[:, :, layer.L0:]
    t.cuda.synchronize()
    for s in (0, 7):
        L = layer.L0 + s + 1
        say(f"[oracle index decode] step {s}")
        out, lse, sel = layer.decode(idx, x.q[s], L, 9)
        tl.oracle_decode_check(layer, idx, x.q[s], L, 9, out, lse, sel)


def wi_index_from_oracle(lay):
    import kv_vector_index_amd as wi
    t = tl.torch()
    st = lambda f: lay.stacked(f)  # noqa: E731
    return wi.IndexTensors(
        tl.to_dev(st("centroid_mean")), tl.to_dev(st("value_sum")),
        t.from_numpy(st("size").astype(np.int32)).cuda(),
        t.from_numpy(st("offset").astype(np.int32)).cuda(),
        t.from_numpy(st("labels").astype(np.int32)).cuda(),
        t.from_numpy(st("perm").astype(np.int32)).cuda(),
        tl.to_dev(st("last_centroids")), None)


def test_retrieve_all_equals_dense_equals_full_attention(tiny):
    w, x, layer = tiny
    idx = layer.build()
    L = layer.L0 + 5
    say("[retrieve-all] decode + dense")
    out, lse, _ = layer.decode(idx, x.q[4], L, layer.C)
    dout, dlse, _ = layer.decode(idx, x.q[4], L, 0, dense=True)
    kc, vc = tl.to_np16(layer.k_out), tl.to_np16(layer.v_out)
    G = layer.Hq // layer.H
    for g in range(layer.H):
        ref, rlse = wo.full_attention(x.q[4][0, g * G:(g + 1) * G], kc[0, g], vc[0, g], L)
        assert tl.row_rel_err(out[0, g * G:(g + 1) * G], ref) <= tl.OUT_TOL
        assert tl.row_rel_err(dout[0, g * G:(g + 1) * G], ref) <= tl.OUT_TOL
        assert np.all(np.abs(dlse[0, g * G:(g + 1) * G] - rlse) <= tl.OUT_TOL)
        assert np.all(np.abs(lse[0, g * G:(g + 1) * G] - rlse) <= tl.OUT_TOL)


def test_zero_query_gives_the_mean_value(tiny):
    """q = 0: every logit is 0. Against the oracle on the same index (2e-3), and against the
    closed form mean(v) within the error the bf16 value sums allow (each stored sum carries
    a relative rounding error up to 2^-9, so 1e-2 of the row scale), with lse = ln L."""
    w, x, layer = tiny
    idx = layer.build()
    L = layer.L0 + 3
    q0 = np.zeros_like(x.q[0])
    for n_r in (0, 6):
        say(f"[zero query] n_r={n_r}")
        out, lse, sel = layer.decode(idx, q0, L, n_r)
        tl.oracle_decode_check(layer, idx, q0, L, n_r, out, lse, sel)
        vmean = wo.bf16_to_f64(tl.to_np16(layer.v_out)[:, :, :L]).mean(axis=2)  # [B, H, d]
        G = layer.Hq // layer.H
        assert tl.row_rel_err(out, np.repeat(vmean, G, axis=1)) <= 1e-2
        assert np.all(np.abs(lse - np.log(L)) <= 1e-4)


CASES = {
    # name: (ragged_layer kwargs, decode budgets)
    "gqa4_ragged": (dict(), (0, 5, 40)),
    "mha_g1": (dict(H=2, Hq=2), (3,)),
    # every other group size the kernels are instantiated for, up to the largest (G = 8)
    "gqa3": (dict(H=2, Hq=6), (5,)),
    "gqa5_batch2": (dict(B=2, H=1, Hq=5), (0, 9)),
    "gqa6": (dict(H=2, Hq=12), (40,)),
    "gqa8": (dict(H=2, Hq=16), (0, 5, 40)),
    "qwen_g7_batch2": (dict(B=2, H=2, Hq=14, L0=600, S=200, kseg=13), (4, 26)),
    "short_last_segment": (dict(L0=530, S=256, kseg=40, n_recent=3), (7,)),
    "no_steady_zone": (dict(n_sink=0, n_recent=0, steps=1), (2,)),
    "one_cluster_per_segment": (dict(kseg=1, S=128), (1,)),
    "singletons": (dict(L0=300, S=64, kseg=64, n_sink=1, n_recent=2), (0, 11)),
    "many_clusters": (dict(L0=2200, S=1024, kseg=300, T=4), (12, 300)),
    # more clusters per segment than the segment-resident assignment holds in LDS
    "tiled_assignment": (dict(L0=1500, S=1024, kseg=600, T=2), (20,)),
    # 32 (b, kv-head) x 28 retrieve workgroups: more than three per CU, so the retrieve
    # kernel merges its share of the earlier partials element by element
    "wide_retrieve_grid": (dict(B=4, H=8, Hq=32, L0=3000, S=1024, kseg=64, steps=1), (150,)),
    # the largest segment and cluster count the library takes (S = 16384, k_seg = 2048): a
    # first segment of 16381 points (every 64-point block of the sort's per-wave chunks),
    # a ragged second one of 9003
    "max_segment_and_clusters": (dict(H=1, Hq=4, L0=25404, S=16384, kseg=2048, T=2, steps=1),
                                 (40, 2048)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_shapes_and_edge_cases(case):
    kw, budgets = CASES[case]
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    layer, q = tl.ragged_layer(rng, **kw)
    say(f"[edge {case}] seed {zlib.crc32(case.encode())} build B={layer.B} H={layer.H} "
        f"Hq={layer.Hq} L0={layer.L0} "
        f"S={layer.S} kseg={layer.kseg}")
    idx = layer.build()
    labels = idx.labels.cpu().numpy()
    K = wo.bf16_to_f64(layer.k_np)
    last = tl.to_np16(idx.last_centroids)
    for b in range(layer.B):
        for g in range(layer.H):
            for s, (lo, hi) in enumerate(tl.segment_ranges(layer)):
                k = layer.kseg
                Xhat = wo.normalise_rows(K[b, g, lo:hi])
                tl.check_assignment(Xhat, last[b, g, s * k:(s + 1) * k], tl.n_valid(k, hi - lo),
                                    labels[b, g, lo:hi] - s * k)
            ref, ko, _ = wo.build_head(layer.k_np[b, g], layer.v_np[b, g], layer.L0, layer.S,
                                       layer.kseg, layer.T, layer.n_sink, layer.n_recent,
                                       labels_override=labels[b, g])
            hi_ = tl.head_index(idx, b, g)
            assert np.array_equal(hi_.size, ref.size) and np.array_equal(hi_.offset, ref.offset)
            assert np.array_equal(hi_.perm, ref.perm)
            assert np.array_equal(tl.to_np16(layer.k_out)[b, g, :layer.L0], ko)
            assert tl.bf16_close(hi_.centroid_mean, ref.centroid_mean) <= 1
            assert tl.bf16_close(hi_.value_sum, ref.value_sum) <= 1
    for s in range(q.shape[0]):
        L = layer.L0 + s + 1
        for n_r in budgets:
            n_r = min(n_r, layer.C)
            say(f"[edge {case}] decode step {s} n_r={n_r}")
            out, lse, sel = layer.decode(idx, q[s], L, n_r)
            tl.oracle_decode_check(layer, idx, q[s], L, n_r, out, lse, sel)
        dout, dlse, _ = layer.decode(idx, q[s], L, 0, dense=True)
        kc, vc = tl.to_np16(layer.k_out), tl.to_np16(layer.v_out)
        G = layer.Hq // layer.H
        for b in range(layer.B):
            for g in range(layer.H):
                ref, _ = wo.full_attention(q[s][b, g * G:(g + 1) * G], kc[b, g], vc[b, g], L)
                assert tl.row_rel_err(dout[b, g * G:(g + 1) * G], ref) <= tl.OUT_TOL


@pytest.mark.slow
def test_llama128k_sampled_parity():
    """Full 128K single-layer workload, launched as the bench launches it: sampled segments
    checked at the last pass and through the finalise (labels, sizes, offsets, permuted rows,
    centroid means, value sums), the objective of three heads over all their segments, one
    k-means update step on the sampled segments (a build with one pass fewer), and two decode
    steps checked on every head."""
    w = synth.WORKLOADS["llama128k"]
    say("[128k] generate")
    x = synth.generate_layer(w, rows=w.context + 2)
    layer = tl.Layer(x.k, x.v, w.context, w.segment_size, w.clusters_per_segment, w.n_iters,
                     w.n_sink, w.n_recent, w.n_q_heads)
    say("[128k] build with one pass fewer")
    idx_prev = layer.build(T=w.n_iters - 1)
    say("[128k] build")
    idx = layer.build()
    nseg = layer.nseg
    rng = np.random.default_rng(5)
    picks = [(0, 0, 0), (0, 3, 7), (0, 7, nseg - 1)] + [
        (0, int(rng.integers(8)), int(rng.integers(nseg))) for _ in range(3)]
    say(f"[128k] check segments {picks}")
    tl.check_segments(layer, idx, picks, objective_heads=[(0, 0), (0, 3), (0, 7)])
    say("[128k] check one update step")
    tl.check_update_step(layer, idx_prev, idx, picks)
    for s in range(2):
        L = layer.L0 + s + 1
        say(f"[128k] decode step {s}")
        out, lse, sel = layer.decode(idx, x.q[s], L, w.n_retrieve)
        tl.oracle_decode_check(layer, idx, x.q[s], L, w.n_retrieve, out, lse, sel)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama1m", "llama122k_b8", "qwen256k"])
def test_full_size_sampled_parity(name):
    """The other full-size layers that bench.py times (1M tokens; batch 8 at 122 880; the
    Qwen-shaped batch 4 at 262 144 with seven query heads per KV head), launched as the bench
    launches them: three sampled (b, kv-head, segment) triples checked at the last pass and
    through the finalise (labels, sizes, offsets, permuted rows, centroid means, value sums),
    one update step there, the objective of one head over all its segments, and one decode
    step checked on four sampled (b, kv-head) pairs."""
    w = synth.WORKLOADS[name]
    say(f"[{name}] generate")
    x = synth.generate_layer(w, rows=w.context + 1)
    layer = tl.Layer(x.k, x.v, w.context, w.segment_size, w.clusters_per_segment, w.n_iters,
                     w.n_sink, w.n_recent, w.n_q_heads)
    say(f"[{name}] build with one pass fewer")
    idx_prev = layer.build(T=w.n_iters - 1)
    say(f"[{name}] build")
    idx = layer.build()
    nseg = layer.nseg
    rng = np.random.default_rng(11)
    picks = [(0, 0, 0), (layer.B - 1, layer.H - 1, nseg - 1),
             (int(rng.integers(layer.B)), int(rng.integers(layer.H)), int(rng.integers(nseg)))]
    say(f"[{name}] check segments {picks}")
    tl.check_segments(layer, idx, picks, objective_heads=[picks[2][:2]])
    say(f"[{name}] check one update step")
    tl.check_update_step(layer, idx_prev, idx, picks)
    del idx_prev
    say(f"[{name}] decode")
    L = layer.L0 + 1
    out, lse, sel = layer.decode(idx, x.q[0], L, w.n_retrieve)
    heads = {(0, 0), (layer.B - 1, layer.H - 1),
             (int(rng.integers(layer.B)), int(rng.integers(layer.H))),
             (int(rng.integers(layer.B)), int(rng.integers(layer.H)))}
    worst = tl.oracle_decode_check(layer, idx, x.q[0], L, w.n_retrieve, out, lse, sel, heads=heads)
    say(f"[{name}] worst relative error {worst:.2e}")


def extend_and_check(full, idx_full, prev_len, n_q_steps=1, q=None):
    """Build an index for prev_len tokens, extend it to full.L0 with the rows that the
    extension documents as unread (before max(s0 S, n_sink)) overwritten with other data,
    and check the result: bit for bit equal to the full build idx_full (index and cache), and
    against the oracle on every segment (labels from the GPU's last centroids, sizes,
    offsets, permuted rows, means, value sums) and on one decode step."""
    t = tl.torch()
    prev = tl.Layer(full.k_np, full.v_np, prev_len, full.S, full.kseg, full.T, full.n_sink,
                    full.n_recent, full.Hq)
    idx_prev = prev.build()
    idx_new = wi.alloc_index(full.B, full.H, full.C, full.L0)
    idx_new.objective = None
    p = full.build_params()
    ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
    s0 = (prev_len - full.n_recent) // full.S
    lim = max(s0 * full.S, full.n_sink)
    k_in, v_in = full.k.clone(), full.v.clone()
    k_in[:, :, :lim] = -k_in[:, :, :lim].flip(2)    # other data in the rows not read
    v_in[:, :, :lim] = -v_in[:, :, :lim].flip(2)
    say(f"[extend] prev_len={prev_len} s0={s0} rows not read [0, {lim})")
    wi.wave_index_extend(p, prev_len, k_in, v_in, prev.k_out, prev.v_out, idx_prev, idx_new, ws)
    t.cuda.synchronize()
    for f in ("centroid_mean", "value_sum", "cluster_size", "cluster_offset", "labels", "perm",
              "last_centroids"):
        a, b = getattr(idx_new, f), getattr(idx_full, f)
        assert t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a,
                       b.view(t.int16) if b.dtype == t.bfloat16 else b), f
    L0 = full.L0
    assert t.equal(prev.k_out[:, :, :L0].view(t.int16), full.k_out[:, :, :L0].view(t.int16))
    assert t.equal(prev.v_out[:, :, :L0].view(t.int16), full.v_out[:, :, :L0].view(t.int16))
    # against the oracle: the extended index and cache as a layer of L0 tokens
    ext = tl.Layer.__new__(tl.Layer)
    ext.__dict__.update(full.__dict__)
    ext.k_out, ext.v_out = prev.k_out, prev.v_out
    picks = [(b, g, s) for b in range(full.B) for g in range(full.H) for s in range(full.nseg)]
    tl.check_segments(ext, idx_new, picks)
    if q is not None:
        L = L0 + 1
        n_r = max(1, full.C // 20)
        out, lse, sel = ext.decode(idx_new, q[0], L, n_r)
        tl.oracle_decode_check(ext, idx_new, q[0], L, n_r, out, lse, sel)


@pytest.mark.parametrize("prev_len", [20, 1041, 1100, 1700, 3000])
def test_extension_equals_the_full_build_and_the_oracle(prev_len):
    """An index built for prev_len tokens and extended to 3000 equals the index built for
    3000 directly, bit for bit (clustering is segment-local and the build deterministic), and
    so does the extended cache; the extended index matches the oracle. prev_len 20 =
    n_sink + n_recent (an empty index); 1041 puts the earlier indexed range on a segment
    boundary; 1100 and 1700 end it inside a segment (rebuilt); 3000 extends by nothing. Two
    batch elements and KV heads exercise the cluster and position strides, which differ
    between the two lengths."""
    rng = np.random.default_rng(17)
    full, q = tl.ragged_layer(rng, B=2, H=2, Hq=4, L0=3000, steps=2, S=512, kseg=32, T=3,
                              n_sink=3, n_recent=17)
    idx_full = full.build()
    idx_full.objective = None
    extend_and_check(full, idx_full, prev_len, q=q)


def test_extension_by_nothing_without_a_steady_zone():
    """n_sink = n_recent = 0 and an unchanged length that ends a segment: no segment is
    rebuilt (the first one to build would be past the last); the call copies the earlier
    index and still equals the full build."""
    rng = np.random.default_rng(23)
    full, q = tl.ragged_layer(rng, B=1, H=2, Hq=4, L0=1024, steps=1, S=512, kseg=16, T=2,
                              n_sink=0, n_recent=0)
    idx_full = full.build()
    idx_full.objective = None
    extend_and_check(full, idx_full, 1024, q=q)


def test_chained_extensions_equal_the_full_build():
    """The prefill-fused build: an index extended one segment of new tokens at a time, from
    an empty index (only the steady zone) to the whole context, equals the index built in one
    call, bit for bit, and matches the oracle on every segment and one decode step."""
    t = tl.torch()
    rng = np.random.default_rng(27)
    full, q = tl.ragged_layer(rng, B=1, H=2, Hq=8, L0=2600, steps=1, S=512, kseg=32, T=3,
                              n_sink=3, n_recent=17)
    idx_full = full.build()
    idx_full.objective = None
    lens = [full.n_sink + full.n_recent] + list(range(512, full.L0, 512)) + [full.L0]
    cur = tl.Layer(full.k_np, full.v_np, lens[0], full.S, full.kseg, full.T, full.n_sink,
                   full.n_recent, full.Hq)
    idx = cur.build()
    idx.objective = None
    for n0, n1 in zip(lens[:-1], lens[1:]):
        say(f"[chained extension] {n0} -> {n1}")
        nxt = tl.Layer(full.k_np, full.v_np, n1, full.S, full.kseg, full.T, full.n_sink,
                       full.n_recent, full.Hq)
        new = wi.alloc_index(full.B, full.H, nxt.C, n1)
        new.objective = None
        p = nxt.build_params()
        ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
        wi.wave_index_extend(p, n0, full.k, full.v, cur.k_out, cur.v_out, idx, new, ws)
        t.cuda.synchronize()
        idx = new
    for f in ("centroid_mean", "value_sum", "cluster_size", "cluster_offset", "labels", "perm",
              "last_centroids"):
        a, b = getattr(idx, f), getattr(idx_full, f)
        assert t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a,
                       b.view(t.int16) if b.dtype == t.bfloat16 else b), f
    L0 = full.L0
    assert t.equal(cur.k_out[:, :, :L0].view(t.int16), full.k_out[:, :, :L0].view(t.int16))
    assert t.equal(cur.v_out[:, :, :L0].view(t.int16), full.v_out[:, :, :L0].view(t.int16))
    ext = tl.Layer.__new__(tl.Layer)
    ext.__dict__.update(full.__dict__)
    ext.k_out, ext.v_out = cur.k_out, cur.v_out
    tl.check_segments(ext, idx, [(0, g, s) for g in range(full.H) for s in range(full.nseg)])
    out, lse, sel = ext.decode(idx, q[0], L0 + 1, 9)
    tl.oracle_decode_check(ext, idx, q[0], L0 + 1, 9, out, lse, sel)


def test_decode_continues_after_an_extension():
    """A decode loop across an index extension: decode with the index of 1100 tokens while
    500 generated tokens accumulate in the recent zone, extend the index to the 1600 tokens
    (three segments clustered again), and decode on. Before the extension, against the
    oracle on the earlier index; after it, against the oracle's own index built for 1600
    tokens (same labels as the extended index) and against the oracle on the extended index."""
    t = tl.torch()
    rng = np.random.default_rng(29)
    full, q = tl.ragged_layer(rng, B=1, H=2, Hq=8, L0=1600, steps=2, S=512, kseg=32, T=3,
                              n_sink=3, n_recent=17)
    prev = tl.Layer(full.k_np, full.v_np, 1100, full.S, full.kseg, full.T, full.n_sink,
                    full.n_recent, full.Hq)
    idx_prev = prev.build()
    n_r = 6
    L = 1400
    say(f"[decode loop] decode at L={L} on the index of {prev.L0} tokens")
    out, lse, sel = prev.decode(idx_prev, q[0], L, n_r)
    tl.oracle_decode_check(prev, idx_prev, q[0], L, n_r, out, lse, sel)
    say("[decode loop] extend to 1600 tokens")
    idx_new = wi.alloc_index(full.B, full.H, full.C, full.L0)
    idx_new.objective = None
    p = full.build_params()
    ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
    wi.wave_index_extend(p, prev.L0, full.k, full.v, prev.k_out, prev.v_out, idx_prev, idx_new,
                         ws)
    t.cuda.synchronize()
    ext = tl.Layer.__new__(tl.Layer)
    ext.__dict__.update(full.__dict__)
    ext.k_out, ext.v_out = prev.k_out, prev.v_out
    L = full.L0 + 1
    n_r = 9
    say(f"[decode loop] decode at L={L} on the extended index (C={full.C})")
    out, lse, sel = ext.decode(idx_new, q[1], L, n_r)
    tl.oracle_decode_check(ext, idx_new, q[1], L, n_r, out, lse, sel)
    lay = wo.build_layer(full.k_np, full.v_np, full.L0, full.S, full.kseg, full.T, full.n_sink,
                         full.n_recent)
    assert np.array_equal(lay.stacked("labels"), idx_new.labels.cpu().numpy()), \
        "the oracle's own clustering differs from the extended index"
    kc = np.concatenate([lay.k_out, full.k_np[:, :, full.L0:]], axis=2)
    vc = np.concatenate([lay.v_out, full.v_np[:, :, full.L0:]], axis=2)
    G = full.Hq // full.H
    for g in range(full.H):
        r = wo.decode_group(q[1][0, g * G:(g + 1) * G], kc[0, g], vc[0, g], lay.heads[0][g],
                            full.L0, L, full.n_sink, full.n_recent, n_r)
        assert tl.row_rel_err(out[0, g * G:(g + 1) * G], r.out) <= tl.OUT_TOL
        assert np.all(np.abs(lse[0, g * G:(g + 1) * G] - r.lse) <= tl.OUT_TOL)


def test_extension_with_tiled_assignment():
    """The extension through the other assignment kernel (k_seg > 512 centroids per segment:
    LDS tiles of 128 centroids) and a group of seven query heads."""
    t = tl.torch()
    rng = np.random.default_rng(19)
    full, _ = tl.ragged_layer(rng, B=1, H=2, Hq=14, L0=2600, steps=1, S=1024, kseg=600, T=2,
                              n_sink=3, n_recent=17)
    idx_full = full.build()
    prev = tl.Layer(full.k_np, full.v_np, 1500, full.S, full.kseg, full.T, full.n_sink,
                    full.n_recent, full.Hq)
    idx_prev = prev.build()
    idx_new = wi.alloc_index(full.B, full.H, full.C, full.L0)
    idx_new.objective = None
    p = full.build_params()
    ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
    wi.wave_index_extend(p, 1500, full.k, full.v, prev.k_out, prev.v_out, idx_prev, idx_new, ws)
    t.cuda.synchronize()
    for f in ("centroid_mean", "value_sum", "cluster_size", "cluster_offset", "labels", "perm",
              "last_centroids"):
        a, b = getattr(idx_new, f), getattr(idx_full, f)
        assert t.equal(a.view(t.int16) if a.dtype == t.bfloat16 else a,
                       b.view(t.int16) if b.dtype == t.bfloat16 else b), f
    assert t.equal(prev.k_out[:, :, :full.L0].view(t.int16),
                   full.k_out[:, :, :full.L0].view(t.int16))


def test_extension_rejects_bad_arguments():
    """An earlier length out of range, an objective output, and an index that overlaps the
    earlier one are refused before anything is enqueued."""
    t = tl.torch()
    rng = np.random.default_rng(18)
    full, _ = tl.ragged_layer(rng, B=1, H=1, Hq=2, L0=1200, steps=1, S=256, kseg=16, T=2,
                              n_sink=3, n_recent=17)
    idx_prev = full.build()
    p = full.build_params()
    ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
    out = wi.alloc_index(1, 1, full.C, full.L0)
    with pytest.raises(wi.WaveError, match="UNSUPPORTED"):  # objective requested
        wi.wave_index_extend(p, 600, full.k, full.v, full.k_out, full.v_out, idx_prev, out, ws)
    out.objective = None
    for bad in (10, 1201):
        with pytest.raises(wi.WaveError, match="INVALID_ARG"):
            wi.wave_index_extend(p, bad, full.k, full.v, full.k_out, full.v_out, idx_prev, out,
                                 ws)
    idx_prev.objective = None
    with pytest.raises(wi.WaveError, match="ALIAS"):
        wi.wave_index_extend(p, 600, full.k, full.v, full.k_out, full.v_out, idx_prev,
                             idx_prev, ws)


def host_index_layer(rng, C, n_distinct, Hq=4, n_sink=3, n_recent=9, steps=1, p_empty=0.05,
                     cmean_f32=None, nonempty=()):
    """One KV head whose index is written on the host: cluster sizes 0..3, centroid means
    drawn from only n_distinct bf16 vectors (so thousands of group scores tie exactly) or
    given (cmean_f32, exactly representable in bf16), value sums = the bf16-rounded sums of
    the cluster's value rows."""
    t = tl.torch()
    size = rng.integers(1, 4, C).astype(np.int32)
    size[rng.random(C) < p_empty] = 0
    size[list(nonempty)] = np.maximum(size[list(nonempty)], 1)
    offset = (n_sink + np.concatenate([[0], np.cumsum(size)[:-1]])).astype(np.int32)
    L0 = n_sink + int(size.sum()) + n_recent
    Lcap = L0 + steps
    k = tl.f32_bits(rng.standard_normal((1, 1, Lcap, 128)))
    v = tl.f32_bits(rng.standard_normal((1, 1, Lcap, 128)))
    if cmean_f32 is None:
        protos = tl.f32_bits(rng.standard_normal((n_distinct, 128)) * 0.3)
        cmean = protos[rng.integers(0, n_distinct, C)]
    else:
        cmean = tl.f32_bits(cmean_f32)
    V = wo.bf16_to_f64(v[0, 0])
    csum = np.zeros((C, 128))
    owner = np.repeat(np.arange(C), size)
    np.add.at(csum, owner, V[n_sink:n_sink + len(owner)])
    vsum = wo.round_bf16(csum)
    layer = tl.Layer(k, v, L0, L0, 1, 1, n_sink, n_recent, Hq)
    layer.C = C
    layer.k_out, layer.v_out = layer.k, layer.v
    idx = wi.alloc_index(1, 1, C, L0)
    idx.centroid_mean.copy_(tl.to_dev(cmean[None, None]))
    idx.value_sum.copy_(tl.to_dev(vsum[None, None]))
    idx.cluster_size.copy_(t.from_numpy(size[None, None]))
    idx.cluster_offset.copy_(t.from_numpy(offset[None, None]))
    idx.labels.zero_()
    idx.perm.zero_()
    idx.last_centroids.zero_()
    q = tl.f32_bits(rng.standard_normal((steps, 1, Hq, 128)))
    return layer, idx, q, size


@pytest.mark.parametrize("C", [3000, 8192, 8193, 10241, 12000, 65536])
def test_exact_score_ties_select_lowest_ids(C):
    """Exactly tied group scores are broken towards the lower cluster id, both where one
    workgroup selects a whole head from registers (C <= 8192) and where several workgroups
    per head list candidates and the last ranks them (larger C, down to 8193, where the last
    of 65 chunks holds one cluster, and 10241, a ragged last chunk); the budgets put the cut
    inside a block of ties thousands of clusters wide, and past the number of non-empty
    clusters."""
    rng = np.random.default_rng(C)
    layer, idx, q, size = host_index_layer(rng, C, n_distinct=5)
    for n_r in (1, C // 50, C // 3, C):
        say(f"[ties C={C}] n_r={n_r}")
        out, lse, sel = layer.decode(idx, q[0], layer.L0 + 1, n_r)
        hi = tl.head_index(idx, 0, 0)
        free = wo.decode_group(q[0][0], tl.to_np16(layer.k)[0, 0], tl.to_np16(layer.v)[0, 0], hi,
                               layer.L0, layer.L0 + 1, layer.n_sink, layer.n_recent, n_r)
        got = sel[0, 0]
        want = np.sort(free.selected)
        assert np.array_equal(got[got >= 0], want), "tie-break differs from lowest-id order"
        assert np.all(got[len(want):] == -1)
        tl.oracle_decode_check(layer, idx, q[0], layer.L0 + 1, n_r, out, lse, sel)


@pytest.mark.parametrize("C,skew", [(6000, 0.0), (8192, 0.93), (8193, 0.93), (30000, 0.0),
                                    (65536, 0.93)])
def test_crowded_cut_bin_is_ranked_exactly(C, skew):
    """Thousands of distinct group scores in the cut bin, so the cut pair is found after one
    to three narrowing rounds (C <= 8192: from one workgroup's registers; larger C: from the
    listed candidates); with skew most clusters share the top two score components and
    differ only in the third. The scores are exact in fp32 in any summation order (query
    e0 + 2^-8 e1 + 2^-16 e2 in every head, centroids with few-bit bf16 values in [1, 2) in
    dims 0..2, zero elsewhere, so every score is a 22-bit fraction; one non-empty outlier of
    64 stretches the histogram range so that the rest fall in a few of its bins) and
    distinct scores stay distinct through the scaling, so the selection must equal the
    oracle's exactly, ties to the lower id."""
    rng = np.random.default_rng(C + int(skew * 100))
    cm = np.zeros((C, 128), np.float32)
    k0 = np.where(rng.random(C) < skew, 0, rng.integers(0, 16, C))
    k1 = np.where(rng.random(C) < skew, 0, rng.integers(0, 128, C))
    cm[:, 0] = 1.0 + k0 / 128.0
    cm[:, 1] = 1.0 + k1 / 128.0
    cm[:, 2] = 1.0 + rng.integers(0, 32, C) / 32.0
    j_out = int(rng.integers(0, C))
    cm[j_out, 0] = 64.0
    layer, idx, _, size = host_index_layer(rng, C, 0, cmean_f32=cm, p_empty=0.02,
                                           nonempty=(j_out,))
    qv = np.zeros((1, 1, layer.Hq, 128), np.float32)
    qv[..., 0] = 1.0
    qv[..., 1] = 2.0 ** -8
    qv[..., 2] = 2.0 ** -16
    q = tl.f32_bits(qv)
    hi = tl.head_index(idx, 0, 0)
    for n_r in (C // 50, C // 7, C // 2):
        say(f"[crowded C={C} skew={skew}] n_r={n_r}")
        out, lse, sel = layer.decode(idx, q[0], layer.L0 + 1, n_r)
        free = wo.decode_group(q[0][0], tl.to_np16(layer.k)[0, 0], tl.to_np16(layer.v)[0, 0], hi,
                               layer.L0, layer.L0 + 1, layer.n_sink, layer.n_recent, n_r)
        got = sel[0, 0]
        want = np.sort(free.selected)
        assert np.array_equal(got[got >= 0], want), "selection differs from the exact ranking"
        assert np.all(got[len(want):] == -1)
        tl.oracle_decode_check(layer, idx, q[0], layer.L0 + 1, n_r, out, lse, sel)


def test_assignment_with_negative_best_scores():
    """Points whose dot product with every centroid of their segment is negative still get
    the oracle's assignment (ties within 1e-4): the first pass's centroids are the seeds, the
    unit keys at local positions j floor(n / kseg), all near +8 e0, while the keys halfway
    between seed positions lie near -8 e0, so that their best score is about -0.65 (66 such
    points); the argmax compares fp32 scores of either sign. Checked after one pass and after
    three."""
    rng = np.random.default_rng(1907)
    d, L0, S, kseg, n_sink, n_recent = 128, 1100, 512, 32, 4, 16
    L = L0 + 1
    base = np.zeros(d)
    base[0] = 8.0
    kf = base + 0.5 * rng.standard_normal((L, d))
    neg = []
    for lo, hi in wo.segment_ranges(L0, S, n_sink, n_recent):
        step = (hi - lo) // kseg
        if step >= 2:
            neg.extend(range(lo + step // 2, hi, step))
    kf[neg] = -base + 0.5 * rng.standard_normal((len(neg), d))
    layer = tl.Layer(tl.f32_bits(kf[None, None]), tl.f32_bits(rng.standard_normal((1, 1, L, d))),
                     L0, S, kseg, 3, n_sink, n_recent, 2)
    K = wo.bf16_to_f64(layer.k_np)
    for T in (1, 3):
        say(f"[negative scores] n_iters={T}")
        idx = layer.build(T=T)
        mu = tl.to_np16(idx.last_centroids)
        labels = idx.labels.cpu().numpy()
        n_negative = 0
        for s, (lo, hi) in enumerate(tl.segment_ranges(layer)):
            Xhat = wo.normalise_rows(K[0, 0, lo:hi])
            mus = mu[0, 0, s * kseg:(s + 1) * kseg]
            nv = tl.n_valid(kseg, hi - lo)
            best = (Xhat @ wo.bf16_to_f64(mus)[:nv].T).max(axis=1)
            n_negative += int((best < 0).sum())
            tl.check_assignment(Xhat, mus, nv, labels[0, 0, lo:hi] - s * kseg)
        if T == 1:
            assert n_negative >= 60, n_negative  # (the case this test is for)


def test_traced_calls_time_each_kernel_and_match_the_plain_calls(tiny):
    """The traced variants give bit-identical results and time every kernel with one
    start / end event pair (build: norms, seeds, passes x (assign, sort) + (passes - 1) x
    update, finalise, steady, objective; decode: stream, select, retrieve)."""
    t = tl.torch()
    w, x, layer = tiny
    T = 3
    p = layer.build_params(T)
    ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")

    def events(n):
        ev = [t.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:
            e.record()
        return ev

    idx_a = wi.alloc_index(layer.B, layer.H, layer.C, layer.L0)
    idx_b = wi.alloc_index(layer.B, layer.H, layer.C, layer.L0)
    wi.wave_index_build(p, layer.k, layer.v, layer.k_out, layer.v_out, idx_a, ws)
    ko_a = layer.k_out.clone()
    n_build = 2 * (3 * T + 4)
    bev = events(n_build + 4)                    # room to spare: only what is used is counted
    got = wi.wave_index_build(p, layer.k, layer.v, layer.k_out, layer.v_out, idx_b, ws,
                              events=[e.cuda_event for e in bev])
    t.cuda.synchronize()
    assert got == n_build
    for f in ("centroid_mean", "value_sum", "cluster_size", "cluster_offset", "labels", "perm"):
        assert t.equal(getattr(idx_a, f), getattr(idx_b, f)), f
    assert t.equal(ko_a, layer.k_out)
    durs = [bev[2 * i].elapsed_time(bev[2 * i + 1]) for i in range(n_build // 2)]
    assert all(d > 0 for d in durs), durs
    layer.k_out[:, :, layer.L0:] = layer.k[:, :, layer.L0:]
    layer.v_out[:, :, layer.L0:] = layer.v[:, :, layer.L0:]
    L, n_r = layer.L0 + 1, w.n_retrieve
    dp = layer.decode_params(L, n_r)
    q = tl.to_dev(x.q[0])
    outs = []
    for traced in (False, True):
        out = t.empty(layer.B, layer.Hq, 128, dtype=t.float32, device="cuda")
        dws = wi.alloc_decode_workspace(dp)
        ev = events(8) if traced else None
        n = wi.wave_decode_attention(dp, q, layer.k_out, layer.v_out, idx_b, out, None, None,
                                     dws, events=None if ev is None else [e.cuda_event for e in ev])
        t.cuda.synchronize()
        if traced:
            assert n == 6
            assert all(ev[2 * i].elapsed_time(ev[2 * i + 1]) > 0 for i in range(3))
        outs.append(out.cpu())
    assert t.equal(outs[0], outs[1])
