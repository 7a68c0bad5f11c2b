"""Helpers for the GPU parity tests: run the HIP library through its binding, read results back,
and compare with the CPU oracle under the tolerance protocol.

Tolerance protocol (integer decisions exact unless the scores tie within 1e-4; floating point
within 2e-3 of the row's largest magnitude):
  * k-means labels: GPU label g is accepted against oracle label o when g == o or
    cos(x, mu_g) >= cos(x, mu_o) - 1e-4 (both from the same centroids, fp64).
  * retrieved clusters: same count; every cluster in the symmetric difference has a group
    score within 1e-4 * max(1, |tau|) of the oracle's n_r-th best score tau; the outputs are
    then compared with the oracle run on the GPU's own retrieved set.
  * sizes, offsets, permutation, permuted rows: bit-exact given the GPU labels; centroid means,
    value sums and unit centroids within 1 bf16 ulp, or within 2^-17 of the row's scale where
    that is larger (fp32 sums on the GPU vs fp64 in the oracle may round to neighbouring bf16
    values; near zero the fp32 summation error spans several of bf16's tiny spacings).
  * outputs: per (b, h) row, max|gpu - oracle| <= 2e-3 * max|oracle|; lse within 2e-3.
"""
from __future__ import annotations

import math

import numpy as np

import kv_vector_index_amd as wi
from oracle import wave_oracle as wo

TIE = 1e-4
OUT_TOL = 2e-3


def torch():
    import torch as t
    return t


def to_dev(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).cuda()


def to_np16(x) -> np.ndarray:
    t = torch()
    return x.detach().contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def bf16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between bit patterns (+0 and -0 are equal)."""
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def bf16_close(got: np.ndarray, ref: np.ndarray, abs_rel: float = 2.0 ** -17) -> float:
    """Worst violation ratio of |got - ref| <= max(1 ulp of ref, abs_rel * max(1, max|ref row|)).

    bf16 results rounded from fp32 (GPU) and fp64 (oracle) sums may land on neighbouring
    values (1 ulp); near zero, where bf16 spacing is tiny, the fp32 summation error of a
    cluster sum (about n * 2^-24 of the row's scale) can span several ulps, hence the
    absolute floor. Returns max |diff| / allowed (<= 1 passes)."""
    g = wo.bf16_to_f64(got)
    r = wo.bf16_to_f64(ref)
    _, e = np.frexp(np.abs(r))
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    row = np.maximum(1.0, np.abs(r).max(axis=-1, keepdims=True))
    allowed = np.maximum(ulp, abs_rel * row)
    return float((np.abs(g - r) / allowed).max()) if g.size else 0.0


class Layer:
    """One layer's inputs on the device plus the parameters of a build / decode."""

    def __init__(self, k: np.ndarray, v: np.ndarray, L0: int, S: int, kseg: int, T: int,
                 n_sink: int, n_recent: int, n_q_heads: int):
        t = torch()
        self.k_np, self.v_np = k, v
        self.B, self.H, self.Lcap, self.d = k.shape
        self.L0, self.S, self.kseg, self.T = L0, S, kseg, T
        self.n_sink, self.n_recent, self.Hq = n_sink, n_recent, n_q_heads
        self.nseg = -(-L0 // S)
        self.C = self.nseg * kseg
        self.k, self.v = to_dev(k), to_dev(v)
        self.k_out = t.zeros_like(self.k)
        self.v_out = t.zeros_like(self.v)

    def build_params(self, T=None):
        return wi.wave_build_params(self.B, self.Hq, self.H, 128, self.L0, self.Lcap, self.S,
                                    self.kseg, self.T if T is None else T, self.n_sink,
                                    self.n_recent)

    def build(self, T=None, stream=None):
        t = torch()
        p = self.build_params(T)
        ws = t.empty(wi.wave_index_workspace_size(p), dtype=t.uint8, device="cuda")
        idx = wi.alloc_index(self.B, self.H, self.C, self.L0)
        wi.wave_index_build(p, self.k, self.v, self.k_out, self.v_out, idx, ws, stream)
        # decode tokens appended after the prefill keep their generator rows
        self.k_out[:, :, self.L0:] = self.k[:, :, self.L0:]
        self.v_out[:, :, self.L0:] = self.v[:, :, self.L0:]
        t.cuda.synchronize()
        return idx

    def decode_params(self, L, n_r, scale=None):
        return wi.wave_decode_params(self.B, self.Hq, self.H, 128, L, self.L0, self.Lcap, self.C,
                                     self.n_sink, self.n_recent, n_r,
                                     scale if scale is not None else 128 ** -0.5)

    def decode(self, idx, q_np: np.ndarray, L: int, n_r: int, dense=False, ws=None):
        t = torch()
        p = self.decode_params(L, n_r)
        if ws is None:
            ws = wi.alloc_decode_workspace(p)
        q = to_dev(q_np)
        out = t.empty(self.B, self.Hq, 128, dtype=t.float32, device="cuda")
        lse = t.empty(self.B, self.Hq, dtype=t.float32, device="cuda")
        sel = t.full((self.B, self.H, max(n_r, 1)), -7, dtype=t.int32, device="cuda")
        if dense:
            wi.wave_dense_decode_attention(p, q, self.k_out, self.v_out, out, lse, ws)
        else:
            wi.wave_decode_attention(p, q, self.k_out, self.v_out, idx, out, lse, sel, ws)
        t.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()[:, :, :n_r]


def head_index(idx: wi.IndexTensors, b: int, g: int) -> wo.HeadIndex:
    """The GPU index of one (b, kv-head) as the oracle's HeadIndex."""
    return wo.HeadIndex(
        centroid_mean=to_np16(idx.centroid_mean[b, g]), value_sum=to_np16(idx.value_sum[b, g]),
        size=idx.cluster_size[b, g].cpu().numpy(), offset=idx.cluster_offset[b, g].cpu().numpy(),
        labels=idx.labels[b, g].cpu().numpy(), perm=idx.perm[b, g].cpu().numpy(),
        last_centroids=to_np16(idx.last_centroids[b, g]),
        objective=np.zeros(1))


def check_assignment(Xhat: np.ndarray, mu_bits: np.ndarray, n_valid: int, got: np.ndarray):
    """GPU labels vs the oracle's assignment from the same centroids, ties within 1e-4."""
    ref = wo.kmeans_assign(Xhat, mu_bits, n_valid)
    bad = np.nonzero(ref != got)[0]
    if len(bad):
        mu = wo.bf16_to_f64(mu_bits)
        assert np.all((got[bad] >= 0) & (got[bad] < n_valid)), "label out of range"
        cg = np.einsum("ij,ij->i", Xhat[bad], mu[got[bad]])
        co = np.einsum("ij,ij->i", Xhat[bad], mu[ref[bad]])
        assert np.all(cg >= co - TIE), f"{len(bad)} labels differ beyond ties: {(co - cg).max()}"
    return len(bad)


def check_selection(shat_ref: np.ndarray, size: np.ndarray, n_r: int, got: np.ndarray):
    """GPU retrieved set vs the oracle's, ties within 1e-4 of the n_r-th score."""
    ref = wo.select_clusters(shat_ref, size, n_r)
    got = np.sort(got[got >= 0])
    assert len(got) == len(ref), (len(got), len(ref))
    if len(ref) and not np.array_equal(got, ref):
        tau = np.sort(shat_ref[size > 0])[::-1][len(ref) - 1]
        diff = np.setxor1d(got, ref)
        assert np.all(np.abs(shat_ref[diff] - tau) <= TIE * max(1.0, abs(tau))), \
            "retrieved sets differ beyond ties"
    return got


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max|out - ref| / max|ref| (rows = last axis)."""
    num = np.abs(out - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def oracle_decode_check(layer: Layer, idx: wi.IndexTensors, q_np, L, n_r, out, lse, sel,
                        heads=None):
    """Compare one GPU decode step with the oracle (run on the GPU's index and selection)."""
    G = layer.Hq // layer.H
    kc = to_np16(layer.k_out)
    vc = to_np16(layer.v_out)
    worst = 0.0
    for b in range(layer.B):
        for g in range(layer.H):
            if heads is not None and (b, g) not in heads:
                continue
            hi = head_index(idx, b, g)
            qg = q_np[b, g * G:(g + 1) * G]
            free = wo.decode_group(qg, kc[b, g], vc[b, g], hi, layer.L0, L, layer.n_sink,
                                   layer.n_recent, n_r)
            chosen = check_selection(free.group_score, hi.size, n_r, sel[b, g])
            r = wo.decode_group(qg, kc[b, g], vc[b, g], hi, layer.L0, L, layer.n_sink,
                                layer.n_recent, n_r, selected=chosen)
            e = row_rel_err(out[b, g * G:(g + 1) * G], r.out)
            assert e <= OUT_TOL, (b, g, e)
            assert np.all(np.abs(lse[b, g * G:(g + 1) * G] - r.lse) <= OUT_TOL), (b, g)
            worst = max(worst, e)
    return worst


def ragged_layer(rng, B=1, H=2, Hq=4, L0=700, steps=3, S=256, kseg=24, T=3, n_sink=3,
                 n_recent=17, n_topics=12, spread=0.6):
    """Small topic-structured keys (RoPE-free) for shape / edge-case tests."""
    d = 128
    L = L0 + steps
    k = np.empty((B, H, L, d), np.uint16)
    v = np.empty((B, H, L, d), np.uint16)
    for b in range(B):
        for g in range(H):
            topics = rng.standard_normal((n_topics, d))
            z = np.repeat(rng.integers(0, n_topics, size=L // 16 + 1), 16)[:L]
            k[b, g] = f32_bits(topics[z] + spread * rng.standard_normal((L, d)))
            v[b, g] = f32_bits(rng.standard_normal((L, d)))
    q = f32_bits(rng.standard_normal((steps, B, Hq, d)) * 1.5)
    return Layer(k, v, L0, S, kseg, T, n_sink, n_recent, Hq), q


def f32_bits(x) -> np.ndarray:
    t = torch()
    return t.from_numpy(np.asarray(x, np.float32)).to(t.bfloat16).view(t.int16).numpy().view(
        np.uint16)


def segment_ranges(layer: Layer):
    return wo.segment_ranges(layer.L0, layer.S, layer.n_sink, layer.n_recent)


def n_valid(kseg: int, n: int) -> int:
    return kseg if n >= kseg else n


def sqrt_d() -> float:
    return math.sqrt(128)


def check_segments(layer: Layer, idx: wi.IndexTensors, picks, objective_heads=()):
    """Index parity on sampled segments and heads, given the GPU's own labels.

    For each (b, g, s) in picks: labels = the oracle's assignment from the GPU's last
    centroids (ties within 1e-4); sizes, offsets and permuted K / V rows bit-exact; centroid
    means and value sums within 1 bf16 ulp (bf16_close). For each (b, g) in objective_heads:
    the GPU objective equals the oracle's J of the GPU labels over every segment of the head
    (1e-4 relative). Works segment by segment, so that it stays cheap at 1M tokens."""
    segs = segment_ranges(layer)
    k = layer.kseg
    labels_all = idx.labels.cpu().numpy()
    for (b, g, s) in picks:
        lo, hi = segs[s]
        c0, c1 = s * k, (s + 1) * k
        loc = labels_all[b, g, lo:hi] - c0
        Kseg = wo.bf16_to_f64(layer.k_np[b, g, lo:hi])
        Vseg = wo.bf16_to_f64(layer.v_np[b, g, lo:hi])
        Xhat = wo.normalise_rows(Kseg)
        last = to_np16(idx.last_centroids[b, g, c0:c1])
        check_assignment(Xhat, last, n_valid(k, hi - lo), loc)
        size, off, order = wo.finalise_segment(lo, loc, k)
        assert np.array_equal(idx.cluster_size[b, g, c0:c1].cpu().numpy(), size), (b, g, s)
        assert np.array_equal(idx.cluster_offset[b, g, c0:c1].cpu().numpy(), off), (b, g, s)
        if hi > lo:
            assert np.array_equal(to_np16(layer.k_out[b, g, lo:hi]), layer.k_np[b, g, order])
            assert np.array_equal(to_np16(layer.v_out[b, g, lo:hi]), layer.v_np[b, g, order])
        cm, vs = wo.cluster_stats(Kseg, Vseg, 0, loc, k)
        assert bf16_close(to_np16(idx.centroid_mean[b, g, c0:c1]), cm) <= 1, (b, g, s)
        assert bf16_close(to_np16(idx.value_sum[b, g, c0:c1]), vs) <= 1, (b, g, s)
    if objective_heads:
        obj = idx.objective.cpu().numpy()
        for (b, g) in objective_heads:
            J = 0.0
            for s, (lo, hi) in enumerate(segs):
                loc = labels_all[b, g, lo:hi] - s * k
                Xhat = wo.normalise_rows(wo.bf16_to_f64(layer.k_np[b, g, lo:hi]))
                J += wo.kmeans_objective(wo.kmeans_cluster_sums(Xhat, loc, k))
            assert abs(obj[b, g] - J) <= 1e-4 * abs(J), (b, g, obj[b, g], J)


def check_update_step(layer: Layer, idx_prev: wi.IndexTensors, idx_next: wi.IndexTensors,
                      picks):
    """One k-means update at full size: idx_prev was built with T - 1 passes and idx_next
    with T. The unit centroids of idx_next's last pass (mu^(T-1)) must equal the oracle's
    update of the (T-1)-th pass's labels (idx_prev.labels) from the centroids that pass used
    (idx_prev.last_centroids, mu^(T-2)), within 1 bf16 ulp, on the sampled (b, g, s)."""
    segs = segment_ranges(layer)
    k = layer.kseg
    for (b, g, s) in picks:
        lo, hi = segs[s]
        c0, c1 = s * k, (s + 1) * k
        loc = idx_prev.labels[b, g, lo:hi].cpu().numpy() - c0
        Xhat = wo.normalise_rows(wo.bf16_to_f64(layer.k_np[b, g, lo:hi]))
        mu_prev = to_np16(idx_prev.last_centroids[b, g, c0:c1])
        u = wo.kmeans_cluster_sums(Xhat, loc, k)
        ref = wo.kmeans_update(u, np.bincount(loc, minlength=k), mu_prev)
        got = to_np16(idx_next.last_centroids[b, g, c0:c1])
        assert bf16_close(got, ref) <= 1, (b, g, s)
