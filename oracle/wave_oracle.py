"""Wave-index oracle: a plain, slow, fp64 CPU implementation of the hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU-baseline leg
may import or call this module; the product path never does, and this module imports nothing
from the product package. It shares no code with the HIP library.

What it computes (the RetroInfer wave index, per batch element b and KV head g):

* Index build (segmented spherical k-means). The summaries say the index clusters the
  keys of each segment of the context locally (gist.science/de §2A "Segmented Clustering";
  gist.science/fr §2A; gist.science/zh §2A 分段聚类), that the clustering is spherical
  k-means (gist.science/fr §2A item 2), and that estimation uses cluster centroids together
  with precomputed per-cluster value sums (gist.science/zh §2A 估计区). Sizes n_j follow
  from the estimate, the member map from "compute the retrieved clusters' tokens exactly".
* Tripartite decode attention (all three summaries §2A, and the abstract's "tripartite
  attention approximation"): exact attention over the steady zone (tokens at the start and
  the end of the context) and over the tokens of the clusters most similar to the query
  (retrieval zone), plus a centroid-based estimate for every other cluster (estimation
  zone), combined into one softmax.

Readings taken where the pages are silent (each is listed in the design notes):
  R1  the centroid that scores retrieval and drives estimation is the arithmetic mean of
      the cluster's raw keys (Jensen's bound, gist.science/zh §2A, needs the mean);
      the unit centroid mu_j of spherical k-means is build-internal.
  R2  steady tokens are not clustered; every token is in exactly one zone.
  R3  segments are aligned to absolute positions [sS, (s+1)S); each has k_seg clusters.
  R4  spherical k-means: cosine assignment, normalised-sum update, an empty cluster keeps
      its centroid, T = number of assignment passes, seeds at stride floor(n_s/k_seg).
  R5  assignment ties go to the lowest local cluster id.
  R6  GQA: one retrieval set per KV head, ranked by the mean of the group's logits;
      estimation uses each query head's own logits.
  R7  top-k ties go to the lower global cluster id; the budget is an integer n_r.
  R8  empty clusters are never retrieved and add nothing to the estimate.
  R9  softmax scale 1/sqrt(d) unless given.
  R11 centroid means and value sums are stored in bf16 (round to nearest even).

Precision: every sum is fp64 over the exact values of the bf16 inputs; stored bf16
outputs are rounded once, to nearest even, from fp64.

Pins: every function here is checked in tests/test_oracle_pins.py against closed forms,
invariants, library routines (torch scaled_dot_product_attention in fp64, Python's sort)
and a hand-worked example (tests/golden/). The accuracy of the approximation against
exact attention on real models has no pin in the pages ("parity unpinned"); it is only
measured.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# --------------------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) in one rounding; return bits.

    bf16 keeps 8 significant bits. For |x| in [2^(e-1), 2^e) the spacing of bf16 numbers is
    2^(e-8); below the smallest normal (2^-126) it is the fixed subnormal spacing 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2^e with 0.5 <= |m| < 1 (e = 0 for x = 0)
    e = np.maximum(e, -125)                  # subnormal range: fixed spacing 2^-133
    quantum = np.ldexp(1.0, e - 8)
    y = np.rint(x / quantum) * quantum       # np.rint rounds half to even; both steps exact
    y = np.where(np.abs(y) > 3.3895313892515355e38, np.copysign(np.inf, x), y)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------------------
# Index build: segmented spherical k-means, then per-cluster statistics
# --------------------------------------------------------------------------------------


def segment_ranges(L0: int, S: int, n_sink: int, n_recent: int) -> list[tuple[int, int]]:
    """Indexed positions of each segment (reading R2/R3).

    Indexed positions are [n_sink, L0 - n_recent); segment s covers the absolute positions
    [s*S, min((s+1)*S, L0)). Returns (lo, hi) per segment (hi <= lo means no points).
    """
    n_seg = -(-L0 // S)
    lo_all, hi_all = n_sink, L0 - n_recent
    out = []
    for s in range(n_seg):
        lo = max(s * S, lo_all)
        hi = min((s + 1) * S, L0, hi_all)
        out.append((lo, max(hi, lo)))
    return out


def normalise_rows(X: np.ndarray) -> np.ndarray:
    """x_hat_i = x_i / ||x_i|| (a zero row stays zero)."""
    r = np.sqrt(np.sum(X * X, axis=1))
    out = np.zeros_like(X)
    nz = r > 0
    out[nz] = X[nz] / r[nz, None]
    return out


def kmeans_seeds(Xhat: np.ndarray, k_seg: int) -> tuple[np.ndarray, int]:
    """Initial unit centroids (reading R4): strided points of the segment.

    With n_s >= k_seg points, centroid j starts at point j*floor(n_s/k_seg); with fewer, the
    first n_s clusters start at points 0..n_s-1 and the rest stay empty for good.
    Returns (mu bf16 bits [k_seg, d], n_valid).
    """
    n_s, d = Xhat.shape
    mu = np.zeros((k_seg, d), dtype=np.uint16)
    if n_s >= k_seg:
        stride = n_s // k_seg
        mu[:] = round_bf16(Xhat[np.arange(k_seg) * stride])
        return mu, k_seg
    mu[:n_s] = round_bf16(Xhat)
    return mu, n_s


def kmeans_assign(Xhat: np.ndarray, mu_bits: np.ndarray, n_valid: int) -> np.ndarray:
    """a_i = argmax_j cos(x_i, mu_j) over the n_valid usable centroids; ties -> lowest j."""
    if Xhat.shape[0] == 0:
        return np.zeros(0, dtype=np.int64)
    scores = Xhat @ bf16_to_f64(mu_bits[:n_valid]).T
    return np.argmax(scores, axis=1)          # first maximum = lowest index


def kmeans_cluster_sums(Xhat: np.ndarray, labels: np.ndarray, k_seg: int) -> np.ndarray:
    """u_j = sum of the unit points assigned to cluster j (fp64)."""
    u = np.zeros((k_seg, Xhat.shape[1]))
    for j in range(k_seg):
        u[j] = Xhat[labels == j].sum(axis=0)
    return u


def kmeans_update(u: np.ndarray, counts: np.ndarray, mu_prev_bits: np.ndarray) -> np.ndarray:
    """mu_j = bf16(u_j / ||u_j||) for a non-empty cluster; an empty cluster keeps mu_j."""
    mu = mu_prev_bits.copy()
    for j in range(u.shape[0]):
        if counts[j] > 0:
            nrm = math.sqrt(float(u[j] @ u[j]))
            mu[j] = round_bf16(u[j] / nrm) if nrm > 0 else round_bf16(np.zeros_like(u[j]))
    return mu


def kmeans_objective(u: np.ndarray) -> float:
    """Spherical k-means objective J = sum_j ||u_j|| (= sum_i cos(x_i, direction of u_{a_i}))."""
    return float(np.sum(np.sqrt(np.sum(u * u, axis=1))))


@dataclass
class SegmentClustering:
    labels: np.ndarray            # final local labels a^(T), [n_s]
    last_centroids: np.ndarray    # bf16 bits [k_seg, d]: the centroids used by the last pass
    objective: float              # J from the final labels
    n_valid: int
    history: list                 # mu^(0..T-1) bf16 bits (for step-wise checks)


def cluster_segment(X: np.ndarray, k_seg: int, n_iters: int) -> SegmentClustering:
    """Spherical k-means over one segment's raw keys X (fp64 [n_s, d]), n_iters passes."""
    Xhat = normalise_rows(X)
    mu, n_valid = kmeans_seeds(Xhat, k_seg)
    history = []
    labels = np.zeros(X.shape[0], dtype=np.int64)
    u = np.zeros((k_seg, X.shape[1]))
    for t in range(1, n_iters + 1):
        history.append(mu)
        labels = kmeans_assign(Xhat, mu, n_valid)
        u = kmeans_cluster_sums(Xhat, labels, k_seg)
        if t < n_iters:
            counts = np.bincount(labels, minlength=k_seg)
            mu = kmeans_update(u, counts, mu)
    return SegmentClustering(labels, history[-1] if history else mu, kmeans_objective(u),
                             n_valid, history)


@dataclass
class HeadIndex:
    """The wave index of one (batch element, KV head), in the library's layout."""
    centroid_mean: np.ndarray     # bf16 bits [C, d]: mean raw key of each cluster (R1)
    value_sum: np.ndarray         # bf16 bits [C, d]: sum of the cluster's value rows
    size: np.ndarray              # int32 [C]
    offset: np.ndarray            # int32 [C]: first slot of the cluster in the permuted cache
    labels: np.ndarray            # int32 [L0]: global cluster id, -1 for steady tokens
    perm: np.ndarray              # int32 [L0]: perm[slot] = source position of that row
    last_centroids: np.ndarray    # bf16 bits [C, d]
    objective: np.ndarray         # float64 [n_seg]: J per segment


def finalise_segment(lo: int, local_labels: np.ndarray, k_seg: int):
    """Sizes, offsets and the cluster-contiguous order of one segment's slots [lo, lo+n_s).

    Clusters are laid out in ascending local id; inside a cluster, in ascending position.
    Returns (size [k_seg], offset [k_seg], order: source positions in slot order).
    """
    size = np.bincount(local_labels, minlength=k_seg).astype(np.int64)
    offset = lo + np.concatenate([[0], np.cumsum(size)[:-1]])
    order = []
    for j in range(k_seg):
        order.extend((lo + np.nonzero(local_labels == j)[0]).tolist())
    return size, offset, np.asarray(order, dtype=np.int64)


def cluster_stats(K: np.ndarray, V: np.ndarray, lo: int, local_labels: np.ndarray,
                  k_seg: int) -> tuple[np.ndarray, np.ndarray]:
    """Mean raw key and value sum of each cluster of the segment whose points start at
    position lo (K, V: fp64 rows indexed by absolute position), both bf16 (reading R1, R11;
    gist.science/zh §2A: centroids plus precomputed value sums). Empty clusters are zero."""
    d = K.shape[1]
    cmean = np.zeros((k_seg, d), dtype=np.uint16)
    vsum = np.zeros((k_seg, d), dtype=np.uint16)
    for j in range(k_seg):
        members = lo + np.nonzero(local_labels == j)[0]
        if len(members):
            cmean[j] = round_bf16(K[members].sum(axis=0) / len(members))
            vsum[j] = round_bf16(V[members].sum(axis=0))
    return cmean, vsum


def build_head(Kb: np.ndarray, Vb: np.ndarray, L0: int, S: int, k_seg: int, n_iters: int,
               n_sink: int, n_recent: int, labels_override: np.ndarray | None = None,
               ) -> tuple[HeadIndex, np.ndarray, np.ndarray]:
    """Build the wave index of one (b, KV head) from bf16 key/value bits [>=L0, d].

    If labels_override (global ids [L0], -1 for steady) is given, clustering is skipped and
    the statistics and layout are computed from those labels (used to check a given label
    set step-wise). Returns (index, K_out bits [L0, d], V_out bits [L0, d]).
    """
    K = bf16_to_f64(Kb[:L0])
    V = bf16_to_f64(Vb[:L0])
    d = K.shape[1]
    segs = segment_ranges(L0, S, n_sink, n_recent)
    C = len(segs) * k_seg
    cmean = np.zeros((C, d), dtype=np.uint16)
    vsum = np.zeros((C, d), dtype=np.uint16)
    size = np.zeros(C, dtype=np.int32)
    offset = np.zeros(C, dtype=np.int32)
    labels = np.full(L0, -1, dtype=np.int32)
    perm = np.arange(L0, dtype=np.int32)
    last = np.zeros((C, d), dtype=np.uint16)
    obj = np.zeros(len(segs))
    for s, (lo, hi) in enumerate(segs):
        base = s * k_seg
        if labels_override is None:
            cl = cluster_segment(K[lo:hi], k_seg, n_iters)
            loc = cl.labels
            last[base:base + k_seg] = cl.last_centroids
            obj[s] = cl.objective
        else:
            loc = labels_override[lo:hi].astype(np.int64) - base
            assert np.all((loc >= 0) & (loc < k_seg)), "label outside its segment"
            u = kmeans_cluster_sums(normalise_rows(K[lo:hi]), loc, k_seg)
            obj[s] = kmeans_objective(u)
        labels[lo:hi] = base + loc
        sz, off, order = finalise_segment(lo, loc, k_seg)
        size[base:base + k_seg] = sz
        offset[base:base + k_seg] = off
        perm[lo:hi] = order
        cmean[base:base + k_seg], vsum[base:base + k_seg] = cluster_stats(K, V, lo, loc, k_seg)
    K_out = Kb[:L0][perm]
    V_out = Vb[:L0][perm]
    return HeadIndex(cmean, vsum, size, offset, labels, perm, last, obj), K_out, V_out


# --------------------------------------------------------------------------------------
# Decode: tripartite attention
# --------------------------------------------------------------------------------------


@dataclass
class HeadGroupDecode:
    out: np.ndarray        # [G, d] float64
    lse: np.ndarray        # [G]
    selected: np.ndarray   # retrieved global cluster ids, ascending
    group_score: np.ndarray  # s_hat [C] (-inf for empty clusters)
    score: np.ndarray      # s [G, C]


def select_clusters(group_score: np.ndarray, size: np.ndarray, n_retrieve: int) -> np.ndarray:
    """Retrieval zone (R6-R8): the n_r highest group scores among non-empty clusters, ties to
    the lower id; all non-empty clusters if there are fewer. Returned in ascending id order."""
    ids = np.nonzero(size > 0)[0]
    order = np.lexsort((ids, -group_score[ids]))   # primary: -score, secondary: id
    return np.sort(ids[order[:n_retrieve]])


def decode_group(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, idx: HeadIndex, L0: int, L: int,
                 n_sink: int, n_recent: int, n_retrieve: int, scale: float | None = None,
                 selected: np.ndarray | None = None) -> HeadGroupDecode:
    """Tripartite attention of the G query heads that share one KV head.

    q: bf16 bits [G, d]. Kc, Vc: bf16 bits [>=L, d], the permuted cache (slots of the index
    layout for [0, L0), appended decode tokens at [L0, L)). `selected` forces the retrieved
    set (used to compare with a given selection).
    """
    Q = bf16_to_f64(q)
    G, d = Q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cmean = bf16_to_f64(idx.centroid_mean)
    vsum = bf16_to_f64(idx.value_sum)
    nonempty = idx.size > 0
    # 1. logits of every cluster centroid, per query head, and their group mean (R1, R6)
    s = scale * (Q @ cmean.T)
    s[:, ~nonempty] = -np.inf
    s_hat = s.mean(axis=0)
    # 2. retrieval zone
    R = select_clusters(s_hat, idx.size, n_retrieve) if selected is None else np.sort(selected)
    # 3. exact tokens: steady zone (sink + recent, plus appended tokens) and retrieved members
    steady = list(range(0, n_sink)) + list(range(L0 - n_recent, L))
    members = [t for j in R for t in range(idx.offset[j], idx.offset[j] + idx.size[j])]
    E = np.asarray(steady + members, dtype=np.int64)
    U = np.setdiff1d(np.nonzero(nonempty)[0], R)
    Ke = bf16_to_f64(Kc[E])
    Ve = bf16_to_f64(Vc[E])
    out = np.zeros((G, d))
    lse = np.zeros(G)
    for h in range(G):
        a = scale * (Ke @ Q[h])                  # exact logits
        su = s[h, U]                             # centroid logits of the estimation zone
        M = max(a.max() if a.size else -np.inf, su.max() if su.size else -np.inf)
        pe = np.exp(a - M)
        pu = np.exp(su - M)
        num = pe @ Ve + pu @ vsum[U]             # estimate: e^{s_j} * (sum of values)
        den = pe.sum() + pu @ idx.size[U]        # estimate: n_j * e^{s_j}
        out[h] = num / den
        lse[h] = M + math.log(den)
    return HeadGroupDecode(out, lse, R, s_hat, s)


def full_attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, L: int,
                   scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of q (bf16 bits [G, d]) over the first L cache rows."""
    Q = bf16_to_f64(q)
    K = bf16_to_f64(Kc[:L])
    V = bf16_to_f64(Vc[:L])
    scale = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    a = scale * (Q @ K.T)
    M = a.max(axis=1, keepdims=True)
    p = np.exp(a - M)
    den = p.sum(axis=1)
    return (p @ V) / den[:, None], M[:, 0] + np.log(den)


# --------------------------------------------------------------------------------------
# Whole-layer drivers (loops over batch elements and KV heads)
# --------------------------------------------------------------------------------------


@dataclass
class LayerIndex:
    heads: list            # [B][Hkv] HeadIndex
    k_out: np.ndarray      # bf16 bits [B, Hkv, L0, d]
    v_out: np.ndarray

    def stacked(self, field_name: str) -> np.ndarray:
        return np.stack([np.stack([getattr(h, field_name) for h in row]) for row in self.heads])


def build_layer(K: np.ndarray, V: np.ndarray, L0: int, S: int, k_seg: int, n_iters: int,
                n_sink: int, n_recent: int, labels_override: np.ndarray | None = None,
                heads: list | None = None) -> LayerIndex:
    """Build the index for K, V bf16 bits [B, Hkv, >=L0, d] (optionally only some heads)."""
    B, H = K.shape[:2]
    rows, kout, vout = [], np.zeros((B, H, L0, K.shape[3]), np.uint16), None
    vout = np.zeros_like(kout)
    for b in range(B):
        row = []
        for g in range(H):
            if heads is not None and (b, g) not in heads:
                row.append(None)
                continue
            lab = None if labels_override is None else labels_override[b, g]
            hi, ko, vo = build_head(K[b, g], V[b, g], L0, S, k_seg, n_iters, n_sink, n_recent, lab)
            row.append(hi)
            kout[b, g], vout[b, g] = ko, vo
        rows.append(row)
    return LayerIndex(rows, kout, vout)


def decode_layer(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, index: LayerIndex, L0: int,
                 L: int, n_sink: int, n_recent: int, n_retrieve: int,
                 scale: float | None = None, selected: np.ndarray | None = None):
    """Decode one step for q bf16 bits [B, Hq, d]; returns (out [B,Hq,d], lse [B,Hq],
    selected [B, Hkv] list of id arrays, group scores [B, Hkv, C])."""
    B, Hq, d = q.shape
    H = Kc.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    sel, shat = [], []
    for b in range(B):
        sel_b, sh_b = [], []
        for g in range(H):
            forced = None if selected is None else selected[b][g]
            r = decode_group(q[b, g * G:(g + 1) * G], Kc[b, g], Vc[b, g], index.heads[b][g],
                             L0, L, n_sink, n_recent, n_retrieve, scale, forced)
            out[b, g * G:(g + 1) * G] = r.out
            lse[b, g * G:(g + 1) * G] = r.lse
            sel_b.append(r.selected)
            sh_b.append(r.group_score)
        sel.append(sel_b)
        shat.append(sh_b)
    return out, lse, sel, np.asarray(shat)
