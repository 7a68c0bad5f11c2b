"""Attention-aware vector search oracle: a plain, slow CPU implementation of the second
retrieval zone.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU-baseline leg
may import or call this module; the product path never does, and this module imports nothing
from the product package. It shares no code with the HIP library.

What it computes follows the RetrievalAttention abstract (jarxiv.com, "RetrievalAttention:
Accelerating Long-Context LLM Inference via Vector Retrieval", abstract): the keys of the
context are held in an approximate-nearest-neighbour index, a decode step retrieves the
keys most relevant to its query by a vector search, and attention runs over the retrieved
tokens; off-the-shelf indexes fail because decode queries and keys follow different
distributions, so the search structure is adapted to the distribution of the queries. The
abstract gives no algorithm; these readings fill it in (each is listed in the design notes):

  A1  the index covers the indexed zone [n_sink, L0 - n_recent) of the context; node x is
      position n_sink + x. The steady zone (sink and recent tokens, and tokens appended
      during decode) is attended exactly, as in the wave index.
  A2  relevance is the inner product q.k (the attention logit before scaling).
  A3  query awareness comes from training queries (the prefill queries of the KV head's
      group): each training query t lists its M best keys by exact inner product, in
      (score descending, id ascending) order. The list's first key is linked to every
      other key of the list and each of them back to it (a star per training query). A
      key keeps at most R neighbours, taken without repeats in the order of its
      postings (its place r in a list, then the list's index t): where it heads a list,
      the list's other keys in list order, else the list's head.
  A4  GQA: one retrieval set per KV head, searched with the sum of the group's query
      vectors (the ranking of the group-mean logit).
  A5  the search seeds its pool with the heads of the n_entry training queries whose inner
      product with the search vector is largest, then repeats rounds: the W best pool
      entries not yet expanded are expanded (their unvisited neighbours are scored), and
      the pool keeps its ef best entries, until every pool entry is expanded or max_rounds
      rounds have run. The k best pool entries are retrieved.
  A6  precision of the search's decisions: the search vector is the fp32 sum of the bf16
      query rows in head order. A score is an fp32 inner product in a fixed order: the
      fp32 products of each block of 8 consecutive dims are summed in dim order, and the
      d/8 block sums are combined by a balanced pairwise tree (neighbours first); every
      product and sum is rounded to fp32, with no fused multiply-add. Ties go to the lower
      id.
  A7  attention runs over the steady zone and the retrieved tokens only (no estimate of
      the rest), one softmax, in fp64.

Pins: tests/test_oracle_pins_anns.py (exact rational arithmetic for the lists, a
hand-worked graph and search in tests/golden/, a complete graph that must return the exact
top-k, a cancellation case that fixes the summation order, torch's fp64 attention).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .wave_oracle import bf16_to_f64


def node_range(L0: int, n_sink: int, n_recent: int) -> tuple[int, int]:
    """Positions [lo, hi) of the indexed zone (A1); empty when the steady zone covers L0."""
    lo, hi = n_sink, L0 - n_recent
    return (lo, max(lo, hi))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------------------
# Build: training lists (A3) and the graph
# --------------------------------------------------------------------------------------


def train_lists(keys: np.ndarray, train: np.ndarray, M: int) -> tuple[np.ndarray, np.ndarray]:
    """For each training query (bf16 bits [n_t, d]) the M nodes (bf16 key rows [N, d]) of
    largest inner product, in (score descending, id ascending) order, computed in fp64; -1
    pads when N < M. Returns (ids int32 [n_t, M], scores fp64 [n_t, M])."""
    K = bf16_to_f64(keys)
    T = bf16_to_f64(train)
    n_t, N = T.shape[0], K.shape[0]
    ids = np.full((n_t, M), -1, dtype=np.int32)
    sc = np.full((n_t, M), -np.inf)
    if N == 0:
        return ids, sc
    S = T @ K.T
    node = np.arange(N)
    m = min(M, N)
    for t in range(n_t):
        order = np.lexsort((node, -S[t]))[:m]    # primary: -score, secondary: id
        ids[t, :m] = order
        sc[t, :m] = S[t, order]
    return ids, sc


def link(lists: np.ndarray, N: int, R: int) -> np.ndarray:
    """The graph of A3 from the training lists (int [n_t, M], -1 padded): adjacency int32
    [N, R], -1 padded."""
    n_t, M = lists.shape
    postings = [[] for _ in range(N)]
    for t in range(n_t):
        for r in range(M):
            x = int(lists[t, r])
            if x >= 0:
                postings[x].append((r, t))
    adj = np.full((N, R), -1, dtype=np.int32)
    for x in range(N):
        taken: list[int] = []
        for r, t in sorted(postings[x]):
            cands = [int(y) for y in lists[t, 1:]] if r == 0 else [int(lists[t, 0])]
            for y in cands:
                if len(taken) == R:
                    break
                if y >= 0 and y not in taken:
                    taken.append(y)
            if len(taken) == R:
                break
        adj[x, :len(taken)] = taken
    return adj


@dataclass
class HeadGraph:
    lists: np.ndarray      # [n_t, M] training lists (node ids)
    adj: np.ndarray        # [N, R]
    entry: np.ndarray      # [n_t] each training query's first node (-1 if none)


def build_head(Kb: np.ndarray, train: np.ndarray, L0: int, n_sink: int, n_recent: int, M: int,
               R: int, lists: np.ndarray | None = None) -> HeadGraph:
    """The graph of one (b, kv-head): K bf16 bits [>=L0, d] (positions), training queries
    bf16 bits [n_t, d]. `lists` replaces the training lists (to link a given set)."""
    lo, hi = node_range(L0, n_sink, n_recent)
    if lists is None:
        lists, _ = train_lists(Kb[lo:hi], train, M)
    adj = link(lists, hi - lo, R)
    return HeadGraph(lists, adj, lists[:, 0].copy())


# --------------------------------------------------------------------------------------
# Search (A4-A6)
# --------------------------------------------------------------------------------------


def group_vector(q: np.ndarray) -> np.ndarray:
    """Sum of the group's query rows (bf16 bits [G, d]) in fp32, head by head (A4, A6)."""
    Q = bf16_to_f32(q)
    s = Q[0].copy()
    for h in range(1, Q.shape[0]):
        s = (s + Q[h]).astype(np.float32)
    return s


SCORE_BLOCK = 8   # dims summed in order before the pairwise tree (A6)


def scores_f32(u: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """fp32 inner products of u (float32 [d]) with bf16 rows [n, d] in the order of A6: each
    block of 8 dims (the whole row when d < 8) summed in dim order, then the block sums
    combined pairwise, neighbours first; every product and sum rounded to fp32. The number
    of blocks must be a power of two."""
    X = bf16_to_f32(rows)
    n, d = X.shape
    blk = min(SCORE_BLOCK, d)
    nb = d // blk
    assert nb * blk == d and nb & (nb - 1) == 0, "d / 8 must be a power of two"
    sums = []
    for b in range(nb):
        acc = np.zeros(n, dtype=np.float32)
        for i in range(b * blk, (b + 1) * blk):
            acc = (acc + (u[i] * X[:, i]).astype(np.float32)).astype(np.float32)
        sums.append(acc)
    while len(sums) > 1:
        sums = [(sums[j] + sums[j + 1]).astype(np.float32) for j in range(0, len(sums), 2)]
    return sums[0]


def best_first(score: np.ndarray, ids: np.ndarray, n: int) -> np.ndarray:
    """Positions of the n best (score descending, id ascending) entries."""
    return np.lexsort((ids, -score.astype(np.float64)))[:n]


@dataclass
class SearchResult:
    ids: np.ndarray        # [k] retrieved nodes, best first (-1 pads)
    scores: np.ndarray     # [k] their fp32 scores
    rounds: int            # expansion rounds run
    visited: int           # nodes scored


def search(u: np.ndarray, keys: np.ndarray, train: np.ndarray, entry: np.ndarray,
           adj: np.ndarray, n_entry: int, ef: int, W: int, k: int,
           max_rounds: int) -> SearchResult:
    """Beam search of A5 for the search vector u (float32 [d]) over the nodes (bf16 key rows
    [N, d]) with the graph `adj` [N, R] and the training queries' heads `entry` [n_t]."""
    n_t = train.shape[0]
    # seeds: the heads of the n_entry training queries nearest u
    ts = scores_f32(u, train)
    top_t = best_first(ts, np.arange(n_t), min(n_entry, n_t))
    seeds = sorted({int(entry[t]) for t in top_t if entry[t] >= 0})
    visited = set(seeds)
    pool_id = np.asarray(seeds, dtype=np.int64)
    pool_sc = scores_f32(u, keys[pool_id]) if len(seeds) else np.zeros(0, np.float32)
    keep = best_first(pool_sc, pool_id, ef)
    pool_id, pool_sc = pool_id[keep], pool_sc[keep]
    expanded = np.zeros(len(pool_id), dtype=bool)
    rounds = 0
    while rounds < max_rounds:
        todo = np.nonzero(~expanded)[0][:W]
        if len(todo) == 0:
            break
        expanded[todo] = True
        new = []
        for pos in todo:
            for y in adj[pool_id[pos]]:
                y = int(y)
                if y >= 0 and y not in visited:
                    visited.add(y)
                    new.append(y)
        new_id = np.asarray(new, dtype=np.int64)
        new_sc = scores_f32(u, keys[new_id]) if len(new) else np.zeros(0, np.float32)
        all_id = np.concatenate([pool_id, new_id])
        all_sc = np.concatenate([pool_sc, new_sc])
        all_ex = np.concatenate([expanded, np.zeros(len(new), dtype=bool)])
        keep = best_first(all_sc, all_id, ef)
        pool_id, pool_sc, expanded = all_id[keep], all_sc[keep], all_ex[keep]
        rounds += 1
    out_id = np.full(k, -1, dtype=np.int32)
    out_sc = np.full(k, -np.inf, dtype=np.float32)
    m = min(k, len(pool_id))
    out_id[:m] = pool_id[:m]
    out_sc[:m] = pool_sc[:m]
    return SearchResult(out_id, out_sc, rounds, len(visited))


# --------------------------------------------------------------------------------------
# Attention over the steady zone and the retrieved tokens (A7)
# --------------------------------------------------------------------------------------


def steady_rows(L0: int, L: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Cache rows of the steady zone: the sink, then the recent rows and appended tokens
    (n_sink + n_recent <= L0)."""
    return np.asarray(list(range(0, n_sink)) + list(range(L0 - n_recent, L)), dtype=np.int64)


def attend(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, rows: np.ndarray,
           scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of q (bf16 bits [G, d]) over the cache rows `rows` in fp64:
    (out [G, d], lse [G])."""
    Q = bf16_to_f64(q)
    K = bf16_to_f64(Kc[rows])
    V = bf16_to_f64(Vc[rows])
    scale = 1.0 / math.sqrt(Q.shape[1]) if scale is None else scale
    a = scale * (Q @ K.T)
    M = a.max(axis=1, keepdims=True)
    p = np.exp(a - M)
    den = p.sum(axis=1)
    return (p @ V) / den[:, None], M[:, 0] + np.log(den)


@dataclass
class GroupStep:
    out: np.ndarray        # [G, d]
    lse: np.ndarray        # [G]
    retrieved: np.ndarray  # [k] positions, best first (-1 pads)
    search: SearchResult


def decode_group(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, graph: HeadGraph,
                 train: np.ndarray, L0: int, L: int, n_sink: int, n_recent: int, n_entry: int,
                 ef: int, W: int, k: int, max_rounds: int, scale: float | None = None,
                 retrieved: np.ndarray | None = None) -> GroupStep:
    """One decode step of the G query heads of a KV head: the search over the graph, then
    attention over the steady zone and the retrieved tokens. `retrieved` (positions) forces
    the retrieved set."""
    lo, hi = node_range(L0, n_sink, n_recent)
    res = search(group_vector(q), Kc[lo:hi], train, graph.entry, graph.adj, n_entry, ef, W, k,
                 max_rounds)
    pos = np.where(res.ids >= 0, res.ids + lo, -1) if retrieved is None else np.asarray(retrieved)
    rows = np.concatenate([steady_rows(L0, L, n_sink, n_recent), pos[pos >= 0].astype(np.int64)])
    out, lse = attend(q, Kc, Vc, rows, scale)
    return GroupStep(out, lse, pos.astype(np.int32), res)
