"""Pins for the attention-aware vector search oracle (oracle/anns_oracle.py).

The expected values come from exact rational arithmetic (Python's fractions and integers),
hand-worked examples (tests/golden/anns_hand_worked.json), reductions to brute force (a
complete graph), a library routine (torch's scaled_dot_product_attention in fp64) and
cancellation cases whose fp32 results are worked by hand. None compares the oracle with
itself.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import anns_oracle as ao

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "anns_hand_worked.json")


def bits(x):
    """float values -> bf16 bit patterns via torch's own conversion (round to nearest even)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def vals(b):
    return torch.from_numpy(np.asarray(b, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).double().numpy()


@pytest.fixture
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# training lists: exact rational ranking
# ------------------------------------------------------------------------------------------

def test_train_lists_equal_the_exact_rational_ranking(rng):
    """Each list is the M best nodes by the exact inner product (fractions of the bf16
    values), ties to the lower id; duplicate keys make exact ties."""
    N, n_t, d, M = 40, 6, 8, 7
    K = bits(rng.standard_normal((N, d)))
    K[3] = bits(4 * vals(K[3]))   # long enough to rank first for a query along it
    K[7] = K[3]          # exact ties
    K[30] = K[3]
    T = bits(rng.standard_normal((n_t, d)))
    T[2] = K[3]          # a training query that ranks the duplicates first
    ids, sc = ao.train_lists(K, T, M)
    Kf = [[Fraction(float(v)) for v in row] for row in vals(K)]
    Tf = [[Fraction(float(v)) for v in row] for row in vals(T)]
    for t in range(n_t):
        exact = [sum(a * b for a, b in zip(Tf[t], Kf[x])) for x in range(N)]
        want = sorted(range(N), key=lambda x: (-exact[x], x))[:M]
        assert ids[t].tolist() == want, t
        assert np.allclose(sc[t], [float(exact[x]) for x in want], rtol=1e-12, atol=0)
    assert ids[2, :3].tolist() == [3, 7, 30]


def test_train_lists_pad_when_there_are_fewer_nodes_than_m(rng):
    K = bits(rng.standard_normal((3, 4)))
    T = bits(rng.standard_normal((2, 4)))
    ids, _ = ao.train_lists(K, T, 5)
    assert (ids[:, 3:] == -1).all() and sorted(ids[0, :3].tolist()) == [0, 1, 2]
    ids0, _ = ao.train_lists(K[:0], T, 5)
    assert (ids0 == -1).all()


# ------------------------------------------------------------------------------------------
# the graph
# ------------------------------------------------------------------------------------------

def test_link_hand_worked(golden):
    g = golden["link"]
    lists = np.asarray(g["lists"], dtype=np.int32)
    adj = ao.link(lists, g["N"], g["R"])
    assert adj.tolist() == g["adj"]
    assert lists[:, 0].tolist() == g["entry"]


def test_link_invariants(rng):
    """Every edge joins two nodes of one list, one of them its head; no self loops or repeats;
    a row holds all of its node's neighbours when they number at most R; a node in no list
    has none."""
    N, n_t, M, R = 120, 60, 8, 6
    lists = np.stack([rng.permutation(N)[:M] for _ in range(n_t)]).astype(np.int32)
    lists[5, 6:] = -1                      # a short list
    adj = ao.link(lists, N, R)
    pairs = set()
    for t in range(n_t):
        row = [int(x) for x in lists[t] if x >= 0]
        for y in row[1:]:
            pairs.add((row[0], y))
            pairs.add((y, row[0]))
    in_lists = set(int(x) for x in lists.ravel() if x >= 0)
    for x in range(N):
        nb = [int(y) for y in adj[x] if y >= 0]
        assert (adj[x, len(nb):] == -1).all()
        assert len(set(nb)) == len(nb) and x not in nb
        assert all((x, y) in pairs for y in nb)
        allnb = {y for (a, y) in pairs if a == x}
        if len(allnb) <= R:
            assert set(nb) == allnb
        else:
            assert len(nb) == R
        if x not in in_lists:
            assert not nb


def test_link_prefers_the_nodes_own_lists_then_the_best_places():
    """A node heading a list takes that list's members before the heads of lists it merely
    belongs to; among those, the list where it ranks higher comes first."""
    lists = np.asarray([[9, 0, 1], [8, 2, 0], [0, 5, 6], [7, 0, 3]], dtype=np.int32)
    adj = ao.link(lists, 10, 4)
    # node 0 heads list 2 (members 5, 6), is 2nd in lists 0 and 3 (heads 9, 7), 3rd in list 1
    assert adj[0].tolist() == [5, 6, 9, 7]


# ------------------------------------------------------------------------------------------
# fp32 scores in a fixed order (A6)
# ------------------------------------------------------------------------------------------

def test_scores_accumulate_a_block_in_dim_order():
    """1 + 2^24 rounds to 2^24 in fp32 (tie to even), so the sum over dims in order of
    (2^24, 1, -2^24, 1) is 1; the reverse order, or an exact sum, gives 2."""
    u = np.ones(4, dtype=np.float32)
    row = bits([[2.0 ** 24, 1.0, -(2.0 ** 24), 1.0]])
    assert ao.scores_f32(u, row).tolist() == [1.0]
    assert ao.scores_f32(u, row[:, ::-1].copy()).tolist() == [2.0]


def test_scores_combine_blocks_pairwise():
    """Four blocks of 8 dims whose sums are (1, 2^24, 1, -2^24): pairwise, (1 + 2^24) rounds
    to 2^24 and (1 - 2^24) is exact, so the score is 1; a sum of the blocks in order would
    give 0 (2^24 + 1 rounds back to 2^24), the exact sum is 2."""
    u = np.ones(32, dtype=np.float32)
    x = np.zeros(32)
    x[0], x[8], x[16], x[24] = 1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)
    assert ao.scores_f32(u, bits([x])).tolist() == [1.0]
    # 16 blocks (d = 128): the same four sums in blocks 0, 1, 2, 3 meet first in pairs (0,1)
    # and (2,3), then in the pair of pairs; blocks 4..15 are zero
    u = np.ones(128, dtype=np.float32)
    x = np.zeros(128)
    x[0], x[8], x[16], x[24] = 1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)
    assert ao.scores_f32(u, bits([x])).tolist() == [1.0]
    # moved to blocks 0, 2, 1, 3 the pairs are (1, 1) and (2^24, -2^24): exact, 2
    x = np.zeros(128)
    x[0], x[16], x[8], x[24] = 1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)
    assert ao.scores_f32(u, bits([x])).tolist() == [2.0]


def test_scores_round_each_product():
    """(1 + 2^-23)(1 + 2^-7) = 1 + 2^-7 + 2^-23 + 2^-30 rounds to 1 + 2^-7 + 2^-23, which
    cancels the first term exactly; a fused multiply-add would leave 2^-30."""
    a = np.float32(1 + 2.0 ** -7 + 2.0 ** -23)
    u = np.asarray([-a, np.float32(1 + 2.0 ** -23)], dtype=np.float32)
    row = bits([[1.0, 1 + 2.0 ** -7]])
    assert ao.scores_f32(u, row).tolist() == [0.0]


def test_scores_are_exact_on_small_integers(rng):
    u = rng.integers(-8, 9, size=32).astype(np.float32)
    X = rng.integers(-8, 9, size=(50, 32))
    exact = X @ u.astype(np.int64)
    assert ao.scores_f32(u, bits(X)).tolist() == exact.astype(np.float32).tolist()


def test_group_vector_sums_heads_in_order():
    q = bits([[2.0 ** 24], [1.0], [-(2.0 ** 24)], [1.0]])
    assert ao.group_vector(q).tolist() == [1.0]


# ------------------------------------------------------------------------------------------
# search
# ------------------------------------------------------------------------------------------

def test_search_hand_worked(golden):
    g = golden["search"]
    keys = bits(g["keys"])
    train = bits(g["train"])
    adj = np.asarray(g["adj"], dtype=np.int32)
    entry = np.asarray(g["entry"], dtype=np.int32)
    for c in g["cases"]:
        r = ao.search(np.asarray(c["u"], dtype=np.float32), keys, train, entry, adj,
                      c["n_entry"], c["ef"], c["W"], c["k"], c["max_rounds"])
        assert r.ids.tolist() == c["ids"], c
        assert r.scores.tolist() == c["scores"], c
        assert (r.rounds, r.visited) == (c["rounds"], c["visited"]), c


def test_search_on_a_complete_graph_returns_the_exact_top_k(rng):
    """With every node adjacent to every other, the first round scores every node, so the
    search returns the exact top-k (integer keys and query: exact scores, by Python ints)."""
    N, d, k = 64, 16, 10
    X = rng.integers(-4, 5, size=(N, d))
    X[11] = X[40]                                   # an exact tie
    u = rng.integers(-4, 5, size=d)
    adj = np.asarray([[y for y in range(N) if y != x] for x in range(N)], dtype=np.int32)
    train = bits(rng.standard_normal((3, d)))
    entry = np.asarray([5, 17, 33], dtype=np.int32)
    r = ao.search(u.astype(np.float32), bits(X), train, entry, adj, 2, 16, 4, k, 100)
    exact = [int(np.dot(X[x].tolist(), u.tolist())) for x in range(N)]
    want = sorted(range(N), key=lambda x: (-exact[x], x))[:k]
    assert r.ids.tolist() == want
    assert r.scores.tolist() == [float(exact[x]) for x in want]
    assert r.visited == N


def test_search_invariants(rng):
    """Random graph: the result is in (score descending, id ascending) order, its scores are
    the nodes' scores, it is made of visited nodes, no round is lost, and zero rounds keep the
    best seeds."""
    N, d, R, n_t = 300, 16, 6, 40
    keys = bits(rng.standard_normal((N, d)))
    adj = rng.integers(-1, N, size=(N, R)).astype(np.int32)
    train = bits(rng.standard_normal((n_t, d)))
    entry = rng.integers(0, N, size=n_t).astype(np.int32)
    u = vals(bits(rng.standard_normal(d))).astype(np.float32)
    sc = ao.scores_f32(u, keys)
    r = ao.search(u, keys, train, entry, adj, 4, 32, 3, 12, 1000)
    ids = r.ids[r.ids >= 0]
    key = [(-float(sc[x]), int(x)) for x in ids]
    assert key == sorted(key)
    assert r.scores[:len(ids)].tolist() == sc[ids].tolist()
    assert len(ids) <= r.visited <= N
    r0 = ao.search(u, keys, train, entry, adj, 4, 32, 3, 12, 0)
    ts = ao.scores_f32(u, train)
    top_t = sorted(range(n_t), key=lambda t: (-float(ts[t]), t))[:4]
    seeds = sorted({int(entry[t]) for t in top_t}, key=lambda x: (-float(sc[x]), x))
    assert r0.ids[:len(seeds)].tolist() == seeds[:12] and r0.rounds == 0
    assert r.scores[0] >= r0.scores[0]


# ------------------------------------------------------------------------------------------
# attention (A7)
# ------------------------------------------------------------------------------------------

def test_attend_over_every_row_is_softmax_attention(rng):
    L, d, G = 50, 16, 3
    K = bits(rng.standard_normal((L, d)))
    V = bits(rng.standard_normal((L, d)))
    q = bits(rng.standard_normal((G, d)))
    out, lse = ao.attend(q, K, V, np.arange(L))
    Q = torch.from_numpy(vals(q))[None, :, None, :]
    Kt = torch.from_numpy(vals(K))[None, None].expand(1, G, -1, -1)
    Vt = torch.from_numpy(vals(V))[None, None].expand(1, G, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt)[0, :, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    a = vals(q) @ vals(K).T / np.sqrt(d)
    assert np.allclose(lse, np.log(np.exp(a).sum(axis=1)), rtol=1e-12)


def test_decode_group_rows_are_the_steady_zone_and_the_retrieved_tokens(rng):
    """The retrieved positions lie in the indexed zone, so the attended rows are the steady
    zone and the retrieved tokens, each once; forcing the retrieved set to every indexed
    position gives full attention over [0, L)."""
    L0, L, d, G, ns, nr = 96, 99, 16, 2, 4, 8
    K = bits(rng.standard_normal((L, d)))
    V = bits(rng.standard_normal((L, d)))
    q = bits(rng.standard_normal((G, d)))
    train = bits(rng.standard_normal((12, d)))
    graph = ao.build_head(K, train, L0, ns, nr, M=6, R=4)
    st = ao.decode_group(q, K, V, graph, train, L0, L, ns, nr, n_entry=3, ef=16, W=2, k=8,
                         max_rounds=50)
    pos = st.retrieved[st.retrieved >= 0]
    assert ((pos >= ns) & (pos < L0 - nr)).all() and len(set(pos.tolist())) == len(pos)
    lo, hi = ao.node_range(L0, ns, nr)
    full = ao.decode_group(q, K, V, graph, train, L0, L, ns, nr, 3, 16, 2, 8, 50,
                           retrieved=np.arange(lo, hi))
    ref, ref_lse = ao.attend(q, K, V, np.arange(L))
    assert np.allclose(full.out, ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(full.lse, ref_lse, rtol=1e-12)
