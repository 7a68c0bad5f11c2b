"""Attention-aware vector search on the GPU against the oracle (oracle/anns_oracle.py).

* build: every training list holds the list_len best nodes up to the fp32 error of the
  matrix-core scores (an exchanged node scores within that error of the list's last one, and
  consecutive entries are in order within it); the graph and the entries equal the oracle's
  link of the GPU's own lists bit for bit (integer work);
* search: the retrieved positions, the rounds and the count of scored nodes equal the
  oracle's search on the GPU's graph bit for bit (both sides decide in fp32 in the same order);
* attention: out and lse within 2e-3 of the oracle's fp64 attention over the same rows.
"""
import zlib

import numpy as np
import pytest

import kv_vector_index_amd as wi
import synth
import wave_testlib as tl
from oracle import anns_oracle as ao
from oracle import wave_oracle as wo

pytestmark = pytest.mark.gpu

GAMMA = 8e-6          # >= 128 * 2^-24 (+ margin): fp32 error bound of a 128-term dot product


def say(*a):
    print("[anns]", *a, flush=True)


def params(B, Hq, H, L0, Lcap, ns, nr, n_t, M, R, E, ef, W, k, rounds, L=None):
    return wi.wave_anns_params(B, Hq, H, 128, L0 if L is None else L, L0, Lcap, ns, nr, n_t, M,
                               R, E, ef, W, k, rounds, 128 ** -0.5)


class Case:
    """Inputs on the device, the built graph, and the parameters."""

    def __init__(self, K, V, T, q, L0, ns, nr, M, R, E, ef, W, k, rounds):
        t = tl.torch()
        self.K, self.V, self.T, self.q = K, V, T, q        # bf16 bits (numpy)
        B, H, Lcap, _ = K.shape
        self.B, self.H, self.Lcap, self.L0, self.ns, self.nr = B, H, Lcap, L0, ns, nr
        self.Hq = q.shape[2]
        self.G = self.Hq // H
        self.n_t = T.shape[2]
        self.cfg = (M, R, E, ef, W, k, rounds)
        self.p = params(B, self.Hq, H, L0, Lcap, ns, nr, self.n_t, *self.cfg)
        self.k_dev, self.v_dev = tl.to_dev(K), tl.to_dev(V)
        self.t_dev = tl.to_dev(T)
        self.index = wi.alloc_anns_index(self.p, self.t_dev)
        ws = t.empty(max(wi.wave_anns_build_workspace_size(self.p), 1), dtype=t.uint8,
                     device="cuda")
        wi.wave_anns_build(self.p, self.k_dev, self.index, ws)
        t.cuda.synchronize()
        self.lists = self.index.lists.cpu().numpy()
        self.graph = self.index.graph.cpu().numpy()
        self.entry = self.index.entry.cpu().numpy()
        self.dws = t.empty(wi.wave_anns_decode_workspace_size(self.p), dtype=t.uint8,
                           device="cuda")

    @property
    def N(self):
        return self.L0 - self.ns - self.nr

    def decode(self, s):
        """GPU step s (query q[s], length L0 + s + 1): out, lse, retrieved, stats."""
        t = tl.torch()
        L = self.L0 + s + 1
        p = params(self.B, self.Hq, self.H, self.L0, self.Lcap, self.ns, self.nr, self.n_t,
                   *self.cfg, L=L)
        out = t.full((self.B, self.Hq, 128), 7.0, dtype=t.float32, device="cuda")
        lse = t.full((self.B, self.Hq), 7.0, dtype=t.float32, device="cuda")
        ret = t.full((self.B, self.H, self.cfg[5]), -7, dtype=t.int32, device="cuda")
        st = t.full((self.B, self.H, 2), -7, dtype=t.int32, device="cuda")
        wi.wave_anns_decode_attention(p, tl.to_dev(self.q[s]), self.k_dev, self.v_dev,
                                      self.index, out, lse, ret, st, self.dws)
        t.cuda.synchronize()
        return L, out.cpu().numpy(), lse.cpu().numpy(), ret.cpu().numpy(), st.cpu().numpy()


def check_lists(c: Case, heads=None, rows=None):
    """GPU lists against exact fp64 scores, within the fp32 error of the products."""
    M = c.cfg[0]
    lo, hi = ao.node_range(c.L0, c.ns, c.nr)
    for b in range(c.B):
        for g in range(c.H):
            if heads is not None and (b, g) not in heads:
                continue
            if hi == lo:
                assert (c.lists[b, g] == -1).all(), (b, g)
                continue
            keys = c.K[b, g, lo:hi]
            Kf = wo.bf16_to_f64(keys)
            ts = range(c.n_t) if rows is None else rows
            Tf = wo.bf16_to_f64(c.T[b, g, list(ts)])
            S = Tf @ Kf.T
            bound = GAMMA * (np.abs(Tf) @ np.abs(Kf).T).max(axis=1)
            for j, t in enumerate(ts):
                got = c.lists[b, g, t]
                m = min(M, hi - lo)
                assert (got[m:] == -1).all() and (got[:m] >= 0).all(), (b, g, t)
                assert len(set(got[:m].tolist())) == m, (b, g, t)
                want = np.lexsort((np.arange(hi - lo), -S[j]))[:m]
                tau = S[j, want[-1]] if m else 0.0
                for x in set(got[:m].tolist()) ^ set(want.tolist()):
                    assert abs(S[j, x] - tau) <= 2 * bound[j], (b, g, t, x)
                sg = S[j, got[:m]]
                assert (sg[:-1] >= sg[1:] - 2 * bound[j]).all(), (b, g, t)


def check_graph(c: Case, heads=None):
    M, R = c.cfg[0], c.cfg[1]
    for b in range(c.B):
        for g in range(c.H):
            if heads is not None and (b, g) not in heads:
                continue
            adj = ao.link(c.lists[b, g], c.N, R)
            assert np.array_equal(c.graph[b, g], adj), (b, g)
            assert np.array_equal(c.entry[b, g], c.lists[b, g, :, 0]), (b, g)


def check_step(c: Case, s, heads=None):
    M, R, E, ef, W, k, rounds = c.cfg
    L, out, lse, ret, st = c.decode(s)
    lo, hi = ao.node_range(c.L0, c.ns, c.nr)
    worst = 0.0
    for b in range(c.B):
        for g in range(c.H):
            if heads is not None and (b, g) not in heads:
                continue
            graph = ao.HeadGraph(c.lists[b, g], c.graph[b, g], c.entry[b, g])
            qg = c.q[s, b, g * c.G:(g + 1) * c.G]
            r = ao.decode_group(qg, c.K[b, g], c.V[b, g], graph, c.T[b, g], c.L0, L, c.ns, c.nr,
                                E, ef, W, k, rounds)
            assert np.array_equal(ret[b, g], r.retrieved), (s, b, g, ret[b, g], r.retrieved)
            assert st[b, g].tolist() == [r.search.rounds, r.search.visited], (s, b, g)
            e = tl.row_rel_err(out[b, g * c.G:(g + 1) * c.G], r.out)
            assert e <= tl.OUT_TOL, (s, b, g, e)
            assert np.all(np.abs(lse[b, g * c.G:(g + 1) * c.G] - r.lse) <= tl.OUT_TOL), (s, b, g)
            worst = max(worst, e)
    return worst


def tiny_case(**cfg):
    w = synth.WORKLOADS["tiny"]
    x = synth.generate_layer(w)
    T = synth.training_queries(w, 64)                 # 256 training queries per KV head
    base = dict(M=16, R=16, E=8, ef=128, W=8, k=64, rounds=1000)
    base.update(cfg)
    return w, Case(x.k, x.v, T, x.q, w.context, w.n_sink, w.n_recent, **base)


@pytest.fixture(scope="module")
def tiny():
    return tiny_case()


def test_tiny_build_lists_and_graph(tiny):
    w, c = tiny
    say("tiny build: N", c.N, "n_t", c.n_t)
    check_lists(c)
    check_graph(c)
    deg = (c.graph >= 0).sum(axis=-1)
    assert min(c.cfg[1], c.cfg[0] - 1) <= deg.max() <= c.cfg[1] and (deg > 0).mean() > 0.02


def test_tiny_every_step_equals_the_oracle(tiny):
    w, c = tiny
    worst = max(check_step(c, s) for s in range(w.steps))
    say("tiny steps: worst row error", worst)


def test_search_finds_the_exact_best_nodes_often(tiny):
    """Not a parity claim: a sanity check that the graph is searchable (recall of the exact
    top-k by the fp32 score, over the tiny workload's steps)."""
    w, c = tiny
    k = c.cfg[5]
    lo, hi = ao.node_range(c.L0, c.ns, c.nr)
    rec = []
    for s in range(4):
        _, _, _, ret, _ = c.decode(s)
        for g in range(c.H):
            u = ao.group_vector(c.q[s, 0, g * c.G:(g + 1) * c.G])
            sc = ao.scores_f32(u, c.K[0, g, lo:hi])
            best = set((np.lexsort((np.arange(hi - lo), -sc.astype(np.float64)))[:k] + lo).tolist())
            rec.append(len(best & set(ret[0, g].tolist())) / k)
    say("tiny recall@k", float(np.mean(rec)))
    assert np.mean(rec) > 0.3


EDGE = {
    # name: (B, Hq, H, L0, steps, ns, nr, n_pos, cfg)
    "ragged_train_and_nodes": (1, 8, 2, 700, 2, 3, 21, 13, dict(M=20, R=12, E=5, ef=96, W=6, k=40)),
    "fewer_nodes_than_m": (1, 8, 2, 60, 2, 4, 16, 8, dict(M=48, R=8, E=4, ef=32, W=4, k=16)),
    "no_nodes": (1, 8, 2, 40, 2, 8, 32, 8, dict(M=8, R=8, E=4, ef=16, W=2, k=8)),
    "zero_rounds": (1, 8, 2, 500, 2, 4, 16, 16, dict(M=16, R=16, E=9, ef=64, W=8, k=32, rounds=0)),
    "one_each": (1, 8, 2, 500, 2, 4, 16, 16, dict(M=1, R=1, E=1, ef=1, W=1, k=1)),
    "wide_rounds": (1, 4, 1, 3000, 2, 4, 64, 100, dict(M=64, R=32, E=64, ef=1024, W=64, k=512)),
    "mha_batch2": (2, 4, 4, 900, 2, 4, 32, 20, dict(M=24, R=20, E=6, ef=80, W=5, k=50)),
    "g7": (1, 14, 2, 900, 2, 4, 32, 10, dict(M=16, R=16, E=8, ef=64, W=8, k=32)),
    "g3": (1, 6, 2, 800, 2, 4, 32, 12, dict(M=16, R=16, E=8, ef=64, W=8, k=32)),
    "g8": (1, 16, 2, 900, 2, 4, 32, 10, dict(M=16, R=16, E=8, ef=64, W=8, k=32)),
    "duplicate_keys": (1, 8, 2, 600, 2, 4, 16, 16, dict(M=16, R=16, E=8, ef=64, W=8, k=32)),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_shapes_and_edge_cases(name):
    B, Hq, H, L0, steps, ns, nr, n_pos, cfg = EDGE[name]
    seed = zlib.crc32(name.encode())
    say("edge case", name, "seed", seed)
    rng = np.random.default_rng(seed)
    G, d = Hq // H, 128
    Lcap = L0 + steps
    topics = rng.standard_normal((6, d))
    z = rng.integers(0, 6, size=(B, H, Lcap))
    K = synth.f32_to_bf16_bits((topics[z] + 0.5 * rng.standard_normal((B, H, Lcap, d)))
                               .astype(np.float32))
    if name == "duplicate_keys":            # exact score ties in the lists and the search
        K[:, :, 100:140] = K[:, :, 60:100]
        K[:, :, 300:303] = K[:, :, 50:51]
    V = synth.f32_to_bf16_bits(rng.standard_normal((B, H, Lcap, d)).astype(np.float32))
    T = synth.f32_to_bf16_bits((topics[rng.integers(0, 6, size=(B, H, n_pos * G))] +
                                rng.standard_normal((B, H, n_pos * G, d))).astype(np.float32))
    q = synth.f32_to_bf16_bits((topics[rng.integers(0, 6, size=(steps, B, 1, 1))][:, :, :, 0] +
                                rng.standard_normal((steps, B, Hq, d))).astype(np.float32))
    base = dict(rounds=1000)
    base.update(cfg)
    c = Case(K, V, T, q, L0, ns, nr, **base)
    check_lists(c)
    check_graph(c)
    for s in range(steps):
        check_step(c, s)


def test_llama128k_sampled_parity():
    """The 128K layer at the bench's settings: sampled training lists against exact scores,
    the graph of two heads against the oracle's link of the GPU's lists, and two steps of two
    heads against the oracle's search and attention."""
    w = synth.WORKLOADS["llama128k"].with_(steps=2)
    x = synth.generate_layer(w)
    T = synth.training_queries(w, 1024)
    say("128K: generated")
    c = Case(x.k, x.v, T, x.q, w.context, w.n_sink, w.n_recent, M=32, R=32, E=16, ef=512, W=32,
             k=256, rounds=1000)
    say("128K: built")
    heads = [(0, 0), (0, 5)]
    check_lists(c, heads=heads, rows=[0, 1, 777, 2048, 4095])
    say("128K: lists")
    check_graph(c, heads=heads)
    say("128K: graph")
    for s in range(2):
        check_step(c, s, heads=heads)
    say("128K: steps")
