"""Host-memory tier (the wave buffer of RetroInfer: gist.science de section 2B "Wave Buffer"):
the cache in pinned host memory behind a device block cache. Every tiered decode step must
give the same out, lse and selection as wave_decode_attention on the same rows, bit for bit,
whatever the cache holds; every row a slot marks as held must equal the host row of the block
its owner names, and the table and the owners must agree; and the row counters must add up
to the retrieved rows."""
import numpy as np
import pytest

import kv_vector_index_amd as wi
import synth
import wave_testlib as tl

pytestmark = pytest.mark.gpu

ALIGN = 256                     # the library's sub-buffer alignment
TC_WORDS = 16


def tier_views(layer, p, n_slots, state):
    """(counters, table, slot owners, slot steps, slot row masks) of the tier state."""
    t = tl.torch()
    BH = layer.B * layer.H
    nblk = -(-layer.Lcap // wi.TIER_BLOCK)
    up = lambda x: -(-x // ALIGN) * ALIGN  # noqa: E731
    o_tab = up(4 * TC_WORDS)
    o_word = o_tab + up(4 * BH * nblk)
    o_valid = o_word + up(8 * n_slots)
    i32 = state.view(t.int32)
    words = state[o_word:o_word + 8 * n_slots].view(t.int32).view(n_slots, 2)
    return (i32[:TC_WORDS], i32[o_tab // 4:o_tab // 4 + BH * nblk].view(BH, nblk),
            words[:, 0], words[:, 1], i32[o_valid // 4:o_valid // 4 + n_slots])


def make_tier(layer, p, n_slots):
    t = tl.torch()
    tier = wi.alloc_tier(p, n_slots)
    # slots the fill has not written hold NaN (bf16 0xffff): a read of one, even under a zero
    # weight, turns the output to NaN
    tier.cache.fill_(0xFF)
    # written by the device (a DMA copy on the stream), as a caller offloading its cache
    # would: the device's reads of host memory need not see host-side writes still held in the
    # CPU's caches
    tier.host_k.copy_(layer.k_out)
    tier.host_v.copy_(layer.v_out)
    ns, nr = layer.n_sink, layer.n_recent
    tier.steady_k.copy_(t.cat([layer.k_out[:, :, :ns], layer.k_out[:, :, layer.L0 - nr:]], dim=2))
    tier.steady_v.copy_(t.cat([layer.v_out[:, :, :ns], layer.v_out[:, :, layer.L0 - nr:]], dim=2))
    wi.wave_tier_reset(p, tier)
    return tier


def check_cache_contents(layer, p, tier):
    """Every block the table names: its slot's owner is the block, and every row the slot
    marks as held equals the host row (K and V); every owned slot's block points back.
    Returns (blocks cached, rows held)."""
    t = tl.torch()
    ctr, tab, owner, step, valid = tier_views(layer, p, tier.n_slots, tier.state)
    tab, owner = tab.cpu().numpy(), owner.cpu().numpy()
    valid = valid.cpu().numpy().view(np.uint32)
    assert (tab >= -1).all(), "a block left being claimed after a step"
    cache = tier.cache.view(t.bfloat16).view(tier.n_slots, 2, wi.TIER_BLOCK, 128).cpu()
    hk = tier.host_k.view(layer.B * layer.H, layer.Lcap, 128)
    hv = tier.host_v.view(layer.B * layer.H, layer.Lcap, 128)
    nblk = tab.shape[1]
    n_cached = n_rows = 0
    for bh, b in zip(*np.nonzero(tab >= 0)):
        s = int(tab[bh, b])
        assert owner[s] == bh * nblk + b, (bh, b, s, owner[s])
        rows = [r for r in range(wi.TIER_BLOCK) if (int(valid[s]) >> r) & 1]
        assert all(b * wi.TIER_BLOCK + r < layer.Lcap for r in rows), (bh, b)
        for r in rows:
            assert t.equal(cache[s, 0, r], hk[bh, b * wi.TIER_BLOCK + r]), (bh, b, r)
            assert t.equal(cache[s, 1, r], hv[bh, b * wi.TIER_BLOCK + r]), (bh, b, r)
        n_cached += 1
        n_rows += len(rows)
    for s in np.nonzero(owner >= 0)[0]:
        bh, b = divmod(int(owner[s]), nblk)
        assert tab[bh, b] == s, "an owner whose block does not point back"
    return n_cached, n_rows


def retrieved_rows(idx, sel):
    """Token rows of the selected clusters, summed over (b, kv-head)."""
    size = idx.cluster_size.cpu().numpy()
    tot = 0
    for b in range(sel.shape[0]):
        for g in range(sel.shape[1]):
            j = sel[b, g][sel[b, g] >= 0]
            tot += int(size[b, g, j].sum())
    return tot


@pytest.fixture(scope="module")
def layer4k():
    w = synth.WORKLOADS["tiny"]
    x = synth.generate_layer(w)
    layer = tl.Layer(x.k, x.v, w.context, w.segment_size, w.clusters_per_segment, w.n_iters,
                     w.n_sink, w.n_recent, w.n_q_heads)
    idx = layer.build()
    return w, x, layer, idx


@pytest.mark.parametrize("n_slots", [4096, 64, 3])
def test_tiered_steps_equal_the_resident_steps(layer4k, n_slots):
    """16 decode steps through the tier (a cache of every block, a small one that must
    replace, one too small for a step's blocks) against the resident decode: out, lse and the
    selection bit for bit at every step; the cache's contents after every step; the counters
    add up."""
    t = tl.torch()
    w, x, layer, idx = layer4k
    n_r = w.n_retrieve
    p_last = layer.decode_params(layer.L0 + w.steps, n_r)
    tier = make_tier(layer, p_last, n_slots)
    ws = wi.alloc_decode_workspace(p_last)
    total_rows = 0
    for s in range(w.steps):
        L = layer.L0 + s + 1
        p = layer.decode_params(L, n_r)
        out_r, lse_r, sel_r = layer.decode(idx, x.q[s], L, n_r)
        q = tl.to_dev(x.q[s])
        out = t.empty(layer.B, layer.Hq, 128, dtype=t.float32, device="cuda")
        lse = t.empty(layer.B, layer.Hq, dtype=t.float32, device="cuda")
        sel = t.full((layer.B, layer.H, n_r), -7, dtype=t.int32, device="cuda")
        wi.wave_decode_attention_tiered(p, q, tier, idx, out, lse, sel, ws)
        t.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), sel_r), f"step {s}: selection"
        assert np.array_equal(out.cpu().numpy(), out_r), f"step {s}: out"
        assert np.array_equal(lse.cpu().numpy(), lse_r), f"step {s}: lse"
        n_cached, n_rows = check_cache_contents(layer, p, tier)
        assert n_cached <= n_slots
        total_rows += retrieved_rows(idx, sel_r)
    c = wi.wave_tier_counters(p_last, tier)
    assert c["rows_cached"] + c["rows_host"] == total_rows, (c, total_rows)
    assert 0 < c["rows_written"] <= c["rows_host"], c
    if n_slots >= 4096:       # every block fits: no claim is refused and rows are reused
        assert c["blocks_refused"] == 0
        assert c["rows_cached"] > 0
        assert n_rows <= c["rows_written"]
    if n_slots == 3:
        assert c["blocks_refused"] > 0


def test_tier_reset_empties_the_cache(layer4k):
    """After a reset nothing is cached: the next step reads every retrieved row from host
    memory and still equals the resident step."""
    t = tl.torch()
    w, x, layer, idx = layer4k
    n_r = w.n_retrieve
    L = layer.L0 + 1
    p = layer.decode_params(L, n_r)
    tier = make_tier(layer, p, 512)
    ws = wi.alloc_decode_workspace(p)
    q = tl.to_dev(x.q[0])
    out = t.empty(layer.B, layer.Hq, 128, dtype=t.float32, device="cuda")
    for _ in range(2):
        wi.wave_decode_attention_tiered(p, q, tier, idx, out, None, None, ws)
    wi.wave_tier_reset(p, tier)
    wi.wave_decode_attention_tiered(p, q, tier, idx, out, None, None, ws)
    c = wi.wave_tier_counters(p, tier)
    out_r, _, sel_r = layer.decode(idx, x.q[0], L, n_r)
    assert np.array_equal(out.cpu().numpy(), out_r)
    assert c["rows_cached"] == 0 and c["rows_host"] == retrieved_rows(idx, sel_r), c


TIER_EDGE = {
    # name: (B, H, Hq, L0, steps, S, kseg, n_sink, n_recent, n_r, n_slots)
    "g7_batch2_partial_last_block": (2, 2, 14, 1500, 4, 512, 32, 3, 17, 9, 16),
    "mha": (1, 4, 4, 1200, 3, 256, 24, 4, 20, 7, 12),
    "no_steady_zone": (1, 2, 8, 1024, 3, 256, 16, 0, 0, 6, 8),
    "one_slot": (1, 2, 8, 900, 4, 300, 20, 2, 11, 5, 1),
    "g5": (1, 1, 5, 800, 3, 256, 20, 2, 9, 6, 6),
    "g8": (1, 2, 16, 1100, 3, 256, 24, 3, 17, 8, 10),
}


@pytest.mark.parametrize("name", sorted(TIER_EDGE))
def test_tier_shapes_and_edge_cases(name):
    """Other shapes through the tier: seven query heads per KV head at batch 2 with a partly
    filled last block, MHA, five and eight query heads per KV head, no steady zone, a single
    slot; every step bit for bit equal to the
    resident decode, the cache's rows checked after every step."""
    import zlib
    B, H, Hq, L0, steps, S, kseg, ns, nr, n_r, n_slots = TIER_EDGE[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    print(f"[tier] edge case {name}", flush=True)
    layer, q = tl.ragged_layer(rng, B=B, H=H, Hq=Hq, L0=L0, steps=steps, S=S, kseg=kseg,
                               n_sink=ns, n_recent=nr)
    idx = layer.build()
    t = tl.torch()
    p_last = layer.decode_params(layer.L0 + steps, n_r)
    tier = make_tier(layer, p_last, n_slots)
    ws = wi.alloc_decode_workspace(p_last)
    total = 0
    for s in range(steps):
        L = layer.L0 + s + 1
        p = layer.decode_params(L, n_r)
        out_r, lse_r, sel_r = layer.decode(idx, q[s], L, n_r)
        out = t.empty(layer.B, layer.Hq, 128, dtype=t.float32, device="cuda")
        lse = t.empty(layer.B, layer.Hq, dtype=t.float32, device="cuda")
        sel = t.full((layer.B, layer.H, n_r), -7, dtype=t.int32, device="cuda")
        wi.wave_decode_attention_tiered(p, tl.to_dev(q[s]), tier, idx, out, lse, sel, ws)
        t.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), sel_r), (name, s)
        assert np.array_equal(out.cpu().numpy(), out_r), (name, s)
        assert np.array_equal(lse.cpu().numpy(), lse_r), (name, s)
        check_cache_contents(layer, p, tier)
        total += retrieved_rows(idx, sel_r)
    c = wi.wave_tier_counters(p_last, tier)
    assert c["rows_cached"] + c["rows_host"] == total, (name, c, total)
