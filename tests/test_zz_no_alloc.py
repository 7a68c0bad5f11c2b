"""The allocation-free decode entry point (the library's own per-GPU scratch instead of a
caller workspace) against the workspace entry point, through the C ABI: two calls in a row,
the second with a smaller problem, each bit for bit equal to wave_decode_attention with a
fresh workspace, and within the oracle's tolerances."""
import sys

import numpy as np
import pytest

import kv_vector_index_amd as wi
import wave_testlib as tl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def decode_both(layer, idx, q_np, L, n_r):
    t = tl.torch()
    p = layer.decode_params(L, n_r)
    q = tl.to_dev(q_np)
    res = []
    for noalloc in (False, True):
        out = t.full((layer.B, layer.Hq, 128), float("nan"), dtype=t.float32, device="cuda")
        lse = t.full((layer.B, layer.Hq), float("nan"), dtype=t.float32, device="cuda")
        sel = t.full((layer.B, layer.H, n_r), -7, dtype=t.int32, device="cuda")
        if noalloc:
            wi.wave_decode_attention_noalloc(p, q, layer.k_out, layer.v_out, idx, out, lse, sel)
        else:
            ws = wi.alloc_decode_workspace(p)
            wi.wave_decode_attention(p, q, layer.k_out, layer.v_out, idx, out, lse, sel, ws)
        t.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()))
    return res


def test_noalloc_decode_equals_the_workspace_entry_point():
    rng = np.random.default_rng(41)
    big, qb = tl.ragged_layer(rng, B=2, H=4, Hq=16, L0=3000, steps=1, S=1024, kseg=64)
    small, qs = tl.ragged_layer(rng, B=1, H=2, Hq=8, L0=900, steps=1, S=256, kseg=24)
    for name, layer, q, n_r in (("larger", big, qb, 40), ("smaller", small, qs, 7)):
        say(f"[noalloc] {name}: B={layer.B} H={layer.H} Hq={layer.Hq} L0={layer.L0} "
            f"C={layer.C} n_r={n_r}")
        need = wi.wave_decode_workspace_size(layer.decode_params(layer.L0 + 1, n_r))
        assert need <= wi.NOALLOC_SCRATCH_BYTES
        idx = layer.build()
        L = layer.L0 + 1
        (o1, l1, s1), (o2, l2, s2) = decode_both(layer, idx, q[0], L, n_r)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2) and np.array_equal(s1, s2)
        tl.oracle_decode_check(layer, idx, q[0], L, n_r, o2, l2, s2)
