"""The C-ABI library loads, exports every symbol its header declares, and validates arguments
on the host (no GPU work is enqueued by any call in this file)."""
import ctypes
import os
import re
import subprocess

import pytest

import kv_vector_index_amd as wi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wave_index.h")

pytestmark = pytest.mark.skipif(not os.path.exists(wi.LIB_PATH),
                                reason="libwave_index.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:wave_status|const char\*)\s+(wave_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(wi.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", wi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    lib = wi.library()
    for f in declared_functions():
        assert getattr(lib, f) is not None


def test_status_strings():
    assert wi.wave_status_string(0) == "ok"
    assert "workspace" in wi.wave_status_string(3)
    assert wi.wave_status_string(99) == "unknown status"


def build_params(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=4096,
                kv_capacity=4112, segment_size=4096, clusters_per_segment=256, n_iters=5,
                n_sink=4, n_recent=64)
    base.update(kw)
    return wi.wave_build_params(**base)


def decode_params(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=4097,
                index_len=4096, kv_capacity=4112, n_clusters=256, n_sink=4, n_recent=64,
                n_retrieve=6, scale=128 ** -0.5)
    base.update(kw)
    return wi.wave_decode_params(**base)


def test_workspace_sizes_are_positive_and_grow_with_the_problem():
    a = wi.wave_index_workspace_size(build_params())
    b = wi.wave_index_workspace_size(build_params(batch=2))
    assert 0 < a < b
    c = wi.wave_decode_workspace_size(decode_params())
    d = wi.wave_decode_workspace_size(decode_params(batch=3))
    assert 0 < c < d
    # independent of the current length: one workspace serves every decode step
    assert wi.wave_decode_workspace_size(decode_params(seq_len=4100)) == c


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(head_dim=0), 1), (dict(n_q_heads=30), 1),
    (dict(batch=0), 1), (dict(seq_len=0), 1), (dict(kv_capacity=100), 1),
    (dict(clusters_per_segment=5000), 1), (dict(segment_size=32768, clusters_per_segment=8), 2),
    (dict(clusters_per_segment=4096, segment_size=8192), 2), (dict(n_iters=0), 1),
    (dict(n_sink=-1), 1), (dict(n_sink=3000, n_recent=2000), 1),
])
def test_build_validation(kw, code):
    with pytest.raises(wi.WaveError) as e:
        wi.wave_index_workspace_size(build_params(**kw))
    assert e.value.code == code


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), 2), (dict(n_q_heads=36, n_kv_heads=4), 2), (dict(n_q_heads=33), 1),
    (dict(seq_len=4000), 1), (dict(seq_len=5000), 1), (dict(n_retrieve=-1), 1),
    (dict(n_retrieve=257), 1), (dict(scale=0.0), 1), (dict(scale=float("nan")), 1),
    (dict(n_clusters=0), 1), (dict(n_sink=4000, n_recent=200), 1), (dict(n_clusters=65537), 2),
])
def test_decode_validation(kw, code):
    with pytest.raises(wi.WaveError) as e:
        wi.wave_decode_workspace_size(decode_params(**kw))
    assert e.value.code == code


def test_build_rejects_null_small_workspace_and_aliasing_before_any_launch():
    """Pointer checks run on the host before anything is enqueued (fake addresses are never
    dereferenced because every call here fails validation)."""
    lib = wi.library()
    p = build_params()
    ws = wi.wave_index_workspace_size(p)
    cache = 1 * 8 * 4112 * 128 * 2
    K, V, KO, VO, WS = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40
    idx = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
    call = lambda *a: lib.wave_index_build(ctypes.byref(p), *a)  # noqa: E731
    assert call(None, V, KO, VO, ctypes.byref(idx), WS, ws, None) == 1
    assert call(K, V, KO, VO, ctypes.byref(idx), WS, ws - 1, None) == 3
    assert call(K, V, KO, VO, ctypes.byref(idx), None, ws, None) == 3
    assert call(K, V, K + cache // 2, VO, ctypes.byref(idx), WS, ws, None) == 4
    assert call(K, V, KO, KO + 256, ctypes.byref(idx), WS, ws, None) == 4
    bad = wi.wave_index(6 << 40, None, 8 << 40, 9 << 40, None, None, None, None)
    assert call(K, V, KO, VO, ctypes.byref(bad), WS, ws, None) == 1


def test_extend_validates_before_any_launch():
    """The extension's own checks (earlier length, earlier index, objective output, overlap
    with the earlier index) run on the host before anything is enqueued."""
    lib = wi.library()
    p = build_params()
    ws = wi.wave_index_workspace_size(p)
    K, V, KO, VO, WS = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40
    idx = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
    prev = wi.wave_index(10 << 40, 11 << 40, 12 << 40, 13 << 40, None, None, None, None)
    lo = p.n_sink + p.n_recent

    def call(n, pr, ix):
        return lib.wave_index_extend(ctypes.byref(p), n, K, V, KO, VO,
                                     ctypes.byref(pr) if pr is not None else None,
                                     ctypes.byref(ix), WS, ws, None)
    assert call(lo, None, idx) == 1                      # no earlier index
    assert call(lo - 1, prev, idx) == 1                  # shorter than the steady zone
    assert call(p.seq_len + 1, prev, idx) == 1           # longer than the new length
    no_size = wi.wave_index(10 << 40, 11 << 40, None, 13 << 40, None, None, None, None)
    assert call(lo, no_size, idx) == 1                   # an earlier required array missing
    with_obj = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, 14 << 40)
    assert call(lo, prev, with_obj) == 2                 # objective output
    assert call(lo, idx, idx) == 4                       # earlier index overlaps the output
    # an optional output of idx must exist in prev (it is copied for the unchanged segments)
    for field, addr in (("labels", 15 << 40), ("perm", 16 << 40), ("last_centroids", 17 << 40)):
        want = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
        setattr(want, field, addr)
        assert call(lo, prev, want) == 1, field


def test_decode_rejects_null_small_workspace_and_aliasing_before_any_launch():
    lib = wi.library()
    p = decode_params()
    ws = wi.wave_decode_workspace_size(p)
    Q, K, V, OUT, WS = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40
    idx = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
    call = lambda *a: lib.wave_decode_attention(ctypes.byref(p), *a)  # noqa: E731
    assert call(Q, K, V, ctypes.byref(idx), None, None, None, WS, ws, None) == 1
    assert call(Q, K, V, ctypes.byref(idx), OUT, None, None, WS, ws - 256, None) == 3
    assert call(Q, K, V, ctypes.byref(idx), K + 512, None, None, WS, ws, None) == 4
    assert call(Q, K, V, ctypes.byref(idx), OUT, OUT + 64, None, WS, ws, None) == 4
    bad = decode_params(n_retrieve=-1)
    assert lib.wave_decode_attention(ctypes.byref(bad), Q, K, V, ctypes.byref(idx), OUT, None,
                                     None, WS, ws, None) == 1
    dense = lib.wave_dense_decode_attention
    assert dense(ctypes.byref(p), Q, K, V, None, None, WS, ws, None) == 1
    assert dense(ctypes.byref(p), Q, K, V, OUT, None, None, ws, None) == 3


def test_noalloc_decode_rejects_a_problem_larger_than_its_scratch_before_any_launch():
    """The allocation-free entry point checks its fixed scratch size on the host: a problem
    whose workspace exceeds it is refused (WAVE_ERR_WORKSPACE) before anything is enqueued,
    and argument errors come first."""
    lib = wi.library()
    big = decode_params(batch=64, n_clusters=65536, index_len=1 << 20, seq_len=(1 << 20) + 1,
                        kv_capacity=(1 << 20) + 16, n_retrieve=1180)
    assert wi.wave_decode_workspace_size(big) > wi.NOALLOC_SCRATCH_BYTES
    Q, K, V, OUT = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    idx = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
    call = lib.wave_decode_attention_noalloc
    assert call(ctypes.byref(big), Q, K, V, ctypes.byref(idx), OUT, None, None, None) == 3
    bad = decode_params(n_retrieve=-1)
    assert call(ctypes.byref(bad), Q, K, V, ctypes.byref(idx), OUT, None, None, None) == 1


def test_tier_validates_before_any_launch():
    """The host-memory tier's checks run on the host before anything is enqueued: slot count,
    missing buffers, a block cache overlapping the tier state or an output."""
    lib = wi.library()
    p = decode_params()
    n = ctypes.c_size_t(0)
    assert lib.wave_tier_state_size(ctypes.byref(p), 0, ctypes.byref(n)) == 1
    assert lib.wave_tier_state_size(ctypes.byref(p), 64, ctypes.byref(n)) == 0
    st_bytes = n.value
    assert st_bytes > 0
    assert lib.wave_tier_state_size(ctypes.byref(p), 128, ctypes.byref(n)) == 0
    assert n.value > st_bytes                   # owners and stamps per slot
    ws = wi.wave_decode_workspace_size(p)
    Q, OUT, WS = 1 << 40, 4 << 40, 5 << 40
    HK, HV, SK, SV, CA, STT = 20 << 40, 21 << 40, 22 << 40, 23 << 40, 24 << 40, 25 << 40
    idx = wi.wave_index(6 << 40, 7 << 40, 8 << 40, 9 << 40, None, None, None, None)
    call = lib.wave_decode_attention_tiered

    def tier(**kw):
        base = dict(host_k=HK, host_v=HV, steady_k=SK, steady_v=SV, cache=CA, state=STT,
                    n_slots=64)
        base.update(kw)
        return wi.wave_tier(**base)
    assert call(ctypes.byref(p), Q, None, ctypes.byref(idx), OUT, None, None, WS, ws, None) == 1
    for f in ("host_k", "host_v", "steady_k", "steady_v", "cache", "state"):
        t = tier(**{f: None})
        assert call(ctypes.byref(p), Q, ctypes.byref(t), ctypes.byref(idx), OUT, None, None, WS,
                    ws, None) == 1, f
    t = tier(n_slots=0)
    assert call(ctypes.byref(p), Q, ctypes.byref(t), ctypes.byref(idx), OUT, None, None, WS, ws,
                None) == 1
    t = tier(state=CA + 4096)                   # the cache (64 x 16 KiB) covers the state
    assert call(ctypes.byref(p), Q, ctypes.byref(t), ctypes.byref(idx), OUT, None, None, WS, ws,
                None) == 4
    t = tier(cache=OUT)                         # the cache over out
    assert call(ctypes.byref(p), Q, ctypes.byref(t), ctypes.byref(idx), OUT, None, None, WS, ws,
                None) == 4
    t = tier()
    assert call(ctypes.byref(p), Q, ctypes.byref(t), ctypes.byref(idx), OUT, None, None, WS,
                ws - 256, None) == 3
    assert lib.wave_tier_reset(ctypes.byref(p), None, None) == 1
    c = (ctypes.c_uint64 * 5)()
    assert lib.wave_tier_counters(ctypes.byref(p), None, c, None) == 1


def anns_params(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=4097,
                index_len=4096, kv_capacity=4112, n_sink=4, n_recent=64, n_train=256,
                list_len=32, degree=32, n_entry=16, pool=512, expand=32, n_retrieve=256,
                max_rounds=100, scale=128 ** -0.5)
    base.update(kw)
    return wi.wave_anns_params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), 2), (dict(n_q_heads=30), 1), (dict(n_q_heads=72, n_kv_heads=8), 2),
    (dict(n_train=0), 1), (dict(n_train=16385), 1), (dict(list_len=65), 1),
    (dict(degree=0), 1), (dict(n_entry=65), 1), (dict(pool=1025), 1), (dict(expand=0), 1),
    (dict(expand=64, degree=64), 1), (dict(n_retrieve=513), 1), (dict(max_rounds=-1), 1),
    (dict(n_sink=3000, n_recent=2000), 1), (dict(index_len=5000), 1),
    # a visited set larger than the workgroup's LDS
    (dict(index_len=2_000_000, kv_capacity=2_000_016, seq_len=2_000_001), 2),
])
def test_anns_validation(kw, code):
    p = anns_params(**kw)
    n = ctypes.c_size_t(0)
    assert wi.library().wave_anns_build_workspace_size(ctypes.byref(p), ctypes.byref(n)) == code


def test_anns_validates_before_any_launch():
    """The vector search's checks run on the host before anything is enqueued: missing
    buffers, a small workspace, an output over an input or another output, the step's own
    length and scale."""
    lib = wi.library()
    p = anns_params()
    bws, dws = wi.wave_anns_build_workspace_size(p), wi.wave_anns_decode_workspace_size(p)
    assert bws > 0 and dws > 0
    K, V, Q, TR, GR, EN, LI, WS, OUT = (i << 40 for i in range(1, 10))
    idx = wi.wave_anns_index(TR, GR, EN, LI)
    build = lambda i, ws=WS, n=bws: lib.wave_anns_build(  # noqa: E731
        ctypes.byref(p), K, ctypes.byref(i), ws, n, None)
    assert build(wi.wave_anns_index(TR, GR, EN, None)) == 1
    assert build(wi.wave_anns_index(None, GR, EN, LI)) == 1
    assert build(idx, n=bws - 256) == 3
    assert build(idx, ws=None) == 3
    assert build(wi.wave_anns_index(TR, K + 4096, EN, LI)) == 4       # graph over the cache
    assert build(wi.wave_anns_index(TR, GR, GR + 64, LI)) == 4        # entry over the graph
    dec = lambda pp=p, out=OUT, lse=None, ret=None, st=None, n=dws: (  # noqa: E731
        lib.wave_anns_decode_attention(ctypes.byref(pp), Q, K, V, ctypes.byref(idx), out, lse,
                                       ret, st, WS, n, None))
    assert dec(out=None) == 1
    assert dec(n=dws - 256) == 3
    assert dec(out=Q) == 4                                             # out over q
    assert dec(ret=GR + 128) == 4                                      # retrieved over the graph
    assert dec(lse=OUT + 256) == 4                                     # lse over out
    assert dec(pp=anns_params(seq_len=4095)) == 1                      # L below L0
    assert dec(pp=anns_params(scale=0.0)) == 1
