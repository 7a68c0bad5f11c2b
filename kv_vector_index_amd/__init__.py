"""Python binding of libwave_index (MI355X wave index): argument marshalling only.

Every computation runs in the HIP library; this module only converts torch tensors (device
memory) and the current HIP stream into the C ABI's plain pointers, and raises on error.
The names mirror the C entry points declared in include/wave_index.h. PyTorch serves as
the device-memory allocator and stream provider.

If the compiled library is missing, importing the package still works but every call
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

__all__ = [
    "WaveError", "wave_build_params", "wave_index", "wave_decode_params", "library",
    "wave_status_string", "wave_index_workspace_size", "wave_index_build", "wave_index_extend",
    "wave_decode_workspace_size", "wave_decode_attention", "wave_dense_decode_attention",
    "IndexTensors", "alloc_index", "EXPORTED_SYMBOLS", "LIB_PATH", "wave_trace",
    "alloc_decode_workspace", "wave_decode_attention_noalloc", "NOALLOC_SCRATCH_BYTES",
    "wave_tier", "TierTensors", "alloc_tier", "wave_tier_state_size", "wave_tier_reset",
    "wave_decode_attention_tiered", "wave_tier_counters", "TIER_BLOCK",
    "wave_anns_params", "wave_anns_index", "AnnsTensors", "alloc_anns_index",
    "wave_anns_build_workspace_size", "wave_anns_build", "wave_anns_decode_workspace_size",
    "wave_anns_decode_attention",
]

# WAVE_INDEX_LIB selects another build of the library (e.g. the sanitized host-only one)
LIB_PATH = os.environ.get("WAVE_INDEX_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libwave_index.so")
EXPORTED_SYMBOLS = (
    "wave_status_string", "wave_index_workspace_size", "wave_index_build", "wave_index_extend",
    "wave_decode_workspace_size", "wave_decode_attention", "wave_dense_decode_attention",
    "wave_index_build_traced", "wave_decode_attention_traced", "wave_decode_attention_noalloc",
    "wave_tier_state_size", "wave_tier_reset", "wave_decode_attention_tiered",
    "wave_tier_counters", "wave_anns_build_workspace_size", "wave_anns_build",
    "wave_anns_decode_workspace_size", "wave_anns_decode_attention", "wave_anns_build_traced",
    "wave_anns_decode_attention_traced",
)
TIER_BLOCK = 32                    # cache rows per block of the host-memory tier
NOALLOC_SCRATCH_BYTES = 64 << 20   # WAVE_NOALLOC_SCRATCH_BYTES
STATUS = {0: "WAVE_OK", 1: "WAVE_ERR_INVALID_ARG", 2: "WAVE_ERR_UNSUPPORTED",
          3: "WAVE_ERR_WORKSPACE", 4: "WAVE_ERR_ALIAS", 5: "WAVE_ERR_HIP"}


class WaveError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__(f"{fn}: {self.name} ({wave_status_string(code)})")


class wave_build_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("kv_capacity", ctypes.c_int64),
                ("segment_size", ctypes.c_int32), ("clusters_per_segment", ctypes.c_int32),
                ("n_iters", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_recent", ctypes.c_int32)]


class wave_index(ctypes.Structure):
    _fields_ = [("centroid_mean", ctypes.c_void_p), ("value_sum", ctypes.c_void_p),
                ("cluster_size", ctypes.c_void_p), ("cluster_offset", ctypes.c_void_p),
                ("labels", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("last_centroids", ctypes.c_void_p), ("objective", ctypes.c_void_p)]


class wave_decode_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("index_len", ctypes.c_int64),
                ("kv_capacity", ctypes.c_int64), ("n_clusters", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("n_retrieve", ctypes.c_int32), ("scale", ctypes.c_float)]


class wave_tier(ctypes.Structure):
    _fields_ = [("host_k", ctypes.c_void_p), ("host_v", ctypes.c_void_p),
                ("steady_k", ctypes.c_void_p), ("steady_v", ctypes.c_void_p),
                ("cache", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32)]


class wave_anns_params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("index_len", ctypes.c_int64),
                ("kv_capacity", ctypes.c_int64), ("n_sink", ctypes.c_int32),
                ("n_recent", ctypes.c_int32), ("n_train", ctypes.c_int32),
                ("list_len", ctypes.c_int32), ("degree", ctypes.c_int32),
                ("n_entry", ctypes.c_int32), ("pool", ctypes.c_int32),
                ("expand", ctypes.c_int32), ("n_retrieve", ctypes.c_int32),
                ("max_rounds", ctypes.c_int32), ("scale", ctypes.c_float)]


class wave_anns_index(ctypes.Structure):
    _fields_ = [("train", ctypes.c_void_p), ("graph", ctypes.c_void_p),
                ("entry", ctypes.c_void_p), ("lists", ctypes.c_void_p)]


class wave_trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int32),
                ("recorded", ctypes.c_int32)]


_LIB = None


def library() -> ctypes.CDLL:
    """The loaded libwave_index.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.wave_status_string.restype = ctypes.c_char_p
        lib.wave_status_string.argtypes = [ctypes.c_int]
        lib.wave_index_workspace_size.argtypes = [P(wave_build_params), P(sz)]
        lib.wave_index_build.argtypes = [P(wave_build_params), vp, vp, vp, vp, P(wave_index),
                                         vp, sz, vp]
        lib.wave_index_extend.argtypes = [P(wave_build_params), ctypes.c_int64, vp, vp, vp, vp,
                                          P(wave_index), P(wave_index), vp, sz, vp]
        lib.wave_decode_workspace_size.argtypes = [P(wave_decode_params), P(sz)]
        lib.wave_decode_attention.argtypes = [P(wave_decode_params), vp, vp, vp, P(wave_index),
                                              vp, vp, vp, vp, sz, vp]
        lib.wave_dense_decode_attention.argtypes = [P(wave_decode_params), vp, vp, vp, vp, vp,
                                                    vp, sz, vp]
        lib.wave_decode_attention_noalloc.argtypes = [P(wave_decode_params), vp, vp, vp,
                                                      P(wave_index), vp, vp, vp, vp]
        lib.wave_tier_state_size.argtypes = [P(wave_decode_params), ctypes.c_int32, P(sz)]
        lib.wave_tier_reset.argtypes = [P(wave_decode_params), P(wave_tier), vp]
        lib.wave_decode_attention_tiered.argtypes = [P(wave_decode_params), vp, P(wave_tier),
                                                     P(wave_index), vp, vp, vp, vp, sz, vp]
        lib.wave_tier_counters.argtypes = [P(wave_decode_params), P(wave_tier),
                                           P(ctypes.c_uint64), vp]
        lib.wave_anns_build_workspace_size.argtypes = [P(wave_anns_params), P(sz)]
        lib.wave_anns_build.argtypes = [P(wave_anns_params), vp, P(wave_anns_index), vp, sz, vp]
        lib.wave_anns_decode_workspace_size.argtypes = [P(wave_anns_params), P(sz)]
        lib.wave_anns_decode_attention.argtypes = [P(wave_anns_params), vp, vp, vp,
                                                   P(wave_anns_index), vp, vp, vp, vp, vp, sz,
                                                   vp]
        lib.wave_anns_build_traced.argtypes = lib.wave_anns_build.argtypes + [P(wave_trace)]
        lib.wave_anns_decode_attention_traced.argtypes = (
            lib.wave_anns_decode_attention.argtypes + [P(wave_trace)])
        lib.wave_index_build_traced.argtypes = lib.wave_index_build.argtypes + [P(wave_trace)]
        lib.wave_decode_attention_traced.argtypes = (lib.wave_decode_attention.argtypes
                                                     + [P(wave_trace)])
        for name in EXPORTED_SYMBOLS[1:]:
            getattr(lib, name).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise WaveError(fn, code)


def wave_status_string(code: int) -> str:
    return library().wave_status_string(code).decode()


def wave_index_workspace_size(p: wave_build_params) -> int:
    n = ctypes.c_size_t(0)
    _check("wave_index_workspace_size", library().wave_index_workspace_size(ctypes.byref(p),
                                                                             ctypes.byref(n)))
    return n.value


def wave_decode_workspace_size(p: wave_decode_params) -> int:
    n = ctypes.c_size_t(0)
    _check("wave_decode_workspace_size", library().wave_decode_workspace_size(ctypes.byref(p),
                                                                               ctypes.byref(n)))
    return n.value


def alloc_decode_workspace(p: wave_decode_params, device="cuda"):
    """A decode workspace for this shape (allocated with torch; needs no clearing)."""
    import torch
    return torch.empty(wave_decode_workspace_size(p), dtype=torch.uint8, device=device)


@dataclass
class IndexTensors:
    """Device tensors of one layer's index, in the library layout."""
    centroid_mean: object      # bf16 [B, Hkv, C, d]
    value_sum: object          # bf16 [B, Hkv, C, d]
    cluster_size: object       # int32 [B, Hkv, C]
    cluster_offset: object     # int32 [B, Hkv, C]
    labels: object = None      # int32 [B, Hkv, L0]
    perm: object = None        # int32 [B, Hkv, L0]
    last_centroids: object = None
    objective: object = None   # float32 [B, Hkv]

    def c_struct(self) -> wave_index:
        return wave_index(*[_ptr(getattr(self, f)) for f, _ in wave_index._fields_])


def alloc_index(batch: int, n_kv_heads: int, n_clusters: int, seq_len: int, device="cuda",
                optional: bool = True) -> IndexTensors:
    import torch
    B, H, C, d = batch, n_kv_heads, n_clusters, 128
    e = dict(device=device)
    return IndexTensors(
        torch.empty(B, H, C, d, dtype=torch.bfloat16, **e),
        torch.empty(B, H, C, d, dtype=torch.bfloat16, **e),
        torch.empty(B, H, C, dtype=torch.int32, **e),
        torch.empty(B, H, C, dtype=torch.int32, **e),
        torch.empty(B, H, seq_len, dtype=torch.int32, **e) if optional else None,
        torch.empty(B, H, seq_len, dtype=torch.int32, **e) if optional else None,
        torch.empty(B, H, C, d, dtype=torch.bfloat16, **e) if optional else None,
        torch.empty(B, H, dtype=torch.float32, **e) if optional else None,
    )


def _trace(events):
    arr = (ctypes.c_void_p * len(events))(*events)
    return wave_trace(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), len(events), 0), arr


def wave_index_extend(p: wave_build_params, prev_seq_len: int, k, v, k_out, v_out,
                      prev: IndexTensors, index: IndexTensors, workspace, stream=None) -> None:
    """Enqueue the extension of `prev` (built for prev_seq_len tokens) to p.seq_len tokens
    into `index` (see wave_index_extend in include/wave_index.h)."""
    pi, ni = prev.c_struct(), index.c_struct()
    _check("wave_index_extend", library().wave_index_extend(
        ctypes.byref(p), int(prev_seq_len), _ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out),
        ctypes.byref(pi), ctypes.byref(ni), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def wave_index_build(p: wave_build_params, k, v, k_out, v_out, index: IndexTensors, workspace,
                     stream=None, events=None) -> int:
    """Enqueue the index build (see wave_index_build in include/wave_index.h).

    With `events` (a list of created hipEvent_t handles) the traced variant times its
    kernels: events 2i and 2i + 1 bracket the execution of kernel i; returns the number of
    events used (0 without events)."""
    idx = index.c_struct()
    args = (ctypes.byref(p), _ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out), ctypes.byref(idx),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if events is None:
        _check("wave_index_build", library().wave_index_build(*args))
        return 0
    tr, keep = _trace(events)
    _check("wave_index_build_traced", library().wave_index_build_traced(*args, ctypes.byref(tr)))
    return tr.recorded


def wave_decode_attention(p: wave_decode_params, q, k_cache, v_cache, index: IndexTensors, out,
                          lse=None, selected=None, workspace=None, stream=None,
                          events=None) -> int:
    """Enqueue one tripartite decode step (see include/wave_index.h); `events` as for
    wave_index_build."""
    idx = index.c_struct()
    args = (ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(idx), _ptr(out),
            _ptr(lse), _ptr(selected), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream))
    if events is None:
        _check("wave_decode_attention", library().wave_decode_attention(*args))
        return 0
    tr, keep = _trace(events)
    _check("wave_decode_attention_traced",
           library().wave_decode_attention_traced(*args, ctypes.byref(tr)))
    return tr.recorded


def wave_decode_attention_noalloc(p: wave_decode_params, q, k_cache, v_cache,
                                  index: IndexTensors, out, lse=None, selected=None,
                                  stream=None) -> None:
    """Enqueue one decode step that allocates nothing: the workspace is the library's own
    per-GPU scratch (see wave_decode_attention_noalloc in include/wave_index.h)."""
    idx = index.c_struct()
    _check("wave_decode_attention_noalloc", library().wave_decode_attention_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(idx), _ptr(out),
        _ptr(lse), _ptr(selected), _stream(stream)))


def wave_dense_decode_attention(p: wave_decode_params, q, k_cache, v_cache, out, lse=None,
                                workspace=None, stream=None) -> None:
    """Enqueue dense (full) decode attention over all seq_len rows."""
    _check("wave_dense_decode_attention", library().wave_dense_decode_attention(
        ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


def default_scale(head_dim: int = 128) -> float:
    return 1.0 / math.sqrt(head_dim)


# ------------------------------------------------------------------------------------
# host-memory tier
# ------------------------------------------------------------------------------------
@dataclass
class TierTensors:
    """One layer's host-memory tier: the cache in pinned host memory, the steady zone and the
    block cache in device memory, and the tier state (see wave_tier in include/wave_index.h)."""
    host_k: object     # pinned host bf16 [B, Hkv, Lcap, d]
    host_v: object
    steady_k: object   # device bf16 [B, Hkv, n_sink + n_recent + Lcap - L0, d]
    steady_v: object
    cache: object      # device uint8 [n_slots * 16384]
    state: object      # device uint8 [wave_tier_state_size]
    n_slots: int

    def c_struct(self) -> wave_tier:
        return wave_tier(_ptr(self.host_k), _ptr(self.host_v), _ptr(self.steady_k),
                         _ptr(self.steady_v), _ptr(self.cache), _ptr(self.state),
                         int(self.n_slots))


def wave_tier_state_size(p: wave_decode_params, n_slots: int) -> int:
    n = ctypes.c_size_t(0)
    _check("wave_tier_state_size", library().wave_tier_state_size(ctypes.byref(p), int(n_slots),
                                                                   ctypes.byref(n)))
    return n.value


def alloc_tier(p: wave_decode_params, n_slots: int, device="cuda") -> TierTensors:
    """Host and device buffers of a tier for these decode parameters (contents unset: copy the
    cache rows in, then wave_tier_reset)."""
    import torch
    B, H, Lcap, d = p.batch, p.n_kv_heads, p.kv_capacity, 128
    rows = p.n_sink + p.n_recent + (p.kv_capacity - p.index_len)
    hk = torch.empty(B, H, Lcap, d, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(B, H, Lcap, d, dtype=torch.bfloat16, pin_memory=True)
    sk = torch.empty(B, H, rows, d, dtype=torch.bfloat16, device=device)
    sv = torch.empty(B, H, rows, d, dtype=torch.bfloat16, device=device)
    cache = torch.empty(n_slots * 2 * TIER_BLOCK * d * 2, dtype=torch.uint8, device=device)
    state = torch.empty(wave_tier_state_size(p, n_slots), dtype=torch.uint8, device=device)
    return TierTensors(hk, hv, sk, sv, cache, state, n_slots)


def wave_tier_reset(p: wave_decode_params, tier: TierTensors, stream=None) -> None:
    """Enqueue the emptying of the tier's block cache."""
    t = tier.c_struct()
    _check("wave_tier_reset", library().wave_tier_reset(ctypes.byref(p), ctypes.byref(t),
                                                         _stream(stream)))


def wave_decode_attention_tiered(p: wave_decode_params, q, tier: TierTensors,
                                 index: IndexTensors, out, lse=None, selected=None,
                                 workspace=None, stream=None) -> None:
    """Enqueue one decode step with the cache in the host-memory tier."""
    t, idx = tier.c_struct(), index.c_struct()
    _check("wave_decode_attention_tiered", library().wave_decode_attention_tiered(
        ctypes.byref(p), _ptr(q), ctypes.byref(t), ctypes.byref(idx), _ptr(out), _ptr(lse),
        _ptr(selected), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


def wave_tier_counters(p: wave_decode_params, tier: TierTensors, stream=None) -> dict:
    """Totals since the last reset (synchronizes the stream): token rows read from the block
    cache and from host memory, slots claimed and claims refused, rows written into the
    cache."""
    t = tier.c_struct()
    c = (ctypes.c_uint64 * 5)()
    _check("wave_tier_counters", library().wave_tier_counters(ctypes.byref(p), ctypes.byref(t),
                                                               c, _stream(stream)))
    return {"rows_cached": c[0], "rows_host": c[1], "blocks_admitted": c[2],
            "blocks_refused": c[3], "rows_written": c[4]}


# ------------------------------------------------------------------------------------
# attention-aware vector search (a second retrieval zone)
# ------------------------------------------------------------------------------------
@dataclass
class AnnsTensors:
    """One layer's vector-search index (see wave_anns_index in include/wave_index.h)."""
    train: object      # bf16 [B, Hkv, n_train, d]
    graph: object      # int32 [B, Hkv, N, degree]
    entry: object      # int32 [B, Hkv, n_train]
    lists: object      # int32 [B, Hkv, n_train, list_len]

    def c_struct(self) -> wave_anns_index:
        return wave_anns_index(_ptr(self.train), _ptr(self.graph), _ptr(self.entry),
                               _ptr(self.lists))


def alloc_anns_index(p: wave_anns_params, train, device="cuda") -> AnnsTensors:
    """Buffers of the graph for these parameters around the training queries `train`."""
    import torch
    B, H = p.batch, p.n_kv_heads
    N = max(p.index_len - p.n_sink - p.n_recent, 0)
    e = dict(device=device, dtype=torch.int32)
    return AnnsTensors(train, torch.empty(B, H, N, p.degree, **e),
                       torch.empty(B, H, p.n_train, **e),
                       torch.empty(B, H, p.n_train, p.list_len, **e))


def wave_anns_build_workspace_size(p: wave_anns_params) -> int:
    n = ctypes.c_size_t(0)
    _check("wave_anns_build_workspace_size",
           library().wave_anns_build_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def wave_anns_decode_workspace_size(p: wave_anns_params) -> int:
    n = ctypes.c_size_t(0)
    _check("wave_anns_decode_workspace_size",
           library().wave_anns_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def wave_anns_build(p: wave_anns_params, k_cache, index: AnnsTensors, workspace, stream=None,
                    events=None) -> int:
    """Enqueue the graph build (see wave_anns_build in include/wave_index.h); `events` as for
    wave_index_build."""
    idx = index.c_struct()
    args = (ctypes.byref(p), _ptr(k_cache), ctypes.byref(idx), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream))
    if events is None:
        _check("wave_anns_build", library().wave_anns_build(*args))
        return 0
    tr, keep = _trace(events)
    _check("wave_anns_build_traced", library().wave_anns_build_traced(*args, ctypes.byref(tr)))
    return tr.recorded


def wave_anns_decode_attention(p: wave_anns_params, q, k_cache, v_cache, index: AnnsTensors,
                               out, lse=None, retrieved=None, stats=None, workspace=None,
                               stream=None, events=None) -> int:
    """Enqueue one decode step through the vector search (see wave_anns_decode_attention in
    include/wave_index.h); `events` as for wave_index_build."""
    idx = index.c_struct()
    args = (ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(idx),
            _ptr(out), _ptr(lse), _ptr(retrieved), _ptr(stats), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream))
    if events is None:
        _check("wave_anns_decode_attention", library().wave_anns_decode_attention(*args))
        return 0
    tr, keep = _trace(events)
    _check("wave_anns_decode_attention_traced",
           library().wave_anns_decode_attention_traced(*args, ctypes.byref(tr)))
    return tr.recorded
