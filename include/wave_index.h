/*
 * wave_index.h -- C ABI of the MI355X (gfx950) wave-index library.
 *
 * The library implements the data-parallel hot path of RetroInfer's wave index
 * ("Attention-aWare VEctor index"): building the index with segmented spherical k-means
 * over each KV head's keys, and the per-step tripartite decode attention that combines
 * exact attention over the steady and retrieval zones with a centroid estimate of the
 * estimation zone.
 *
 * Sources (web summaries of the RetroInfer paper, arXiv 2505.02922):
 *   - abstract (chatpaper.ai): wave index = tripartite attention approximation,
 *     accuracy-bounded attention estimation, segmented clustering;
 *   - gist.science/de, section 2A; gist.science/fr, section 2A; gist.science/zh,
 *     section 2A: the three zones, centroids plus precomputed value sums for the
 *     estimate with a Jensen lower bound, spherical k-means (fr), segment-local
 *     clustering that exploits RoPE locality (zh);
 *   - gist.science/zh section 3: a retrieval budget of about 1.8 % of the clusters.
 *
 * Conventions shared by every entry point
 *   - Layout. bf16 tensors are IEEE bfloat16 (round to nearest even). K/V caches are
 *     [B, Hkv, Lcap, d] row-major (one 2*d-byte row per token); query head h uses KV head
 *     h / G with G = Hq / Hkv. Only d = 128 is supported.
 *   - Ownership. The caller allocates and owns every buffer (device memory), including the
 *     workspace, whose size the *_workspace_size functions report. The library allocates
 *     no device memory and keeps no state between calls.
 *   - Asynchrony. Compute entry points validate their arguments on the host, enqueue
 *     kernels on `stream` and return; outputs are valid once the stream has reached them.
 *     Calls that share a workspace must not overlap.
 *   - Errors. Invalid arguments are reported before anything is enqueued; a failed kernel
 *     launch returns WAVE_ERR_HIP. Nothing is written on error.
 */
#ifndef WAVE_INDEX_H
#define WAVE_INDEX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WAVE_OK = 0,
  WAVE_ERR_INVALID_ARG = 1,  /* a size, count or pointer is out of range or null */
  WAVE_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement (d != 128,
                                G > 8, an objective output of an extension) */
  WAVE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the reported size */
  WAVE_ERR_ALIAS = 4,        /* an output buffer overlaps an input buffer */
  WAVE_ERR_HIP = 5           /* a HIP launch or runtime call failed */
} wave_status;

/* ------------------------------------------------------------------------------------
 * Index build: segmented spherical k-means over the keys of each (batch element, KV head)
 * ------------------------------------------------------------------------------------
 * Positions [0, n_sink) and [seq_len - n_recent, seq_len) form the steady zone and are not
 * clustered. The indexed positions of segment s are [s*S, (s+1)*S) intersected with
 * [n_sink, seq_len - n_recent). Each segment has clusters_per_segment clusters (global id
 * s * clusters_per_segment + j), so C = ceil(seq_len / S) * clusters_per_segment.
 * Spherical k-means (gist.science/fr section 2A) per segment: unit keys x = k/||k||; seeds
 * mu_j = bf16(x at local point j*floor(n_s/k_seg)) (first n_s points if n_s < k_seg; the
 * remaining clusters stay empty); n_iters passes of "assign each point to the centroid of
 * largest cosine (lowest id on ties), then mu_j = bf16(normalised sum of its unit points)"
 * (an empty cluster keeps its centroid; the last pass is not followed by an update).
 * From the final labels: size n_j, mean raw key bf16(sum k / n_j), value sum bf16(sum v)
 * (gist.science/zh section 2A: centroids and precomputed value sums), and a segment-local
 * permutation of K and V into cluster order (ascending cluster id, ascending position
 * inside a cluster) so that every cluster's tokens are contiguous.
 */
typedef struct {
  int32_t batch;                 /* B >= 1 */
  int32_t n_q_heads;             /* Hq, a multiple of n_kv_heads (only checked, not used) */
  int32_t n_kv_heads;            /* Hkv >= 1 */
  int32_t head_dim;              /* d; must be 128 */
  int64_t seq_len;               /* L0 >= 1: tokens indexed, rows [0, L0) of k and v */
  int64_t kv_capacity;           /* Lcap >= L0: row stride (in tokens) of k, v, k_out, v_out */
  int32_t segment_size;          /* S, 1..16384 */
  int32_t clusters_per_segment;  /* k_seg, 1..min(S, 2048) */
  int32_t n_iters;               /* T, 1..1000 assignment passes */
  int32_t n_sink;                /* >= 0 */
  int32_t n_recent;              /* >= 0, n_sink + n_recent <= L0 */
} wave_build_params;

/* The index of one layer. All arrays are device memory, indexed [B, Hkv, ...]. */
typedef struct {
  void* centroid_mean;     /* bf16 [B, Hkv, C, d]: mean raw key of each cluster (0 if empty) */
  void* value_sum;         /* bf16 [B, Hkv, C, d]: sum of the cluster's value rows (0 if empty) */
  int32_t* cluster_size;   /* [B, Hkv, C]: n_j */
  int32_t* cluster_offset; /* [B, Hkv, C]: first row of cluster j in k_out / v_out */
  int32_t* labels;         /* optional [B, Hkv, L0]: global cluster id per position, -1 steady */
  int32_t* perm;           /* optional [B, Hkv, L0]: perm[row] = source position of k_out row */
  void* last_centroids;    /* optional bf16 [B, Hkv, C, d]: unit centroids of the last pass */
  float* objective;        /* optional [B, Hkv]: sum over clusters of ||sum of unit points|| */
} wave_index;

/* Bytes of workspace wave_index_build needs for these parameters (host only). */
wave_status wave_index_workspace_size(const wave_build_params* p, size_t* bytes);

/* Build the index of one layer.
 *   k, v         bf16 [B, Hkv, Lcap, d] inputs; rows [0, L0) are read.
 *   k_out, v_out bf16 [B, Hkv, Lcap, d] outputs: rows [0, L0) receive the permuted cache
 *                (steady rows unchanged); rows [L0, Lcap) are not touched. They must not
 *                overlap k or v (WAVE_ERR_ALIAS).
 *   idx          output arrays (the optional ones may be NULL).
 *   workspace    device memory of at least wave_index_workspace_size bytes (no clearing
 *                needed). */
wave_status wave_index_build(const wave_build_params* p, const void* k, const void* v,
                             void* k_out, void* v_out, const wave_index* idx,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Extend an index after tokens were appended: the index prev was built (or extended) for
 * prev_seq_len tokens with the same parameters otherwise; idx receives the index for
 * p->seq_len tokens (its arrays sized for that length, not overlapping prev's).
 * Clustering is segment-local (gist.science de/fr/zh, section 2A, "segmented clustering"),
 * so the segments whose indexed range is unchanged keep their clusters: with
 * s0 = floor((prev_seq_len - n_recent) / S), clusters [0, s0 k_seg) and the labels / perm
 * of positions [0, s0 S) are copied from prev, and segments [s0, nseg) are built from k, v
 * as wave_index_build builds them. The result equals wave_index_build for p->seq_len.
 *   k, v         bf16 [B, Hkv, Lcap, d]: the tokens in their original order for rows
 *                [max(s0 S, n_sink), seq_len) (rows before, the sink rows included, are
 *                not read)
 *   k_out, v_out the cache of the earlier build, extended in place: rows
 *                [max(s0 S, n_sink), seq_len) are written as a build writes them, rows
 *                [0, max(s0 S, n_sink)) (the sink rows included) are not touched
 *   prev         the earlier index (only read). Each optional array of idx (labels, perm,
 *                last_centroids) is copied from prev's for the unchanged segments, so prev
 *                must have it too (WAVE_ERR_INVALID_ARG otherwise)
 *   idx          output; idx->objective must be NULL (WAVE_ERR_UNSUPPORTED), since the
 *                objective needs every cluster's pass sums
 *   workspace    as for wave_index_build with p.
 * An extension by nothing (prev_seq_len = seq_len) is valid; it copies prev into idx.
 * WAVE_ERR_INVALID_ARG when prev_seq_len < n_sink + n_recent or > p->seq_len;
 * WAVE_ERR_ALIAS when prev overlaps an output. */
wave_status wave_index_extend(const wave_build_params* p, int64_t prev_seq_len, const void* k,
                              const void* v, void* k_out, void* v_out, const wave_index* prev,
                              const wave_index* idx, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Tripartite decode attention (one step, one layer)
 * ------------------------------------------------------------------------------------
 * For every batch element b and query head h (KV head g = h / G), with scale = p->scale:
 *   s_j = scale * q_h . centroid_mean_j for non-empty clusters, and the group score
 *   s^_j = mean over the G heads of KV head g. The retrieval zone R is the n_retrieve
 *   clusters of largest s^_j (ties to the lower id; all non-empty clusters if fewer).
 *   Exact zone E = [0, n_sink) U [index_len - n_recent, seq_len) U the rows of R's clusters
 *   (the steady zone of the summaries, section 2A, plus the tokens appended since the
 *   build). Estimation zone U = the other non-empty clusters.
 *   out_h = (sum_E e^{a_i} v_i + sum_U e^{s_j} V_j) / (sum_E e^{a_i} + sum_U n_j e^{s_j}),
 *   a_i = scale * q_h . k_i, V_j = value_sum_j; lse_h = log of the denominator.
 * Accumulation is fp32 over bf16 inputs.
 */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;  /* head_dim must be 128; G <= 8 */
  int64_t seq_len;       /* L: rows [0, L) of the cache are attended (L0 <= L <= Lcap) */
  int64_t index_len;     /* L0: rows covered by the index */
  int64_t kv_capacity;   /* Lcap: row stride of the caches */
  int32_t n_clusters;    /* C >= 1 */
  int32_t n_sink;        /* as in the build */
  int32_t n_recent;      /* as in the build; the recent zone extends to L */
  int32_t n_retrieve;    /* 0 <= n_r <= C: clusters attended exactly */
  float scale;           /* > 0, usually 1/sqrt(d) */
} wave_decode_params;

/* Bytes of decode workspace for these parameters (host only). The workspace needs no
 * clearing or other preparation, and a workspace of this size also serves any call whose
 * parameters need no more (the size does not depend on seq_len, so one workspace serves
 * every step up to kv_capacity). Calls that share a workspace must not overlap in time. */
wave_status wave_decode_workspace_size(const wave_decode_params* p, size_t* bytes);

/* One decode step.
 *   q          bf16 [B, Hq, d]
 *   k_cache, v_cache  bf16 [B, Hkv, Lcap, d]: k_out / v_out of the build, with decode
 *              tokens appended at rows [L0, L)
 *   idx        the build's index (only the four required arrays are read)
 *   out        fp32 [B, Hq, d]
 *   lse        optional fp32 [B, Hq]
 *   selected   optional int32 [B, Hkv, n_retrieve]: R in ascending id order, -1 padded
 *   workspace  at least wave_decode_workspace_size bytes (no clearing needed).
 * n_clusters is at most 65536 (WAVE_ERR_UNSUPPORTED above). */
wave_status wave_decode_attention(const wave_decode_params* p, const void* q,
                                  const void* k_cache, const void* v_cache,
                                  const wave_index* idx, float* out, float* lse,
                                  int32_t* selected, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Bytes of the library's own decode scratch used by wave_decode_attention_noalloc. */
#define WAVE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* wave_decode_attention for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same step with
 * the workspace taken from a scratch array of WAVE_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on, from the code object's load until the process
 * ends. The call allocates nothing. Arguments as for wave_decode_attention without the
 * workspace; WAVE_ERR_WORKSPACE when the parameters need more than
 * WAVE_NOALLOC_SCRATCH_BYTES of workspace (wave_decode_workspace_size reports it), checked
 * before anything is enqueued. Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other host threads) race and must not be
 * made; calls on different GPUs do not interfere. */
wave_status wave_decode_attention_noalloc(const wave_decode_params* p, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const wave_index* idx, float* out, float* lse,
                                          int32_t* selected, hipStream_t stream);

/* Dense decode attention over all L rows (the "full attention" the summaries compare
 * against, section 4). Same parameters; the index fields of p are ignored. */
wave_status wave_dense_decode_attention(const wave_decode_params* p, const void* q,
                                        const void* k_cache, const void* v_cache, float* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Host-memory tier: the cache in host memory behind a device block cache
 * ------------------------------------------------------------------------------------
 * The wave buffer of RetroInfer (gist.science de section 2B "Wave Buffer", fr section 2B,
 * zh section 2B) keeps the bulk of the KV cache in CPU memory and a cache of hot blocks on
 * the GPU, exploiting that successive decode steps retrieve largely the same clusters. Here
 * the index (centroids, value sums, sizes, offsets) and the steady zone stay in device
 * memory; the index's layout of the cache (k_out / v_out of the build) lives in pinned host
 * memory; a device cache of n_slots slots holds rows of blocks of 32 consecutive cache rows
 * (K and V, 16 KiB a slot). A decode step selects clusters as wave_decode_attention does and
 * reads each retrieved row from its block's slot when the slot holds the row, else from host
 * memory; a row read from host memory is also written into its block's slot (a slot is
 * claimed for a block that has none: the next slot in a rotating order that the step has not
 * used, a second-chance replacement; a block that finds none stays in host memory). The
 * result is bit-identical to wave_decode_attention on the same rows; only where the rows are
 * read from differs.
 */
typedef struct {
  const void* host_k;    /* pinned host memory (hipHostMalloc), bf16 [B, Hkv, Lcap, d]: the
                            cache in the index's layout (rows of the indexed zone are read) */
  const void* host_v;
  const void* steady_k;  /* device, bf16 [B, Hkv, S_rows, d]: rows [0, n_sink) of the cache,
                            then rows [L0 - n_recent, L) (decode tokens appended in order);
                            S_rows = n_sink + n_recent + Lcap - L0 */
  const void* steady_v;
  void* cache;           /* device, n_slots * 16384 bytes: the block cache */
  void* state;           /* device, wave_tier_state_size bytes: block table, slot owners and
                            stamps, counters; wave_tier_reset sets it up */
  int32_t n_slots;       /* >= 1 */
} wave_tier;

/* Bytes of tier state for these decode parameters and n_slots (host only). */
wave_status wave_tier_state_size(const wave_decode_params* p, int32_t n_slots, size_t* bytes);

/* Empty the block cache: no block cached, step counters and totals zero (enqueued on
 * stream). Needed once before the first tiered step, and after host_k / host_v change. */
wave_status wave_tier_reset(const wave_decode_params* p, const wave_tier* tier,
                            hipStream_t stream);

/* One decode step with the cache in the tier (arguments otherwise as for
 * wave_decode_attention; the workspace is the same size). Steps that share a tier are
 * ordered on one stream. */
wave_status wave_decode_attention_tiered(const wave_decode_params* p, const void* q,
                                         const wave_tier* tier, const wave_index* idx,
                                         float* out, float* lse, int32_t* selected,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* Totals since the last reset, copied to the host (synchronizes stream): retrieved token rows
 * read from the block cache, read from host memory, slots claimed for a block, claims that
 * found no free slot, rows read from host memory and written into the cache. */
wave_status wave_tier_counters(const wave_decode_params* p, const wave_tier* tier,
                               uint64_t counters[5], hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Attention-aware vector search: a second retrieval zone
 * ------------------------------------------------------------------------------------
 * RetrievalAttention (jarxiv.com, "RetrievalAttention: Accelerating Long-Context LLM
 * Inference via Vector Retrieval", abstract) retrieves, at each decode step, the keys most
 * relevant to the query from an approximate-nearest-neighbour index over the KV vectors, and
 * attends to the retrieved tokens; because decode queries and keys follow different
 * distributions, its index adapts to the distribution of the queries. Here, per (b, KV head),
 * the nodes are the keys of the indexed zone [n_sink, L0 - n_recent) of the cache (node x =
 * position n_sink + x; the cache is in position order, not the wave index's layout):
 *   build: each of n_train training queries (the caller's, e.g. prefill queries of the
 *     group's heads) lists its list_len nodes of largest inner product, best first (ties to
 *     the lower id). The list's first node is linked to every other node of the list, and
 *     each of them back to it. A node keeps at most `degree` neighbours, taken without
 *     repeats in the order of (its place in a list, the list's index): where it heads a
 *     list, the list's other nodes in order, else the list's head. The list heads are the
 *     training queries' entries.
 *   search (per step): u = the fp32 sum of the group's query rows (head order); a node's
 *     score is the fp32 dot product of u with its key in a fixed order: each block of 8
 *     dims summed in dim order, then the 16 block sums pairwise, neighbours first; each
 *     product and sum rounded (no fused multiply-add); ties to the lower id. The pool
 *     starts with the entries of the n_entry training queries of largest score; each round
 *     expands the `expand` best unexpanded pool entries (their unvisited neighbours are
 *     scored) and the pool keeps its `pool` best entries, until no entry is left to expand
 *     or max_rounds rounds have run. The n_retrieve best pool entries are retrieved.
 *   attention: softmax over the steady zone [0, n_sink) U [L0 - n_recent, L) and the
 *     retrieved tokens, scale * q . k logits, fp32 accumulation (no estimate of the rest).
 */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;  /* head_dim must be 128; G <= 8 */
  int64_t seq_len;       /* L (decode): rows [0, L) exist; index_len <= L <= kv_capacity */
  int64_t index_len;     /* L0: the graph covers positions [n_sink, L0 - n_recent) */
  int64_t kv_capacity;   /* Lcap: row stride of the caches */
  int32_t n_sink, n_recent;   /* n_sink + n_recent <= L0 */
  int32_t n_train;       /* 1..16384 training queries per (b, KV head) */
  int32_t list_len;      /* 1..64 nodes per training list */
  int32_t degree;        /* 1..64 neighbours per node */
  int32_t n_entry;       /* 1..64 training queries that seed a search */
  int32_t pool;          /* 1..1024 pool entries kept */
  int32_t expand;        /* 1..64 entries expanded per round; expand * degree <= 2048 */
  int32_t n_retrieve;    /* 1..pool nodes retrieved */
  int32_t max_rounds;    /* >= 0 */
  float scale;           /* > 0 (decode), usually 1/sqrt(d) */
} wave_anns_params;

typedef struct {
  const void* train;     /* bf16 [B, Hkv, n_train, d] training queries (build and search) */
  int32_t* graph;        /* [B, Hkv, N, degree] neighbours, -1 padded (N = L0 - n_sink -
                            n_recent; may be NULL when N = 0) */
  int32_t* entry;        /* [B, Hkv, n_train] each training query's first node (-1: none) */
  int32_t* lists;        /* [B, Hkv, n_train, list_len] training lists, -1 padded (written by
                            the build; the search does not read them) */
} wave_anns_index;

/* Bytes of build workspace (host only; no clearing needed). The visited set of a search
 * lives on chip: N is limited to about a million nodes at pool = 1024 (WAVE_ERR_UNSUPPORTED
 * beyond). */
wave_status wave_anns_build_workspace_size(const wave_anns_params* p, size_t* bytes);

/* Build the graph from the cache's keys (k_cache bf16 [B, Hkv, Lcap, d], rows [n_sink,
 * L0 - n_recent) are read) and idx->train; writes graph, entry and lists. */
wave_status wave_anns_build(const wave_anns_params* p, const void* k_cache,
                            const wave_anns_index* idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Bytes of decode workspace (host only; no clearing needed; independent of seq_len). */
wave_status wave_anns_decode_workspace_size(const wave_anns_params* p, size_t* bytes);

/* One decode step: search, then attention.
 *   q          bf16 [B, Hq, d]
 *   k_cache, v_cache  bf16 [B, Hkv, Lcap, d], decode tokens appended at rows [L0, L)
 *   out        fp32 [B, Hq, d];  lse  optional fp32 [B, Hq]
 *   retrieved  optional int32 [B, Hkv, n_retrieve]: retrieved positions, best first, -1
 *              padded
 *   stats      optional int32 [B, Hkv, 2]: rounds run, nodes scored. */
wave_status wave_anns_decode_attention(const wave_anns_params* p, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const wave_anns_index* idx, float* out, float* lse,
                                       int32_t* retrieved, int32_t* stats, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Tracing: per-kernel timing events
 * ------------------------------------------------------------------------------------
 * The *_traced variants behave exactly like their plain counterparts and additionally time
 * their kernels with caller-created HIP events: events[2i] and events[2i + 1] are recorded
 * at the start and at the end of the execution of the i-th kernel of the call (through
 * hipExtLaunchKernel), so hipEventElapsedTime(events[2i], events[2i + 1]) is that kernel's
 * duration. Kernels beyond capacity / 2 run untimed; `recorded` returns the number of events
 * used (twice the number of timed kernels).
 * Kernel order, build: key norms (if any indexed token), seeds, then per pass: assign,
 * sort, and (all passes but the last) update; then finalise, steady-row copy (if
 * n_sink + n_recent > 0), objective (if requested). Decode: score, histogram (only when
 * n_clusters > 8192), gather, retrieve (tiered: then step).
 * Dense decode: partial, merge. Vector-search build: lists, zero (if N > 0), count, and
 * if N > 0 scan, scatter, link. Vector-search decode: seed, search, partial, merge.
 */
typedef struct {
  hipEvent_t* events;   /* capacity events created by the caller (hipEventCreate) */
  int32_t capacity;
  int32_t recorded;     /* out */
} wave_trace;

wave_status wave_index_build_traced(const wave_build_params* p, const void* k, const void* v,
                                    void* k_out, void* v_out, const wave_index* idx,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    wave_trace* trace);

wave_status wave_decode_attention_traced(const wave_decode_params* p, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const wave_index* idx, float* out, float* lse,
                                         int32_t* selected, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream,
                                         wave_trace* trace);

wave_status wave_anns_build_traced(const wave_anns_params* p, const void* k_cache,
                                   const wave_anns_index* idx, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   wave_trace* trace);

wave_status wave_anns_decode_attention_traced(const wave_anns_params* p, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const wave_anns_index* idx, float* out,
                                              float* lse, int32_t* retrieved, int32_t* stats,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, wave_trace* trace);

/* Static, human-readable name of a status code. */
const char* wave_status_string(wave_status s);

#ifdef __cplusplus
}
#endif

#endif /* WAVE_INDEX_H */
