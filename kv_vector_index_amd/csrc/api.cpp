// C ABI of the wave-index library: argument validation, workspace layout, launch order.
// Nothing here allocates device memory or synchronises; kernels are enqueued on the
// caller's stream.
#include "../../include/wave_index.h"

#include <math.h>

#include <algorithm>
#include <string.h>

#include "wave_kernels.h"

static_assert(wave::kNoAllocScratchBytes == WAVE_NOALLOC_SCRATCH_BYTES,
              "the scratch size in the header and in the library agree");

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves aligned sub-buffers out of one workspace; with base == nullptr it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return na && nb && x < y + nb && y < x + na;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

// ---------------------------------------------------------------- build

struct BuildShape {
  int nseg, C;
  int64_t BH, cache_elems;  // elements of one [B, Hkv, Lcap, d] cache
};

wave_status check_build(const wave_build_params* p, BuildShape* sh) {
  if (!p) return WAVE_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1) return WAVE_ERR_INVALID_ARG;
  if (p->n_q_heads % p->n_kv_heads) return WAVE_ERR_INVALID_ARG;
  if (p->head_dim != wave::kHeadDim) return p->head_dim > 0 ? WAVE_ERR_UNSUPPORTED
                                                            : WAVE_ERR_INVALID_ARG;
  if (p->seq_len < 1 || p->kv_capacity < p->seq_len) return WAVE_ERR_INVALID_ARG;
  if (p->seq_len > (int64_t)1 << 30) return WAVE_ERR_UNSUPPORTED;
  if (p->segment_size < 1 || p->clusters_per_segment < 1) return WAVE_ERR_INVALID_ARG;
  if (p->clusters_per_segment > p->segment_size) return WAVE_ERR_INVALID_ARG;
  if (p->segment_size > 16384 || p->clusters_per_segment > 2048) return WAVE_ERR_UNSUPPORTED;
  if (p->n_iters < 1 || p->n_iters > 1000) return WAVE_ERR_INVALID_ARG;
  if (p->n_sink < 0 || p->n_recent < 0) return WAVE_ERR_INVALID_ARG;
  if ((int64_t)p->n_sink + p->n_recent > p->seq_len) return WAVE_ERR_INVALID_ARG;
  const int64_t nseg = (p->seq_len + p->segment_size - 1) / p->segment_size;
  const int64_t C = nseg * p->clusters_per_segment;
  if (C > INT32_MAX / 2) return WAVE_ERR_UNSUPPORTED;
  int64_t bh, rows, elems;
  if (!mul_ok(p->batch, p->n_kv_heads, &bh) || !mul_ok(bh, p->kv_capacity, &rows) ||
      !mul_ok(rows, wave::kHeadDim, &elems) || elems > INT64_MAX / 4)
    return WAVE_ERR_INVALID_ARG;
  sh->nseg = (int)nseg;
  sh->C = (int)C;
  sh->BH = bh;
  sh->cache_elems = elems;
  return WAVE_OK;
}

// Workspace of the build; returns its size (and fills a when base != nullptr).
size_t layout_build(const wave_build_params* p, const BuildShape& sh, void* base,
                    wave::BuildArgs* a) {
  Carver cv(base);
  const size_t BH = (size_t)sh.BH, L0 = (size_t)p->seq_len, C = (size_t)sh.C;
  float* inv = cv.take<float>(BH * L0);
  uint16_t* mu0 = cv.take<uint16_t>(BH * C * wave::kHeadDim);
  uint16_t* mu1 = cv.take<uint16_t>(BH * C * wave::kHeadDim);
  int32_t* lab = cv.take<int32_t>(BH * L0);
  int32_t* order = cv.take<int32_t>(BH * L0);
  int32_t* cstart = cv.take<int32_t>(BH * sh.nseg * (size_t)(p->clusters_per_segment + 1));
  float* cnorm = cv.take<float>(BH * C);
  if (a) {
    a->inv_norm = inv;
    a->mu[0] = mu0;
    a->mu[1] = mu1;
    a->lab = lab;
    a->order = order;
    a->cstart = cstart;
    a->cnorm = cnorm;
  }
  return cv.off;
}

// ---------------------------------------------------------------- decode

struct DecodeShape {
  int G, nS, nSW, nEW, nStMax, nH, nB, nG, nBDense, rcap;
  int64_t BH, cache_elems;
};

int clampi(int64_t x, int lo, int hi) { return (int)(x < lo ? lo : (x > hi ? hi : x)); }

wave_status check_decode(const wave_decode_params* p, DecodeShape* sh) {
  if (!p) return WAVE_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1) return WAVE_ERR_INVALID_ARG;
  if (p->n_q_heads % p->n_kv_heads) return WAVE_ERR_INVALID_ARG;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G > wave::kMaxGroup) return WAVE_ERR_UNSUPPORTED;
  if (p->head_dim != wave::kHeadDim) return p->head_dim > 0 ? WAVE_ERR_UNSUPPORTED
                                                            : WAVE_ERR_INVALID_ARG;
  if (p->index_len < 1 || p->seq_len < p->index_len || p->kv_capacity < p->seq_len)
    return WAVE_ERR_INVALID_ARG;
  if (p->kv_capacity > (int64_t)1 << 30) return WAVE_ERR_UNSUPPORTED;
  if (p->n_clusters < 1) return WAVE_ERR_INVALID_ARG;
  if (p->n_clusters > wave::kMaxClusters) return WAVE_ERR_UNSUPPORTED;
  if (p->n_sink < 0 || p->n_recent < 0) return WAVE_ERR_INVALID_ARG;
  if ((int64_t)p->n_sink + p->n_recent > p->index_len) return WAVE_ERR_INVALID_ARG;
  if (p->n_retrieve < 0 || p->n_retrieve > p->n_clusters) return WAVE_ERR_INVALID_ARG;
  if (!(p->scale > 0.f) || !isfinite(p->scale)) return WAVE_ERR_INVALID_ARG;
  int64_t bh, rows, elems;
  if (!mul_ok(p->batch, p->n_kv_heads, &bh) || !mul_ok(bh, p->kv_capacity, &rows) ||
      !mul_ok(rows, wave::kHeadDim, &elems) || elems > INT64_MAX / 4)
    return WAVE_ERR_INVALID_ARG;
  if (bh > 65536) return WAVE_ERR_UNSUPPORTED;
  sh->G = G;
  sh->BH = bh;
  sh->cache_elems = elems;
  sh->nS = (p->n_clusters + wave::kChunk - 1) / wave::kChunk;
  const int64_t steady_max = (int64_t)p->n_sink + p->n_recent + (p->kv_capacity - p->index_len);
  sh->nStMax = (int)((steady_max + wave::kTokChunk - 1) / wave::kTokChunk);
  // retrieve workgroups: about kRowsPerItem virtual rows each (a retrieved cluster's tokens
  // plus its estimate-removal row) at 1.5x the average cluster size (the retrieved clusters
  // run larger than average)
  const int64_t indexed = p->index_len - p->n_sink - p->n_recent;
  const int64_t avg = indexed > p->n_clusters ? indexed / p->n_clusters : 1;
  // and at most about four workgroups per CU over all (b, kv-heads), so that they all run
  // in one round
  const int nb_cap = clampi(wave::kRetrieveWGPerCall / bh, 1, wave::kMaxRetrieveWG);
  sh->nB = clampi(((int64_t)p->n_retrieve * (avg + 1) * 3 / 2 + wave::kRowsPerItem - 1) /
                      wave::kRowsPerItem, 1, nb_cap);
  // score workgroups: one per chunk of 128 clusters
  sh->nSW = sh->nS;
  // estimate workgroups: kEstChunks chunks each
  sh->nEW = (sh->nS + wave::kEstChunks - 1) / wave::kEstChunks;
  // retrieve merge groups: one merge of all partials for up to two groups' worth, else
  // groups of about kMergeGroup and a second level
  sh->nG = sh->nB <= 2 * wave::kMergeGroup
               ? 1 : (sh->nB + wave::kMergeGroup - 1) / wave::kMergeGroup;
  // selection workgroups per (b, kv-head): one for heads of at most kLocalSelectMax clusters
  // (it holds all of the head's scores), else one per kSelSpan scores
  const int64_t cp = (int64_t)sh->nS * wave::kChunk;
  sh->nH = cp <= wave::kLocalSelectMax ? 1 : (int)((cp + wave::kSelSpan - 1) / wave::kSelSpan);
  sh->nBDense = clampi((p->kv_capacity + 1023) / 1024, 1, 512);
  sh->rcap = p->n_retrieve > 0 ? p->n_retrieve : 1;
  return WAVE_OK;
}

// Decode workspace (no preparation needed: the score kernel clears the counters in every
// call). Returns the total size.
size_t layout_decode(const wave_decode_params* p, const DecodeShape& sh, void* base,
                     wave::DecodeArgs* a) {
  Carver cv(base);
  const size_t BH = (size_t)sh.BH, G = (size_t)sh.G, C = (size_t)p->n_clusters;
  const size_t Cp = (size_t)sh.nS * wave::kChunk;
  const size_t nP = (size_t)sh.nEW + sh.nStMax + sh.nB + sh.nG;
  const size_t nPmax = nP > (size_t)sh.nBDense ? nP : (size_t)sh.nBDense;
  uint32_t* counter = cv.take<uint32_t>(BH * wave::kCtrStride);
  float* smm = cv.take<float>(BH * (size_t)sh.nSW * 2);
  uint32_t* hist = cv.take<uint32_t>(BH * wave::kHistBins);
  int32_t* sure = cv.take<int32_t>(BH * (size_t)sh.rcap);
  float* tie_key = cv.take<float>(BH * C);
  int32_t* tie_id = cv.take<int32_t>(BH * C);
  float* scores = cv.take<float>(BH * C * G);
  float* shat = cv.take<float>(BH * Cp);
  int32_t* sel_id = cv.take<int32_t>(BH * (size_t)sh.rcap);
  int32_t* sel_ts = cv.take<int32_t>(BH * ((size_t)sh.rcap + 1));
  int32_t* sel_coff = cv.take<int32_t>(BH * (size_t)sh.rcap);
  int32_t* sel_n = cv.take<int32_t>(BH);
  int32_t* wg_info = cv.take<int32_t>(BH * wave::kMaxRetrieveWG * 4);
  float* part = cv.take<float>(BH * nPmax * G * wave::kPartStride);
  if (a) {
    a->counter = counter;
    a->smm = smm;
    a->hist = hist;
    a->sure = sure;
    a->tie_key = tie_key;
    a->tie_id = tie_id;
    a->scores = scores;
    a->shat = shat;
    a->sel_id = sel_id;
    a->sel_ts = sel_ts;
    a->sel_coff = sel_coff;
    a->sel_n = sel_n;
    a->wg_info = wg_info;
    a->part = part;
  }
  return cv.off;
}

void fill_decode_shape(const wave_decode_params* p, const DecodeShape& sh, wave::DecodeArgs* a) {
  a->B = p->batch;
  a->Hq = p->n_q_heads;
  a->Hkv = p->n_kv_heads;
  a->G = sh.G;
  a->L = p->seq_len;
  a->L0 = p->index_len;
  a->Lcap = p->kv_capacity;
  a->C = p->n_clusters;
  a->Cp = sh.nS * wave::kChunk;
  a->n_sink = p->n_sink;
  a->n_recent = p->n_recent;
  a->n_retrieve = p->n_retrieve;
  a->rcap = sh.rcap;
  a->scale = p->scale;
  a->scale_log2 = p->scale * wave::kLog2eHost;
}

}  // namespace

extern "C" {

const char* wave_status_string(wave_status s) {
  switch (s) {
    case WAVE_OK: return "ok";
    case WAVE_ERR_INVALID_ARG: return "invalid argument";
    case WAVE_ERR_UNSUPPORTED: return "unsupported shape";
    case WAVE_ERR_WORKSPACE: return "workspace missing or too small";
    case WAVE_ERR_ALIAS: return "output buffer overlaps an input buffer";
    case WAVE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

wave_status wave_index_workspace_size(const wave_build_params* p, size_t* bytes) {
  if (!bytes) return WAVE_ERR_INVALID_ARG;
  BuildShape sh;
  wave_status st = check_build(p, &sh);
  if (st != WAVE_OK) return st;
  *bytes = layout_build(p, sh, nullptr, nullptr);
  return WAVE_OK;
}

namespace {

// prev != nullptr: an extension of the index prev built for prev_len tokens (segments before
// the first one whose indexed range grew are copied from it, the rest are built).
wave_status build_impl(const wave_build_params* p, const void* k, const void* v, void* k_out,
                       void* v_out, const wave_index* idx, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, wave::Tracer* tr,
                       const wave_index* prev = nullptr, int64_t prev_len = 0) {
  BuildShape sh;
  wave_status st = check_build(p, &sh);
  if (st != WAVE_OK) return st;
  if (!k || !v || !k_out || !v_out || !idx || !idx->centroid_mean || !idx->value_sum ||
      !idx->cluster_size || !idx->cluster_offset)
    return WAVE_ERR_INVALID_ARG;
  const size_t need = layout_build(p, sh, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return WAVE_ERR_WORKSPACE;
  const size_t cache_bytes = (size_t)sh.cache_elems * 2;
  const size_t L0 = (size_t)p->seq_len, BH = (size_t)sh.BH, C = (size_t)sh.C;
  const size_t meta_bytes = BH * C * wave::kHeadDim * 2;
  // outputs must not overlap the inputs (k, v) or each other
  const void* outs[] = {k_out, v_out, idx->centroid_mean, idx->value_sum, idx->cluster_size,
                        idx->cluster_offset, idx->labels, idx->perm, idx->last_centroids,
                        idx->objective, workspace};
  const size_t out_sz[] = {cache_bytes, cache_bytes, meta_bytes, meta_bytes, BH * C * 4,
                           BH * C * 4, BH * L0 * 4, BH * L0 * 4, meta_bytes, BH * 4,
                           workspace_bytes};
  const int nout = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < nout; ++i) {
    if (!outs[i]) continue;
    if (overlaps(outs[i], out_sz[i], k, cache_bytes) || overlaps(outs[i], out_sz[i], v, cache_bytes))
      return WAVE_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (outs[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return WAVE_ERR_ALIAS;
  }

  wave::BuildArgs a{};
  layout_build(p, sh, workspace, &a);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  a.cmean = static_cast<uint16_t*>(idx->centroid_mean);
  a.vsum = static_cast<uint16_t*>(idx->value_sum);
  a.csize = idx->cluster_size;
  a.coff = idx->cluster_offset;
  a.labels = idx->labels;
  a.perm = idx->perm;
  a.last_mu = static_cast<uint16_t*>(idx->last_centroids);
  a.objective = idx->objective;
  a.B = p->batch;
  a.Hkv = p->n_kv_heads;
  a.L0 = p->seq_len;
  a.Lcap = p->kv_capacity;
  a.S = p->segment_size;
  a.kseg = p->clusters_per_segment;
  a.nseg = sh.nseg;
  a.C = sh.C;
  a.T = p->n_iters;
  a.n_sink = p->n_sink;
  a.n_recent = p->n_recent;
  a.idx_lo = p->n_sink;
  a.idx_hi = p->seq_len - p->n_recent;
  a.seg0 = 0;
  if (prev) {
    // the earlier index: prev_len tokens, the same segments and clusters per segment
    if (prev_len < (int64_t)p->n_sink + p->n_recent || prev_len > p->seq_len)
      return WAVE_ERR_INVALID_ARG;
    if (!prev->centroid_mean || !prev->value_sum || !prev->cluster_size ||
        !prev->cluster_offset)
      return WAVE_ERR_INVALID_ARG;
    if (idx->objective) return WAVE_ERR_UNSUPPORTED;  // needs every cluster's pass sums
    // an optional output is copied from the earlier index for the unchanged segments
    if ((idx->labels && !prev->labels) || (idx->perm && !prev->perm) ||
        (idx->last_centroids && !prev->last_centroids))
      return WAVE_ERR_INVALID_ARG;
    const int64_t S = p->segment_size, K = p->clusters_per_segment;
    const int64_t nseg_prev = (prev_len + S - 1) / S, C_prev = nseg_prev * K;
    const int seg0 = (int)((prev_len - p->n_recent) / S);
    const size_t prev_meta = BH * (size_t)C_prev * wave::kHeadDim * 2;
    const void* ins[] = {prev->centroid_mean, prev->value_sum, prev->cluster_size,
                         prev->cluster_offset, prev->labels, prev->perm, prev->last_centroids};
    const size_t in_sz[] = {prev_meta, prev_meta, BH * C_prev * 4, BH * C_prev * 4,
                            BH * (size_t)prev_len * 4, BH * (size_t)prev_len * 4, prev_meta};
    for (int i = 0; i < 7; ++i)
      for (int j = 0; j < nout; ++j)
        if (ins[i] && outs[j] && overlaps(ins[i], in_sz[i], outs[j], out_sz[j]))
          return WAVE_ERR_ALIAS;
    // clusters of segments [0, seg0) and positions [0, seg0 S) keep the earlier index's
    // values (the optional arrays when both indexes have them)
    wave::CopyArgs c{};
    c.BH = (int)BH;
    const int64_t nc = (int64_t)seg0 * K, np = std::min<int64_t>((int64_t)seg0 * S, prev_len);
    auto add = [&](const void* src, void* dst, int64_t words, int64_t ss, int64_t ds) {
      if (src && dst && words > 0)
        c.blk[c.n++] = {static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), words,
                        ss, ds};
    };
    constexpr int64_t kRowWords = wave::kHeadDim / 2;
    add(prev->centroid_mean, idx->centroid_mean, nc * kRowWords, C_prev * kRowWords,
        (int64_t)C * kRowWords);
    add(prev->value_sum, idx->value_sum, nc * kRowWords, C_prev * kRowWords,
        (int64_t)C * kRowWords);
    add(prev->cluster_size, idx->cluster_size, nc, C_prev, C);
    add(prev->cluster_offset, idx->cluster_offset, nc, C_prev, C);
    add(prev->last_centroids, idx->last_centroids, nc * kRowWords, C_prev * kRowWords,
        (int64_t)C * kRowWords);
    add(prev->labels, idx->labels, np, prev_len, (int64_t)L0);
    add(prev->perm, idx->perm, np, prev_len, (int64_t)L0);
    if (wave::launch_copy_blocks(c, stream, tr) != hipSuccess) return WAVE_ERR_HIP;
    a.seg0 = seg0;
    a.extend = 1;
  }
  return wave::launch_build(a, stream, tr) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

}  // namespace

wave_status wave_index_build(const wave_build_params* p, const void* k, const void* v,
                             void* k_out, void* v_out, const wave_index* idx, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return build_impl(p, k, v, k_out, v_out, idx, workspace, workspace_bytes, stream, nullptr);
}

wave_status wave_index_extend(const wave_build_params* p, int64_t prev_seq_len, const void* k,
                              const void* v, void* k_out, void* v_out, const wave_index* prev,
                              const wave_index* idx, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (!prev) return WAVE_ERR_INVALID_ARG;
  return build_impl(p, k, v, k_out, v_out, idx, workspace, workspace_bytes, stream, nullptr,
                    prev, prev_seq_len);
}

wave_status wave_index_build_traced(const wave_build_params* p, const void* k, const void* v,
                                    void* k_out, void* v_out, const wave_index* idx,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    wave_trace* trace) {
  if (!trace || (trace->capacity > 0 && !trace->events)) return WAVE_ERR_INVALID_ARG;
  wave::Tracer tr{trace->events, trace->capacity, 0};
  const wave_status st =
      build_impl(p, k, v, k_out, v_out, idx, workspace, workspace_bytes, stream, &tr);
  trace->recorded = tr.n;
  return st;
}

wave_status wave_decode_workspace_size(const wave_decode_params* p, size_t* bytes) {
  if (!bytes) return WAVE_ERR_INVALID_ARG;
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  *bytes = layout_decode(p, sh, nullptr, nullptr);
  return WAVE_OK;
}

namespace {

// Tier state: counters, block table, slot owners and stamps, the request list.
struct TierShape {
  int64_t nblk, steady_rows;
};
wave_status check_tier(const wave_decode_params* p, const DecodeShape& sh, int32_t n_slots,
                       TierShape* ts) {
  if (n_slots < 1) return WAVE_ERR_INVALID_ARG;
  if (n_slots > (1 << 24)) return WAVE_ERR_UNSUPPORTED;
  ts->nblk = (p->kv_capacity + wave::kTierBlock - 1) / wave::kTierBlock;
  ts->steady_rows = (int64_t)p->n_sink + p->n_recent + (p->kv_capacity - p->index_len);
  if (sh.BH * ts->nblk >= INT32_MAX) return WAVE_ERR_UNSUPPORTED;   // (block ids are int32)
  return WAVE_OK;
}
size_t layout_tier(const DecodeShape& sh, const TierShape& ts, int32_t n_slots, void* base,
                   wave::DecodeArgs* a) {
  Carver cv(base);
  uint32_t* tctr = cv.take<uint32_t>(wave::kTcWords);
  int32_t* tab = cv.take<int32_t>((size_t)sh.BH * ts.nblk);
  uint64_t* slotw = cv.take<uint64_t>((size_t)n_slots);
  uint32_t* valid = cv.take<uint32_t>((size_t)n_slots);
  if (a) {
    a->tctr = tctr;
    a->tab = tab;
    a->slotw = slotw;
    a->valid = valid;
    a->nslots = n_slots;
    a->nblk = (int)ts.nblk;
    a->Ls = ts.steady_rows;
  }
  return cv.off;
}

// tier: null for the cache in device memory (k_cache, v_cache), else the host-memory tier
// (k_cache, v_cache unused).
wave_status decode_impl(const wave_decode_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const wave_index* idx, float* out, float* lse,
                        int32_t* selected, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, wave::Tracer* tr, const wave_tier* tier = nullptr) {
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  TierShape ts{};
  if (tier) {
    st = check_tier(p, sh, tier->n_slots, &ts);
    if (st != WAVE_OK) return st;
    if (!tier->host_k || !tier->host_v || !tier->steady_k || !tier->steady_v || !tier->cache ||
        !tier->state)
      return WAVE_ERR_INVALID_ARG;
    k_cache = tier->host_k;
    v_cache = tier->host_v;
  }
  if (!q || !k_cache || !v_cache || !idx || !idx->centroid_mean || !idx->value_sum ||
      !idx->cluster_size || !idx->cluster_offset || !out)
    return WAVE_ERR_INVALID_ARG;
  const size_t need = layout_decode(p, sh, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return WAVE_ERR_WORKSPACE;
  const size_t BH = (size_t)sh.BH, C = (size_t)p->n_clusters;
  const size_t cache_bytes = (size_t)sh.cache_elems * 2;
  const size_t qb = (size_t)p->batch * p->n_q_heads * wave::kHeadDim;
  const size_t steady_bytes = BH * (size_t)ts.steady_rows * wave::kHeadDim * 2;
  const void* ins[] = {q, k_cache, v_cache, idx->centroid_mean, idx->value_sum,
                       idx->cluster_size, idx->cluster_offset,
                       tier ? tier->steady_k : nullptr, tier ? tier->steady_v : nullptr};
  const size_t in_sz[] = {qb * 2, cache_bytes, cache_bytes, BH * C * wave::kHeadDim * 2,
                          BH * C * wave::kHeadDim * 2, BH * C * 4, BH * C * 4, steady_bytes,
                          steady_bytes};
  const void* outs[] = {out, lse, selected, workspace, tier ? tier->cache : nullptr,
                        tier ? tier->state : nullptr};
  const size_t out_sz[] = {qb * 4, (size_t)p->batch * p->n_q_heads * 4,
                           BH * (size_t)p->n_retrieve * 4, workspace_bytes,
                           tier ? (size_t)tier->n_slots * 2 * wave::kTierBlock * wave::kRowBytes : 0,
                           tier ? layout_tier(sh, ts, tier->n_slots, nullptr, nullptr) : 0};
  for (int i = 0; i < 6; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 9; ++j)
      if (ins[j] && overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return WAVE_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (outs[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return WAVE_ERR_ALIAS;
  }
  wave::DecodeArgs a{};
  layout_decode(p, sh, workspace, &a);
  if (tier) {
    layout_tier(sh, ts, tier->n_slots, tier->state, &a);
    a.tier = 1;
    a.hk = static_cast<const uint16_t*>(tier->host_k);
    a.hv = static_cast<const uint16_t*>(tier->host_v);
    a.sk = static_cast<const uint16_t*>(tier->steady_k);
    a.sv = static_cast<const uint16_t*>(tier->steady_v);
    a.cache = static_cast<uint16_t*>(tier->cache);
  }
  fill_decode_shape(p, sh, &a);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.cmean = static_cast<const uint16_t*>(idx->centroid_mean);
  a.vsum = static_cast<const uint16_t*>(idx->value_sum);
  a.csize = idx->cluster_size;
  a.coff = idx->cluster_offset;
  a.out = out;
  a.lse = lse;
  a.selected = p->n_retrieve > 0 ? selected : nullptr;
  const int64_t n_steady = (int64_t)p->n_sink + p->n_recent + (p->seq_len - p->index_len);
  a.nS = sh.nS;
  a.nSt = (int)((n_steady + wave::kTokChunk - 1) / wave::kTokChunk);
  a.nSW = sh.nSW;
  a.nEW = sh.nEW;
  a.nH = sh.nH;
  a.hist_kernel = sh.nS * wave::kChunk > wave::kLocalSelectMax ? 1 : 0;
  a.nB = sh.nB;
  a.nG = sh.nG;
  a.nP = a.nEW + a.nSt + a.nB + a.nG;
  return wave::launch_decode(a, stream, tr) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

}  // namespace

wave_status wave_decode_attention(const wave_decode_params* p, const void* q, const void* k_cache,
                                  const void* v_cache, const wave_index* idx, float* out,
                                  float* lse, int32_t* selected, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(p, q, k_cache, v_cache, idx, out, lse, selected, workspace,
                     workspace_bytes, stream, nullptr);
}

wave_status wave_decode_attention_traced(const wave_decode_params* p, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const wave_index* idx, float* out, float* lse,
                                         int32_t* selected, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream,
                                         wave_trace* trace) {
  if (!trace || (trace->capacity > 0 && !trace->events)) return WAVE_ERR_INVALID_ARG;
  wave::Tracer tr{trace->events, trace->capacity, 0};
  const wave_status st = decode_impl(p, q, k_cache, v_cache, idx, out, lse, selected, workspace,
                                     workspace_bytes, stream, &tr);
  trace->recorded = tr.n;
  return st;
}

wave_status wave_decode_attention_noalloc(const wave_decode_params* p, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          const wave_index* idx, float* out, float* lse,
                                          int32_t* selected, hipStream_t stream) {
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  const size_t need = layout_decode(p, sh, nullptr, nullptr);
  if (need > wave::kNoAllocScratchBytes) return WAVE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (wave::noalloc_scratch(&ws) != hipSuccess) return WAVE_ERR_HIP;
  return decode_impl(p, q, k_cache, v_cache, idx, out, lse, selected, ws, need, stream,
                     nullptr);
}

wave_status wave_tier_state_size(const wave_decode_params* p, int32_t n_slots, size_t* bytes) {
  if (!bytes) return WAVE_ERR_INVALID_ARG;
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  TierShape ts;
  st = check_tier(p, sh, n_slots, &ts);
  if (st != WAVE_OK) return st;
  *bytes = layout_tier(sh, ts, n_slots, nullptr, nullptr);
  return WAVE_OK;
}

wave_status wave_tier_reset(const wave_decode_params* p, const wave_tier* tier,
                            hipStream_t stream) {
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  if (!tier || !tier->state) return WAVE_ERR_INVALID_ARG;
  TierShape ts;
  st = check_tier(p, sh, tier->n_slots, &ts);
  if (st != WAVE_OK) return st;
  wave::DecodeArgs a{};
  fill_decode_shape(p, sh, &a);
  layout_tier(sh, ts, tier->n_slots, tier->state, &a);
  return wave::launch_tier_reset(a, stream) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

wave_status wave_decode_attention_tiered(const wave_decode_params* p, const void* q,
                                         const wave_tier* tier, const wave_index* idx,
                                         float* out, float* lse, int32_t* selected,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (!tier) return WAVE_ERR_INVALID_ARG;
  return decode_impl(p, q, nullptr, nullptr, idx, out, lse, selected, workspace,
                     workspace_bytes, stream, nullptr, tier);
}

wave_status wave_tier_counters(const wave_decode_params* p, const wave_tier* tier,
                               uint64_t counters[5], hipStream_t stream) {
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  if (!tier || !tier->state || !counters) return WAVE_ERR_INVALID_ARG;
  uint32_t c[wave::kTcWords];
  if (wave::tier_counters_copy(c, tier->state, stream) != hipSuccess) return WAVE_ERR_HIP;
  counters[0] = c[wave::kTcRowsCached];
  counters[1] = c[wave::kTcRowsHost];
  counters[2] = c[wave::kTcAdmitted];
  counters[3] = c[wave::kTcRefused];
  counters[4] = c[wave::kTcRowsWritten];
  return WAVE_OK;
}

wave_status wave_dense_decode_attention(const wave_decode_params* p, const void* q,
                                        const void* k_cache, const void* v_cache, float* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  DecodeShape sh;
  wave_status st = check_decode(p, &sh);
  if (st != WAVE_OK) return st;
  if (!q || !k_cache || !v_cache || !out) return WAVE_ERR_INVALID_ARG;
  const size_t need = layout_decode(p, sh, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return WAVE_ERR_WORKSPACE;
  const size_t cache_bytes = (size_t)sh.cache_elems * 2;
  const size_t qb = (size_t)p->batch * p->n_q_heads * wave::kHeadDim;
  const void* ins[] = {q, k_cache, v_cache};
  const size_t in_sz[] = {qb * 2, cache_bytes, cache_bytes};
  const void* outs[] = {out, lse, workspace};
  const size_t out_sz[] = {qb * 4, (size_t)p->batch * p->n_q_heads * 4, workspace_bytes};
  for (int i = 0; i < 3; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return WAVE_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (outs[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return WAVE_ERR_ALIAS;
  }
  wave::DecodeArgs a{};
  layout_decode(p, sh, workspace, &a);
  fill_decode_shape(p, sh, &a);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.out = out;
  a.lse = lse;
  a.nB = sh.nBDense;
  a.nP = sh.nBDense;
  return wave::launch_dense_decode(a, stream, nullptr) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- attention-aware vector search

namespace {

struct AnnsShape {
  int G;
  int64_t N;        // nodes: the indexed zone [n_sink, L0 - n_recent)
  int64_t BH;
  int nB;           // attention workgroups per (b, kv-head)
};

// Checks shared by the build and the decode (decode = 1 also checks seq_len and scale).
wave_status check_anns(const wave_anns_params* p, int decode, AnnsShape* sh) {
  if (!p) return WAVE_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1 ||
      p->n_q_heads % p->n_kv_heads != 0)
    return WAVE_ERR_INVALID_ARG;
  if (p->head_dim != wave::kHeadDim) return WAVE_ERR_UNSUPPORTED;
  sh->G = p->n_q_heads / p->n_kv_heads;
  if (sh->G > wave::kMaxGroup) return WAVE_ERR_UNSUPPORTED;
  if (p->n_sink < 0 || p->n_recent < 0 || p->index_len < 0 ||
      (int64_t)p->n_sink + p->n_recent > p->index_len || p->index_len > p->kv_capacity ||
      p->kv_capacity > ((int64_t)1 << 40))
    return WAVE_ERR_INVALID_ARG;
  if (decode && (p->seq_len < p->index_len || p->seq_len > p->kv_capacity || !(p->scale > 0.f)))
    return WAVE_ERR_INVALID_ARG;
  if (p->n_train < 1 || p->n_train > wave::kAnnsMaxTrain || p->list_len < 1 ||
      p->list_len > wave::kAnnsMaxList || p->degree < 1 || p->degree > wave::kAnnsMaxDegree ||
      p->n_entry < 1 || p->n_entry > wave::kAnnsMaxEntry || p->pool < 1 ||
      p->pool > wave::kAnnsMaxPool || p->expand < 1 || p->expand > wave::kAnnsMaxExpand ||
      p->expand * p->degree > wave::kAnnsMaxCand || p->n_retrieve < 1 ||
      p->n_retrieve > p->pool || p->max_rounds < 0)
    return WAVE_ERR_INVALID_ARG;
  sh->N = p->index_len - p->n_sink - p->n_recent;
  sh->BH = (int64_t)p->batch * p->n_kv_heads;
  if (sh->N >= ((int64_t)1 << 30) ||
      wave::anns_search_lds(sh->N, p->pool) > wave::kAnnsMaxLds)   // (visited set on chip)
    return WAVE_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(sh->BH, sh->N, &t) || !mul_ok(t, p->degree, &t) || t > ((int64_t)1 << 40))
    return WAVE_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)p->n_sink + p->n_recent + (p->kv_capacity - p->index_len) +
                       p->n_retrieve;
  sh->nB = (int)std::min<int64_t>(std::max<int64_t>((rows + 31) / 32, 1), 64);
  return WAVE_OK;
}

size_t anns_graph_bytes(const wave_anns_params* p, const AnnsShape& sh) {
  return (size_t)sh.BH * sh.N * p->degree * 4;
}
size_t anns_entry_bytes(const wave_anns_params* p, const AnnsShape& sh) {
  return (size_t)sh.BH * p->n_train * 4;
}
size_t anns_lists_bytes(const wave_anns_params* p, const AnnsShape& sh) {
  return (size_t)sh.BH * p->n_train * p->list_len * 4;
}

size_t layout_anns_build(const wave_anns_params* p, const AnnsShape& sh, void* base,
                         wave::AnnsArgs* a) {
  Carver c(base);
  int32_t* cnt = c.take<int32_t>((size_t)sh.BH * sh.N);
  int32_t* off = c.take<int32_t>((size_t)sh.BH * (sh.N + 1));
  int32_t* post = c.take<int32_t>((size_t)sh.BH * p->n_train * p->list_len);
  if (a) {
    a->cnt = cnt;
    a->off = off;
    a->post = post;
  }
  return c.off;
}

size_t layout_anns_decode(const wave_anns_params* p, const AnnsShape& sh, void* base,
                          wave::AnnsArgs* a, wave::DecodeArgs* d) {
  Carver c(base);
  int32_t* pos = c.take<int32_t>((size_t)sh.BH * p->n_retrieve);
  int32_t* n = c.take<int32_t>((size_t)sh.BH);
  float* part = c.take<float>((size_t)sh.BH * sh.nB * sh.G * wave::kPartStride);
  float* seed_s = c.take<float>((size_t)sh.BH * wave::kAnnsMaxSeedWG * p->n_entry);
  int32_t* seed_i = c.take<int32_t>((size_t)sh.BH * wave::kAnnsMaxSeedWG * p->n_entry);
  if (a) {
    a->found_pos = pos;
    a->found_n = n;
    a->seed_s = seed_s;
    a->seed_i = seed_i;
  }
  if (d) {
    d->rows_pos = pos;
    d->rows_n = n;
    d->part = part;
  }
  return c.off;
}

void fill_anns_shape(const wave_anns_params* p, const AnnsShape& sh, wave::AnnsArgs* a) {
  a->B = p->batch;
  a->Hq = p->n_q_heads;
  a->Hkv = p->n_kv_heads;
  a->G = sh.G;
  a->Lcap = p->kv_capacity;
  a->L0 = p->index_len;
  a->n_sink = p->n_sink;
  a->n_recent = p->n_recent;
  a->N = (int)sh.N;
  a->n_t = p->n_train;
  a->M = p->list_len;
  a->R = p->degree;
  a->n_entry = p->n_entry;
  a->ef = p->pool;
  a->W = p->expand;
  a->n_ret = p->n_retrieve;
  a->max_rounds = p->max_rounds;
  a->search_lds = (uint32_t)wave::anns_search_lds(sh.N, p->pool);
  a->nseed = std::min(wave::kAnnsMaxSeedWG, (p->n_train + 255) / 256);
  a->seed_chunk = (p->n_train + a->nseed - 1) / a->nseed;
}

wave_status anns_build_impl(const wave_anns_params* p, const void* k_cache,
                            const wave_anns_index* idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream, wave::Tracer* tr) {
  AnnsShape sh;
  wave_status st = check_anns(p, 0, &sh);
  if (st != WAVE_OK) return st;
  if (!k_cache || !idx || !idx->train || (!idx->graph && sh.N > 0) || !idx->entry ||
      !idx->lists)
    return WAVE_ERR_INVALID_ARG;
  const size_t need = layout_anns_build(p, sh, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return WAVE_ERR_WORKSPACE;
  const size_t cache_bytes = (size_t)sh.BH * p->kv_capacity * wave::kHeadDim * 2;
  const size_t train_bytes = (size_t)sh.BH * p->n_train * wave::kHeadDim * 2;
  const void* ins[] = {k_cache, idx->train};
  const size_t in_sz[] = {cache_bytes, train_bytes};
  const void* outs[] = {idx->graph, idx->entry, idx->lists, workspace};
  const size_t out_sz[] = {anns_graph_bytes(p, sh), anns_entry_bytes(p, sh),
                           anns_lists_bytes(p, sh), workspace_bytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return WAVE_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return WAVE_ERR_ALIAS;
  }
  wave::AnnsArgs a{};
  fill_anns_shape(p, sh, &a);
  layout_anns_build(p, sh, workspace, &a);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.train = static_cast<const uint16_t*>(idx->train);
  a.graph = idx->graph;
  a.entry = idx->entry;
  a.lists = idx->lists;
  return wave::launch_anns_build(a, stream, tr) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

wave_status anns_decode_impl(const wave_anns_params* p, const void* q, const void* k_cache,
                             const void* v_cache, const wave_anns_index* idx, float* out,
                             float* lse, int32_t* retrieved, int32_t* stats, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, wave::Tracer* tr) {
  AnnsShape sh;
  wave_status st = check_anns(p, 1, &sh);
  if (st != WAVE_OK) return st;
  if (!q || !k_cache || !v_cache || !idx || !idx->train || (!idx->graph && sh.N > 0) ||
      !idx->entry || !out)
    return WAVE_ERR_INVALID_ARG;
  const size_t need = layout_anns_decode(p, sh, nullptr, nullptr, nullptr);
  if (!workspace || workspace_bytes < need) return WAVE_ERR_WORKSPACE;
  const size_t cache_bytes = (size_t)sh.BH * p->kv_capacity * wave::kHeadDim * 2;
  const size_t qn = (size_t)p->batch * p->n_q_heads;
  const void* ins[] = {q, k_cache, v_cache, idx->train, idx->graph, idx->entry};
  const size_t in_sz[] = {qn * wave::kHeadDim * 2, cache_bytes, cache_bytes,
                          (size_t)sh.BH * p->n_train * wave::kHeadDim * 2,
                          anns_graph_bytes(p, sh), anns_entry_bytes(p, sh)};
  const void* outs[] = {out, lse, retrieved, stats, workspace};
  const size_t out_sz[] = {qn * wave::kHeadDim * 4, qn * 4,
                           (size_t)sh.BH * p->n_retrieve * 4, (size_t)sh.BH * 8,
                           workspace_bytes};
  for (int i = 0; i < 5; ++i) {
    if (!outs[i]) continue;
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return WAVE_ERR_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (outs[j] && overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return WAVE_ERR_ALIAS;
  }
  wave::AnnsArgs a{};
  wave::DecodeArgs d{};
  fill_anns_shape(p, sh, &a);
  layout_anns_decode(p, sh, workspace, &a, &d);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.train = static_cast<const uint16_t*>(idx->train);
  a.q = static_cast<const uint16_t*>(q);
  a.graph = idx->graph;
  a.entry = idx->entry;
  a.stats = stats;
  d.q = a.q;
  d.k = a.k;
  d.v = static_cast<const uint16_t*>(v_cache);
  d.out = out;
  d.lse = lse;
  d.B = p->batch;
  d.Hq = p->n_q_heads;
  d.Hkv = p->n_kv_heads;
  d.G = sh.G;
  d.L = p->seq_len;
  d.L0 = p->index_len;
  d.Lcap = p->kv_capacity;
  d.n_sink = p->n_sink;
  d.n_recent = p->n_recent;
  d.scale = p->scale;
  d.scale_log2 = p->scale * wave::kLog2eHost;
  d.nB = sh.nB;
  d.nP = sh.nB;
  d.rows_k = p->n_retrieve;
  if (retrieved) {   // (the search writes the caller's buffer, and the attention reads it)
    a.found_pos = retrieved;
    d.rows_pos = retrieved;
  }
  if (wave::launch_anns_search(a, stream, tr) != hipSuccess) return WAVE_ERR_HIP;
  return wave::launch_listed_attention(d, stream, tr) == hipSuccess ? WAVE_OK : WAVE_ERR_HIP;
}

}  // namespace

extern "C" {

wave_status wave_anns_build_workspace_size(const wave_anns_params* p, size_t* bytes) {
  AnnsShape sh;
  const wave_status st = check_anns(p, 0, &sh);
  if (st != WAVE_OK) return st;
  if (!bytes) return WAVE_ERR_INVALID_ARG;
  *bytes = layout_anns_build(p, sh, nullptr, nullptr);
  return WAVE_OK;
}

wave_status wave_anns_build(const wave_anns_params* p, const void* k_cache,
                            const wave_anns_index* idx, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return anns_build_impl(p, k_cache, idx, workspace, workspace_bytes, stream, nullptr);
}

wave_status wave_anns_build_traced(const wave_anns_params* p, const void* k_cache,
                                   const wave_anns_index* idx, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   wave_trace* trace) {
  if (!trace || (trace->capacity > 0 && !trace->events)) return WAVE_ERR_INVALID_ARG;
  wave::Tracer tr{trace->events, trace->capacity, 0};
  const wave_status st = anns_build_impl(p, k_cache, idx, workspace, workspace_bytes, stream,
                                         &tr);
  trace->recorded = tr.n;
  return st;
}

wave_status wave_anns_decode_workspace_size(const wave_anns_params* p, size_t* bytes) {
  AnnsShape sh;
  const wave_status st = check_anns(p, 0, &sh);
  if (st != WAVE_OK) return st;
  if (!bytes) return WAVE_ERR_INVALID_ARG;
  *bytes = layout_anns_decode(p, sh, nullptr, nullptr, nullptr);
  return WAVE_OK;
}

wave_status wave_anns_decode_attention(const wave_anns_params* p, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const wave_anns_index* idx, float* out, float* lse,
                                       int32_t* retrieved, int32_t* stats, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return anns_decode_impl(p, q, k_cache, v_cache, idx, out, lse, retrieved, stats, workspace,
                          workspace_bytes, stream, nullptr);
}

wave_status wave_anns_decode_attention_traced(const wave_anns_params* p, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const wave_anns_index* idx, float* out,
                                              float* lse, int32_t* retrieved, int32_t* stats,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, wave_trace* trace) {
  if (!trace || (trace->capacity > 0 && !trace->events)) return WAVE_ERR_INVALID_ARG;
  wave::Tracer tr{trace->events, trace->capacity, 0};
  const wave_status st = anns_decode_impl(p, q, k_cache, v_cache, idx, out, lse, retrieved,
                                          stats, workspace, workspace_bytes, stream, &tr);
  trace->recorded = tr.n;
  return st;
}

}  // extern "C"
