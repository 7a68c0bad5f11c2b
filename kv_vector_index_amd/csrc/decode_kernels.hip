// Tripartite decode attention of the wave index (gfx950).
//
// The summaries of RetroInfer (gist.science de/fr/zh, section 2A) split attention into a
// steady zone (tokens at the start and end of the context, attended exactly), a retrieval
// zone (the clusters most similar to the query, whose tokens are attended exactly) and an
// estimation zone (every other cluster, approximated from its centroid and its precomputed
// value sum; the zh summary notes that Jensen's inequality makes the estimate a lower bound).
// With logits a_i = scale q.k_i, centroid logits s_j = scale q.c_j, sizes n_j and value
// sums V_j, one query head's output is
//     out = (sum_E e^{a_i} v_i + sum_U e^{s_j} V_j) / (sum_E e^{a_i} + sum_U n_j e^{s_j}).
//
// MI355X design: one persistent kernel per call. Workgroups take work items from an atomic
// ticket, in this order:
//   1. score      (b, kv-head, 256 clusters): stream the centroid rows once, store each query
//                 head's logit and the group-mean score, add the scores to a histogram of
//                 their ordered bit patterns. The workgroup that finishes the last score item
//                 of a (b, kv-head) runs the exact top-n_r selection for it right away
//                 (histogram -> candidate bin -> refinement in LDS; ties to the lower id) and
//                 publishes the retrieved ids and their token list.
//   2. steady     exact attention over the steady zone (no dependency).
//   3. estimate   (b, kv-head, 256 clusters): stream the value sums and fold the estimate of
//                 ALL non-empty clusters into a partial softmax; it waits only for its own
//                 score item. Streaming every value sum (instead of only the unretrieved
//                 ones) lets this run while the selection is still being made.
//   4. retrieved  waits for the selection, attends the retrieved tokens exactly and removes
//                 the estimate terms that step 3 added for the retrieved clusters.
// The workgroup that writes the last partial of a (b, kv-head) merges its partials by
// log-sum-exp into out / lse. Every wait is on an item with a smaller ticket, which a running
// workgroup has already claimed, so the waits always end; each wait is also bounded.
// Rows are read 16 lanes per 256-byte row (4 rows per wave instruction, fully coalesced);
// each K/V row is shared by the G query heads of its group.
#include "wave_common.h"
#include "wave_kernels.h"

namespace wave {

// Per-lane online-softmax state for the G heads of one KV group. A lane owns 8 of the 128
// output dims (dims 8c..8c+7 with c = lane % 16); m and l are replicated across the 16
// lanes of a row group. m is kept in log2 units.
template <int G>
struct Online {
  float m[G], l[G], o[G][8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[h][d] = 0.f;
    }
  }
};

__device__ __forceinline__ float vdim(const u32x4& v, int d) {
  const uint32_t w = v[d >> 1];
  return (d & 1) ? bf_hi(w) : bf_lo(w);
}

// Fold R rows into the state. s2: log2-domain logits (-inf = skip row), w: denominator
// weight of the row (1 for a token, n_j for a cluster estimate, -n_j to remove one),
// vsign: +1 / -1 multiplier of the value row.
template <int G, int R>
__device__ __forceinline__ void fold_rows(Online<G>& st, const float (&s2)[R][G],
                                          const float (&w)[R], const u32x4 (&v)[R],
                                          float vsign) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float tm = s2[0][h];
#pragma unroll
    for (int i = 1; i < R; ++i) tm = fmaxf(tm, s2[i][h]);
    const float mn = fmaxf(st.m[h], tm);
    if (mn == kNegInf) continue;
    const float alpha = fast_exp2(st.m[h] - mn);
    float p[R];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      p[i] = fast_exp2(s2[i][h] - mn);
      ls += w[i] * p[i];
      p[i] *= vsign;
    }
    st.l[h] = alpha * st.l[h] + ls;
    st.m[h] = mn;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      float acc = alpha * st.o[h][d];
#pragma unroll
      for (int i = 0; i < R; ++i) acc += p[i] * vdim(v[i], d);
      st.o[h][d] = acc;
    }
  }
}

// Scale factors of two partial states (m in log2 units) for their merge.
__device__ __forceinline__ void lse_pair(float m1, float m2, float& a1, float& a2, float& mn) {
  mn = fmaxf(m1, m2);
  if (mn == kNegInf) {
    a1 = a2 = 0.f;
  } else {
    a1 = fast_exp2(m1 - mn);
    a2 = fast_exp2(m2 - mn);
  }
}

// Combine the four 16-lane row groups of a wave; afterwards every lane holds the wave state.
template <int G>
__device__ __forceinline__ void merge_row_groups(Online<G>& st) {
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(st.m[h], off);
      const float lo = __shfl_xor(st.l[h], off);
      float a1, a2, mn;
      lse_pair(st.m[h], mo, a1, a2, mn);
      st.m[h] = mn;
      st.l[h] = a1 * st.l[h] + a2 * lo;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float oo = __shfl_xor(st.o[h][d], off);
        st.o[h][d] = a1 * st.o[h][d] + a2 * oo;
      }
    }
  }
}

// Combine the waves of the workgroup and write one partial [G][kPartStride] to dst.
template <int G>
__device__ __forceinline__ void write_block_partial(Online<G>& st, float* __restrict__ dst) {
  constexpr int W = kDecThreads / 64;
  __shared__ float sm[W][G][kPartStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  merge_row_groups<G>(st);
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int d = 0; d < 8; ++d) sm[wave][h][lane * 8 + d] = st.o[h][d];
      if (lane == 0) {
        sm[wave][h][128] = st.m[h];
        sm[wave][h][129] = st.l[h];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * 128; idx += kDecThreads) {
    const int h = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm[w][h][128]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float s = fast_exp2(sm[w][h][128] - M);
        o += s * sm[w][h][d];
        l += s * sm[w][h][129];
      }
    }
    st_dev(dst + h * kPartStride + d, o);
    if (d == 0) {
      st_dev(dst + h * kPartStride + 128, M);
      st_dev(dst + h * kPartStride + 129, l);
    }
  }
  __syncthreads();
}

template <int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int g, int c, u32x4 (&q)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
    q[h] = ld16(a.q + ((size_t)(b * a.Hq + g * G + h) * kHeadDim + c * 8));
}

// logits of R rows for the G heads (all 16 lanes of a row group receive them)
template <int G, int R>
__device__ __forceinline__ void row_logits(const u32x4 (&q)[G], const u32x4 (&k)[R],
                                           float scale, float (&s)[R][G]) {
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int h = 0; h < G; ++h) s[i][h] = sum16(dot8(q[h], k[i])) * scale;
}

// Steady zone: position t of [0, n_steady) -> cache row
__device__ __forceinline__ int64_t steady_row(const DecodeArgs& a, int64_t t) {
  return t < a.n_sink ? t : a.L0 - a.n_recent + (t - a.n_sink);
}

// order-preserving map of a float to uint32 (larger float -> larger key); 0 is reserved
// for empty clusters (score -inf)
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == kNegInf) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------------------------
// block-wide helpers (256 threads)
// ------------------------------------------------------------------------------------
struct ScanTmp {
  uint32_t w[kDecThreads / 64];
};

// exclusive scan over the block; *total = block sum
__device__ __forceinline__ uint32_t scan_excl(uint32_t x, ScanTmp& tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) tmp.w[wave] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kDecThreads / 64; ++w) {
    const uint32_t t = tmp.w[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// Bounded wait until *flag != 0 (thread 0 polls; the block then acquires).
__device__ __forceinline__ void wait_flag(const DecodeArgs& a, const uint32_t* flag) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (ld_dev(flag) == 0u) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 20)) {  // about a second: a missing producer, never expected
        atomicOr(&a.ctl->error, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Data published through flags and counters is written with device-coherent stores
// (st_dev) and read with device-coherent loads (ld_dev); draining each wave's stores
// before the flag update orders the data before the flag for every reader.

// Publish this block's device-coherent writes, then set *flag.
__device__ __forceinline__ void publish_flag(uint32_t* flag) {
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) st_dev(flag, 1u);
}

// Publish this block's device-coherent writes and count one more arrival on *counter;
// true (in every thread) for the block that brings it to n.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n) {
  __shared__ uint32_t s_last;
  drain_vmem();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == n - 1) ? 1u : 0u;
  __syncthreads();
  return s_last != 0u;
}

// ------------------------------------------------------------------------------------
// selection of the retrieval zone for one (b, kv-head), by one workgroup
// ------------------------------------------------------------------------------------
constexpr int kSweep = 32;                     // ids per thread per sweep
constexpr int kSweepIds = kSweep * kDecThreads;

// group scores [j0, j0 + kSweep) as ordered keys (0 past the end); scalar loads, all issued
// before use (rows of these arrays need not be 16-byte aligned)
__device__ __forceinline__ void load_keys(const float* shat, int C, int j0,
                                          uint32_t (&key)[kSweep]) {
  float v[kSweep];
#pragma unroll
  for (int i = 0; i < kSweep; ++i) v[i] = (j0 + i < C) ? ld_dev(shat + j0 + i) : kNegInf;
#pragma unroll
  for (int i = 0; i < kSweep; ++i) key[i] = order_key(v[i]);
}

__device__ __forceinline__ void do_select(const DecodeArgs& a, int bh, uint32_t* s_buf) {
  const int tid = threadIdx.x;
  __shared__ ScanTmp tmp;
  __shared__ uint32_t s_h[256];
  __shared__ uint32_t s_b[2];
  const int C = a.C;
  const float* shat = a.shat + (size_t)bh * C;

  // ---- pass 1: the histogram the score items built (thread t owns the top bins first)
  uint32_t* H = a.hist + (size_t)bh * kHistBins;
  uint32_t h[16];
  const int hb0 = kHistBins - 16 * (tid + 1);    // bins hb0 .. hb0+15, visited descending
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = ld_dev(H + hb0 + i);
#pragma unroll
  for (int i = 0; i < 16; ++i) st_dev(H + hb0 + i, 0u);
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) loc += h[i];
  uint32_t ne;
  const uint32_t above_me = scan_excl(loc, tmp, &ne);
  const uint32_t nr = min((uint32_t)a.n_retrieve, ne);

  // Selection = {key > T} plus the keq lowest ids with key == T.
  uint32_t T, keq;
  if (nr == ne) {
    T = 0u;            // every non-empty cluster (keys > 0)
    keq = 0u;
  } else if (nr == 0) {
    T = 0xffffffffu;   // nothing
    keq = 0u;
  } else {
    uint32_t run = above_me;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (run < nr && run + h[i] >= nr) {
        s_b[0] = (uint32_t)(hb0 + i);
        s_b[1] = run;
      }
      run += h[i];
    }
    __syncthreads();
    const uint32_t bstar = s_b[0];
    uint32_t need = nr - s_b[1];
    __syncthreads();
    // ---- pass 2: candidates = keys in bin bstar, ascending id order
    uint32_t* ckey = a.cand_key + (size_t)bh * C;
    int32_t* cid = a.cand_id + (size_t)bh * C;
    uint32_t n_c = 0;
    for (int base = 0; base < C; base += kSweepIds) {
      const int j0 = base + tid * kSweep;
      uint32_t key[kSweep];
      load_keys(shat, C, j0, key);
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < kSweep; ++i) cnt += (key[i] != 0u && (key[i] >> kHistShift) == bstar);
      uint32_t tot;
      uint32_t pos = n_c + scan_excl(cnt, tmp, &tot);
#pragma unroll
      for (int i = 0; i < kSweep; ++i) {
        if (key[i] != 0u && (key[i] >> kHistShift) == bstar) {
          st_dev(ckey + pos, key[i]);
          st_dev(cid + pos, j0 + i);
          if (pos < (uint32_t)kCandLds) s_buf[pos] = key[i];
          ++pos;
        }
      }
      n_c += tot;
    }
    const bool staged = n_c <= (uint32_t)kCandLds;
    drain_vmem();  // candidates may be re-read from global memory below
    __syncthreads();
    // ---- refine inside the bin: the need-th largest candidate key (256 bins per round)
    uint32_t lo = bstar << kHistShift, hi = lo | ((1u << kHistShift) - 1u);
    for (;;) {
      if (lo == hi) break;
      const uint32_t width = (uint32_t)(((uint64_t)hi - lo + 1 + 255) / 256);
      s_h[tid] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < n_c; i += kDecThreads) {
        const uint32_t k = staged ? s_buf[i] : ld_dev(ckey + i);
        if (k >= lo && k <= hi) atomicAdd(&s_h[(k - lo) / width], 1u);
      }
      __syncthreads();
      const uint32_t cnt = s_h[255 - tid];
      uint32_t tot;
      const uint32_t incl = scan_excl(cnt, tmp, &tot) + cnt;
      if (incl >= need && incl - cnt < need) {
        s_b[0] = 255u - tid;
        s_b[1] = incl - cnt;
      }
      __syncthreads();
      const uint32_t b2 = s_b[0], above = s_b[1];
      __syncthreads();
      need -= above;
      const uint64_t nlo = (uint64_t)lo + (uint64_t)b2 * width;
      const uint64_t nhi = min((uint64_t)hi, nlo + width - 1);
      lo = (uint32_t)nlo;
      hi = (uint32_t)nhi;
      if (width == 1) break;
    }
    T = lo;
    keq = need;
  }

  // ---- pass 3: ordered compaction of the retrieved ids and their token list
  const int32_t* csize = a.csize + (size_t)bh * C;
  const int32_t* coff = a.coff + (size_t)bh * C;
  int32_t* sel = a.sel + (size_t)bh * a.rcap;
  int32_t* slots = a.slots + (size_t)bh * a.L0;
  uint32_t eq_run = 0, sel_run = 0, tok_run = 0;
  for (int base = 0; base < C; base += kSweepIds) {
    const int j0 = base + tid * kSweep;
    uint32_t key[kSweep];
    load_keys(shat, C, j0, key);
    int32_t sz[kSweep];
#pragma unroll
    for (int i = 0; i < kSweep; ++i) sz[i] = (j0 + i < C) ? csize[j0 + i] : 0;
    uint32_t n_eq = 0;
#pragma unroll
    for (int i = 0; i < kSweep; ++i) n_eq += (T != 0u && key[i] == T);
    uint32_t tot_eq;
    uint32_t e = eq_run + scan_excl(n_eq, tmp, &tot_eq);
    uint32_t n_sel = 0, n_tok = 0, take = 0u;  // take: bit i = id j0 + i retrieved
#pragma unroll
    for (int i = 0; i < kSweep; ++i) {
      bool t = key[i] > T;
      if (T != 0u && key[i] == T) {
        t = e < keq;
        ++e;
      }
      take |= (t ? 1u : 0u) << i;
      n_sel += t;
      n_tok += t ? (uint32_t)sz[i] : 0u;
    }
    uint32_t tot_sel, tot_tok;
    uint32_t ps = sel_run + scan_excl(n_sel, tmp, &tot_sel);
    uint32_t pt = tok_run + scan_excl(n_tok, tmp, &tot_tok);
    while (take) {  // few ids per thread; sizes and offsets re-read from memory
      const int i = __builtin_ctz(take);
      take &= take - 1u;
      const int j = j0 + i;
      if (ps < (uint32_t)a.rcap) st_dev(sel + ps, j);
      if (a.selected && ps < (uint32_t)a.n_retrieve)
        a.selected[(size_t)bh * a.n_retrieve + ps] = j;
      ++ps;
      const int n = csize[j], o = coff[j];
      for (int r = 0; r < n && pt + r < (uint32_t)a.L0; ++r) st_dev(slots + pt + r, o + r);
      pt += (uint32_t)n;
    }
    eq_run += tot_eq;
    sel_run += tot_sel;
    tok_run += tot_tok;
  }
  if (a.selected)
    for (int r = (int)sel_run + tid; r < a.n_retrieve; r += kDecThreads)
      a.selected[(size_t)bh * a.n_retrieve + r] = -1;
  if (tid == 0) {
    st_dev(a.nsel + bh, (int32_t)min(sel_run, (uint32_t)a.rcap));
    st_dev(a.ntok + bh, (int32_t)min(tok_run, (uint32_t)a.L0));
  }
  publish_flag(a.sel_ready + bh);
}

// ------------------------------------------------------------------------------------
// work items
// ------------------------------------------------------------------------------------

// Merge the n partials of one (b, kv-head) into out / lse.
template <int G>
__device__ __forceinline__ void final_merge(const DecodeArgs& a, int bh, const float* parts, int n) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  for (int idx = threadIdx.x; idx < G * 128; idx += kDecThreads) {
    const int h = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll 8
    for (int p = 0; p < n; ++p) M = fmaxf(M, ld_dev(parts + (p * G + h) * kPartStride + 128));
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll 8
      for (int p = 0; p < n; ++p) {
        const float* pp = parts + (p * G + h) * kPartStride;
        const float s = fast_exp2(ld_dev(pp + 128) - M);
        o += s * ld_dev(pp + d);
        l += s * ld_dev(pp + 129);
      }
    }
    const size_t qh = (size_t)b * a.Hq + g * G + h;
    a.out[qh * kHeadDim + d] = o / l;
    if (d == 0 && a.lse) a.lse[qh] = (M + log2f(l)) * kLn2;
  }
}

template <int G>
__device__ __forceinline__ void finish_partial(const DecodeArgs& a, int bh, Online<G>& st,
                                               int p) {
  float* parts = a.part + (size_t)bh * a.nP * G * kPartStride;
  write_block_partial<G>(st, parts + (size_t)p * G * kPartStride);
  if (arrive_last(a.part_done + bh, (uint32_t)a.nP)) {
    final_merge<G>(a, bh, parts, a.nP);
    if (a.local_select)  // every reader of this head's histogram is done: clear it
      for (int i = threadIdx.x; i < kHistBins; i += kDecThreads)
        st_dev(a.hist + (size_t)bh * kHistBins + i, 0u);
  }
}

template <int G>
__device__ __forceinline__ void item_score(const DecodeArgs& a, int bh, int c, uint32_t* s_buf) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, cc = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  for (int i = tid; i < kHistBins; i += kDecThreads) s_buf[i] = 0u;
  __syncthreads();
  const size_t base = (size_t)bh * a.C;
  const int wbeg = c * kChunk + wave * (kChunk / 4);
  const int wend = min(a.C, wbeg + kChunk / 4);
  const float sl2 = a.scale_log2;
  // two tiles of 4 rows per row group in flight (8 rows, 32 per wave)
  for (int t = wbeg; t < wend; t += 32) {
    u32x4 kr[8];
    int32_t n[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = t + 4 * i + grp;
      if (j < wend) {
        kr[i] = ld16_stream(a.cmean + (base + j) * kHeadDim + cc * 8);
        n[i] = a.csize[base + j];
      } else {
        kr[i] = u32x4{0, 0, 0, 0};
        n[i] = -1;
      }
    }
    float s[8][G];
    row_logits<G, 8>(q, kr, 1.f, s);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = t + 4 * i + grp;
      if (n[i] < 0) continue;
      float mean = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) mean += s[i][h] * a.scale;
      mean = mean / (float)G;
      const float sh = n[i] > 0 ? mean : kNegInf;
      if (cc < G) {
        float mine = s[i][0];
#pragma unroll
        for (int h = 1; h < G; ++h) mine = (cc == h) ? s[i][h] : mine;
        st_dev(a.scores + (base + j) * G + cc, mine * sl2);
      }
      if (cc == 0) {
        st_dev(a.shat + base + j, sh);
        const uint32_t key = order_key(sh);
        if (key) atomicAdd(&s_buf[key >> kHistShift], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* H = a.hist + (size_t)bh * kHistBins;
  for (int i = tid; i < kHistBins; i += kDecThreads)
    if (s_buf[i]) atomicAdd(&H[i], s_buf[i]);
  publish_flag(a.chunk_ready + (size_t)bh * a.nS + c);
  if (arrive_last(a.score_done + bh, (uint32_t)a.nS) && !a.local_select) do_select(a, bh, s_buf);
}

template <int G>
__device__ __forceinline__ void item_steady(const DecodeArgs& a, int bh, int i_item) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, cc = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  Online<G> st;
  st.init();
  const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
  const int64_t wbeg = (int64_t)i_item * kTokChunk + wave * (kTokChunk / 4);
  const int64_t wend = min(n_steady, wbeg + kTokChunk / 4);
  const size_t base = (size_t)bh * a.Lcap;
  for (int64_t t = wbeg; t < wend; t += 32) {
    u32x4 kr[8], vr[8];
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tt = t + 4 * i + grp;
      if (tt < wend) {
        const size_t row = (base + steady_row(a, tt)) * kHeadDim + cc * 8;
        kr[i] = ld16_stream(a.k + row);
        vr[i] = ld16_stream(a.v + row);
        w[i] = 1.f;
      } else {
        kr[i] = vr[i] = u32x4{0, 0, 0, 0};
        w[i] = 0.f;
      }
    }
    float s[8][G];
    row_logits<G, 8>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (w[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, 8>(st, s, w, vr, 1.f);
  }
  finish_partial<G>(a, bh, st, i_item);
}

template <int G>
__device__ __forceinline__ void item_estimate(const DecodeArgs& a, int bh, int c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, cc = lane & 15;
  wait_flag(a, a.chunk_ready + (size_t)bh * a.nS + c);
  Online<G> st;
  st.init();
  const size_t base = (size_t)bh * a.C;
  const int wbeg = c * kChunk + wave * (kChunk / 4);
  const int wend = min(a.C, wbeg + kChunk / 4);
  for (int t = wbeg; t < wend; t += 32) {
    u32x4 vr[8];
    float w[8], s[8][G];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = t + 4 * i + grp;
      if (j < wend) {
        vr[i] = ld16_stream(a.vsum + (base + j) * kHeadDim + cc * 8);
        w[i] = (float)a.csize[base + j];
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = ld_dev(a.scores + (base + j) * G + h);
      } else {
        vr[i] = u32x4{0, 0, 0, 0};
        w[i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (w[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, 8>(st, s, w, vr, 1.f);
  }
  finish_partial<G>(a, bh, st, a.nSt + c);
}

// Exact attention over the rows given by row_of(t) for t in [wb, we) (rows are cache rows).
template <int G, typename RowOf>
__device__ __forceinline__ void attend_rows(const DecodeArgs& a, int bh, const u32x4 (&q)[G],
                                            Online<G>& st, int64_t wb, int64_t we, RowOf row_of) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, cc = lane & 15;
  const size_t base = (size_t)bh * a.Lcap;
  for (int64_t t = wb; t < we; t += 32) {
    int64_t sl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tt = t + 4 * i + grp;
      sl[i] = tt < we ? (int64_t)row_of(tt) : -1;
    }
    u32x4 kr[8], vr[8];
    float wt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (sl[i] >= 0) {
        const size_t row = (base + sl[i]) * kHeadDim + cc * 8;
        kr[i] = ld16_stream(a.k + row);
        vr[i] = ld16_stream(a.v + row);
        wt[i] = 1.f;
      } else {
        kr[i] = vr[i] = u32x4{0, 0, 0, 0};
        wt[i] = 0.f;
      }
    }
    float s[8][G];
    row_logits<G, 8>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (wt[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, 8>(st, s, wt, vr, 1.f);
  }
}

// Remove the estimate terms of the clusters id_of(k), k in [wb, we), from the state: the
// same stored logits, weight -n_j and value -V_j (the estimate items added them).
template <int G, typename IdOf>
__device__ __forceinline__ void remove_estimates(const DecodeArgs& a, int bh, Online<G>& st,
                                                 int wb, int we, IdOf id_of) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, cc = lane & 15;
  const size_t base = (size_t)bh * a.C;
  for (int t = wb; t < we; t += 16) {
    int32_t jr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = t + 4 * i + grp;
      jr[i] = tt < we ? id_of(tt) : -1;
    }
    u32x4 vr[4];
    float wt[4], s[4][G];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (jr[i] >= 0) {
        vr[i] = ld16(a.vsum + (base + jr[i]) * kHeadDim + cc * 8);
        wt[i] = -(float)a.csize[base + jr[i]];
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = ld_dev(a.scores + (base + jr[i]) * G + h);
      } else {
        vr[i] = u32x4{0, 0, 0, 0};
        wt[i] = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
      }
    }
    fold_rows<G, 4>(st, s, wt, vr, -1.f);
  }
}

// Retrieved item, published selection (many clusters): the select of the last score item
// listed the retrieved ids and their cache rows.
template <int G>
__device__ __forceinline__ void item_retrieved_published(const DecodeArgs& a, int bh, int w_item) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, cc = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  wait_flag(a, a.sel_ready + bh);
  Online<G> st;
  st.init();
  const int nB = a.nB;
  const int64_t ntok = ld_dev(a.ntok + bh);
  const int64_t t0 = ntok * w_item / nB, t1 = ntok * (w_item + 1) / nB;
  const int32_t* slots = a.slots + (size_t)bh * a.L0;
  attend_rows<G>(a, bh, q, st, t0 + (t1 - t0) * wave / 4, t0 + (t1 - t0) * (wave + 1) / 4,
                 [&](int64_t t) { return ld_dev(slots + t); });
  const int ns = ld_dev(a.nsel + bh);
  const int k0 = (int)((int64_t)ns * w_item / nB), k1 = (int)((int64_t)ns * (w_item + 1) / nB);
  const int32_t* sel = a.sel + (size_t)bh * a.rcap;
  remove_estimates<G>(a, bh, st, k0 + (k1 - k0) * wave / 4, k0 + (k1 - k0) * (wave + 1) / 4,
                      [&](int k) { return ld_dev(sel + k); });
  finish_partial<G>(a, bh, st, a.nSt + a.nS + w_item);
}

// Bounded wait until *counter >= n (thread 0 polls; the block then proceeds).
__device__ __forceinline__ void wait_count(const DecodeArgs& a, const uint32_t* counter,
                                           uint32_t n) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (ld_dev(counter) < n) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 20)) {  // about a second: a missing producer, never expected
        atomicOr(&a.ctl->error, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Retrieved item, local selection (up to kLocalSelMax clusters): every retrieved item of a
// (b, kv-head) recomputes the same exact selection from the histogram and the group scores
// staged in LDS as soon as the head's score items are done, then attends its share of the
// selected tokens. This saves the round trips of publishing a list and waiting for it.
// Dynamic LDS (words): keys [per][256] (entry (i, t) = cluster t*per + i, so that thread t
// walks its own ids without bank conflicts), sizes u16 [per][256], then three windows of
// kWin words.
template <int G>
__device__ __forceinline__ void item_retrieved_local(const DecodeArgs& a, int bh, int w_item,
                                                     uint32_t* dyn) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cc = lane & 15;
  const int C = a.C;
  const int per = (C + kDecThreads - 1) / kDecThreads;
  uint32_t* s_key = dyn;
  uint16_t* s_sz = reinterpret_cast<uint16_t*>(dyn + per * kDecThreads);
  uint32_t* wp = dyn + per * kDecThreads + (per * kDecThreads + 1) / 2;
  uint32_t* wn = wp + kWin;
  int32_t* wo = reinterpret_cast<int32_t*>(wn + kWin);
  __shared__ ScanTmp tmp;
  __shared__ uint32_t s_h[256];
  __shared__ uint32_t s_b[2];
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  wait_count(a, a.score_done + bh, (uint32_t)a.nS);
  const size_t cb = (size_t)bh * C;

  // ---- one round trip: histogram, group scores and sizes
  const uint32_t* H = a.hist + (size_t)bh * kHistBins;
  const int hb0 = kHistBins - 16 * (tid + 1);  // this thread's bins, visited descending
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = ld_dev(H + hb0 + i);
  for (int i0 = 0; i0 < per; i0 += 16) {
    float v[16];
    int32_t z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = tid * per + i0 + e;
      const bool ok = (i0 + e < per) && j < C;
      v[e] = ok ? ld_dev(a.shat + cb + j) : kNegInf;
      z[e] = ok ? a.csize[cb + j] : 0;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (i0 + e < per) {
        s_key[(i0 + e) * kDecThreads + tid] = order_key(v[e]);
        s_sz[(i0 + e) * kDecThreads + tid] = (uint16_t)z[e];
      }
  }
  uint32_t loc = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) loc += h[i];
  uint32_t ne;
  const uint32_t above_me = scan_excl(loc, tmp, &ne);  // also publishes the LDS stores
  const uint32_t nr = min((uint32_t)a.n_retrieve, ne);

  // ---- threshold: selection = {key > T} plus the keq lowest ids with key == T
  uint32_t T, keq;
  if (nr == ne) {
    T = 0u;
    keq = 0u;
  } else if (nr == 0) {
    T = 0xffffffffu;
    keq = 0u;
  } else {
    uint32_t run = above_me;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (run < nr && run + h[i] >= nr) {
        s_b[0] = (uint32_t)(hb0 + i);
        s_b[1] = run;
      }
      run += h[i];
    }
    __syncthreads();
    uint32_t lo = s_b[0] << kHistShift, need = nr - s_b[1];
    uint32_t hi = lo | ((1u << kHistShift) - 1u);
    __syncthreads();
    for (;;) {  // 256 bins per round over the keys inside [lo, hi]
      if (lo == hi) break;
      const uint32_t width = (uint32_t)(((uint64_t)hi - lo + 1 + 255) / 256);
      s_h[tid] = 0u;
      __syncthreads();
      for (int i = 0; i < per; ++i) {
        const uint32_t k = s_key[i * kDecThreads + tid];
        if (k >= lo && k <= hi) atomicAdd(&s_h[(k - lo) / width], 1u);
      }
      __syncthreads();
      const uint32_t cnt = s_h[255 - tid];
      uint32_t tot;
      const uint32_t incl = scan_excl(cnt, tmp, &tot) + cnt;
      if (incl >= need && incl - cnt < need) {
        s_b[0] = 255u - tid;
        s_b[1] = incl - cnt;
      }
      __syncthreads();
      const uint32_t b2 = s_b[0], above = s_b[1];
      __syncthreads();
      need -= above;
      const uint64_t nlo = (uint64_t)lo + (uint64_t)b2 * width;
      const uint64_t nhi = min((uint64_t)hi, nlo + width - 1);
      lo = (uint32_t)nlo;
      hi = (uint32_t)nhi;
      if (width == 1) break;
    }
    T = lo;
    keq = need;
  }

  // ---- ranks and token offsets of this thread's retrieved ids (ascending id order)
  uint32_t n_eq = 0;
  for (int i = 0; i < per; ++i) n_eq += (T != 0u && s_key[i * kDecThreads + tid] == T);
  uint32_t tot;
  const uint32_t eq0 = scan_excl(n_eq, tmp, &tot);
  // walk(f): f(rank, token offset, size, id) for each retrieved id of this thread
  auto walk = [&](uint32_t r, uint32_t p, auto f) {
    uint32_t e = eq0;
    for (int i = 0; i < per; ++i) {
      const uint32_t k = s_key[i * kDecThreads + tid];
      bool take = k > T;
      if (T != 0u && k == T) {
        take = e < keq;
        ++e;
      }
      if (take) {
        const uint32_t n = s_sz[i * kDecThreads + tid];
        f(r, p, n, tid * per + i);
        ++r;
        p += n;
      }
    }
  };
  uint32_t my_sel = 0, my_tok = 0;
  walk(0u, 0u, [&](uint32_t, uint32_t, uint32_t n, int) {
    ++my_sel;
    my_tok += n;
  });
  uint32_t nsel, ntok;
  const uint32_t r0 = scan_excl(my_sel, tmp, &nsel);
  const uint32_t p0 = scan_excl(my_tok, tmp, &ntok);
  if (w_item == 0 && a.selected) {
    walk(r0, p0, [&](uint32_t r, uint32_t, uint32_t, int j) {
      if (r < (uint32_t)a.n_retrieve) a.selected[(size_t)bh * a.n_retrieve + r] = j;
    });
    for (int r = (int)nsel + tid; r < a.n_retrieve; r += kDecThreads)
      a.selected[(size_t)bh * a.n_retrieve + r] = -1;
  }
  Online<G> st;
  st.init();
  const int nB = a.nB;
  // tokens [T0, T1) of the selection belong to this item; clusters [R0, R1) overlap them
  const uint32_t T0 = (uint32_t)((uint64_t)ntok * w_item / nB);
  const uint32_t T1 = (uint32_t)((uint64_t)ntok * (w_item + 1) / nB);
  uint32_t c_before = 0, c_upto = 0;
  walk(r0, p0, [&](uint32_t, uint32_t p, uint32_t n, int) {
    c_before += (p + n <= T0);
    c_upto += (p < T1);
  });
  uint32_t R0, R1;
  scan_excl(c_before, tmp, &R0);
  scan_excl(c_upto, tmp, &R1);
  for (uint32_t Rw = R0; Rw < R1; Rw += kWin) {
    const uint32_t cnt = min((uint32_t)kWin, R1 - Rw);
    walk(r0, p0, [&](uint32_t r, uint32_t p, uint32_t n, int j) {
      if (r >= Rw && r < Rw + cnt) {
        wp[r - Rw] = p;
        wn[r - Rw] = n;
        wo[r - Rw] = j;
      }
    });
    __syncthreads();
    for (uint32_t i = tid; i < cnt; i += kDecThreads) wo[i] = a.coff[cb + wo[i]];
    __syncthreads();
    const int64_t ts = max(T0, wp[0]), te = min(T1, wp[cnt - 1] + wn[cnt - 1]);
    attend_rows<G>(a, bh, q, st, ts + (te - ts) * wave / 4, ts + (te - ts) * (wave + 1) / 4,
                   [&](int64_t t) {
                     // the window cluster holding token t (token starts ascend)
                     uint32_t lo = 0, hi = cnt - 1;
                     while (lo < hi) {
                       const uint32_t mid = (lo + hi + 1) >> 1;
                       if (wp[mid] <= (uint32_t)t) lo = mid; else hi = mid - 1;
                     }
                     return (int64_t)wo[lo] + (t - wp[lo]);
                   });
    __syncthreads();
  }
  // the estimate terms of the selected clusters [K0, K1) (by rank) are removed here
  const uint32_t K0 = (uint32_t)((uint64_t)nsel * w_item / nB);
  const uint32_t K1 = (uint32_t)((uint64_t)nsel * (w_item + 1) / nB);
  for (uint32_t Kw = K0; Kw < K1; Kw += kWin) {
    const uint32_t cnt = min((uint32_t)kWin, K1 - Kw);
    walk(r0, p0, [&](uint32_t r, uint32_t, uint32_t, int j) {
      if (r >= Kw && r < Kw + cnt) wo[r - Kw] = j;
    });
    __syncthreads();
    remove_estimates<G>(a, bh, st, (int)(cnt * wave / 4), (int)(cnt * (wave + 1) / 4),
                        [&](int k) { return wo[k]; });
    __syncthreads();
  }
  finish_partial<G>(a, bh, st, a.nSt + a.nS + w_item);
}

// ------------------------------------------------------------------------------------
// the persistent decode kernel
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_decode(DecodeArgs a) {
  __shared__ uint32_t s_buf[kHistBins];
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_ticket;
  const int BH = a.B * a.Hkv;
  const uint32_t nScore = (uint32_t)BH * a.nS;
  const uint32_t nSteady = nScore + (uint32_t)BH * a.nSt;
  const uint32_t nEst = nSteady + (uint32_t)BH * a.nS;
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.ctl->ticket, 1u);
  __syncthreads();
  for (;;) {
    const uint32_t t = s_ticket;
    __syncthreads();
    if (t >= a.total_items) break;
    uint32_t next = 0;
    if (threadIdx.x == 0) next = atomicAdd(&a.ctl->ticket, 1u);  // prefetch the next item
    if (t < nScore) {
      item_score<G>(a, (int)(t % BH), (int)(t / BH), s_buf);
    } else if (t < nSteady) {
      const uint32_t u = t - nScore;
      item_steady<G>(a, (int)(u % BH), (int)(u / BH));
    } else if (t < nEst) {
      const uint32_t u = t - nSteady;
      item_estimate<G>(a, (int)(u % BH), (int)(u / BH));
    } else {
      const uint32_t u = t - nEst;
      if (a.local_select)
        item_retrieved_local<G>(a, (int)(u % BH), (int)(u / BH), s_dyn);
      else
        item_retrieved_published<G>(a, (int)(u % BH), (int)(u / BH));
    }
    __syncthreads();
    if (threadIdx.x == 0) s_ticket = next;
    __syncthreads();
  }
  // the last workgroup to leave returns the control words to zero for the next call
  if (arrive_last(&a.ctl->exited, gridDim.x)) {
    for (int i = threadIdx.x; i < BH; i += kDecThreads) {
      a.score_done[i] = 0u;
      a.part_done[i] = 0u;
      a.sel_ready[i] = 0u;
    }
    for (int i = threadIdx.x; i < BH * a.nS; i += kDecThreads) a.chunk_ready[i] = 0u;
    if (threadIdx.x == 0) {
      a.ctl->ticket = 0u;
      a.ctl->exited = 0u;
    }
  }
}

// ------------------------------------------------------------------------------------
// Dense decode (full attention over [0, L)): split-K partials + merge
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dense_partial(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, c = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, c, q);
  Online<G> st;
  st.init();
  const int nB = a.nB, w = blockIdx.x;
  const int64_t t0 = a.L * w / nB, t1 = a.L * (w + 1) / nB;
  const int64_t wb = t0 + (t1 - t0) * wave / 4, we = t0 + (t1 - t0) * (wave + 1) / 4;
  const size_t base = (size_t)bh * a.Lcap;
  for (int64_t t = wb; t < we; t += 32) {
    u32x4 kr[8], vr[8];
    float wt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t tt = t + 4 * i + grp;
      if (tt < we) {
        const size_t row = (base + tt) * kHeadDim + c * 8;
        kr[i] = ld16_stream(a.k + row);
        vr[i] = ld16_stream(a.v + row);
        wt[i] = 1.f;
      } else {
        kr[i] = vr[i] = u32x4{0, 0, 0, 0};
        wt[i] = 0.f;
      }
    }
    float s[8][G];
    row_logits<G, 8>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (wt[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, 8>(st, s, wt, vr, 1.f);
  }
  write_block_partial<G>(st, a.part + ((size_t)bh * nB + w) * G * kPartStride);
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dense_merge(DecodeArgs a) {
  const int bh = blockIdx.x;
  final_merge<G>(a, bh, a.part + (size_t)bh * a.nB * G * kPartStride, a.nB);
}

__global__ __launch_bounds__(256) void k_zero(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

// ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const uint32_t grid = a.total_items < 2048u ? a.total_items : 2048u;
  if (a.dyn_lds > 0) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<G>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)a.dyn_lds);
    if (e != hipSuccess) return e;
  }
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_decode<G>, dim3(grid), dim3(kDecThreads), a.dyn_lds, s, a);
  const hipError_t e = hipGetLastError();
  Tracer::mark(tr, s);
  return e;
}

template <int G>
static hipError_t launch_dense_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_dense_partial<G>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_dense_merge<G>, dim3(BH), dim3(kDecThreads), 0, s, a);
  e = hipGetLastError();
  Tracer::mark(tr, s);
  return e;
}

#define WAVE_DISPATCH_G(FN, A, S, T)          \
  switch ((A).G) {                            \
    case 1: return FN<1>(A, S, T);            \
    case 2: return FN<2>(A, S, T);            \
    case 3: return FN<3>(A, S, T);            \
    case 4: return FN<4>(A, S, T);            \
    case 5: return FN<5>(A, S, T);            \
    case 6: return FN<6>(A, S, T);            \
    case 7: return FN<7>(A, S, T);            \
    case 8: return FN<8>(A, S, T);            \
    default: return hipErrorInvalidValue;     \
  }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  WAVE_DISPATCH_G(launch_decode_g, a, s, tr)
}
hipError_t launch_dense_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  WAVE_DISPATCH_G(launch_dense_g, a, s, tr)
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const size_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace wave
