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
// MI355X design, two compact kernels per call (a third, the published select, only for
// indexes with more than kLocalSelMax clusters per head):
//   stream    one workgroup per 128 clusters or 128 steady tokens of a (b, kv-head): stream
//             the centroid rows, value-sum rows and sizes once (HBM-bound), store each query
//             head's logit and the group-mean score, and fold the estimate of ALL non-empty
//             clusters (or the exact steady tokens) into one partial softmax state.
//   retrieve  nB workgroups per (b, kv-head). Each recomputes the same exact top-n_r
//             selection from the group scores staged in LDS (histogram of their ordered bit
//             patterns, then refinement; ties to the lower id), attends its share of the
//             retrieved tokens exactly (a retrieved cluster is a contiguous run of cache rows
//             in the index layout) and removes the estimate terms the stream kernel added for
//             the retrieved clusters. The last workgroup of a (b, kv-head) merges all partials
//             by log-sum-exp into out / lse.
// Streaming every value sum in the first kernel (rather than only the unretrieved ones after
// the selection) keeps the selection off the critical path of the big reads. Rows are read
// 16 lanes per 256-byte row (4 rows per wave instruction, fully coalesced) and each K/V row
// is shared by the G query heads of its group. Both kernels stay small: the instruction
// cache is shared by neighbouring CUs, and large fused kernels run far slower.
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


// Exact attention over the rows row_of(t), t in [wb, we) (cache rows), 8 rows per row group
// in flight.
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

// Remove the estimate terms of the clusters id_of(k), k in [wb, we): the same stored logits,
// weight -n_j and value -V_j (the stream kernel added them).
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
        for (int h = 0; h < G; ++h) s[i][h] = a.scores[(base + jr[i]) * G + h];
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

// ------------------------------------------------------------------------------------
// kernel 1: stream (scores + estimate of every cluster, and the steady zone)
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dec_stream(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, cc = lane & 15;
  if (blockIdx.x == 0 && blockIdx.y == 0)  // arrival counters of the retrieve kernel
    for (int i = tid; i < a.B * a.Hkv; i += kDecThreads) a.counter[i] = 0u;
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  Online<G> st;
  st.init();
  if ((int)blockIdx.x < a.nS) {
    const size_t base = (size_t)bh * a.C;
    const int wbeg = blockIdx.x * kChunk + wave * (kChunk / 4);
    const int wend = min(a.C, wbeg + kChunk / 4);
    const float sl2 = a.scale_log2;
    for (int t = wbeg; t < wend; t += 32) {
      u32x4 kr[8], vr[8];
      int32_t n[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = t + 4 * i + grp;
        if (j < wend) {
          const size_t row = (base + j) * kHeadDim + cc * 8;
          kr[i] = ld16_stream(a.cmean + row);
          vr[i] = ld16_stream(a.vsum + row);
          n[i] = a.csize[base + j];
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          n[i] = -1;
        }
      }
      float s[8][G], w[8];
      row_logits<G, 8>(q, kr, 1.f, s);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = t + 4 * i + grp;
        if (n[i] >= 0) {
          float mean = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) mean += s[i][h] * a.scale;
          mean = mean / (float)G;
          if (cc == 0) a.shat[base + j] = n[i] > 0 ? mean : kNegInf;
          if (cc < G) {
            float mine = s[i][0];
#pragma unroll
            for (int h = 1; h < G; ++h) mine = (cc == h) ? s[i][h] : mine;
            a.scores[(base + j) * G + cc] = mine * sl2;
          }
        }
        w[i] = n[i] > 0 ? (float)n[i] : 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = n[i] > 0 ? s[i][h] * sl2 : kNegInf;
      }
      fold_rows<G, 8>(st, s, w, vr, 1.f);
    }
  } else {
    const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
    const int64_t wbeg = (int64_t)(blockIdx.x - a.nS) * kTokChunk + wave * (kTokChunk / 4);
    const int64_t wend = min(n_steady, wbeg + kTokChunk / 4);
    attend_rows<G>(a, bh, q, st, wbeg, wend, [&](int64_t t) { return steady_row(a, t); });
  }
  write_block_partial<G>(st, a.part + ((size_t)bh * a.nP + blockIdx.x) * G * kPartStride);
}

// ------------------------------------------------------------------------------------
// selection helpers (one workgroup)
// ------------------------------------------------------------------------------------

// From an LDS histogram of the top 12 key bits: the number of non-empty clusters ne, the
// size nr of the selection, and (if 0 < nr < ne) the bin holding its smallest key and how
// many keys of that bin belong to the selection.
__device__ __forceinline__ void hist_cut(const uint32_t* s_hist, uint32_t n_req, ScanTmp& tmp,
                                         uint32_t* s_b, uint32_t& ne, uint32_t& nr,
                                         uint32_t& bstar, uint32_t& need) {
  const int tid = threadIdx.x;
  const int hb0 = kHistBins - 16 * (tid + 1);  // this thread's bins, visited descending
  uint32_t h[16], loc = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    h[i] = s_hist[hb0 + i];
    loc += h[i];
  }
  const uint32_t above_me = scan_excl(loc, tmp, &ne);
  nr = min(n_req, ne);
  bstar = 0u;
  need = 0u;
  if (nr == 0u || nr == ne) return;
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
  bstar = s_b[0];
  need = nr - s_b[1];
  __syncthreads();
}

// Narrow [lo, hi] to the need-th largest key (256 equal-width bins per round over the keys
// key_at(k), k in [0, n), that fall inside). On return lo == hi == that key and need = how
// many keys equal to it belong to the selection.
template <typename KeyAt>
__device__ __forceinline__ void refine(KeyAt key_at, int n, uint32_t& lo, uint32_t& hi,
                                       uint32_t& need, ScanTmp& tmp, uint32_t* s_h,
                                       uint32_t* s_b) {
  const int tid = threadIdx.x;
  for (;;) {
    if (lo == hi) return;
    const uint32_t width = (uint32_t)(((uint64_t)hi - lo + 1 + 255) / 256);
    s_h[tid] = 0u;
    __syncthreads();
    for (int k0 = tid; k0 < n; k0 += 8 * kDecThreads) {
      uint32_t kk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + e * kDecThreads;
        kk[e] = k < n ? key_at(k) : 0u;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kk[e] != 0u && kk[e] >= lo && kk[e] <= hi) atomicAdd(&s_h[(kk[e] - lo) / width], 1u);
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
    if (width == 1) return;
  }
}

// Visit this thread's ids (thread t owns ids t*per + i, i < per, stored in LDS at
// i * 256 + t) in ascending order, with whether each belongs to the selection
// {key > T} + {the keq lowest ids with key == T} (e counts the keys == T seen so far).
template <typename F>
__device__ __forceinline__ void walk_ids(const uint32_t* s_key, int per, uint32_t T,
                                         uint32_t keq, uint32_t e, F f) {
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < per; i0 += 8) {
    uint32_t kk[8];
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) kk[e2] = (i0 + e2 < per) ? s_key[(i0 + e2) * kDecThreads + tid] : 0u;
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) {
      if (i0 + e2 >= per) break;
      bool take = kk[e2] > T;
      if (T != 0u && kk[e2] == T) {
        take = e < keq;
        ++e;
      }
      f(i0 + e2, take);
    }
  }
}

// ------------------------------------------------------------------------------------
// kernel 2: retrieve (selection, exact retrieved tokens, estimate removal, final merge)
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dec_retrieve(DecodeArgs a) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ ScanTmp tmp;
  __shared__ uint32_t s_h[256];
  __shared__ uint32_t s_b[2];
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv, w_item = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cc = lane & 15;
  const int C = a.C, nB = a.nB;
  const size_t cb = (size_t)bh * C;
  const int per = (C + kDecThreads - 1) / kDecThreads;
  const int nkeys = a.local_select ? per * kDecThreads : 0;
  uint32_t* s_key = s_dyn;                                       // [per][256]
  uint16_t* s_sz = reinterpret_cast<uint16_t*>(s_dyn + nkeys);   // [per][256]
  uint32_t* wp = s_dyn + nkeys + (nkeys + 1) / 2;                // window: token starts
  uint32_t* wn = wp + kWin;                                      //         sizes
  int32_t* wo = reinterpret_cast<int32_t*>(wn + kWin);           //         ids / cache rows
  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);

  uint32_t nsel, ntok, T = 0u, keq = 0u, eq0 = 0u, r0 = 0u, p0 = 0u;
  if (a.local_select) {
    // ---- group scores and sizes into LDS (one round trip), histogram of the keys
    for (int i = tid; i < kHistBins; i += kDecThreads) s_hist[i] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < per; i0 += 16) {
      float v[16];
      int32_t z[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = tid * per + i0 + e;
        const bool ok = (i0 + e < per) && j < C;
        v[e] = ok ? a.shat[cb + j] : kNegInf;
        z[e] = ok ? a.csize[cb + j] : 0;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (i0 + e < per) {
          const uint32_t key = order_key(v[e]);
          s_key[(i0 + e) * kDecThreads + tid] = key;
          s_sz[(i0 + e) * kDecThreads + tid] = (uint16_t)z[e];
          if (key) atomicAdd(&s_hist[key >> kHistShift], 1u);
        }
    }
    __syncthreads();
    uint32_t ne, nr, bstar, need;
    hist_cut(s_hist, (uint32_t)a.n_retrieve, tmp, s_b, ne, nr, bstar, need);
    if (nr == ne) {
      T = 0u;            // every non-empty cluster (keys > 0)
    } else if (nr == 0) {
      T = 0xffffffffu;   // nothing
    } else {
      uint32_t lo = bstar << kHistShift, hi = lo | ((1u << kHistShift) - 1u);
      refine([&](int k) { return s_key[k]; }, nkeys, lo, hi, need, tmp, s_h, s_b);
      T = lo;
      keq = need;
    }
    // ---- ranks and token offsets of this thread's retrieved ids
    uint32_t n_eq = 0, tot;
    for (int i = 0; i < per; ++i) n_eq += (T != 0u && s_key[i * kDecThreads + tid] == T);
    eq0 = scan_excl(n_eq, tmp, &tot);
    uint32_t my_sel = 0, my_tok = 0;
    walk_ids(s_key, per, T, keq, eq0, [&](int i, bool take) {
      if (take) {
        ++my_sel;
        my_tok += s_sz[i * kDecThreads + tid];
      }
    });
    r0 = scan_excl(my_sel, tmp, &nsel);
    p0 = scan_excl(my_tok, tmp, &ntok);
    if (w_item == 0 && a.selected) {
      uint32_t r = r0;
      walk_ids(s_key, per, T, keq, eq0, [&](int i, bool take) {
        if (take) {
          if (r < (uint32_t)a.n_retrieve) a.selected[(size_t)bh * a.n_retrieve + r] = tid * per + i;
          ++r;
        }
      });
      for (int r2 = (int)nsel + tid; r2 < a.n_retrieve; r2 += kDecThreads)
        a.selected[(size_t)bh * a.n_retrieve + r2] = -1;
    }
  } else {
    nsel = (uint32_t)a.sel_n[bh];
    ntok = (uint32_t)a.sel_tok[(size_t)bh * (a.rcap + 1) + nsel];
  }

  Online<G> st;
  st.init();
  const int32_t* stok = a.sel_tok + (size_t)bh * (a.rcap + 1);
  const int32_t* sid = a.sel_id + (size_t)bh * a.rcap;
  // tokens [T0, T1) of the selection belong to this workgroup; clusters [R0, R1) overlap them
  const uint32_t T0 = (uint32_t)((uint64_t)ntok * w_item / nB);
  const uint32_t T1 = (uint32_t)((uint64_t)ntok * (w_item + 1) / nB);
  uint32_t R0, R1;
  if (a.local_select) {
    uint32_t c_before = 0, c_upto = 0, p = p0;
    walk_ids(s_key, per, T, keq, eq0, [&](int i, bool take) {
      if (take) {
        const uint32_t n = s_sz[i * kDecThreads + tid];
        c_before += (p + n <= T0);
        c_upto += (p < T1);
        p += n;
      }
    });
    scan_excl(c_before, tmp, &R0);
    scan_excl(c_upto, tmp, &R1);
  } else {
    // first cluster ending after T0, first cluster starting at or after T1 (binary search)
    uint32_t lo = 0, hi = nsel;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if ((uint32_t)stok[mid + 1] <= T0) lo = mid + 1; else hi = mid;
    }
    R0 = lo;
    hi = nsel;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if ((uint32_t)stok[mid] < T1) lo = mid + 1; else hi = mid;
    }
    R1 = lo;
  }
  for (uint32_t Rw = R0; Rw < R1; Rw += kWin) {
    const uint32_t cnt = min((uint32_t)kWin, R1 - Rw);
    if (a.local_select) {
      uint32_t r = r0, p = p0;
      walk_ids(s_key, per, T, keq, eq0, [&](int i, bool take) {
        if (take) {
          const uint32_t n = s_sz[i * kDecThreads + tid];
          if (r >= Rw && r < Rw + cnt) {
            wp[r - Rw] = p;
            wn[r - Rw] = n;
            wo[r - Rw] = tid * per + i;
          }
          ++r;
          p += n;
        }
      });
    } else {
      for (uint32_t i = tid; i < cnt; i += kDecThreads) {
        wp[i] = (uint32_t)stok[Rw + i];
        wn[i] = (uint32_t)(stok[Rw + i + 1] - stok[Rw + i]);
        wo[i] = sid[Rw + i];
      }
    }
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
  // the estimate terms of the retrieved clusters [K0, K1) (by rank) are removed here
  const uint32_t K0 = (uint32_t)((uint64_t)nsel * w_item / nB);
  const uint32_t K1 = (uint32_t)((uint64_t)nsel * (w_item + 1) / nB);
  for (uint32_t Kw = K0; Kw < K1; Kw += kWin) {
    const uint32_t cnt = min((uint32_t)kWin, K1 - Kw);
    if (a.local_select) {
      uint32_t r = r0;
      walk_ids(s_key, per, T, keq, eq0, [&](int i, bool take) {
        if (take) {
          if (r >= Kw && r < Kw + cnt) wo[r - Kw] = tid * per + i;
          ++r;
        }
      });
    } else {
      for (uint32_t i = tid; i < cnt; i += kDecThreads) wo[i] = sid[Kw + i];
    }
    __syncthreads();
    remove_estimates<G>(a, bh, st, (int)(cnt * wave / 4), (int)(cnt * (wave + 1) / 4),
                        [&](int k) { return wo[k]; });
    __syncthreads();
  }
  float* parts = a.part + (size_t)bh * a.nP * G * kPartStride;
  write_block_partial<G>(st, parts + (size_t)(a.nS + a.nSt + w_item) * G * kPartStride);
  if (arrive_last(a.counter + bh, (uint32_t)nB)) final_merge<G>(a, bh, parts, a.nP);
}

// ------------------------------------------------------------------------------------
// published select (more than kLocalSelMax clusters per head): one workgroup per
// (b, kv-head) selects and lists the retrieved ids and their token offsets. LDS holds the
// top 16 bits of every key; full keys are re-read only around the cut.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kDecThreads) void k_dec_select(DecodeArgs a) {
  extern __shared__ uint32_t s_dyn[];
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ ScanTmp tmp;
  __shared__ uint32_t s_h[256];
  __shared__ uint32_t s_b[2];
  const int bh = blockIdx.x, tid = threadIdx.x, C = a.C;
  const size_t cb = (size_t)bh * C;
  const float* shat = a.shat + cb;
  const int per = (C + kDecThreads - 1) / kDecThreads;
  uint16_t* s_top = reinterpret_cast<uint16_t*>(s_dyn);          // [per][256] key >> 16
  uint32_t* s_cand = s_dyn + (per * kDecThreads + 1) / 2;        // [kCandLds]
  for (int i = tid; i < kHistBins; i += kDecThreads) s_hist[i] = 0u;
  __syncthreads();
  for (int i0 = 0; i0 < per; i0 += 16) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = tid * per + i0 + e;
      v[e] = ((i0 + e < per) && j < C) ? shat[j] : kNegInf;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (i0 + e < per) {
        const uint32_t key = order_key(v[e]);
        s_top[(i0 + e) * kDecThreads + tid] = (uint16_t)(key >> 16);
        if (key) atomicAdd(&s_hist[key >> kHistShift], 1u);
      }
  }
  __syncthreads();
  uint32_t ne, nr, bstar, need;
  hist_cut(s_hist, (uint32_t)a.n_retrieve, tmp, s_b, ne, nr, bstar, need);
  uint32_t T = 0u, keq = 0u;
  if (nr == 0) {
    T = 0xffffffffu;
  } else if (nr < ne) {
    // second level on the 16-bit keys: which of the 16 sub-bins of bstar holds the cut
    s_h[tid] = 0u;
    __syncthreads();
    for (int i = 0; i < per; ++i) {
      const uint32_t t16 = s_top[i * kDecThreads + tid];
      if ((t16 >> 4) == bstar) atomicAdd(&s_h[t16 & 15u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t run = 0;
      for (int sb = 15; sb >= 0; --sb) {
        if (run < need && run + s_h[sb] >= need) {
          s_b[0] = (bstar << 4) | (uint32_t)sb;
          s_b[1] = need - run;
        }
        run += s_h[sb];
      }
    }
    __syncthreads();
    const uint32_t b16 = s_b[0];
    need = s_b[1];
    __syncthreads();
    // candidates: full keys of the ids whose top 16 bits equal b16
    uint32_t cnt = 0;
    for (int i = 0; i < per; ++i) cnt += s_top[i * kDecThreads + tid] == b16 && tid * per + i < C;
    uint32_t n_c;
    uint32_t pos = scan_excl(cnt, tmp, &n_c);
    const bool staged = n_c <= (uint32_t)kCandLds;
    if (staged)
      for (int i = 0; i < per; ++i)
        if (s_top[i * kDecThreads + tid] == b16 && tid * per + i < C)
          s_cand[pos++] = order_key(shat[tid * per + i]);
    __syncthreads();
    uint32_t lo = b16 << 16, hi = lo | 0xffffu;
    if (staged) {
      refine([&](int k) { return s_cand[k]; }, (int)n_c, lo, hi, need, tmp, s_h, s_b);
    } else {  // many equal top bits: read the full keys of every id again
      refine([&](int k) {
               const int j = (k % kDecThreads) * per + k / kDecThreads;
               return j < C ? order_key(shat[j]) : 0u;
             },
             per * kDecThreads, lo, hi, need, tmp, s_h, s_b);
    }
    T = lo;
    keq = need;
  }
  // ordered compaction: ranks, token offsets, ids
  auto full_key = [&](int i) -> uint32_t {
    const uint32_t t16 = s_top[i * kDecThreads + tid];
    const int j = tid * per + i;
    if (t16 != (T >> 16) || T == 0u || j >= C) return (uint32_t)t16 << 16;  // enough vs T
    return order_key(shat[j]);
  };
  uint32_t n_eq = 0, tot;
  for (int i = 0; i < per; ++i) n_eq += (T != 0u && full_key(i) == T);
  uint32_t e = scan_excl(n_eq, tmp, &tot);
  uint32_t my_sel = 0, my_tok = 0;
  const uint32_t e0 = e;
  for (int i = 0; i < per; ++i) {
    const int j = tid * per + i;
    if (j >= C) break;
    const uint32_t k = full_key(i);
    bool take = (T == 0u) ? (s_top[i * kDecThreads + tid] != 0u || order_key(shat[j]) != 0u)
                          : k > T;
    if (T != 0u && k == T) {
      take = e < keq;
      ++e;
    }
    if (take) {
      ++my_sel;
      my_tok += (uint32_t)a.csize[cb + j];
    }
  }
  uint32_t nsel, ntok;
  uint32_t r = scan_excl(my_sel, tmp, &nsel);
  uint32_t p = scan_excl(my_tok, tmp, &ntok);
  e = e0;
  int32_t* sid = a.sel_id + (size_t)bh * a.rcap;
  int32_t* stok = a.sel_tok + (size_t)bh * (a.rcap + 1);
  for (int i = 0; i < per; ++i) {
    const int j = tid * per + i;
    if (j >= C) break;
    const uint32_t k = full_key(i);
    bool take = (T == 0u) ? (s_top[i * kDecThreads + tid] != 0u || order_key(shat[j]) != 0u)
                          : k > T;
    if (T != 0u && k == T) {
      take = e < keq;
      ++e;
    }
    if (take) {
      if (r < (uint32_t)a.rcap) {
        sid[r] = j;
        stok[r] = (int32_t)p;
      }
      if (a.selected && r < (uint32_t)a.n_retrieve) a.selected[(size_t)bh * a.n_retrieve + r] = j;
      ++r;
      p += (uint32_t)a.csize[cb + j];
    }
  }
  if (a.selected)
    for (int r2 = (int)nsel + tid; r2 < a.n_retrieve; r2 += kDecThreads)
      a.selected[(size_t)bh * a.n_retrieve + r2] = -1;
  if (tid == 0) {
    const uint32_t ns = min(nsel, (uint32_t)a.rcap);
    a.sel_n[bh] = (int32_t)ns;
    stok[ns] = (int32_t)ntok;
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


// ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_dec_stream<G>, dim3(a.nS + a.nSt, BH), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.local_select) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_select),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds_select);
    if (e != hipSuccess) return e;
    Tracer::mark(tr, s);
    hipLaunchKernelGGL(k_dec_select, dim3(BH), dim3(kDecThreads), a.lds_select, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dec_retrieve<G>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.lds_retrieve);
  if (e != hipSuccess) return e;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_dec_retrieve<G>, dim3(a.nB, BH), dim3(kDecThreads), a.lds_retrieve, s, a);
  e = hipGetLastError();
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

}  // namespace wave
