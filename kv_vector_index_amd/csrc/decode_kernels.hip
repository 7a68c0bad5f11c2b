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
// MI355X layout of the work (one call = three kernels on one stream):
//   1. stream:    for each (b, kv-head), workgroups stream every centroid row and value-sum
//                 row once (HBM-bound), score them for the G query heads of the group, store
//                 the group-mean score, and accumulate a partial softmax (m, l, o) of the
//                 estimate over ALL non-empty clusters. Extra workgroups attend the steady
//                 zone exactly.
//   2. select:    one 1024-thread workgroup per (b, kv-head) merges those partials, picks the
//                 retrieved clusters exactly (radix-style range refinement over the ordered
//                 bit patterns of the scores; ties to the lower id) and lists their tokens.
//   3. retrieved: workgroups attend the retrieved tokens exactly and subtract the estimate
//                 terms of the retrieved clusters (added in step 1), then the last workgroup
//                 of each (b, kv-head) merges everything by log-sum-exp.
// Streaming the value sums of all clusters in step 1 (instead of only the unretrieved ones
// after selection) takes the selection off the critical path between the two big reads.
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

// Merge two partial states (m in log2 units).
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
__device__ void write_block_partial(Online<G>& st, float* __restrict__ dst) {
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
    dst[h * kPartStride + d] = o;
    if (d == 0) {
      dst[h * kPartStride + 128] = M;
      dst[h * kPartStride + 129] = l;
    }
  }
}

template <int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int g, int c, u32x4 (&q)[G]) {
#pragma unroll
  for (int h = 0; h < G; ++h)
    q[h] = ld16(a.q + ((size_t)(b * a.Hq + g * G + h) * kHeadDim + c * 8));
}

// log2-domain logits of 4 rows for the G heads (all 16 lanes of a row group get them)
template <int G>
__device__ __forceinline__ void row_logits(const u32x4 (&q)[G], const u32x4 (&k)[4],
                                           float scale, float (&s)[4][G]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < G; ++h) s[i][h] = sum16(dot8(q[h], k[i])) * scale;
}

// Steady zone: position t of [0, n_steady) -> cache row
__device__ __forceinline__ int64_t steady_row(const DecodeArgs& a, int64_t t) {
  return t < a.n_sink ? t : a.L0 - a.n_recent + (t - a.n_sink);
}

// ------------------------------------------------------------------------------------
// 1. stream: estimate over all clusters + group scores, and the steady zone
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_decode_stream(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, c = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, c, q);
  Online<G> st;
  st.init();
  const float sl2 = a.scale_log2;
  if ((int)blockIdx.x < a.nEst) {
    const size_t base = (size_t)bh * a.C;
    const int wbeg = blockIdx.x * kEstChunk + wave * (kEstChunk / 4);
    const int wend = min(a.C, wbeg + kEstChunk / 4);
    for (int t = wbeg; t < wend; t += 16) {
      u32x4 kr[4], vr[4];
      float w[4];
      int jr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = t + 4 * i + grp;
        jr[i] = j;
        if (j < wend) {
          const size_t row = (base + j) * kHeadDim + c * 8;
          kr[i] = ld16_stream(a.cmean + row);
          vr[i] = ld16_stream(a.vsum + row);
          w[i] = (float)a.csize[base + j];
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          w[i] = 0.f;
        }
      }
      float s[4][G];
      row_logits<G>(q, kr, 1.f, s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mean = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) mean += s[i][h] * a.scale;
        mean = mean / (float)G;
        if (c == 0 && jr[i] < wend) a.shat[base + jr[i]] = (w[i] > 0.f) ? mean : kNegInf;
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = (w[i] > 0.f) ? s[i][h] * sl2 : kNegInf;
      }
      fold_rows<G, 4>(st, s, w, vr, 1.f);
    }
  } else {
    const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
    const int64_t wbeg = (int64_t)(blockIdx.x - a.nEst) * kTokChunk + wave * (kTokChunk / 4);
    const int64_t wend = min(n_steady, wbeg + kTokChunk / 4);
    const size_t base = (size_t)bh * a.Lcap;
    for (int64_t t = wbeg; t < wend; t += 16) {
      u32x4 kr[4], vr[4];
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tt = t + 4 * i + grp;
        if (tt < wend) {
          const size_t row = (base + steady_row(a, tt)) * kHeadDim + c * 8;
          kr[i] = ld16_stream(a.k + row);
          vr[i] = ld16_stream(a.v + row);
          w[i] = 1.f;
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          w[i] = 0.f;
        }
      }
      float s[4][G];
      row_logits<G>(q, kr, sl2, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (w[i] == 0.f)
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
      fold_rows<G, 4>(st, s, w, vr, 1.f);
    }
  }
  write_block_partial<G>(st, a.partA + ((size_t)bh * a.nA + blockIdx.x) * G * kPartStride);
}

// ------------------------------------------------------------------------------------
// 2. select: merge stream partials, exact top-n_r clusters, token list
// ------------------------------------------------------------------------------------

// order-preserving map of a float to uint32 (larger float -> larger key); 0 is reserved
// for empty clusters (score -inf)
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == kNegInf) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inclusive scan over the 1024 threads of the block (wave scan + scan of wave totals)
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t x, uint32_t* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kSelThreads / 64 ? s_tmp[lane] : 0u;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < kSelThreads / 64) s_tmp[lane] = t;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? s_tmp[wave - 1] : 0u;
  __syncthreads();
  return x + before;
}

template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T x, T* s_tmp, Op op) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = op(x, __shfl_xor(x, off));
  if (lane == 0) s_tmp[wave] = x;
  __syncthreads();
  T r = s_tmp[0];
  for (int w = 1; w < kSelThreads / 64; ++w) r = op(r, s_tmp[w]);
  __syncthreads();
  return r;
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void k_decode_select(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ uint32_t s_keys[kSelStageMax];
  __shared__ uint32_t s_hist[1024];
  __shared__ uint32_t s_tmp[32];
  __shared__ uint32_t s_b[4];

  if (tid == 0) a.counter[bh] = 0u;

  // ---- merge the stream partials of this (b, kv-head)
  {
    const float* P = a.partA + (size_t)bh * a.nA * G * kPartStride;
    float* D = a.mergedA + (size_t)bh * G * kPartStride;
    for (int idx = tid; idx < G * 128; idx += kSelThreads) {
      const int h = idx >> 7, d = idx & 127;
      float M = kNegInf;
      for (int p = 0; p < a.nA; ++p) M = fmaxf(M, P[(p * G + h) * kPartStride + 128]);
      float o = 0.f, l = 0.f;
      if (M != kNegInf) {
        for (int p = 0; p < a.nA; ++p) {
          const float* pp = P + (p * G + h) * kPartStride;
          const float s = fast_exp2(pp[128] - M);
          o += s * pp[d];
          l += s * pp[129];
        }
      }
      D[h * kPartStride + d] = o;
      if (d == 0) {
        D[h * kPartStride + 128] = M;
        D[h * kPartStride + 129] = l;
      }
    }
  }

  // ---- keys, count of non-empty clusters, key range
  const int C = a.C;
  const float* shat = a.shat + (size_t)bh * C;
  const bool staged = C <= kSelStageMax;
  uint32_t ne = 0, kmin = 0xffffffffu, kmax = 0u;
  for (int j = tid; j < C; j += kSelThreads) {
    const uint32_t key = order_key(shat[j]);
    if (staged) s_keys[j] = key;
    if (key) {
      ++ne;
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  }
  ne = block_reduce<uint32_t>(ne, s_tmp, [](uint32_t x, uint32_t y) { return x + y; });
  kmin = block_reduce<uint32_t>(kmin, s_tmp, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = block_reduce<uint32_t>(kmax, s_tmp, [](uint32_t x, uint32_t y) { return max(x, y); });
  auto key_at = [&](int j) -> uint32_t { return staged ? s_keys[j] : order_key(shat[j]); };

  // Selection = {key > T} plus the keq lowest ids with key == T.
  uint32_t T, keq;
  const uint32_t nr = min((uint32_t)a.n_retrieve, ne);
  if (nr == ne) {
    T = 0u;            // every non-empty cluster (keys > 0)
    keq = 0u;
  } else if (nr == 0) {
    T = 0xffffffffu;   // nothing
    keq = 0u;
  } else {
    // the nr-th largest key by range refinement: 1024 equal-width bins per pass
    uint32_t lo = kmin, hi = kmax, need = nr;
    for (;;) {
      if (lo == hi) break;
      const uint64_t span = (uint64_t)hi - lo + 1;
      const uint64_t width = (span + 1023) / 1024;
      s_hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < C; j += kSelThreads) {
        const uint32_t key = key_at(j);
        if (key >= lo && key <= hi) atomicAdd(&s_hist[(uint32_t)((key - lo) / width)], 1u);
      }
      __syncthreads();
      // bins from the top: thread t owns bin 1023 - t
      const uint32_t cnt = s_hist[1023 - tid];
      const uint32_t incl = block_scan_incl(cnt, s_tmp);
      if (incl >= need && incl - cnt < need) {
        s_b[0] = 1023 - tid;
        s_b[1] = incl - cnt;
      }
      __syncthreads();
      const uint32_t bstar = s_b[0], above = s_b[1];
      __syncthreads();
      need -= above;
      const uint64_t nlo = (uint64_t)lo + (uint64_t)bstar * width;
      const uint64_t nhi = min((uint64_t)hi, nlo + width - 1);
      lo = (uint32_t)nlo;
      hi = (uint32_t)nhi;
      if (width == 1) break;
    }
    T = lo;
    keq = need;
  }

  // ---- ordered compaction: thread t owns ids [t*per, (t+1)*per)
  const int per = (C + kSelThreads - 1) / kSelThreads;
  const int j0 = min(C, tid * per), j1 = min(C, j0 + per);
  uint32_t n_eq = 0;
  for (int j = j0; j < j1; ++j) n_eq += (key_at(j) == T && T != 0u) ? 1u : 0u;
  const uint32_t eq_before = block_scan_incl(n_eq, s_tmp) - n_eq;
  const int32_t* csize = a.csize + (size_t)bh * C;
  const int32_t* coff = a.coff + (size_t)bh * C;
  uint32_t n_sel = 0, n_tok = 0;
  {
    uint32_t e = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = key_at(j);
      bool take = key > T;
      if (key == T && T != 0u) {
        take = e < keq;
        ++e;
      }
      if (take) {
        ++n_sel;
        n_tok += (uint32_t)csize[j];
      }
    }
  }
  const uint32_t sel_incl = block_scan_incl(n_sel, s_tmp);
  const uint32_t tok_incl = block_scan_incl(n_tok, s_tmp);
  {
    uint32_t e = eq_before, ps = sel_incl - n_sel, pt = tok_incl - n_tok;
    int32_t* sel = a.sel + (size_t)bh * a.rcap;
    int32_t* slots = a.slots + (size_t)bh * a.L0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = key_at(j);
      bool take = key > T;
      if (key == T && T != 0u) {
        take = e < keq;
        ++e;
      }
      if (take) {
        if (ps < (uint32_t)a.rcap) sel[ps] = j;
        if (a.selected && ps < (uint32_t)a.n_retrieve)
          a.selected[(size_t)bh * a.n_retrieve + ps] = j;
        ++ps;
        const int n = csize[j], o = coff[j];
        for (int r = 0; r < n && pt + r < (uint32_t)a.L0; ++r) slots[pt + r] = o + r;
        pt += (uint32_t)n;
      }
    }
  }
  if (tid == kSelThreads - 1) {
    a.nsel[bh] = (int32_t)min(sel_incl, (uint32_t)a.rcap);
    a.ntok[bh] = (int32_t)min(tok_incl, (uint32_t)a.L0);
  }
  if (a.selected)
    for (int r = (int)nr + tid; r < a.n_retrieve; r += kSelThreads)
      a.selected[(size_t)bh * a.n_retrieve + r] = -1;
}

// ------------------------------------------------------------------------------------
// 3. retrieved: exact retrieved tokens, removal of their clusters' estimate, final merge
// ------------------------------------------------------------------------------------

// Merge a base partial (may be null) and n partials into out / lse of the G heads.
template <int G>
__device__ void final_merge(const DecodeArgs& a, int bh, const float* base, const float* parts,
                            int n) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  for (int idx = threadIdx.x; idx < G * 128; idx += kDecThreads) {
    const int h = idx >> 7, d = idx & 127;
    float M = base ? base[h * kPartStride + 128] : kNegInf;
    for (int p = 0; p < n; ++p) M = fmaxf(M, parts[(p * G + h) * kPartStride + 128]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
      if (base) {
        const float s = fast_exp2(base[h * kPartStride + 128] - M);
        o = s * base[h * kPartStride + d];
        l = s * base[h * kPartStride + 129];
      }
      for (int p = 0; p < n; ++p) {
        const float* pp = parts + (p * G + h) * kPartStride;
        const float s = fast_exp2(pp[128] - M);
        o += s * pp[d];
        l += s * pp[129];
      }
    }
    const size_t qh = (size_t)b * a.Hq + g * G + h;
    a.out[qh * kHeadDim + d] = o / l;
    if (d == 0 && a.lse) a.lse[qh] = (M + __log2f(l)) * kLn2;
  }
}

template <int G>
__device__ __forceinline__ bool last_block(uint32_t* counter, int n) {
  __shared__ uint32_t s_last;
  __threadfence();  // this thread's partial-result stores, device-wide
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    s_last = (prev == (uint32_t)(n - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last) __threadfence();
  return s_last != 0u;
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void k_decode_retrieved(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, c = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, c, q);
  Online<G> st;
  st.init();
  const float sl2 = a.scale_log2;
  const int nB = a.nB, w = blockIdx.x;
  // exact attention over this workgroup's share of the retrieved tokens
  {
    const int64_t ntok = a.ntok[bh];
    const int64_t t0 = ntok * w / nB, t1 = ntok * (w + 1) / nB;
    const int64_t wb = t0 + (t1 - t0) * wave / 4, we = t0 + (t1 - t0) * (wave + 1) / 4;
    const int32_t* slots = a.slots + (size_t)bh * a.L0;
    const size_t base = (size_t)bh * a.Lcap;
    for (int64_t t = wb; t < we; t += 16) {
      u32x4 kr[4], vr[4];
      float wt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tt = t + 4 * i + grp;
        if (tt < we) {
          const size_t row = (base + slots[tt]) * kHeadDim + c * 8;
          kr[i] = ld16_stream(a.k + row);
          vr[i] = ld16_stream(a.v + row);
          wt[i] = 1.f;
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          wt[i] = 0.f;
        }
      }
      float s[4][G];
      row_logits<G>(q, kr, sl2, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (wt[i] == 0.f)
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
      fold_rows<G, 4>(st, s, wt, vr, 1.f);
    }
  }
  // remove the estimate terms that the stream kernel added for the retrieved clusters
  {
    const int ns = a.nsel[bh];
    const int k0 = (int)((int64_t)ns * w / nB), k1 = (int)((int64_t)ns * (w + 1) / nB);
    const int wb = k0 + (k1 - k0) * wave / 4, we = k0 + (k1 - k0) * (wave + 1) / 4;
    const int32_t* sel = a.sel + (size_t)bh * a.rcap;
    const size_t base = (size_t)bh * a.C;
    for (int t = wb; t < we; t += 16) {
      u32x4 kr[4], vr[4];
      float wt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t + 4 * i + grp;
        if (tt < we) {
          const int j = sel[tt];
          const size_t row = (base + j) * kHeadDim + c * 8;
          kr[i] = ld16(a.cmean + row);
          vr[i] = ld16(a.vsum + row);
          wt[i] = -(float)a.csize[base + j];
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          wt[i] = 0.f;
        }
      }
      // same arithmetic as the stream kernel: logits at scale 1, then * scale * log2(e)
      float s[4][G];
      row_logits<G>(q, kr, 1.f, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = (wt[i] != 0.f) ? s[i][h] * sl2 : kNegInf;
      fold_rows<G, 4>(st, s, wt, vr, -1.f);
    }
  }
  float* part = a.partB + ((size_t)bh * nB + w) * G * kPartStride;
  write_block_partial<G>(st, part);
  if (last_block<G>(a.counter + bh, nB)) {
    final_merge<G>(a, bh, a.mergedA + (size_t)bh * G * kPartStride,
                   a.partB + (size_t)bh * nB * G * kPartStride, nB);
    if (threadIdx.x == 0) a.counter[bh] = 0u;
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
  for (int64_t t = wb; t < we; t += 16) {
    u32x4 kr[4], vr[4];
    float wt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    float s[4][G];
    row_logits<G>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (wt[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, 4>(st, s, wt, vr, 1.f);
  }
  write_block_partial<G>(st, a.partB + ((size_t)bh * nB + w) * G * kPartStride);
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dense_merge(DecodeArgs a) {
  const int bh = blockIdx.x;
  final_merge<G>(a, bh, nullptr, a.partB + (size_t)bh * a.nB * G * kPartStride, a.nB);
}

// ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_decode_stream<G>, dim3(a.nA, BH), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_decode_select<G>, dim3(BH), dim3(kSelThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  Tracer::mark(tr, s);
  hipLaunchKernelGGL(k_decode_retrieved<G>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
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
