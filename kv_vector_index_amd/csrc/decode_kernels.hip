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
// MI355X design, two small kernels per call (plus a one-workgroup-per-head select kernel
// when an index has more than kLocalSelMax clusters per head or the budget exceeds kSelMax):
//   stream    one workgroup per 128 clusters or 128 steady tokens of a (b, kv-head): stream
//             the centroid rows, value-sum rows and sizes once (HBM-bound), store each query
//             head's logit and the group-mean score, and fold the estimate of ALL non-empty
//             clusters (or the exact steady tokens) into one partial softmax state.
//   retrieve  nB workgroups per (b, kv-head). Each recomputes the same exact top-n_r
//             selection from the group scores held in registers (a histogram over the
//             scores' value range, then an exact rank of the few keys in the bin of the cut;
//             ties to the lower id), lists the retrieved clusters in LDS, and walks its share
//             of their "virtual rows": every token of a retrieved cluster (exact attention;
//             a retrieved cluster is a contiguous run of cache rows in the index layout) and
//             one row per cluster that removes the estimate term the stream kernel added.
//             Each workgroup also folds a share of the stream partials; the last workgroup
//             of a (b, kv-head) merges the retrieve partials by log-sum-exp into out / lse.
// Rows are read 16 lanes per 256-byte row (4 rows per wave instruction, fully coalesced) and
// each K/V row is shared by the G query heads of its group.
#include <float.h>

#include "wave_common.h"
#include "wave_kernels.h"

namespace wave {

constexpr float kPosInf = __builtin_huge_valf();

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

// rows in flight per row group and loop step: fewer for large groups (register budget)
template <int G>
struct Rows {
  static constexpr int R = G <= 4 ? 8 : 4;
};

__device__ __forceinline__ float vdim(const u32x4& v, int d) {
  const uint32_t w = v[d >> 1];
  return (d & 1) ? bf_hi(w) : bf_lo(w);
}

// Fold R rows into the state. s2: log2-domain logits (-inf = skip row), w: denominator
// weight of the row (1 for a token, n_j for a cluster estimate, -n_j to remove one),
// sg: +1 / -1 multiplier of the value row.
template <int G, int R>
__device__ __forceinline__ void fold_rows(Online<G>& st, const float (&s2)[R][G],
                                          const float (&w)[R], const u32x4 (&v)[R],
                                          const float (&sg)[R]) {
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
      p[i] *= sg[i];
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

// Combine the waves of the workgroup (and, if xp is not null, one more partial
// [G][kPartStride] held in LDS) and write one partial [G][kPartStride] to dst.
template <int G>
__device__ __forceinline__ void write_block_partial(Online<G>& st, const float* xp,
                                                    float* __restrict__ dst) {
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
    const float* x = xp ? xp + h * kPartStride : nullptr;
    float M = x ? x[128] : kNegInf;
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
      if (x) {
        const float s = fast_exp2(x[128] - M);
        o += s * x[d];
        l += s * x[129];
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

// Log-sum-exp merge of the partials p0, p0 + step, ... (< n) of parts, for the head/dim
// element idx = h * 128 + d; 8 partials in flight per round. DEV: device-coherent loads
// (partials written by other workgroups of the same kernel).
template <bool DEV>
__device__ __forceinline__ void merge_partials(const float* parts, int G, int idx, int p0,
                                               int step, int n, float& M, float& Ls, float& O) {
  const int h = idx >> 7, d = idx & 127;
  M = kNegInf;
  Ls = 0.f;
  O = 0.f;
  for (int p = p0; p < n; p += 8 * step) {
    float pm[8], pl[8], po[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pk = p + k * step;
      const float* pp = parts + ((size_t)pk * G + h) * kPartStride;
      if (pk < n) {
        pm[k] = DEV ? ld_dev(pp + 128) : pp[128];
        pl[k] = DEV ? ld_dev(pp + 129) : pp[129];
        po[k] = DEV ? ld_dev(pp + d) : pp[d];
      } else {
        pm[k] = kNegInf;
        pl[k] = po[k] = 0.f;
      }
    }
    float mx = M;
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, pm[k]);
    if (mx == kNegInf) continue;
    const float sc = fast_exp2(M - mx);
    O *= sc;
    Ls *= sc;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float f = fast_exp2(pm[k] - mx);
      O += f * po[k];
      Ls += f * pl[k];
    }
    M = mx;
  }
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

// Exact attention over the cache rows row_of(t), t in [wb, we).
template <int G, typename RowOf>
__device__ __forceinline__ void attend_rows(const DecodeArgs& a, int bh, const u32x4 (&q)[G],
                                            Online<G>& st, int64_t wb, int64_t we, RowOf row_of) {
  constexpr int R = Rows<G>::R;
  const int lane = threadIdx.x & 63, grp = lane >> 4, cc = lane & 15;
  const size_t base = (size_t)bh * a.Lcap;
  for (int64_t t = wb; t < we; t += 4 * R) {
    u32x4 kr[R], vr[R];
    float wt[R], sg[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t tt = t + 4 * i + grp;
      sg[i] = 1.f;
      if (tt < we) {
        const size_t row = (base + row_of(tt)) * kHeadDim + cc * 8;
        kr[i] = ld16_stream(a.k + row);
        vr[i] = ld16_stream(a.v + row);
        wt[i] = 1.f;
      } else {
        kr[i] = vr[i] = u32x4{0, 0, 0, 0};
        wt[i] = 0.f;
      }
    }
    float s[R][G];
    row_logits<G, R>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (wt[i] == 0.f)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = kNegInf;
    fold_rows<G, R>(st, s, wt, vr, sg);
  }
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

// Exclusive prefix of small counts c in [0, 7] over the lanes of a wave (ballot bit planes).
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t c, uint32_t& wave_total) {
  const uint64_t lt = (1ull << (threadIdx.x & 63)) - 1ull;
  const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
  wave_total = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2);
  return __popcll(b0 & lt) + 2u * __popcll(b1 & lt) + 4u * __popcll(b2 & lt);
}

struct Red3 {
  float mn, mx;
  uint32_t n;
};

// block min / max / count
__device__ __forceinline__ Red3 block_red3(Red3 r, float (*s)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    r.mn = fminf(r.mn, __shfl_xor(r.mn, off));
    r.mx = fmaxf(r.mx, __shfl_xor(r.mx, off));
    r.n += __shfl_xor(r.n, off);
  }
  if (lane == 0) {
    s[wave][0] = r.mn;
    s[wave][1] = r.mx;
    s[wave][2] = __uint_as_float(r.n);
  }
  __syncthreads();
  Red3 t{kPosInf, kNegInf, 0u};
#pragma unroll
  for (int w = 0; w < kDecThreads / 64; ++w) {
    t.mn = fminf(t.mn, s[w][0]);
    t.mx = fmaxf(t.mx, s[w][1]);
    t.n += __float_as_uint(s[w][2]);
  }
  __syncthreads();
  return t;
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
// selection: the n_r clusters of largest group score s^ (ties to the lower id) are exactly
// { j : s^_j > Tkey or (s^_j == Tkey and j <= Tid) } for the n_r-th pair (Tkey, Tid) in
// (score descending, id ascending) order. Empty clusters have s^ = -inf and never qualify.
// ------------------------------------------------------------------------------------
struct SelShared {
  uint32_t hist[kHistBins];  // value-range histogram; reused for the LDS cluster lists
  float ck[kCand];
  int32_t ci[kCand];
  uint32_t wt[kKeySlices * 4];
  float red[4][3];
  uint32_t u[4];
  float tkey;
  int32_t tid;
  ScanTmp tmp;
};
static_assert(3 * kSelMax + 1 <= kHistBins, "cluster lists must fit in the histogram space");

__device__ __forceinline__ float4 neg4() { return make_float4(kNegInf, kNegInf, kNegInf, kNegInf); }

__device__ __forceinline__ bool is_selected(float v, int j, float tkey, int tid) {
  return v != kNegInf && (v > tkey || (v == tkey && j <= tid));
}

// order-preserving map of a float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram bins over a score range [lo, hi], monotone in the score (every step rounds
// monotonically). Linear in the value when the range allows it; otherwise, and on every
// narrowing round, linear in the order-preserving integer key. Either way lo lands in bin 0
// and hi in a later bin, so each narrowing round strictly shrinks the candidate range.
struct Binner {
  float lo, inv;   // value mode: bin = (v - lo) * inv
  uint32_t klo;    // key mode:   bin = (key(v) - klo) * kinv
  float kinv;
  bool by_value;
  __device__ __forceinline__ Binner(float lo_, float hi_, bool first) : lo(lo_) {
    const float d = hi_ - lo_;
    inv = (float)kHistBins / d;
    by_value = first && d > FLT_MIN && d <= FLT_MAX && inv <= FLT_MAX;
    klo = order_key(lo_);
    kinv = (float)kHistBins / ((float)(order_key(hi_) - klo) + 1.f);
  }
  __device__ __forceinline__ int operator()(float v) const {
    const float t = by_value ? (v - lo) * inv : (float)(order_key(v) - klo) * kinv;
    return t >= (float)(kHistBins - 1) ? kHistBins - 1 : (int)t;
  }
};

// Find (Tkey, Tid) given the block-uniform range [lo, hi] of finite scores and
// need in [1, #finite]. each(f) visits every (score, id) this thread owns; tie_id(v, need)
// returns the need-th lowest id whose score equals v (block-uniform).
template <typename Each, typename TieId>
__device__ __forceinline__ void find_threshold(Each each, TieId tie_id, float lo, float hi,
                                               uint32_t need, SelShared& sh, float& Tkey,
                                               int& Tid) {
  const int tid = threadIdx.x;
  bool first = true;
  for (;;) {
    if (lo == hi) {  // every remaining candidate has the same score
      Tkey = lo;
      Tid = tie_id(lo, need);
      return;
    }
    const Binner bin(lo, hi, first);
    first = false;
    for (int i = tid; i < kHistBins; i += kDecThreads) sh.hist[i] = 0u;
    __syncthreads();
    each([&](float v, int) {
      if (v >= lo && v <= hi) atomicAdd(&sh.hist[bin(v)], 1u);
    });
    __syncthreads();
    // bin b* of the need-th largest score: thread t owns 16 bins, visited descending
    const int hb0 = kHistBins - 16 * (tid + 1);
    uint32_t hc[16], loc = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hc[i] = sh.hist[hb0 + i];
      loc += hc[i];
    }
    uint32_t tot;
    uint32_t run = scan_excl(loc, sh.tmp, &tot);
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (run < need && run + hc[i] >= need) {
        sh.u[0] = (uint32_t)(hb0 + i);
        sh.u[1] = run;
      }
      run += hc[i];
    }
    if (tid == 0) sh.u[2] = 0u;
    __syncthreads();
    const int bstar = (int)sh.u[0];
    const uint32_t need2 = need - sh.u[1];
    const uint32_t cnt = sh.hist[bstar];
    if (cnt <= (uint32_t)kCand) {
      // rank the keys of bin b* exactly
      each([&](float v, int j) {
        if (v >= lo && v <= hi && bin(v) == bstar) {
          const uint32_t k = atomicAdd(&sh.u[2], 1u);
          sh.ck[k] = v;
          sh.ci[k] = j;
        }
      });
      __syncthreads();
      if (tid < (int)cnt) {
        const float mv = sh.ck[tid];
        const int mj = sh.ci[tid];
        uint32_t rank = 0;
        for (uint32_t c = 0; c < cnt; ++c) {
          const float cv = sh.ck[c];
          rank += (cv > mv || (cv == mv && sh.ci[c] < mj)) ? 1u : 0u;
        }
        if (rank == need2 - 1) {
          sh.tkey = mv;
          sh.tid = mj;
        }
      }
      __syncthreads();
      Tkey = sh.tkey;
      Tid = sh.tid;
      __syncthreads();
      return;
    }
    // too many keys in b*: narrow the range to that bin's keys and repeat
    Red3 r{kPosInf, kNegInf, 0u};
    each([&](float v, int) {
      if (v >= lo && v <= hi && bin(v) == bstar) {
        r.mn = fminf(r.mn, v);
        r.mx = fmaxf(r.mx, v);
      }
    });
    r = block_red3(r, sh.red);
    lo = r.mn;
    hi = r.mx;
    need = need2;
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
    constexpr int R = Rows<G>::R;
    __shared__ float s_mm[kDecThreads / 64][3];
    const size_t base = (size_t)bh * a.C;
    float* shat = a.shat + (size_t)bh * a.Cp;
    const int j0 = blockIdx.x * kChunk + wave * (kChunk / 4);  // this wave's 32 clusters
    const float sl2 = a.scale_log2, gmean = a.scale / (float)G;
    float mn = kPosInf, mx = kNegInf, cnt = 0.f;
    for (int t = j0; t < j0 + kChunk / 4; t += 4 * R) {
      u32x4 kr[R], vr[R];
      int32_t n[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int j = t + 4 * i + grp;
        if (j < a.C) {
          const size_t row = (base + j) * kHeadDim + cc * 8;
          kr[i] = ld16_stream(a.cmean + row);
          vr[i] = ld16_stream(a.vsum + row);
          n[i] = a.csize[base + j];
        } else {
          kr[i] = vr[i] = u32x4{0, 0, 0, 0};
          n[i] = -1;
        }
      }
      float s[R][G], w[R], sg[R];
      row_logits<G, R>(q, kr, 1.f, s);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int j = t + 4 * i + grp;
        const bool ok = n[i] > 0;
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) sum += s[i][h];
        const float mean = sum * gmean;
        if (cc == 0) shat[j] = ok ? mean : kNegInf;
        if (ok) {
          mn = fminf(mn, mean);
          mx = fmaxf(mx, mean);
          cnt += 1.f;
        }
        if (n[i] >= 0 && cc < G) {
          float mine = s[i][0];
#pragma unroll
          for (int h = 1; h < G; ++h) mine = (cc == h) ? s[i][h] : mine;
          a.scores[(base + j) * G + cc] = mine * sl2;
        }
        w[i] = ok ? (float)n[i] : 0.f;
        sg[i] = 1.f;
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = ok ? s[i][h] * sl2 : kNegInf;
      }
      fold_rows<G, R>(st, s, w, vr, sg);
    }
    // min / max / count of this chunk's finite scores (the 16 lanes of a row group agree)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, off));
      mx = fmaxf(mx, __shfl_xor(mx, off));
      cnt += __shfl_xor(cnt, off);
    }
    if (lane == 0) {
      s_mm[wave][0] = mn;
      s_mm[wave][1] = mx;
      s_mm[wave][2] = cnt;
    }
    __syncthreads();
    if (tid < 3) {
      float r = s_mm[0][tid];
#pragma unroll
      for (int w = 1; w < kDecThreads / 64; ++w)
        r = tid == 0 ? fminf(r, s_mm[w][0]) : tid == 1 ? fmaxf(r, s_mm[w][1]) : r + s_mm[w][2];
      a.mm[((size_t)bh * a.nS + blockIdx.x) * 4 + tid] = r;
    }
  } else {
    const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
    const int64_t wbeg = (int64_t)(blockIdx.x - a.nS) * kTokChunk + wave * (kTokChunk / 4);
    const int64_t wend = min(n_steady, wbeg + kTokChunk / 4);
    attend_rows<G>(a, bh, q, st, wbeg, wend, [&](int64_t t) { return steady_row(a, t); });
  }
  write_block_partial<G>(st, nullptr,
                         a.part + ((size_t)bh * a.nP + blockIdx.x) * G * kPartStride);
}

// ------------------------------------------------------------------------------------
// kernel 2: retrieve
// ------------------------------------------------------------------------------------

// Exact attention and estimate removal over the virtual rows [wb, we) of the listed
// clusters [r_lo, r_hi) (LDS lists: first virtual row ts[] with ts[r_hi] = end, first cache
// row co[], cluster id id[]). A removal row carries weight -n_j (wt < 0); its stored logits
// travel in the registers of its (unused) key row, and in kx for heads 4..7.
template <int G>
__device__ __forceinline__ void attend_virtual(const DecodeArgs& a, int bh, const u32x4 (&q)[G],
                                               Online<G>& st, int wb, int we, const int32_t* ts,
                                               const int32_t* co, const int32_t* id, int r_lo,
                                               int r_hi) {
  constexpr int R = Rows<G>::R;
  constexpr int GX = G > 4 ? G - 4 : 1;
  const int lane = threadIdx.x & 63, grp = lane >> 4, cc = lane & 15;
  const size_t kb = (size_t)bh * a.Lcap, cb = (size_t)bh * a.C;
  for (int t = wb; t < we; t += 4 * R) {
    u32x4 kr[R], vr[R];
    float wt[R], kx[R][GX];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int tt = t + 4 * i + grp;
      kr[i] = vr[i] = u32x4{0, 0, 0, 0};
      wt[i] = 0.f;
#pragma unroll
      for (int h = 0; h < GX; ++h) kx[i][h] = 0.f;
      if (tt < we) {
        int lo = r_lo, hi = r_hi - 1;  // the listed cluster holding virtual row tt
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (ts[mid] <= tt) lo = mid; else hi = mid - 1;
        }
        const int off = tt - ts[lo], n = ts[lo + 1] - ts[lo] - 1;
        if (off < n) {
          const size_t row = (kb + co[lo] + off) * kHeadDim + cc * 8;
          kr[i] = ld16_stream(a.k + row);
          vr[i] = ld16_stream(a.v + row);
          wt[i] = 1.f;
        } else {
          const size_t j = cb + id[lo];
          vr[i] = ld16(a.vsum + j * kHeadDim + cc * 8);
          const float* sp = a.scores + j * G;
#pragma unroll
          for (int h = 0; h < G && h < 4; ++h) kr[i][h] = __float_as_uint(sp[h]);
#pragma unroll
          for (int h = 4; h < G; ++h) kx[i][h - 4] = sp[h];
          wt[i] = -(float)n;
        }
      }
    }
    float s[R][G], sg[R];
    row_logits<G, R>(q, kr, a.scale_log2, s);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      sg[i] = wt[i] < 0.f ? -1.f : 1.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float rs = h < 4 ? __uint_as_float(kr[i][h < 4 ? h : 0]) : kx[i][h < 4 ? 0 : h - 4];
        s[i][h] = wt[i] < 0.f ? rs : (wt[i] == 0.f ? kNegInf : s[i][h]);
      }
    }
    fold_rows<G, R>(st, s, wt, vr, sg);
  }
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dec_retrieve(DecodeArgs a) {
  extern __shared__ float s_key[];       // local select: the group scores, -inf padded
  __shared__ SelShared sh;
  __shared__ float s_x[G][kPartStride];  // this workgroup's share of the stream partials
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv, w_item = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cc = lane & 15;
  const int nB = a.nB, nSP = a.nS + a.nSt;
  float* parts = a.part + (size_t)bh * a.nP * G * kPartStride;
  int32_t* l_ts = reinterpret_cast<int32_t*>(sh.hist);  // [kSelMax + 1]
  int32_t* l_co = l_ts + kSelMax + 1;                      // [kSelMax]
  int32_t* l_id = l_co + kSelMax;                          // [kSelMax]
  const bool local = a.local_select != 0;
  const int Cp = a.Cp, ns = (Cp + 4 * kDecThreads - 1) / (4 * kDecThreads);

  // ---- group scores into LDS (coalesced float4; ids 4 * (i * 256 + tid) + e)
  if (local) {
    const float* shat = a.shat + (size_t)bh * Cp;
    for (int i0 = 0; i0 < ns; i0 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j4 = 4 * ((i0 + u) * kDecThreads + tid);
        v[u] = (i0 + u < ns && j4 < Cp) ? *reinterpret_cast<const float4*>(shat + j4) : neg4();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < ns) *reinterpret_cast<float4*>(s_key + 4 * ((i0 + u) * kDecThreads + tid)) = v[u];
    }
  }
  // ---- this workgroup's stream partials w_item, w_item + nB, ... merged into s_x
  for (int idx = tid; idx < G * 128; idx += kDecThreads) {
    float M, Ls, O;
    merge_partials<false>(parts, G, idx, w_item, nB, nSP, M, Ls, O);
    const int h = idx >> 7, d = idx & 127;
    s_x[h][d] = O;
    if (d == 0) {
      s_x[h][128] = M;
      s_x[h][129] = Ls;
    }
  }
  __syncthreads();

  int nsel, V;  // retrieved clusters, their virtual rows
  int r_lo = 0, r_hi = 0;
  if (local) {
    auto each = [&](auto f) {
      for (int i = 0; i < ns; ++i) {
        const int j4 = 4 * (i * kDecThreads + tid);
        const float4 x = *reinterpret_cast<const float4*>(s_key + j4);
        f(x.x, j4);
        f(x.y, j4 + 1);
        f(x.z, j4 + 2);
        f(x.w, j4 + 3);
      }
    };
    // Ordered visit of the ids with pred(v, j) true (ids ascend with slice, then thread,
    // then element): each is passed with its rank; returns the count.
    auto ordered = [&](auto pred, auto visit) -> uint32_t {
      for (int i = 0; i < ns; ++i) {
        const int j4 = 4 * (i * kDecThreads + tid);
        const float4 x = *reinterpret_cast<const float4*>(s_key + j4);
        const uint32_t c = pred(x.x, j4) + pred(x.y, j4 + 1) + pred(x.z, j4 + 2) +
                           pred(x.w, j4 + 3);
        uint32_t wt;
        wave_prefix_small(c, wt);
        if (lane == 0) sh.wt[i * 4 + wave] = wt;
      }
      __syncthreads();
      uint32_t acc = 0;
      for (int i = 0; i < ns; ++i) {
        const int j4 = 4 * (i * kDecThreads + tid);
        const float4 x = *reinterpret_cast<const float4*>(s_key + j4);
        const float e4[4] = {x.x, x.y, x.z, x.w};
        bool p4[4];
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p4[e] = pred(e4[e], j4 + e);
          c += p4[e];
        }
        uint32_t wt;
        uint32_t k = wave_prefix_small(c, wt) + acc;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = sh.wt[i * 4 + w];
          k += w < wave ? v : 0u;
          acc += v;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (p4[e]) visit(j4 + e, k++);
      }
      __syncthreads();
      return acc;
    };
    auto tie_id = [&](float v, uint32_t need) -> int {
      ordered([&](float x, int) { return x == v; },
              [&](int j, uint32_t k) {
                if (k + 1 == need) sh.tid = j;
              });
      const int r = sh.tid;
      __syncthreads();
      return r;
    };
    Red3 r{kPosInf, kNegInf, 0u};
    each([&](float v, int) {
      if (v != kNegInf) {
        r.mn = fminf(r.mn, v);
        r.mx = fmaxf(r.mx, v);
        ++r.n;
      }
    });
    r = block_red3(r, sh.red);
    const uint32_t nr = min((uint32_t)a.n_retrieve, r.n);
    float Tkey = kPosInf;
    int Tid = -1;
    if (nr == r.n && nr > 0) {
      Tkey = kNegInf;  // every non-empty cluster
    } else if (nr > 0) {
      find_threshold(each, tie_id, r.mn, r.mx, nr, sh, Tkey, Tid);
    }
    // ---- ordered compaction of the selection into the LDS list (ascending ids)
    nsel = (int)ordered([&](float v, int j) { return is_selected(v, j, Tkey, Tid); },
                        [&](int j, uint32_t k) { l_id[k] = j; });
    if (w_item == 0 && a.selected) {
      int32_t* sel = a.selected + (size_t)bh * a.n_retrieve;
      for (int i = tid; i < a.n_retrieve; i += kDecThreads) sel[i] = i < nsel ? l_id[i] : -1;
    }
    // ---- sizes and first cache rows of the listed clusters; virtual row starts
    constexpr int kPer = kSelMax / kDecThreads;
    const int per = (nsel + kDecThreads - 1) / kDecThreads;
    int32_t sz[kPer], co[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int rr = tid * per + k;
      if (k < per && rr < nsel) {
        const size_t j = (size_t)bh * a.C + l_id[rr];
        sz[k] = a.csize[j];
        co[k] = a.coff[j];
      } else {
        sz[k] = -1;
        co[k] = 0;
      }
    }
    uint32_t my = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) my += sz[k] >= 0 ? (uint32_t)sz[k] + 1u : 0u;
    uint32_t tot;
    uint32_t pos = scan_excl(my, sh.tmp, &tot);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int rr = tid * per + k;
      if (sz[k] >= 0) {
        l_ts[rr] = (int)pos;
        l_co[rr] = co[k];
        pos += (uint32_t)sz[k] + 1u;
      }
    }
    V = (int)tot;
    if (tid == 0) l_ts[nsel] = V;
    __syncthreads();
  } else {
    nsel = a.sel_n[bh];
    V = a.sel_ts[(size_t)bh * (a.rcap + 1) + nsel];
  }
  const int T0 = (int)((int64_t)V * w_item / nB), T1 = (int)((int64_t)V * (w_item + 1) / nB);
  if (T0 < T1) {
    if (local) {  // listed clusters overlapping [T0, T1): binary searches in the LDS list
      int lo = 0, hi = nsel - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (l_ts[mid] <= T0) lo = mid; else hi = mid - 1;
      }
      r_lo = lo;
      hi = nsel - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (l_ts[mid] < T1) lo = mid; else hi = mid - 1;
      }
      r_hi = lo + 1;
    } else {
      const int32_t* r0 = a.wg_r0 + (size_t)bh * (kMaxRetrieveWG + 1);
      r_lo = r0[w_item];
      r_hi = w_item + 1 < nB ? min(nsel, r0[w_item + 1] + 1) : nsel;
    }
  }

  u32x4 q[G];
  load_q<G>(a, b, g, cc, q);
  Online<G> st;
  st.init();
  if (local) {
    if (T0 < T1) {
      const int ts = max(T0, l_ts[r_lo]), te = min(T1, l_ts[r_hi]);
      attend_virtual<G>(a, bh, q, st, ts + (te - ts) * wave / 4, ts + (te - ts) * (wave + 1) / 4,
                        l_ts, l_co, l_id, r_lo, r_hi);
    }
  } else {
    const size_t lb = (size_t)bh * a.rcap;
    const int32_t* g_ts = a.sel_ts + (size_t)bh * (a.rcap + 1);
    for (int rw = r_lo; rw < r_hi; rw += kSelMax) {
      const int cnt = min(kSelMax, r_hi - rw);
      for (int i = tid; i <= cnt; i += kDecThreads) {
        l_ts[i] = g_ts[rw + i];
        if (i < cnt) {
          l_co[i] = a.sel_coff[lb + rw + i];
          l_id[i] = a.sel_id[lb + rw + i];
        }
      }
      __syncthreads();
      const int ts = max(T0, l_ts[0]), te = min(T1, l_ts[cnt]);
      if (ts < te)
        attend_virtual<G>(a, bh, q, st, ts + (te - ts) * wave / 4,
                          ts + (te - ts) * (wave + 1) / 4, l_ts, l_co, l_id, 0, cnt);
      __syncthreads();
    }
  }
  write_block_partial<G>(st, &s_x[0][0], parts + (size_t)(nSP + w_item) * G * kPartStride);
  if (arrive_last(a.counter + bh, (uint32_t)nB)) {
    const int bq = b * a.Hq + g * G;
    for (int idx = tid; idx < G * 128; idx += kDecThreads) {
      float M, Ls, O;
      merge_partials<true>(parts, G, idx, nSP, 1, nSP + nB, M, Ls, O);
      const int h = idx >> 7, d = idx & 127;
      a.out[(size_t)(bq + h) * kHeadDim + d] = O / Ls;
      if (d == 0 && a.lse) a.lse[bq + h] = (M + log2f(Ls)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------
// published select (large indexes or budgets): one workgroup per (b, kv-head) selects and
// lists the retrieved clusters (ids, first virtual row, first cache row) in the workspace,
// plus the first listed cluster of every retrieve workgroup. Scores are streamed from the
// workspace (L2-resident) on each pass.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kDecThreads) void k_dec_select(DecodeArgs a) {
  __shared__ SelShared sh;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cp = a.Cp, nsl = (Cp + 4 * kDecThreads - 1) / (4 * kDecThreads);
  const float* shat = a.shat + (size_t)bh * Cp;
  const size_t cb = (size_t)bh * a.C;
  auto each = [&](auto f) {
    for (int i0 = 0; i0 < nsl; i0 += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j4 = 4 * ((i0 + u) * kDecThreads + tid);
        v[u] = (i0 + u < nsl && j4 < Cp) ? *reinterpret_cast<const float4*>(shat + j4) : neg4();
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j4 = 4 * ((i0 + u) * kDecThreads + tid);
        f(v[u].x, j4);
        f(v[u].y, j4 + 1);
        f(v[u].z, j4 + 2);
        f(v[u].w, j4 + 3);
      }
    }
  };
  // slice-by-slice ordered search for the need-th lowest id whose score equals v
  auto tie_id = [&](float v, uint32_t need) -> int {
    uint32_t acc = 0;
    for (int i = 0; i < nsl; ++i) {
      const int j4 = 4 * (i * kDecThreads + tid);
      const float4 x = j4 < Cp ? *reinterpret_cast<const float4*>(shat + j4) : neg4();
      const uint32_t c = (x.x == v) + (x.y == v) + (x.z == v) + (x.w == v);
      uint32_t wt;
      uint32_t pre = wave_prefix_small(c, wt);
      if (lane == 0) sh.wt[wave] = wt;
      __syncthreads();
      uint32_t before = 0, stot = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        stot += sh.wt[w];
        before += w < wave ? sh.wt[w] : 0u;
      }
      pre += acc + before;
      if (pre < need && need <= pre + c) {
        const float e4[4] = {x.x, x.y, x.z, x.w};
        uint32_t k = pre;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e4[e] == v && ++k == need) sh.tid = j4 + e;
      }
      acc += stot;
      __syncthreads();
      if (acc >= need) break;
    }
    const int r = sh.tid;
    __syncthreads();
    return r;
  };
  // range and count of the finite scores from the stream chunks' summaries
  Red3 r{kPosInf, kNegInf, 0u};
  for (int x = tid; x < a.nS; x += kDecThreads) {
    const float* m = a.mm + ((size_t)bh * a.nS + x) * 4;
    r.mn = fminf(r.mn, m[0]);
    r.mx = fmaxf(r.mx, m[1]);
    r.n += (uint32_t)m[2];
  }
  r = block_red3(r, sh.red);
  const uint32_t nr = min((uint32_t)a.n_retrieve, r.n);
  float Tkey = kPosInf;
  int Tid = -1;
  if (nr == r.n && nr > 0) {
    Tkey = kNegInf;
  } else if (nr > 0) {
    find_threshold(each, tie_id, r.mn, r.mx, nr, sh, Tkey, Tid);
  }
  // total virtual rows of the selection
  uint32_t my = 0;
  for (int i = 0; i < nsl; ++i) {
    const int j4 = 4 * (i * kDecThreads + tid);
    if (j4 >= a.C) break;
    const float4 x = *reinterpret_cast<const float4*>(shat + j4);
    const float e4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j4 + e < a.C && is_selected(e4[e], j4 + e, Tkey, Tid))
        my += (uint32_t)a.csize[cb + j4 + e] + 1u;
  }
  uint32_t V;
  scan_excl(my, sh.tmp, &V);
  // ordered compaction, one slice of 1024 ids at a time
  const int nB = a.nB;
  int32_t* sid = a.sel_id + (size_t)bh * a.rcap;
  int32_t* sts = a.sel_ts + (size_t)bh * (a.rcap + 1);
  int32_t* sco = a.sel_coff + (size_t)bh * a.rcap;
  int32_t* r0 = a.wg_r0 + (size_t)bh * (kMaxRetrieveWG + 1);
  int32_t* selo = a.selected ? a.selected + (size_t)bh * a.n_retrieve : nullptr;
  uint32_t rank = 0, row = 0;
  for (int i = 0; i < nsl; ++i) {
    const int j4 = 4 * (i * kDecThreads + tid);
    const float4 x = j4 < Cp ? *reinterpret_cast<const float4*>(shat + j4) : neg4();
    const float e4[4] = {x.x, x.y, x.z, x.w};
    int32_t n4[4];
    uint32_t c = 0, tok = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool s = j4 + e < a.C && is_selected(e4[e], j4 + e, Tkey, Tid);
      n4[e] = s ? a.csize[cb + j4 + e] : -1;
      c += s;
      tok += s ? (uint32_t)n4[e] + 1u : 0u;
    }
    uint32_t wt;
    const uint32_t pre = wave_prefix_small(c, wt);
    uint32_t tp = tok;  // inclusive scan of tok over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(tp, off);
      if (lane >= off) tp += y;
    }
    if (lane == 63) {
      sh.wt[wave] = wt;
      sh.wt[4 + wave] = tp;
    }
    __syncthreads();
    uint32_t before_c = 0, before_t = 0, sc = 0, stk = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc += sh.wt[w];
      stk += sh.wt[4 + w];
      before_c += w < wave ? sh.wt[w] : 0u;
      before_t += w < wave ? sh.wt[4 + w] : 0u;
    }
    __syncthreads();
    uint32_t rr = rank + before_c + pre, ts = row + before_t + tp - tok;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n4[e] >= 0) {
        const int j = j4 + e;
        sid[rr] = j;
        sts[rr] = (int32_t)ts;
        sco[rr] = a.coff[cb + j];
        if (selo) selo[rr] = j;
        // retrieve workgroups whose first virtual row falls in [ts, te)
        const uint32_t te = ts + (uint32_t)n4[e] + 1u;
        const int w0 = (int)(((uint64_t)ts * nB + V - 1) / V);
        const int w1 = (int)(((uint64_t)te * nB + V - 1) / V);
        for (int w = w0; w < w1; ++w) r0[w] = (int32_t)rr;
        ++rr;
        ts = te;
      }
    rank += sc;
    row += stk;
  }
  if (selo)
    for (int i = (int)rank + tid; i < a.n_retrieve; i += kDecThreads) selo[i] = -1;
  if (tid == 0) {
    a.sel_n[bh] = (int32_t)rank;
    sts[rank] = (int32_t)V;
    if (V == 0)
      for (int w = 0; w < nB; ++w) r0[w] = 0;
    r0[nB] = (int32_t)rank;
  }
}

// ------------------------------------------------------------------------------------
// dense decode (full attention over [0, L)): split-K partials + merge
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dense_partial(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, c, q);
  Online<G> st;
  st.init();
  const int nB = a.nB, w = blockIdx.x;
  const int64_t t0 = a.L * w / nB, t1 = a.L * (w + 1) / nB;
  const int64_t wb = t0 + (t1 - t0) * wave / 4, we = t0 + (t1 - t0) * (wave + 1) / 4;
  attend_rows<G>(a, bh, q, st, wb, we, [](int64_t t) { return t; });
  write_block_partial<G>(st, nullptr, a.part + ((size_t)bh * nB + w) * G * kPartStride);
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dense_merge(DecodeArgs a) {
  const int bh = blockIdx.x, b = bh / a.Hkv, g = bh % a.Hkv;
  const float* parts = a.part + (size_t)bh * a.nB * G * kPartStride;
  const int bq = b * a.Hq + g * G;
  for (int idx = threadIdx.x; idx < G * 128; idx += kDecThreads) {
    float M, Ls, O;
    merge_partials<true>(parts, G, idx, 0, 1, a.nB, M, Ls, O);
    const int h = idx >> 7, d = idx & 127;
    a.out[(size_t)(bq + h) * kHeadDim + d] = O / Ls;
    if (d == 0 && a.lse) a.lse[bq + h] = (M + log2f(Ls)) * kLn2;
  }
}

// ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_dec_stream<G>, dim3(a.nS + a.nSt, BH), dim3(kDecThreads), 0, s, a);
  if (e != hipSuccess) return e;
  if (!a.local_select) {
    e = launch(tr, k_dec_select, dim3(BH), dim3(kDecThreads), 0, s, a);
    if (e != hipSuccess) return e;
  }
  // dynamic LDS of the retrieve kernel: the group scores when it selects for itself
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_dec_retrieve<G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLocalSelMax * (int)sizeof(float));
  if (attr != hipSuccess) return attr;
  const size_t lds = a.local_select ? (size_t)(a.Cp + 4 * kDecThreads - 1) /
                                          (4 * kDecThreads) * (4 * kDecThreads) * sizeof(float)
                                    : 0;
  return launch(tr, k_dec_retrieve<G>, dim3(a.nB, BH), dim3(kDecThreads), (uint32_t)lds, s, a);
}

template <int G>
static hipError_t launch_dense_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_dense_partial<G>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
  if (e != hipSuccess) return e;
  return launch(tr, k_dense_merge<G>, dim3(BH), dim3(kDecThreads), 0, s, a);
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
