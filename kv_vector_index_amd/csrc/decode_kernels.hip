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
// MI355X design, three kernels per call (four for heads of more than kLocalSelectMax clusters):
//   score     a few workgroups per CU stream the centroid rows and sizes once (HBM-bound),
//             store each query head's logit, the group-mean score and each workgroup's
//             score range.
//   [hist]    large heads only: a value-range histogram of the group scores.
//   gather    the selection finds the exact top-n_r clusters (ties to the lower id) from a
//             4096-bin histogram over the head's score range and an exact rank of the cut
//             bin: for heads of at most kLocalSelectMax clusters one workgroup does it all
//             with the head's scores in registers; larger heads have one workgroup per
//             2048 scores listing the clusters above and in the cut bin, and the last of a
//             head ranks the cut bin. Either way the selection is published in ascending id
//             order with each cluster's first "virtual row" (see below) and first cache
//             row, and each retrieve workgroup's share; in the same launch, estimate
//             workgroups fold the
//             centroid term of ALL non-empty clusters (value sums streamed beside the
//             selection) and steady workgroups attend to the sink and recent tokens.
//   retrieve  nB workgroups per (b, kv-head) walk the virtual rows of the retrieved clusters:
//             every token of a retrieved cluster (exact attention; a retrieved cluster is a
//             contiguous run of cache rows in the index layout) and one row per cluster that
//             removes the estimate term added above. Each workgroup also folds a share of the
//             estimate and steady partials; partials are merged by log-sum-exp in one or two
//             levels into out / lse.
// Rows are read 16 lanes per 256-byte row (4 rows per wave instruction, fully coalesced) and
// each K/V row is shared by the G query heads of its group.
#include <float.h>

#include <mutex>

#include <type_traits>

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
// sg: +1 / -1 multiplier of the value row. All weights first, then one pass over the 8
// dims in which each value is unpacked from bf16 once and used by all G heads.
template <int G, int R>
__device__ __forceinline__ void fold_rows(Online<G>& st, const float (&s2)[R][G],
                                          const float (&w)[R], const u32x4 (&v)[R],
                                          const float (&sg)[R]) {
  float alpha[G], p[G][R];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float tm = s2[0][h];
#pragma unroll
    for (int i = 1; i < R; ++i) tm = fmaxf(tm, s2[i][h]);
    const float mn = fmaxf(st.m[h], tm);
    const bool none = mn == kNegInf;  // nothing folded yet and nothing in these rows
    alpha[h] = none ? 1.f : fast_exp2(st.m[h] - mn);
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float e = none ? 0.f : fast_exp2(s2[i][h] - mn);
      ls += w[i] * e;
      p[h][i] = e * sg[i];
    }
    st.l[h] = alpha[h] * st.l[h] + ls;
    st.m[h] = mn;
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    float vd[R];
#pragma unroll
    for (int i = 0; i < R; ++i) vd[i] = vdim(v[i], d);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = alpha[h] * st.o[h][d];
#pragma unroll
      for (int i = 0; i < R; ++i) acc += p[h][i] * vd[i];
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

// The value of lane l ^ 16 (resp. l ^ 32), without LDS: the permlane swaps exchange
// 16-lane rows 0 <-> 1 and 2 <-> 3 (resp. the two 32-lane halves) between two registers.
__device__ __forceinline__ float xor16(float x) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __int_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  const int xi = __float_as_int(x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Combine the four 16-lane row groups of a wave; afterwards every lane holds the wave state.
template <int G>
__device__ __forceinline__ void merge_row_groups(Online<G>& st) {
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    auto other = [&](float x) { return step == 0 ? xor16(x) : xor32(x); };
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = other(st.m[h]);
      const float lo = other(st.l[h]);
      float a1, a2, mn;
      lse_pair(st.m[h], mo, a1, a2, mn);
      st.m[h] = mn;
      st.l[h] = a1 * st.l[h] + a2 * lo;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float oo = other(st.o[h][d]);
        st.o[h][d] = a1 * st.o[h][d] + a2 * oo;
      }
    }
  }
}

// Combine the waves of the workgroup (and, if xp is not null, one more partial
// [G][kPartStride] held in LDS) and write one partial [G][kPartStride] to dst: with
// device-coherent stores when DEV (read by other workgroups of the same kernel), else plain
// stores (read by a later kernel).
// sm: LDS exchange [waves][G][kPartStride] (write_block_partial below brings its own).
template <int G, bool DEV = true>
__device__ __forceinline__ void write_block_partial_in(Online<G>& st, const float* xp,
                                                       float* __restrict__ dst,
                                                       float (*sm)[G][kPartStride]) {
  constexpr int W = kDecThreads / 64;
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
    if constexpr (DEV) {
      st_dev(dst + h * kPartStride + d, o);
      if (d == 0) {
        st_dev(dst + h * kPartStride + 128, M);
        st_dev(dst + h * kPartStride + 129, l);
      }
    } else {
      dst[h * kPartStride + d] = o;
      if (d == 0) {
        dst[h * kPartStride + 128] = M;
        dst[h * kPartStride + 129] = l;
      }
    }
  }
  __syncthreads();
}

template <int G, bool DEV = true>
__device__ __forceinline__ void write_block_partial(Online<G>& st, const float* xp,
                                                    float* __restrict__ dst) {
  __shared__ float sm[kDecThreads / 64][G][kPartStride];
  write_block_partial_in<G, DEV>(st, xp, dst, sm);
}

// Log-sum-exp merge of the partials p0, p0 + step, ... (< n) of parts, for the head/dim
// element idx = h * 128 + d, NBATCH partials in flight per round. DEV: device-coherent loads
// (partials written by other workgroups of the same kernel). NBATCH partials per round.
template <bool DEV, int NBATCH = 8>
__device__ __forceinline__ void merge_partials(const float* parts, int G, int idx, int p0,
                                               int step, int n, float& M, float& Ls, float& O) {
  const int h = idx >> 7, d = idx & 127;
  M = kNegInf;
  Ls = 0.f;
  O = 0.f;
  for (int p = p0; p < n; p += NBATCH * step) {
    float pm[NBATCH], pl[NBATCH], po[NBATCH];
#pragma unroll
    for (int k = 0; k < NBATCH; ++k) {
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
    for (int k = 0; k < NBATCH; ++k) mx = fmaxf(mx, pm[k]);
    if (mx == kNegInf) continue;
    const float sc = fast_exp2(M - mx);
    O *= sc;
    Ls *= sc;
#pragma unroll
    for (int k = 0; k < NBATCH; ++k) {
      const float f = fast_exp2(pm[k] - mx);
      O += f * po[k];
      Ls += f * pl[k];
    }
    M = mx;
  }
}

// Eight (two) floats of a partial: device-coherent 64-bit loads when DEV (partials written by
// other workgroups of the same kernel), else plain loads.
template <bool DEV>
__device__ __forceinline__ float2 part_ld2(const float* p) {
  if constexpr (DEV) {
    const uint64_t u = ld_dev(reinterpret_cast<const uint64_t*>(p));
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}
template <bool DEV>
__device__ __forceinline__ float4 part_ld4(const float* p) {
  const float2 a = part_ld2<DEV>(p), b = part_ld2<DEV>(p + 2);
  return make_float4(a.x, a.y, b.x, b.y);
}

// Log-sum-exp merge of the n partials in slots p0, p0 + step, ... of parts ([slot][G]
// [kPartStride]) by the whole workgroup, in one round of loads when n <= 2 MB: item i
// (thread t % 128, then further items for G > 4) takes head i / 32 and dims 4 (i % 32) ..
// + 3; the two halves of the workgroup take the even and the odd partials, each loading all
// of its partials before combining them, and meet in LDS. emit(h, d4, M, L, o) runs in the
// first half (M in log2 units, o unnormalised).
template <int G, bool DEV, int MB, typename Emit>
__device__ __forceinline__ void merge_block(const float* parts, int p0, int step, int n,
                                            float (*xh)[6], Emit emit) {
  const int tid = threadIdx.x, half = tid >> 7, item = tid & 127;
  for (int it0 = 0; it0 < G * 32; it0 += 128) {
    const int it = it0 + item;
    const bool live = it < G * 32;
    const int h = live ? it >> 5 : 0, d4 = (it & 31) * 4;
    float M = kNegInf, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = half; k0 < n; k0 += 2 * MB) {
      float2 ml[MB];
      float4 ov[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {  // (clamped, unconditional loads: issued together)
        const int k = min(k0 + 2 * b, n - 1);
        const float* pp = parts + ((size_t)(p0 + k * step) * G + h) * kPartStride;
        ml[b] = part_ld2<DEV>(pp + 128);
        ov[b] = part_ld4<DEV>(pp + d4);
        if (k0 + 2 * b >= n) ml[b].x = kNegInf;
      }
      float mx = M;
#pragma unroll
      for (int b = 0; b < MB; ++b) mx = fmaxf(mx, ml[b].x);
      if (mx != kNegInf) {
        const float sc = fast_exp2(M - mx);
        L *= sc;
        o.x *= sc;
        o.y *= sc;
        o.z *= sc;
        o.w *= sc;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          const float f = fast_exp2(ml[b].x - mx);
          L += f * ml[b].y;
          o.x += f * ov[b].x;
          o.y += f * ov[b].y;
          o.z += f * ov[b].z;
          o.w += f * ov[b].w;
        }
        M = mx;
      }
    }
    if (half == 1) {
      xh[item][0] = M;
      xh[item][1] = L;
      xh[item][2] = o.x;
      xh[item][3] = o.y;
      xh[item][4] = o.z;
      xh[item][5] = o.w;
    }
    __syncthreads();
    if (half == 0 && live) {
      const float M2 = xh[item][0], mx = fmaxf(M, M2);
      if (mx != kNegInf) {
        const float f1 = fast_exp2(M - mx), f2 = fast_exp2(M2 - mx);
        L = f1 * L + f2 * xh[item][1];
        o.x = f1 * o.x + f2 * xh[item][2];
        o.y = f1 * o.y + f2 * xh[item][3];
        o.z = f1 * o.z + f2 * xh[item][4];
        o.w = f1 * o.w + f2 * xh[item][5];
        M = mx;
      }
      emit(h, d4, M, L, o);
    }
    __syncthreads();
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

// Exact attention over the rows base + row_of(t), t in [wb, we), of the arrays kc, vc.
template <int G, typename RowOf>
__device__ __forceinline__ void attend_rows(const DecodeArgs& a, const uint16_t* kc,
                                            const uint16_t* vc, size_t base,
                                            const u32x4 (&q)[G], Online<G>& st, int64_t wb,
                                            int64_t we, RowOf row_of) {
  constexpr int R = Rows<G>::R;
  const int lane = threadIdx.x & 63, grp = lane >> 4, cc = lane & 15;
  for (int64_t t = wb; t < we; t += 4 * R) {
    u32x4 kr[R], vr[R];
    float wt[R], sg[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t tt = t + 4 * i + grp;
      sg[i] = 1.f;
      if (tt < we) {
        const size_t row = (base + row_of(tt)) * kHeadDim + cc * 8;
        kr[i] = ld16_stream(kc + row);
        vr[i] = ld16_stream(vc + row);
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
// block-wide helpers for NT-thread workgroups
// ------------------------------------------------------------------------------------

// Exclusive prefix of small counts c in [0, 7] over the lanes of a wave (ballot bit planes).
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t c, uint32_t& wave_total) {
  const uint64_t lt = (1ull << (threadIdx.x & 63)) - 1ull;
  const uint64_t b0 = __ballot(c & 1u), b1 = __ballot(c & 2u), b2 = __ballot(c & 4u);
  wave_total = __popcll(b0) + 2u * __popcll(b1) + 4u * __popcll(b2);
  return __popcll(b0 & lt) + 2u * __popcll(b1 & lt) + 4u * __popcll(b2 & lt);
}

// Reductions over the 64 lanes of a wave without LDS: four DPP steps make each 16-lane row
// uniform, then the four rows are read back as scalars. Every lane gets the result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  auto mv = [](T v, auto ctrl) {
    return __builtin_bit_cast(T, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                          decltype(ctrl)::value, 0xF, 0xF,
                                                          false));
  };
  x = op(x, mv(x, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  x = op(x, mv(x, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  x = op(x, mv(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  x = op(x, mv(x, std::integral_constant<int, 0x140>{}));  // row_mirror
  const int xi = __builtin_bit_cast(int, x);
  const T r0 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(xi, 0));
  const T r1 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(xi, 16));
  const T r2 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(xi, 32));
  const T r3 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(xi, 48));
  return op(op(r0, r1), op(r2, r3));
}

struct Red3 {
  float mn, mx;
  uint32_t n;
};

// block min / max / count
template <int NT>
__device__ __forceinline__ Red3 block_red3(Red3 r, float (*s)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  r.mn = wave_reduce(r.mn, [](float a, float b) { return fminf(a, b); });
  r.mx = wave_reduce(r.mx, [](float a, float b) { return fmaxf(a, b); });
  r.n = wave_reduce(r.n, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 0) {
    s[wave][0] = r.mn;
    s[wave][1] = r.mx;
    s[wave][2] = __uint_as_float(r.n);
  }
  __syncthreads();
  Red3 t{kPosInf, kNegInf, 0u};
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    t.mn = fminf(t.mn, s[w][0]);
    t.mx = fmaxf(t.mx, s[w][1]);
    t.n += __float_as_uint(s[w][2]);
  }
  __syncthreads();
  return t;
}

// LDS histograms whose bins are scanned in runs of 2^SHIFT per thread keep one spare word
// after every run, so that the threads of a wave read their runs from distinct banks.
template <int SHIFT>
__device__ __forceinline__ int padded(int bin) {
  return bin + (bin >> SHIFT);
}
constexpr int kFullPad = 4;    // full histogram (kHistBins): runs of 16 bins
constexpr int kNarrowPad = 2;  // narrowing histogram (kNarrowBins): runs of 4 bins

// Histogram increment with the lanes of a wave that hit the same bin combined first (wave
// ballots over the BITS bits of the bin give each lane its peers), so a bin receives at most
// one LDS atomic per wave instead of one per lane. Lanes with active = false take part in
// the ballots only. PAD: the histogram's padding shift (31: none).
template <int BITS, int PAD = 31>
__device__ __forceinline__ void hist_add(uint32_t* hist, int bin, bool active) {
  uint64_t peers = __ballot(active);
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const bool bit = (bin >> b) & 1;
    const uint64_t m = __ballot(active && bit);
    peers &= bit ? m : ~m;
  }
  const uint64_t below = (1ull << (threadIdx.x & 63)) - 1ull;
  if (active && (peers & below) == 0) atomicAdd(&hist[padded<PAD>(bin)], (uint32_t)__popcll(peers));
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
__device__ __forceinline__ float4 neg4() { return make_float4(kNegInf, kNegInf, kNegInf, kNegInf); }

__device__ __forceinline__ bool is_selected(float v, int j, float tkey, int tid) {
  return v != kNegInf && (v > tkey || (v == tkey && j <= tid));
}

// order-preserving map of a float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram bins (kHistBins) over a score range [lo, hi], monotone in the score (every step
// rounds monotonically). Linear in the value when the range allows it; otherwise, and on
// every narrowing round, linear in the order-preserving integer key. Either way lo lands in
// bin 0 and hi in a later bin, so each narrowing round strictly shrinks the candidate range.
// The same (lo, hi) always gives the same bins, in every kernel.
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

// ------------------------------------------------------------------------------------
// kernel 1: score (centroid logits of every cluster)
// ------------------------------------------------------------------------------------
// One workgroup per chunk of 128 clusters of a (b, kv-head) (the dispatcher balances the
// stream), 32 clusters per wave. The logits of the G heads are a dense product
// [16 x 128] . [128 x 16] per 16 clusters on v_mfma_f32_16x16x32_bf16 (A: the group's query
// rows, zero beyond G; B: 16 centroids, four lanes of 16 bytes per 64 bytes of a row, read
// from the rows staged in LDS; D: lane l < 16 holds heads 0..3 of cluster l, lane 16 + l
// heads 4..7). Every query head's log2-domain logit goes to scores[], the group mean
// (natural units) to shat[] (-inf for empty and padding clusters), and the workgroup's
// finite min / max to smm[]. Workgroup 0 of each (b, kv-head) also clears its counters (and
// its histogram, for the histogram kernel).
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_dec_score(DecodeArgs a) {
  typedef __attribute__((ext_vector_type(4))) float floatx4;
  __shared__ float s_mm[kDecThreads / 64][2];
  __shared__ uint32_t s_rows[kDecThreads / 64][8][256];  // per wave: 8 loads of 4 rows
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kg = lane >> 4;  // MFMA column (cluster) and k group
  if (blockIdx.x == 0) {
    if (tid < kCtrStride) a.counter[(size_t)bh * kCtrStride + tid] = 0u;
    if (a.hist_kernel) {
      uint32_t* h = a.hist + (size_t)bh * kHistBins;
      for (int i = tid; i < kHistBins; i += kDecThreads) h[i] = 0u;
    }
  }
  // A operand: query head `col` (zero beyond G), dims 32 s + 8 kg .. + 7 for k step s
  bf16x8 qa[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    u32x4 v = {0, 0, 0, 0};
    if (col < G)
      v = ld16(a.q + ((size_t)(b * a.Hq + g * G + col) * kHeadDim + st * 32 + kg * 8));
    qa[st] = __builtin_bit_cast(bf16x8, v);
  }
  const size_t base = (size_t)bh * a.C;
  float* shat = a.shat + (size_t)bh * a.Cp;
  const float sl2 = a.scale_log2, gmean = a.scale / (float)G;
  // the wave's 32 centroid rows, whole, into LDS: direct load i brings rows 4 i .. 4 i + 3
  // (slot s = lane / 16), each row rotated by 4 s 16-byte chunks so that the operand reads
  // below (16 rows, one 16-byte column chunk each) spread over all banks
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int t = blockIdx.x * kChunk + wave * 32;  // this wave's first cluster
  {
    const int slot = lane >> 4, cidx = ((lane & 15) - 4 * slot) & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t row = base + min(t + 4 * i + slot, a.C - 1);
      __builtin_amdgcn_global_load_lds(a.cmean + row * kHeadDim + cidx * 8,
                                       (lds_ptr)&s_rows[wave][i][0], 16, 0, 0);
    }
  }
  int32_t n[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    n[u] = __builtin_nontemporal_load(a.csize + base + min(t + 16 * u + col, a.C - 1));
  float mn = kPosInf, mx = kNegInf;
  drain_vmem();  // (this wave's direct loads have landed in LDS)
  __builtin_amdgcn_wave_barrier();
  const char* wr = reinterpret_cast<const char*>(&s_rows[wave][0][0]);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 16 * u + col, blk = r >> 2, sl = r & 3;
    floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 kb = *reinterpret_cast<const u32x4*>(
          wr + blk * 1024 + sl * 256 + (((4 * st + kg + 4 * sl) & 15) << 4));
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], __builtin_bit_cast(bf16x8, kb), d, 0,
                                                  0, 0);
    }
    // lane kg * 16 + col: heads 4 kg + i of cluster t + 16 u + col
    const int j = t + 16 * u + col;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sum += (4 * kg + i < G) ? d[i] : 0.f;
    if (G > 4) sum += __shfl_xor(sum, 16);  // heads 4..7 from lane col + 16
    if (j < a.C && kg < (G + 3) / 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * kg + i < G) a.scores[(base + j) * G + 4 * kg + i] = d[i] * sl2;
    }
    if (kg == 0) {
      const float mean = sum * gmean;
      const bool ok = (j < a.C) & (n[u] > 0);
      if (ok) {
        mn = fminf(mn, mean);
        mx = fmaxf(mx, mean);
      }
      shat[j] = ok ? mean : kNegInf;
    }
  }
  mn = wave_reduce(mn, [](float x, float y) { return fminf(x, y); });
  mx = wave_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
  if (lane == 0) {
    s_mm[wave][0] = mn;
    s_mm[wave][1] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    float* o = a.smm + ((size_t)bh * a.nSW + blockIdx.x) * 2;
    o[0] = fminf(fminf(s_mm[0][0], s_mm[1][0]), fminf(s_mm[2][0], s_mm[3][0]));
    o[1] = fmaxf(fmaxf(s_mm[0][1], s_mm[1][1]), fmaxf(s_mm[2][1], s_mm[3][1]));
  }
}

// ------------------------------------------------------------------------------------
// the head's score range, from the score workgroups' min / max pairs
// ------------------------------------------------------------------------------------
// Value-range bins over [min, max] of the head's finite group scores; every selection
// workgroup of the head recomputes the same (lo, hi) and bins.
__device__ __forceinline__ Red3 score_range(const DecodeArgs& a, int bh, float (*red)[3]) {
  const float* mm = a.smm + (size_t)bh * a.nSW * 2;
  Red3 r{kPosInf, kNegInf, 0u};
  for (int i = threadIdx.x; i < a.nSW; i += kDecThreads) {
    r.mn = fminf(r.mn, mm[2 * i]);
    r.mx = fmaxf(r.mx, mm[2 * i + 1]);
  }
  return block_red3<kDecThreads>(r, red);
}

// Histogram kernel (heads of more than kLocalSelectMax clusters): nH workgroups per (b,
// kv-head), kSelSpan scores each, add their histogram into hist[].
__global__ __launch_bounds__(kDecThreads) void k_dec_hist(DecodeArgs a) {
  constexpr int NT = kDecThreads;
  __shared__ uint32_t hs[kHistBins];
  __shared__ float red[NT / 64][3];
  const int bh = blockIdx.y, tid = threadIdx.x;
  // (the scores are loaded before the range is reduced: one memory round trip for both)
  constexpr int K4 = kSelSpan / (4 * NT);
  const float* sh = a.shat + (size_t)bh * a.Cp;
  float4 sv[K4];
#pragma unroll
  for (int k = 0; k < K4; ++k) {
    const int j4 = blockIdx.x * kSelSpan + k * 4 * NT + 4 * tid;
    sv[k] = j4 < a.Cp ? *reinterpret_cast<const float4*>(sh + j4) : neg4();
  }
  const Red3 r = score_range(a, bh, red);
  if (r.mx == kNegInf) return;  // no finite score in this head
  for (int i = tid; i < kHistBins; i += NT) hs[i] = 0u;
  __syncthreads();
  const Binner bn(r.mn, r.mx, true);
#pragma unroll
  for (int k = 0; k < K4; ++k) {
    const float4 v = sv[k];
    hist_add<12>(hs, v.x != kNegInf ? bn(v.x) : 0, v.x != kNegInf);
    hist_add<12>(hs, v.y != kNegInf ? bn(v.y) : 0, v.y != kNegInf);
    hist_add<12>(hs, v.z != kNegInf ? bn(v.z) : 0, v.z != kNegInf);
    hist_add<12>(hs, v.w != kNegInf ? bn(v.w) : 0, v.w != kNegInf);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)bh * kHistBins;
  for (int i = tid; i < kHistBins; i += NT)
    if (hs[i]) atomicAdd(gh + i, hs[i]);
}

// ------------------------------------------------------------------------------------
// kernel 3: gather (the selection) and estimate (every cluster's centroid term)
// ------------------------------------------------------------------------------------
constexpr int kTieLds = 1024;  // cut-bin clusters staged in LDS by the finishing workgroup
struct FinShared {
  union {
    struct {
      uint32_t bits[kMaxClusters / 32];  // selection bitmap over cluster ids
      uint32_t nzw[kMaxClusters / 32];   // non-empty words: index | first rank << 11
    };
    uint32_t hist[kNarrowBins + kNarrowBins / 4];  // histogram of a crowded cut bin (padded)
    uint32_t full[kHistBins + 1 + kHistBins / 16 + 1];  // all the head's scores (+ a spare
                                                        // bin; padded)
  } u;
  int32_t lst[kMaxClusters / 32];      // the first kMaxClusters / 32 listed ids (before the
                                       // publishing: the clusters above the cut bin)
  float tk[kTieLds];                   // the clusters of the cut bin: scores and ids
  int32_t ti[kTieLds];
  float ck[kCand];
  int32_t ci[kCand];
  int32_t wgr[kMaxRetrieveWG + 1];
  float red[kDecThreads / 64][3];
  ScanTmp<kDecThreads> tmp;
  uint32_t v[4];
  float tkey;
  int32_t tid;
  uint32_t base[2];
};

// The cut of a (b, kv-head) of more than kLocalSelectMax clusters: need = min(n_r, finite
// scores) and the histogram bin b* that holds the need-th largest score (b* = kHistBins when
// need = 0), from the histogram kernel's histogram of all the head's scores. Every selection
// workgroup of the head computes the same values.
struct Cut {
  float lo, hi;
  int bstar;
  uint32_t need;
};
__device__ __forceinline__ Cut find_cut(const DecodeArgs& a, int bh, FinShared& sh) {
  constexpr int NT = kDecThreads, BPT = kHistBins / NT;
  const int tid = threadIdx.x;
  // (the histogram is loaded before the range is reduced: one memory round trip for both)
  const uint32_t* gh = a.hist + (size_t)bh * kHistBins;
  uint32_t hv[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) hv[i] = gh[tid + i * NT];
  const Red3 r = score_range(a, bh, sh.red);
#pragma unroll
  for (int i = 0; i < BPT; ++i)
    sh.u.full[padded<kFullPad>(tid + i * NT)] = r.mx != kNegInf ? hv[i] : 0u;
  __syncthreads();
  const int hb0 = kHistBins - BPT * (tid + 1);  // thread t's bins, visited from the top
  uint32_t hc[BPT], loc = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    hc[i] = sh.u.full[padded<kFullPad>(hb0 + i)];
    loc += hc[i];
  }
  uint32_t ne;
  uint32_t run = scan_excl<NT>(loc, sh.tmp, &ne);
  const uint32_t need = min((uint32_t)a.n_retrieve, ne);
  if (tid == 0) sh.v[0] = kHistBins;
  __syncthreads();
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (run < need && run + hc[i] >= need) sh.v[0] = (uint32_t)(hb0 + i);
    run += hc[i];
  }
  __syncthreads();
  Cut c{r.mn, r.mx, (int)sh.v[0], need};
  __syncthreads();
  return c;
}

// Set bit j of the selection bitmap.
__device__ __forceinline__ void mark(FinShared& sh, int j) {
  atomicOr(&sh.u.bits[j >> 5], 1u << (j & 31));
}

// The id of the need-th set bit (need >= 1, at most the number of set bits) of the bitmap
// words [0, nwords) of sh.u.bits, in every thread.
__device__ __forceinline__ int nth_bit(FinShared& sh, int nwords, uint32_t need) {
  constexpr int NT = kDecThreads, WPT = kMaxClusters / 32 / NT;
  const int tid = threadIdx.x;
  uint32_t w[WPT], c = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    w[i] = tid * WPT + i < nwords ? sh.u.bits[tid * WPT + i] : 0u;
    c += __popc(w[i]);
  }
  uint32_t tot;
  uint32_t run = scan_excl<NT>(c, sh.tmp, &tot);
  if (run < need && run + c >= need) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      uint32_t x = w[i];
      while (x) {
        const int bit = __builtin_ctz(x);
        x &= x - 1u;
        if (++run == need) sh.tid = (tid * WPT + i) * 32 + bit;
      }
    }
  }
  __syncthreads();
  const int r = sh.tid;
  __syncthreads();
  return r;
}

// The need-th lowest id among the n listed clusters whose score equals v (need >= 1).
template <typename LK, typename LI>
__device__ int nth_id_with_score(LK tk, LI ti, uint32_t n, float v, uint32_t need,
                                 FinShared& sh) {
  for (int i = threadIdx.x; i < kMaxClusters / 32; i += kDecThreads) sh.u.bits[i] = 0u;
  __syncthreads();
  for (uint32_t k = threadIdx.x; k < n; k += kDecThreads)
    if (tk(k) == v) mark(sh, ti(k));
  __syncthreads();
  return nth_bit(sh, kMaxClusters / 32, need);
}

// (Tkey, Tid): the need-th pair (score descending, id ascending) among the n listed
// clusters of the cut bin (1 <= need < n). At most kCand of them are ranked exactly at once;
// more, and value-range histograms narrow the range until the bin holding the pair has at
// most kCand scores, which are then ranked exactly. tk(k), ti(k): the k-th listed score and
// id (global memory or LDS).
template <typename LK, typename LI>
__device__ void cut_pair(LK tk, LI ti, uint32_t n, uint32_t need, FinShared& sh, float& Tkey,
                         int& Tid) {
  constexpr int NT = kDecThreads, BPT = kNarrowBins / NT;
  const int tid = threadIdx.x;
  if (n <= (uint32_t)kCand) {
    if (tid < (int)n) {
      const float mv = tk(tid);
      const int mj = ti(tid);
      uint32_t rank = 0;
      for (uint32_t c = 0; c < n; ++c) {
        const float cv = tk(c);
        rank += (cv > mv || (cv == mv && ti(c) < mj)) ? 1u : 0u;
      }
      if (rank == need - 1) {
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
  Red3 r{kPosInf, kNegInf, 0u};
  for (uint32_t k = tid; k < n; k += NT) {
    const float v = tk(k);
    r.mn = fminf(r.mn, v);
    r.mx = fmaxf(r.mx, v);
  }
  r = block_red3<NT>(r, sh.red);
  float lo = r.mn, hi = r.mx;
  bool first = true;
  for (;;) {
    if (lo == hi) {  // every remaining score is lo
      Tkey = lo;
      Tid = nth_id_with_score(tk, ti, n, lo, need, sh);
      return;
    }
    const Binner b4k(lo, hi, first);
    first = false;
    auto bin = [&](float v) { return b4k(v) / (kHistBins / kNarrowBins); };
    for (int i = tid; i < kNarrowBins + kNarrowBins / 4; i += NT) sh.u.hist[i] = 0u;
    __syncthreads();
    for (uint32_t k0 = 0; k0 < n; k0 += NT) {
      const uint32_t k = k0 + tid;
      const float v = k < n ? tk(k) : kNegInf;
      const bool in = k < n && v >= lo && v <= hi;
      hist_add<10, kNarrowPad>(sh.u.hist, in ? bin(v) : 0, in);
    }
    __syncthreads();
    const int hb0 = kNarrowBins - BPT * (tid + 1);
    uint32_t hc[BPT], loc = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      hc[i] = sh.u.hist[padded<kNarrowPad>(hb0 + i)];
      loc += hc[i];
    }
    uint32_t tot;
    uint32_t run = scan_excl<NT>(loc, sh.tmp, &tot);
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (run < need && run + hc[i] >= need) {
        sh.v[0] = (uint32_t)(hb0 + i);
        sh.v[1] = run;
      }
      run += hc[i];
    }
    if (tid == 0) sh.v[2] = 0u;
    __syncthreads();
    const int bstar = (int)sh.v[0];
    const uint32_t need2 = need - sh.v[1], cnt = sh.u.hist[padded<kNarrowPad>(bstar)];
    if (cnt <= (uint32_t)kCand) {
      for (uint32_t k = tid; k < n; k += NT) {
        const float v = tk(k);
        if (v >= lo && v <= hi && bin(v) == bstar) {
          const uint32_t c = atomicAdd(&sh.v[2], 1u);
          sh.ck[c] = v;
          sh.ci[c] = ti(k);
        }
      }
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
    Red3 rb{kPosInf, kNegInf, 0u};
    for (uint32_t k = tid; k < n; k += NT) {
      const float v = tk(k);
      if (v >= lo && v <= hi && bin(v) == bstar) {
        rb.mn = fminf(rb.mn, v);
        rb.mx = fmaxf(rb.mx, v);
      }
    }
    rb = block_red3<NT>(rb, sh.red);
    lo = rb.mn;
    hi = rb.mx;
    need = need2;
  }
}

// Publish the selection marked in the bitmap sh.u.bits (bits of clusters [0, C)) of a (b,
// kv-head): the list in ascending id order (ids, first virtual row, first cache row),
// `selected`, the list length, and each retrieve workgroup's virtual rows and listed
// clusters. Every thread of the workgroup takes part.
__device__ __forceinline__ void publish_selection(const DecodeArgs& a, int bh, FinShared& sh) {
  constexpr int NT = kDecThreads, WPT = kMaxClusters / 32 / NT;
  const int tid = threadIdx.x;
  const size_t cb = (size_t)bh * a.C;
  const int nwords = (a.C + 31) / 32;
  int32_t* sid = a.sel_id + (size_t)bh * a.rcap;
  int32_t* sts = a.sel_ts + (size_t)bh * (a.rcap + 1);
  int32_t* sco = a.sel_coff + (size_t)bh * a.rcap;
  int32_t* selo = a.selected ? a.selected + (size_t)bh * a.n_retrieve : nullptr;
  int32_t* lst = sh.lst;
  constexpr uint32_t kListLds = kMaxClusters / 32;
  // ordered compaction of the bitmap into ranks: the ids go to LDS here, and to the
  // published list with the rest of each cluster's entry below, except where the list is
  // longer than the LDS copy (then all of it goes now). The selection counts make
  // nsel = need <= rcap.
  uint32_t nsel;
  bool long_list;
  auto put = [&](uint32_t r, int j) {
    if (r < nsel) {
      if (r < kListLds) lst[r] = j;
      if (long_list) sid[r] = j;
    }
  };
  if (nwords <= NT) {
    // one word per thread: an exclusive scan of the counts gives each word's first rank
    uint32_t x = tid < nwords ? sh.u.bits[tid] : 0u;
    uint32_t r = scan_excl<NT>(__popc(x), sh.tmp, &nsel);
    nsel = min(nsel, (uint32_t)a.rcap);
    long_list = nsel > kListLds;
    while (x) {
      put(r++, tid * 32 + __builtin_ctz(x));
      x &= x - 1u;
    }
  } else {
    // thread t counts words [t * WPT, (t + 1) * WPT); exclusive scans of the counts give
    // each word's first rank and each non-empty word's place in a compact list, and one
    // lane per listed word writes its ids at consecutive ranks
    uint32_t c = 0, nz = 0;
    uint32_t wcnt[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int w = tid * WPT + i;
      wcnt[i] = w < nwords ? __popc(sh.u.bits[w]) : 0u;
      c += wcnt[i];
      nz += wcnt[i] != 0u ? 1u : 0u;
    }
    uint32_t nnz;
    uint32_t k = scan_excl<NT>(c, sh.tmp, &nsel);
    uint32_t z = scan_excl<NT>(nz, sh.tmp, &nnz);
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      if (wcnt[i]) sh.u.nzw[z++] = (uint32_t)(tid * WPT + i) | (k << 11);
      k += wcnt[i];
    }
    nsel = min(nsel, (uint32_t)a.rcap);
    long_list = nsel > kListLds;
    __syncthreads();
    for (int q = tid; q < (int)nnz; q += NT) {
      const uint32_t e = sh.u.nzw[q];
      const int j0 = (int)(e & 2047u) * 32;
      uint32_t x = sh.u.bits[e & 2047u], r = e >> 11;
      while (x) {
        put(r++, j0 + __builtin_ctz(x));
        x &= x - 1u;
      }
    }
  }
  __syncthreads();
  // sizes and first rows: thread t takes ranks [t * per, (t + 1) * per), loads first
  auto listed = [&](uint32_t r) { return r < kListLds ? lst[r] : sid[r]; };
  constexpr int RB = 8;  // ranks per thread whose loads are issued together
  const uint32_t per = (nsel + NT - 1) / NT, r0 = tid * per, r1 = min(nsel, r0 + per);
  int32_t szb[RB], cob[RB], idb[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    szb[i] = cob[i] = idb[i] = 0;
    if (r0 + i < r1) {
      const int j = listed(r0 + i);
      idb[i] = j;
      szb[i] = a.csize[cb + j];
      cob[i] = a.coff[cb + j];
    }
  }
  uint32_t tok = 0;
#pragma unroll
  for (int i = 0; i < RB; ++i) tok += r0 + i < r1 ? (uint32_t)szb[i] + 1u : 0u;
  for (uint32_t r = r0 + RB; r < r1; ++r) tok += (uint32_t)a.csize[cb + listed(r)] + 1u;
  uint32_t V;
  uint32_t pos = scan_excl<NT>(tok, sh.tmp, &V);
  const int nB = a.nB;
  // retrieve workgroup wi takes virtual rows [wi span, (wi + 1) span) (clipped to V): whole
  // steps of its four waves
  constexpr uint32_t kStep = kRetBlock * (kDecThreads / 64);
  const uint32_t span = kStep * max(1u, (V + kStep * nB - 1) / (kStep * nB));
  auto emit = [&](uint32_t r, int j, int32_t n, int32_t co) {
    const uint32_t te = pos + (uint32_t)n + 1u;
    if (!long_list) sid[r] = j;
    if (selo) selo[r] = j;
    sts[r] = (int32_t)pos;
    sco[r] = co;
    // retrieve workgroups whose first virtual row falls in [pos, te)
    const int w0 = (int)((pos + span - 1) / span);
    const int w1 = (int)((te + span - 1) / span);
    for (int wi = w0; wi < w1; ++wi) sh.wgr[wi] = (int32_t)r;
    pos = te;
  };
#pragma unroll
  for (int i = 0; i < RB; ++i)
    if (r0 + i < r1) emit(r0 + i, idb[i], szb[i], cob[i]);
  for (uint32_t r = r0 + RB; r < r1; ++r) {
    const int j = listed(r);
    emit(r, j, a.csize[cb + j], a.coff[cb + j]);
  }
  if (selo)
    for (int i = (int)nsel + tid; i < a.n_retrieve; i += NT) selo[i] = -1;
  if (tid == 0) {
    a.sel_n[bh] = (int32_t)nsel;
    sts[nsel] = (int32_t)V;
  }
  __syncthreads();
  // per retrieve workgroup: its virtual rows [T0, T1) and listed clusters [r_lo, r_hi)
  for (int wi = tid; wi < nB; wi += NT) {
    const int T0 = (int)min((uint64_t)V, (uint64_t)span * wi);
    const int T1 = (int)min((uint64_t)V, (uint64_t)span * (wi + 1));
    int lo = 0, hi = 0;
    if (T0 < T1) {
      lo = sh.wgr[wi];
      hi = T1 < (int)V ? min((int)nsel, sh.wgr[wi + 1] + 1) : (int)nsel;
    }
    reinterpret_cast<int4*>(a.wg_info)[(size_t)bh * kMaxRetrieveWG + wi] = make_int4(T0, T1, lo, hi);
  }
}


// The last gather workgroup of a (b, kv-head): the exact cut among the clusters of the cut
// bin, the selection bitmap, and from it the published list in ascending id order (ids,
// first virtual row, first cache row), `selected`, and each retrieve workgroup's share.
__device__ __forceinline__ void finish_select(const DecodeArgs& a, int bh, uint32_t need, FinShared& sh) {
  constexpr int NT = kDecThreads;
  const int tid = threadIdx.x;
  const size_t cb = (size_t)bh * a.C;
  const uint32_t* ctr = a.counter + (size_t)bh * kCtrStride;
  const uint32_t nsure = min(ld_dev(ctr + kCtrSure), (uint32_t)a.rcap);
  const uint32_t ntie = min(ld_dev(ctr + kCtrTie), (uint32_t)a.C);
  const float* tk = a.tie_key + cb;
  const int32_t* ti = a.tie_id + cb;
  const int32_t* su = a.sure + (size_t)bh * a.rcap;
  float Tkey = kNegInf;  // default: every listed cluster of the cut bin
  int Tid = 0x7fffffff;
  // the lists in LDS when they fit (one round of loads for both), so that the ranking and
  // the marking below read them from there
  const bool staged = ntie <= (uint32_t)kTieLds && nsure <= (uint32_t)(kMaxClusters / 32);
  if (staged) {
    for (uint32_t k = tid; k < ntie; k += NT) {
      sh.tk[k] = ld_dev(tk + k);
      sh.ti[k] = ld_dev(ti + k);
    }
    for (uint32_t k = tid; k < nsure; k += NT) sh.lst[k] = ld_dev(su + k);
    __syncthreads();
    if (need > nsure && need - nsure < ntie)
      cut_pair([&](uint32_t k) { return sh.tk[k]; }, [&](uint32_t k) { return sh.ti[k]; }, ntie,
               need - nsure, sh, Tkey, Tid);
  } else if (need > nsure && need - nsure < ntie) {
    cut_pair([&](uint32_t k) { return ld_dev(tk + k); }, [&](uint32_t k) { return ld_dev(ti + k); },
             ntie, need - nsure, sh, Tkey, Tid);
  }
  for (int i = tid; i < (a.C + 31) / 32; i += NT) sh.u.bits[i] = 0u;
  __syncthreads();
  if (need > 0) {
    if (staged) {
      for (uint32_t k = tid; k < nsure; k += NT) mark(sh, sh.lst[k]);
      for (uint32_t k = tid; k < ntie; k += NT)
        if (is_selected(sh.tk[k], sh.ti[k], Tkey, Tid)) mark(sh, sh.ti[k]);
    } else {
      for (uint32_t k = tid; k < nsure; k += NT) mark(sh, ld_dev(su + k));
      for (uint32_t k = tid; k < ntie; k += NT) {
        const int j = ld_dev(ti + k);
        if (is_selected(ld_dev(tk + k), j, Tkey, Tid)) mark(sh, j);
      }
    }
  }
  __syncthreads();
  publish_selection(a, bh, sh);
}

// ------------------------------------------------------------------------------------
// selection of a (b, kv-head) of at most kLocalSelectMax clusters by one workgroup, from
// registers: thread t holds the group scores of clusters 4i .. 4i + 3 for i = k * NT + t
// ------------------------------------------------------------------------------------
constexpr int kLocalV = kLocalSelectMax / 4 / kDecThreads;  // float4 of scores per thread

// f(score, cluster id) for every register score of the first nk float4
template <typename F>
__device__ __forceinline__ void for_local(const float4 (&v)[kLocalV], int nk, F f) {
#pragma unroll
  for (int k = 0; k < kLocalV; ++k) {  // (a guard, not an early exit: the loop unrolls)
    if (k < nk) {
      const int j = 4 * (k * kDecThreads + (int)threadIdx.x);
      // (opaque copies: each pass recomputes what it derives from a score, rather than
      // the compiler keeping one pass's values live into the next)
      float x0 = v[k].x, x1 = v[k].y, x2 = v[k].z, x3 = v[k].w;
      asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
      f(x0, j);
      f(x1, j + 1);
      f(x2, j + 2);
      f(x3, j + 3);
    }
  }
}

// OR over each aligned group of 8 lanes (every lane of the group gets it): two quad
// permutations make each quad uniform, then the half-row mirror pairs the two quads.
__device__ __forceinline__ uint32_t or8_lanes(uint32_t w) {
  auto mv = [](uint32_t v, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  w |= mv(w, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  w |= mv(w, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  w |= mv(w, std::integral_constant<int, 0x141>{});  // row_half_mirror
  return w;
}

// sh.u.bits words [0, nk * NT / 8), whole: bit j set where pick(score, j). A thread's four
// clusters are one nibble of a word, so eight lanes OR their nibbles into one word.
template <typename Pick>
__device__ __forceinline__ void local_bitmap(const float4 (&v)[kLocalV], int nk, FinShared& sh,
                                             Pick pick) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kLocalV; ++k) {
    if (k < nk) {
      const int i = k * kDecThreads + tid;
      float x0 = v[k].x, x1 = v[k].y, x2 = v[k].z, x3 = v[k].w;
      asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
      const uint32_t nib = (pick(x0, 4 * i) ? 1u : 0u) | (pick(x1, 4 * i + 1) ? 2u : 0u) |
                           (pick(x2, 4 * i + 2) ? 4u : 0u) | (pick(x3, 4 * i + 3) ? 8u : 0u);
      const uint32_t w = or8_lanes(nib << (4 * (tid & 7)));
      if ((tid & 7) == 0) sh.u.bits[i >> 3] = w;
    }
  }
}

// The bin of sh.v[0] holding the need-th largest of the counts hist[0, NBINS) visited from
// the top, and in sh.v[1] the count above it, with need = min(want, the total) (returned;
// nothing is written when it is 0). Ends on a barrier.
template <int NBINS, int PAD>
__device__ __forceinline__ uint32_t cut_bin(const uint32_t* hist, uint32_t want, FinShared& sh) {
  constexpr int NT = kDecThreads, BPT = NBINS / NT;
  static_assert(BPT == 1 << PAD, "one padding word per thread's run of bins");
  const int tid = threadIdx.x;
  const int hb0 = NBINS - BPT * (tid + 1);  // thread t's bins, visited from the top
  uint32_t hc[BPT], loc = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    hc[i] = hist[padded<PAD>(hb0 + i)];
    loc += hc[i];
  }
  uint32_t tot;
  uint32_t run = scan_excl<NT>(loc, sh.tmp, &tot);
  const uint32_t need = min(want, tot);
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (run < need && run + hc[i] >= need) {
      sh.v[0] = (uint32_t)(hb0 + i);
      sh.v[1] = run;
    }
    run += hc[i];
  }
  __syncthreads();
  return need;
}

// (Tkey, Tid): the need-th pair (score descending, id ascending) among the register scores
// in [lo, hi] (1 <= need < their count), narrowed as cut_pair narrows a listed cut bin.
__device__ __forceinline__ void cut_pair_local(const float4 (&v)[kLocalV], int nk, int nwords, float lo,
                               float hi, uint32_t need, FinShared& sh, float& Tkey, int& Tid) {
  const int tid = threadIdx.x;
  bool first = true;
  for (;;) {
    if (lo == hi) {  // every remaining score is lo
      Tkey = lo;
      local_bitmap(v, nk, sh, [&](float x, int) { return x == lo; });
      __syncthreads();
      Tid = nth_bit(sh, nwords, need);
      return;
    }
    const Binner b4k(lo, hi, first);
    first = false;
    auto bin = [&](float x) { return b4k(x) / (kHistBins / kNarrowBins); };
    for (int i = tid; i < kNarrowBins + kNarrowBins / 4; i += kDecThreads) sh.u.hist[i] = 0u;
    if (tid == 0) sh.v[2] = 0u;
    __syncthreads();
    for_local(v, nk, [&](float x, int) {
      if (x >= lo && x <= hi) atomicAdd(&sh.u.hist[padded<kNarrowPad>(bin(x))], 1u);
    });
    __syncthreads();
    cut_bin<kNarrowBins, kNarrowPad>(sh.u.hist, need, sh);
    const int bstar = (int)sh.v[0];
    const uint32_t need2 = need - sh.v[1], cnt = sh.u.hist[padded<kNarrowPad>(bstar)];
    if (cnt <= (uint32_t)kCand) {
      for_local(v, nk, [&](float x, int j) {
        if (x >= lo && x <= hi && bin(x) == bstar) {
          const uint32_t c = atomicAdd(&sh.v[2], 1u);
          sh.ck[c] = x;
          sh.ci[c] = j;
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
    Red3 rb{kPosInf, kNegInf, 0u};
    for_local(v, nk, [&](float x, int) {
      const bool in = x >= lo && x <= hi && bin(x) == bstar;
      rb.mn = in ? fminf(rb.mn, x) : rb.mn;
      rb.mx = in ? fmaxf(rb.mx, x) : rb.mx;
    });
    rb = block_red3<kDecThreads>(rb, sh.red);
    lo = rb.mn;
    hi = rb.mx;
    need = need2;
  }
}

// The selection of a (b, kv-head) of at most kLocalSelectMax clusters, whole, in one
// workgroup: the head's scores are loaded once into registers; a value-range histogram
// over their [min, max] gives the cut bin b* (the bin of the need-th largest score) and the
// count above it, then the need2-th pair (Tkey, Tid) of b* in (score descending, id
// ascending) order: an exact rank when b* holds at most kCand scores, else narrowing
// histograms over the same registers. Since the bins are monotone in the score, the
// selection is then { j : s_j > Tkey or (s_j == Tkey and j <= Tid) }; the bitmap goes from the
// registers to LDS and is published as the other selection path publishes it.
__device__ __forceinline__ void select_local(const DecodeArgs& a, int bh, FinShared& sh) {
  constexpr int NT = kDecThreads;
  const int tid = threadIdx.x;
  const int n4 = a.Cp / 4, nk = (n4 + NT - 1) / NT, nwords = (a.C + 31) / 32;
  const float4* sh4 = reinterpret_cast<const float4*>(a.shat + (size_t)bh * a.Cp);
  float4 v[kLocalV];
#pragma unroll
  for (int k = 0; k < kLocalV; ++k) {  // (clamped, unconditional loads: issued together)
    const int i = k * NT + tid;
    v[k] = sh4[min(i, n4 - 1)];
    if (i >= n4) v[k] = neg4();
  }
  {
    uint4* z = reinterpret_cast<uint4*>(sh.u.full);
    constexpr int NZ = (kHistBins + 1 + kHistBins / 16 + 1 + 3) / 4;
    for (int i = tid; i < NZ; i += NT) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) sh.v[2] = 0u;
  // the head's finite score range from the score workgroups' (min, max) pairs, read while
  // the scores are in flight (its barriers also end the clearing above)
  const Red3 r = score_range(a, bh, sh.red);
  float Tkey = kPosInf;  // nothing selected (no finite score, or n_r = 0)
  int Tid = 0;
  uint32_t need = 0;
  if (r.mx != kNegInf && a.n_retrieve > 0) {
    // bins (-inf, i.e. empty and padding clusters, to the spare bin), kept two per register
    const Binner bn(r.mn, r.mx, true);
    uint32_t bins[2 * kLocalV];
    auto bin_pass = [&](auto binf) {
#pragma unroll
      for (int k = 0; k < kLocalV; ++k) {
        bins[2 * k] = bins[2 * k + 1] = 0u;
        if (k < nk) {
          float x4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
          asm volatile("" : "+v"(x4[0]), "+v"(x4[1]), "+v"(x4[2]), "+v"(x4[3]));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int b = x4[e] != kNegInf ? binf(x4[e]) : kHistBins;
            atomicAdd(&sh.u.full[padded<kFullPad>(b)], 1u);
            bins[2 * k + (e >> 1)] |= (uint32_t)b << (16 * (e & 1));
          }
        }
      }
    };
    if (bn.by_value) {  // (the mode is the same for the whole head)
      bin_pass([&](float x) {
        const float t = (x - bn.lo) * bn.inv;
        return t >= (float)(kHistBins - 1) ? kHistBins - 1 : (int)t;
      });
    } else {
      bin_pass([&](float x) { return bn(x); });
    }
    auto bin_of = [&](int k, int e) { return (int)((bins[2 * k + (e >> 1)] >> (16 * (e & 1))) & 0xffffu); };
    __syncthreads();
    need = cut_bin<kHistBins, kFullPad>(sh.u.full, (uint32_t)a.n_retrieve, sh);
    const int bstar = (int)sh.v[0];
    const uint32_t need2 = need - sh.v[1], cnt = sh.u.full[padded<kFullPad>(bstar)];
    if (cnt <= (uint32_t)kCand) {
      // rank the scores of b* exactly (need2 = cnt gives its last pair: all of b* is taken);
      // a mask of this thread's scores in b* first, then one LDS slot per set bit
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < kLocalV; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          m |= ((k < nk) & (bin_of(k, e) == bstar)) ? 1u << (4 * k + e) : 0u;
      while (m) {
        const int q = __builtin_ctz(m);
        m &= m - 1u;
        const uint32_t c = atomicAdd(&sh.v[2], 1u);
        float x = 0.f;  // (picked by selects: registers are not indexed dynamically)
#pragma unroll
        for (int k = 0; k < kLocalV; ++k) {
          x = (q >> 2) == k ? ((q & 3) == 0 ? v[k].x : (q & 3) == 1 ? v[k].y
                                : (q & 3) == 2 ? v[k].z : v[k].w) : x;
        }
        sh.ck[c] = x;
        sh.ci[c] = 4 * ((q >> 2) * NT + tid) + (q & 3);
      }
      __syncthreads();
      if (tid < (int)cnt) {
        const float mv = sh.ck[tid];
        const int mj = sh.ci[tid];
        uint32_t rank = 0;
        for (uint32_t c = 0; c < cnt; ++c) {
          const float cv = sh.ck[c];
          const int cj = sh.ci[c];
          rank += ((cv > mv) | ((cv == mv) & (cj < mj))) ? 1u : 0u;
        }
        if (rank == need2 - 1) {
          sh.tkey = mv;
          sh.tid = mj;
        }
      }
      __syncthreads();
      Tkey = sh.tkey;
      Tid = sh.tid;
    } else {
      Red3 rb{kPosInf, kNegInf, 0u};
#pragma unroll
      for (int k = 0; k < kLocalV; ++k) {
        if (k < nk) {
          const float x4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = bin_of(k, e) == bstar;
            rb.mn = in ? fminf(rb.mn, x4[e]) : rb.mn;
            rb.mx = in ? fmaxf(rb.mx, x4[e]) : rb.mx;
          }
        }
      }
      rb = block_red3<NT>(rb, sh.red);
      if (need2 == cnt) {  // all of b*
        Tkey = rb.mn;
        Tid = 0x7fffffff;
      } else {
        cut_pair_local(v, nk, nwords, rb.mn, rb.mx, need2, sh, Tkey, Tid);
      }
    }
  }
  __syncthreads();
  // (the comparisons combined bitwise, here and in the exact rank above: a short-circuit form
  // compiles to exec-mask branches per score)
  local_bitmap(v, nk, sh, [&](float x, int j) { return (x > Tkey) | ((x == Tkey) & (j <= Tid)); });
  __syncthreads();
  publish_selection(a, bh, sh);
}

// Two weights c0, c1 as one bf16 pair of an A operand row: the bf16 parts (round to nearest
// even, one v_cvt_pk_bf16_f32) in rows n < G, the remainders c - bf16(c) in rows G <= n < 2G
// (so that the two rows' fp32 sum carries c to about 2^-17 relative), zero beyond.
template <int G>
__device__ __forceinline__ uint32_t hi_lo_bf16(float c0, float c1, int n) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const uint32_t hi = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)c0, (__bf16)c1});
  const float r0 = c0 - __uint_as_float(hi << 16), r1 = c1 - __uint_as_float(hi & 0xffff0000u);
  const uint32_t lo = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)r0, (__bf16)r1});
  return n < G ? hi : (n < 2 * G ? lo : 0u);
}

constexpr float kLazyMax = 8.f;  // log2 headroom of a retrieve wave's running maximum

// ------------------------------------------------------------------------------------
// estimate: every non-empty cluster's centroid term, on the matrix cores
// ------------------------------------------------------------------------------------
// A workgroup folds kEstChunks chunks of 128 clusters of one (b, kv-head) into one partial
// state; wave w takes clusters 32 w .. 32 w + 31 of each chunk, one K step of
// v_mfma_f32_16x16x32_bf16 per 16 output dims. The product is O[r][dim] = sum_j P[r][j]
// V[j][dim] over the value sums V (exact in bf16): row r < G holds bf16(p) of head r's weight
// p = 2^(s_j - m) (s_j the head's log2-domain logit, m the wave's largest), row G + r holds
// bf16(p - bf16(p)), so that their fp32 sum carries p to about 2^-17 relative; rows from 2G
// are zero. The denominator sum_j n_j p is summed in fp32 from the unrounded p. Lane l holds
// the A operand of row l % 16 and the B operand of dim l % 16, both for the clusters
// 8 (l / 16) .. + 7 of its K step. The value-sum rows reach LDS by direct global-to-LDS
// loads in the layout of the retrieve's value rows (block e of a wave holds the wave's
// clusters 8 g + e in slot g, each row rotated by 2 g 16-byte chunks, blocks 1152 bytes
// apart) and come back as B operands through transposing reads (ds_read_tr16_b64).
struct EstLds {
  // [chunk][wave][e][slot][256 B] with blocks e 1152 bytes apart (as the retrieve's value rows)
  uint32_t rows[kEstChunks][kDecThreads / 64][8][288];
};
struct EstMerge {  // the same LDS after the products: each wave's rows and (m, l) per head
  float o[kDecThreads / 64][2 * kMaxGroup][kHeadDim];
  float m[kDecThreads / 64][kMaxGroup], l[kDecThreads / 64][kMaxGroup];
};

template <int G>
__device__ __forceinline__ void estimate_mfma(const DecodeArgs& a, int bh, int e, EstLds& st,
                                              float* __restrict__ dst) {
  static_assert(2 * G <= 16, "hi and lo rows of every head in one 16-row tile");
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  const size_t base = (size_t)bh * a.C;
  const bool arow = n < 2 * G;
  const int hrow = n < G ? n : (arow ? n - G : 0);  // the head of this lane's A row
  // logits and sizes of this lane's clusters (issued first: they are needed first)
  float sv[kEstChunks][8];
  float nv[kEstChunks][8];
#pragma unroll
  for (int c = 0; c < kEstChunks; ++c) {
    const int j0 = (e * kEstChunks + c) * kChunk + 32 * w + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      const int jc = min(j, a.C - 1);
      const float s = a.scores[(base + jc) * G + hrow];
      const int32_t cnt = a.csize[base + jc];
      const bool ok = arow && j < a.C && cnt > 0;
      sv[c][i] = ok ? s : kNegInf;
      nv[c][i] = ok ? (float)cnt : 0.f;
    }
  }
  // the value-sum rows of the wave's clusters: one direct load of four rows per block
  {
    const int slot = lane >> 4, pos = lane & 15, cidx = (pos - 2 * slot) & 15;
#pragma unroll
    for (int c = 0; c < kEstChunks; ++c) {
#pragma unroll
      for (int ei = 0; ei < 8; ++ei) {
        const int j = (e * kEstChunks + c) * kChunk + 32 * w + 8 * slot + ei;
        const size_t row = base + min(j, a.C - 1);
        __builtin_amdgcn_global_load_lds(a.vsum + row * kHeadDim + cidx * 8,
                                         (lds_ptr)&st.rows[c][w][ei][0], 16, 0, 0);
      }
    }
  }
  // the wave's largest logit per head (lanes of rows h and G + h hold the same)
  float mx = kNegInf;
#pragma unroll
  for (int c = 0; c < kEstChunks; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, sv[c][i]);
  mx = fmaxf(mx, xor16(mx));
  mx = fmaxf(mx, xor32(mx));
  // A operands (hi or lo part of p) and the denominator
  bf16x8 pa[kEstChunks];
  float lsum = 0.f;
#pragma unroll
  for (int c = 0; c < kEstChunks; ++c) {
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float pr[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float s = sv[c][i + u];
        pr[u] = s == kNegInf ? 0.f : fast_exp2(s - mx);
        lsum += nv[c][i + u] * pr[u];
      }
      pk[i >> 1] = hi_lo_bf16<G>(pr[0], pr[1], n);
    }
    pa[c] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
  }
  lsum += xor16(lsum);
  lsum += xor32(lsum);
  typedef __attribute__((ext_vector_type(4))) float floatx4;
  floatx4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  drain_vmem();  // (the direct loads have landed in LDS once the wave's loads completed)
  __syncthreads();
  typedef __attribute__((ext_vector_type(4))) short shortx4;
#pragma unroll
  for (int c = 0; c < kEstChunks; ++c) {
    const char* vb = reinterpret_cast<const char*>(&st.rows[c][w][0][0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // two transposing reads: rows 8 g + 4 hf .. + 3 of dim 16 t + n (see the retrieve)
      shortx4 bh2[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int eb = 4 * hf + (n >> 2);
        const int ch = 2 * t + ((n & 3) >> 1);
        const int off = eb * 1152 + g * 256 + (((ch + 2 * g) & 15) << 4) + ((n & 1) << 3);
        bh2[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(vb + off));
      }
      const u32x4 bw = {(uint32_t)(uint16_t)bh2[0][0] | ((uint32_t)(uint16_t)bh2[0][1] << 16),
                        (uint32_t)(uint16_t)bh2[0][2] | ((uint32_t)(uint16_t)bh2[0][3] << 16),
                        (uint32_t)(uint16_t)bh2[1][0] | ((uint32_t)(uint16_t)bh2[1][1] << 16),
                        (uint32_t)(uint16_t)bh2[1][2] | ((uint32_t)(uint16_t)bh2[1][3] << 16)};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[c], __builtin_bit_cast(bf16x8, bw),
                                                       acc[t], 0, 0, 0);
    }
  }
  __syncthreads();  // (the merge below reuses the staging LDS)
  EstMerge& mg = *reinterpret_cast<EstMerge*>(&st);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      if (r < 2 * G) mg.o[w][r][16 * t + n] = acc[t][i];
    }
  if (g == 0 && n < G) {
    mg.m[w][n] = mx;
    mg.l[w][n] = lsum;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += kDecThreads) {
    const int h = idx >> 7, d = idx & 127;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kDecThreads / 64; ++ww) M = fmaxf(M, mg.m[ww][h]);
    float o = 0.f, l = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kDecThreads / 64; ++ww) {
        const float f = fast_exp2(mg.m[ww][h] - M);
        o += f * (mg.o[ww][h][d] + mg.o[ww][G + h][d]);
        l += f * mg.l[ww][h];
      }
    }
    dst[h * kPartStride + d] = o;
    if (d == 0) {
      dst[h * kPartStride + 128] = M;
      dst[h * kPartStride + 129] = l;
    }
  }
}

// One-dimensional grid, by role (so the selection workgroups of every (b, kv-head) are
// dispatched first): nH per (b, kv-head) select (one for heads of at most kLocalSelectMax
// clusters, which selects and publishes alone; else one per kSelSpan scores, listing the
// clusters above and in the cut bin, the last of them ranking the cut bin and publishing);
// then nSt per (b, kv-head) attend exactly to 128 steady tokens each, into partial slot
// nEW + s; then nEW = nS per (b, kv-head) fold the centroid estimate of a chunk of 128
// clusters each (weight n_j, logit s_j, value sum V_j) into partial slot e. The value-sum
// stream of the estimate does not depend on the selection and runs beside it. HIST: the
// selection of heads of more than kLocalSelectMax clusters (after the histogram kernel);
// each instance holds only its own selection path, so that neither path's code (and its
// placement) depends on the other's.
template <int G, bool HIST>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 1))) void k_dec_gather(DecodeArgs a) {
  const int BH = a.B * a.Hkv, tid = threadIdx.x;
  // (roles use different workgroups: one LDS block serves the selection, an estimate
  // workgroup's staged chunk and the partial exchange of the estimate and steady roles)
  __shared__ union {
    FinShared f;
    EstLds est;
    float sm[kDecThreads / 64][G][kPartStride];
  } lds;
  const int lane = tid & 63, wave = tid >> 6, cc = lane & 15;
  // (roles in dispatch order: selection, steady, estimate; x below numbers a head's
  // workgroups as selection [0, nH), estimate [nH, nH + nEW), steady after those)
  int x = blockIdx.x, bh;
  if (x < a.nH * BH) {
    bh = x / a.nH;
    x -= bh * a.nH;
  } else if (x < (a.nH + a.nSt) * BH) {
    x -= a.nH * BH;
    bh = x / a.nSt;
    x = a.nH + a.nEW + (x - bh * a.nSt);
  } else {
    x -= (a.nH + a.nSt) * BH;
    bh = x / a.nEW;
    x = a.nH + (x - bh * a.nEW);
  }
  if (x >= a.nH) {
    const int b = bh / a.Hkv, g = bh % a.Hkv;
    if (x < a.nH + a.nEW) {
      const int e = x - a.nH;
      estimate_mfma<G>(a, bh, e, lds.est, a.part + ((size_t)bh * a.nP + e) * G * kPartStride);
      return;
    }
    Online<G> st;
    st.init();
    int slot;
    {
      // ---- steady: 128 tokens
      const int s = x - a.nH - a.nEW;
      u32x4 q[G];
      load_q<G>(a, b, g, cc, q);
      const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
      const int64_t wbeg = (int64_t)s * kTokChunk + wave * (kTokChunk / 4);
      const int64_t wend = min(n_steady, wbeg + kTokChunk / 4);
      if (a.tier)  // (the steady zone's own buffer holds its rows in order)
        attend_rows<G>(a, a.sk, a.sv, (size_t)bh * a.Ls, q, st, wbeg, wend,
                       [](int64_t t) { return t; });
      else
        attend_rows<G>(a, a.k, a.v, (size_t)bh * a.Lcap, q, st, wbeg, wend,
                       [&](int64_t t) { return steady_row(a, t); });
      slot = a.nEW + s;
    }
    write_block_partial_in<G, false>(st, nullptr,
                                     a.part + ((size_t)bh * a.nP + slot) * G * kPartStride,
                                     lds.sm);
    return;
  }
  // the selection is the latency-critical chain of the call: its waves issue ahead of the
  // estimate and steady waves that share their SIMDs
  __builtin_amdgcn_s_setprio(3);
  FinShared& sh = lds.f;
  if constexpr (!HIST) {
    select_local(a, bh, sh);
    return;
  }
  // (this workgroup's scores are loaded before the cut is found: their round trip
  // overlaps the cut's)
  constexpr int E = kSelSpan / kDecThreads;  // scores per thread
  const float* shv = a.shat + (size_t)bh * a.Cp;
  float v[E];
#pragma unroll
  for (int k = 0; k < E / 4; ++k) {
    const int j4 = x * kSelSpan + k * 4 * kDecThreads + 4 * tid;
    const float4 v4 = j4 < a.Cp ? *reinterpret_cast<const float4*>(shv + j4) : neg4();
    v[4 * k] = v4.x;
    v[4 * k + 1] = v4.y;
    v[4 * k + 2] = v4.z;
    v[4 * k + 3] = v4.w;
  }
  const Cut cut = find_cut(a, bh, sh);
  uint32_t* ctr = a.counter + (size_t)bh * kCtrStride;
  if (cut.need > 0) {
    const Binner bn(cut.lo, cut.hi, true);
    int bv[E];
    uint32_t ns = 0, nt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      bv[e] = v[e] != kNegInf ? bn(v[e]) : -1;
      ns += bv[e] > cut.bstar ? 1u : 0u;
      nt += bv[e] == cut.bstar ? 1u : 0u;
    }
    // one reservation per workgroup and list
    uint32_t tns, tnt;
    uint32_t ps = scan_excl<kDecThreads>(ns, sh.tmp, &tns);
    uint32_t pt = scan_excl<kDecThreads>(nt, sh.tmp, &tnt);
    if (tid == 0) {
      sh.base[0] = tns ? atomicAdd(ctr + kCtrSure, tns) : 0u;
      sh.base[1] = tnt ? atomicAdd(ctr + kCtrTie, tnt) : 0u;
    }
    __syncthreads();
    ps += sh.base[0];
    pt += sh.base[1];
    int32_t* su = a.sure + (size_t)bh * a.rcap;
    float* tk = a.tie_key + (size_t)bh * a.C;
    int32_t* ti = a.tie_id + (size_t)bh * a.C;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = x * kSelSpan + (e >> 2) * 4 * kDecThreads + 4 * tid + (e & 3);
      if (bv[e] > cut.bstar) {
        if (ps < (uint32_t)a.rcap) st_dev(su + ps, (int32_t)j);
        ++ps;
      } else if (bv[e] == cut.bstar) {
        if (pt < (uint32_t)a.C) {
          st_dev(tk + pt, v[e]);
          st_dev(ti + pt, (int32_t)j);
        }
        ++pt;
      }
    }
  }
  if (arrive_last(ctr + kCtrGather, (uint32_t)a.nH)) finish_select(a, bh, cut.need, sh);
}

// ------------------------------------------------------------------------------------
// kernel 4: retrieve
// ------------------------------------------------------------------------------------

// LDS of one retrieve wave: the value rows of its block of 32 virtual rows, staged for the
// transposing operand reads, the block's logits and its row descriptors.
//   vrows: block e (of 8) holds rows 8 s + e in slot s (s = 0..3), each row rotated by 2 s
//   16-byte chunks; blocks 1152 bytes apart. A ds_read_tr16_b64 of lane (g, L) reads 8 bytes
//   of row 8 g + 4 hf + (L >> 2) and returns that lane's column of four rows, so that two
//   reads give the B operand (8 rows of one dim); the rotation and the block spacing spread
//   the 64 lanes' reads over all LDS banks (each bank twice).
constexpr int kVBlockWords = 288;      // 1024 bytes of rows + 128 bytes of spacing
template <int G>
struct RetWave {
  uint32_t vrows[8][kVBlockWords];
};
template <int G>
struct RetMerge {  // the same LDS after the attend: each wave's rows and (m, l) per head
  float o[kDecThreads / 64][2 * G][kHeadDim];
  float m[kDecThreads / 64][G], l[kDecThreads / 64][G];
};
template <int G>
union RetLds {
  RetWave<G> w[kDecThreads / 64];
  RetMerge<G> mg;
  float xh[128][6];                    // the final merges' exchange (merge_block)
};

// Running softmax state of a wave on the matrix cores: acc[t] holds D rows 4 (lane / 16) + i
// of output dims 16 t + lane % 16, where row r < G is the bf16 part of head r's weights and
// row G + r the remainder; m (log2 units) and l (this lane's rows only) belong to the head
// of the lane's A row (lane % 16 < 2G).
struct MfmaState {
  typedef __attribute__((ext_vector_type(4))) float floatx4;
  floatx4 acc[8];
  float m, l;
};

// Descriptors of the virtual rows [c0, c0 + n) (n <= kDecThreads) of the listed clusters in
// LDS (first virtual row l_ts[] with l_ts[cnt] = end, first cache row l_co[], cluster id
// l_id[]), one row per thread: src = the cache row of a token row, or -1 - j for the removal
// row of cluster j (its centroid key and value sum); wgt = the row's denominator weight (1 for
// a token, -n_j for a removal row). Rows from n on are padding: src -1, wgt 0 (cluster 0's
// removal row, which the build always writes: the padding's zero weights meet finite values in
// the products, never an unwritten cache slot whose contents could be NaN).
//
// TIER (the cache in host memory): a token row is read from its block's slot when the slot
// holds the block, is pinned for this step and has the row (src = slot * kTierBlock + row %
// kTierBlock); else from host memory (src = kHostRow | row), and when the block has a slot
// (pinned, or claimed in this step), the row read over the bus is also written into it (dst =
// slot * 2 kTierBlock + row % kTierBlock, the K row; -1: not written). A slot word holds the
// owner block (low half) and 2 step + claimed (high half): pinning moves a slot of the block
// to this step by compare-and-swap, and a claim takes a slot that nothing of this step pinned
// or claimed, so no slot changes hands while a step reads it. The first row of each run of
// rows of one block pins or claims for the run (t_blk, t_res in LDS), the other rows use its
// result. Rows written in a step are read from the next step on (each row is retrieved once
// a step); a slot claimed in this step is not read at all in it. Returns 1 for a row read
// from a slot, 2 from host memory, 3 from host memory and written into a slot, else 0.
constexpr int32_t kHostRow = 1 << 30;

// Pin slot e for block id in this step: 1 if the slot holds the block and was not claimed in
// this step (it is then stamped with the step: readable and writable), 2 if it was claimed in
// this step for the block (writable only), 0 if it holds another block.
__device__ __forceinline__ int tier_pin(const DecodeArgs& a, int e, int32_t id, uint32_t step) {
  const uint64_t mine = ((uint64_t)(2u * step) << 32) | (uint32_t)id;
  uint64_t w = ld_dev(a.slotw + e);
  for (int tries = 0; tries < 4; ++tries) {
    if ((uint32_t)w != (uint32_t)id) return 0;                // another block holds it now
    const uint32_t hs = (uint32_t)(w >> 32);
    if (hs == 2u * step + 1u) return 2;                       // claimed in this step
    if (hs == 2u * step) return 1;                            // pinned in this step already
    const uint64_t old = atomicCAS(reinterpret_cast<unsigned long long*>(a.slotw + e),
                                   (unsigned long long)w, (unsigned long long)mine);
    if (old == w) return 1;
    w = old;
  }
  return 0;
}

// Claim a slot for block id in this step (the table entry is -2, held by this thread): the
// next slot in the hand's order that nothing of this step pinned or claimed; the hand goes
// round at most once per step. The old block leaves the table, the slot holds no row yet, and
// the table points to the slot. Returns the slot, or -1 (the table entry goes back to -1).
__device__ __forceinline__ int tier_claim(const DecodeArgs& a, int32_t id, uint32_t step) {
  const uint32_t h0 = ld_dev(a.tctr + kTcHandStart);
  const int32_t nid = a.B * a.Hkv * a.nblk;
  const uint64_t want = ((uint64_t)(2u * step + 1u) << 32) | (uint32_t)id;
  for (;;) {
    const uint32_t h = atomicAdd(a.tctr + kTcHand, 1u);
    if (h - h0 >= (uint32_t)a.nslots) break;                  // the revolution is over
    const int s = (int)(h % (uint32_t)a.nslots);
    const uint64_t w = ld_dev(a.slotw + s);
    if ((uint32_t)(w >> 32) >= 2u * step) continue;          // pinned or claimed this step
    if (atomicCAS(reinterpret_cast<unsigned long long*>(a.slotw + s), (unsigned long long)w,
                  (unsigned long long)want) != w)
      continue;
    const int32_t prev = (int32_t)(uint32_t)w;
    if (prev >= 0 && prev < nid) atomicCAS(a.tab + prev, s, -1);
    // (a row of the block that another workgroup marks in the mask before this reset is
    // written but not marked: it is only not reused)
    atomicExch(a.valid + s, 0u);
    atomicExch(a.tab + id, s);
    atomicAdd(a.tctr + kTcAdmitted, 1u);
    return s;
  }
  atomicExch(a.tab + id, -1);
  atomicAdd(a.tctr + kTcRefused, 1u);
  return -1;
}

template <bool TIER>
__device__ __forceinline__ int describe_rows(const DecodeArgs& a, int bh, int c0, int n,
                                             const int32_t* l_ts, const int32_t* l_co,
                                             const int32_t* l_id, int cnt, int32_t* d_src,
                                             float* d_wgt, int32_t* d_dst, int32_t* t_blk,
                                             int32_t* t_res) {
  const int tid = threadIdx.x, t = c0 + tid;
  int32_t src = -1, dst = -1;
  float wgt = 0.f;
  int cls = 0;
  bool token = false;
  if (tid < n) {
    int lo = 0, hi = cnt - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (l_ts[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int off = t - l_ts[lo], nj = l_ts[lo + 1] - l_ts[lo] - 1;
    if (off < nj) {
      src = l_co[lo] + off;
      wgt = 1.f;
      token = true;
    } else {
      src = -1 - l_id[lo];
      wgt = -(float)nj;
    }
  }
  if constexpr (TIER) {
    // the rows of one block are consecutive among the token rows (clusters are contiguous
    // runs of the cache, listed in ascending order; one removal row follows each cluster)
    const int32_t id = token ? bh * a.nblk + src / kTierBlock : -1;
    t_blk[tid] = id;
    t_res[tid] = INT32_MIN;   // (not the first row of a run; a run's first row overwrites it)
    __syncthreads();
    int j = tid - 1;
    if (j >= 0 && t_blk[j] < 0) --j;
    const bool lead = token && (j < 0 || t_blk[j] != id);
    const uint32_t step = ld_dev(a.tctr + kTcStep);
    if (lead) {   // slot and state for the run: (slot << 2) | 1 readable, 2 claimed here, 0 none
      int32_t e = ld_dev(a.tab + id);
      if (e >= a.nslots) e = -3;  // (never set by a claim: a state not reset; not cached)
      int32_t res = 0;
      if (e >= 0) {
        const int pin = tier_pin(a, e, id, step);
        if (pin != 0) res = (e << 2) | pin;
      } else if (e == -1 && atomicCAS(a.tab + id, -1, -2) == -1) {
        const int sl = tier_claim(a, id, step);
        if (sl >= 0) res = (sl << 2) | 2;
      }
      t_res[tid] = res;
    }
    __syncthreads();
    if (token) {
      // the run's first row: the nearest row at or before this one that carries a result
      // (between them lie only rows of this block and removal rows)
      int k = tid;
      while (t_res[k] == INT32_MIN) --k;
      const int32_t res = t_res[k];
      const int e = res >> 2, pin = res & 3, r = src % kTierBlock;
      const uint32_t bit = 1u << r;
      if (pin == 1 && (ld_dev(a.valid + e) & bit)) {
        src = e * kTierBlock + r;
        cls = 1;
      } else {
        if (pin != 0) {
          atomicOr(a.valid + e, bit);
          dst = e * 2 * kTierBlock + r;
        }
        src = kHostRow | src;
        cls = pin != 0 ? 3 : 2;
      }
    }
    d_dst[tid] = dst;
  }
  d_src[tid] = src;
  d_wgt[tid] = wgt;
  return cls;
}

// Exact attention and estimate removal over the described rows [0, nrows) (d_src, d_wgt in
// LDS), in blocks of 32 rows: block k goes to wave k % 4. Per block: the logits as the
// transposed product S^T = K Q^T on v_mfma_f32_16x16x32_bf16, A = the key rows straight from
// memory (a removal row's key is its cluster's centroid, so that its logit is the cluster's
// score), B = the group's queries (column c holds head c mod G for c < 2G, zero beyond).
// Tile tau puts table row 8 (m >> 2) + 4 tau + (m & 3) in its row m, so that lane (g, c) ends
// with the logits of rows 8 g .. 8 g + 7 for its column's head: the A operand layout of the
// weights, without an exchange. The value rows (or value sums) go to LDS by direct loads;
// the weights p = 2^(s - m) (negated for removal rows: their value sum leaves the numerator,
// n_j p the denominator) form the A operand, hi and lo bf16 parts in rows h and G + h,
// against the value rows read back transposed.
template <int G, bool TIER>
__device__ __forceinline__ void attend_rows_mfma(const DecodeArgs& a, int bh,
                                                 const bf16x8 (&qb)[4], MfmaState& st,
                                                 int nrows, const int32_t* d_src,
                                                 const float* d_wgt, const int32_t* d_dst,
                                                 RetWave<G>& W) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  typedef __attribute__((ext_vector_type(4))) float floatx4;
  typedef __attribute__((ext_vector_type(4))) short shortx4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
  const size_t kb = (size_t)bh * a.Lcap, cb = (size_t)bh * a.C;
  const bool arow = n < 2 * G;
  for (int r0 = kRetBlock * wave; r0 < nrows; r0 += kRetBlock * (kDecThreads / 64)) {
    // ---- key rows (A operands of the two tiles), straight from memory
    u32x4 ka[2][4];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int32_t src = d_src[r0 + 8 * (n >> 2) + 4 * tau + (n & 3)];
      const uint16_t* kp;
      if constexpr (TIER)
        kp = src < 0 ? a.cmean + (cb + (-1 - src)) * kHeadDim
             : (src & kHostRow) ? a.hk + (kb + (src & ~kHostRow)) * kHeadDim
             : a.cache + ((size_t)(src / kTierBlock) * 2 * kTierBlock + src % kTierBlock) * kHeadDim;
      else
        kp = src >= 0 ? a.k + (kb + src) * kHeadDim : a.cmean + (cb + (-1 - src)) * kHeadDim;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) ka[tau][s4] = ld16_stream(kp + s4 * 32 + g * 8);
      if constexpr (TIER) {   // a row read over the bus goes into its slot as well
        const int32_t dst = d_dst[r0 + 8 * (n >> 2) + 4 * tau + (n & 3)];
        if (dst >= 0) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            st16(a.cache + (size_t)dst * kHeadDim + s4 * 32 + g * 8, ka[tau][s4]);
        }
      }
    }
    // ---- value rows (or value sums) into LDS
    {
      const int slot = lane >> 4, cidx = (n - 2 * slot) & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int32_t src = d_src[r0 + 8 * slot + e];
        if constexpr (TIER) {
          const bool host = src >= 0 && (src & kHostRow);
          const uint16_t* vp =
              src < 0 ? a.vsum + (cb + (-1 - src)) * kHeadDim
              : host  ? a.hv + (kb + (src & ~kHostRow)) * kHeadDim
                      : a.cache + ((size_t)(src / kTierBlock) * 2 * kTierBlock + kTierBlock +
                                   src % kTierBlock) * kHeadDim;
          // a row in host memory anywhere in this load's four rows: plain loads by every lane,
          // written where the direct load would put them (a direct load is issued by all lanes
          // or by none)
          if (__ballot(host)) {
            const u32x4 v = ld16_stream(vp + cidx * 8);
            *reinterpret_cast<u32x4*>(&W.vrows[e][4 * lane]) = v;
            const int32_t dst = d_dst[r0 + 8 * slot + e];
            if (dst >= 0) st16(a.cache + ((size_t)dst + kTierBlock) * kHeadDim + cidx * 8, v);
          } else {
            __builtin_amdgcn_global_load_lds(vp + cidx * 8, (lds_ptr)&W.vrows[e][0], 16, 0, 0);
          }
        } else {
          const uint16_t* vp = src >= 0 ? a.v + (kb + src) * kHeadDim
                                        : a.vsum + (cb + (-1 - src)) * kHeadDim;
          __builtin_amdgcn_global_load_lds(vp + cidx * 8, (lds_ptr)&W.vrows[e][0], 16, 0, 0);
        }
      }
    }
    // ---- denominator weights of this lane's rows 8 g .. 8 g + 7
    float wv[8];
    {
      const float4* wp = reinterpret_cast<const float4*>(d_wgt + r0 + 8 * g);
      const float4 y0 = wp[0], y1 = wp[1];
      wv[0] = y0.x; wv[1] = y0.y; wv[2] = y0.z; wv[3] = y0.w;
      wv[4] = y1.x; wv[5] = y1.y; wv[6] = y1.z; wv[7] = y1.w;
    }
    // ---- logits: lane (g, c) gets rows 8 g + 4 tau + i of its column's head
    floatx4 dq[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      dq[tau] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        dq[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, ka[tau][s4]), qb[s4], dq[tau], 0, 0, 0);
    }
    float sv[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[4 * tau + i] = wv[4 * tau + i] != 0.f ? dq[tau][i] * a.scale_log2 : kNegInf;
    float mb = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) mb = fmaxf(mb, sv[e]);
    mb = arow ? mb : kNegInf;
    mb = fmaxf(mb, xor16(mb));
    mb = fmaxf(mb, xor32(mb));
    // the running maximum moves only when the block's exceeds it by more than kLazyMax (the
    // weights stay below 2^kLazyMax), so that most blocks leave the accumulators unscaled
    const bool raise = mb > st.m + kLazyMax || (st.m == kNegInf && mb != kNegInf);
    const float mn = raise ? mb : st.m;
    const float alpha = raise ? (st.m == kNegInf ? 0.f : fast_exp2(st.m - mn)) : 1.f;
    st.m = mn;
    float ls = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float c[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x = sv[e + u];
        const float pr = (x == kNegInf || mn == kNegInf) ? 0.f : fast_exp2(x - mn);
        ls += wv[e + u] * pr;
        c[u] = wv[e + u] < 0.f ? -pr : pr;
      }
      pk[e >> 1] = hi_lo_bf16<G>(c[0], c[1], n);
    }
    st.l = alpha * st.l + ls;
    const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    // accumulator rows 4 g + i belong to the head of A row 4 g + i (lane 4 g + i)
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ar = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int t = 0; t < 8; ++t) st.acc[t][i] *= ar;
      }
    }
    // ---- the value rows, read back transposed, against the weights
    drain_vmem();  // (this wave's direct loads have landed in LDS)
    __builtin_amdgcn_wave_barrier();
    const char* vb = reinterpret_cast<const char*>(&W.vrows[0][0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      shortx4 bh2[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int e = 4 * hf + (n >> 2);
        const int c = 2 * t + ((n & 3) >> 1);
        const int off = e * (kVBlockWords * 4) + g * 256 + (((c + 2 * g) & 15) << 4) + ((n & 1) << 3);
        bh2[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(vb + off));
      }
      const u32x4 bw = {(uint32_t)(uint16_t)bh2[0][0] | ((uint32_t)(uint16_t)bh2[0][1] << 16),
                        (uint32_t)(uint16_t)bh2[0][2] | ((uint32_t)(uint16_t)bh2[0][3] << 16),
                        (uint32_t)(uint16_t)bh2[1][0] | ((uint32_t)(uint16_t)bh2[1][1] << 16),
                        (uint32_t)(uint16_t)bh2[1][2] | ((uint32_t)(uint16_t)bh2[1][3] << 16)};
      st.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, bw),
                                                          st.acc[t], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();  // (the next block rewrites this wave's LDS)
  }
}

// The workgroup's waves' states merged with one more partial xp ([G][kPartStride] in LDS,
// may be null) into the partial dst (device-coherent stores: read by other workgroups of
// the same kernel). Ends on a barrier.
template <int G>
__device__ __forceinline__ void write_mfma_partial(MfmaState& st, const float* xp,
                                                   float* __restrict__ dst, RetLds<G>& L) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, n = lane & 15;
  float l = st.l;
  l += xor16(l);
  l += xor32(l);
  __syncthreads();  // (every wave is done with its staging LDS)
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;
      if (r < 2 * G) L.mg.o[w][r][16 * t + n] = st.acc[t][i];
    }
  if (g == 0 && n < G) {
    L.mg.m[w][n] = st.m;
    L.mg.l[w][n] = l;
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += kDecThreads) {
    const int h = idx >> 7, d = idx & 127;
    float M = xp ? xp[h * kPartStride + 128] : kNegInf;
#pragma unroll
    for (int ww = 0; ww < kDecThreads / 64; ++ww) M = fmaxf(M, L.mg.m[ww][h]);
    float o = 0.f, ls = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kDecThreads / 64; ++ww) {
        const float f = fast_exp2(L.mg.m[ww][h] - M);
        o += f * (L.mg.o[ww][h][d] + L.mg.o[ww][G + h][d]);
        ls += f * L.mg.l[ww][h];
      }
      if (xp) {
        const float f = fast_exp2(xp[h * kPartStride + 128] - M);
        o += f * xp[h * kPartStride + d];
        ls += f * xp[h * kPartStride + 129];
      }
    }
    st_dev(dst + h * kPartStride + d, o);
    if (d == 0) {
      st_dev(dst + h * kPartStride + 128, M);
      st_dev(dst + h * kPartStride + 129, ls);
    }
  }
  __syncthreads();
}

// nB workgroups per (b, kv-head): each takes a share of the estimate and steady partials
// and its virtual rows, and writes one partial. The last of each of the nG merge groups
// merges its partials (nG = 1: straight into out / lse); the last of those merges writes
// out / lse.
// XM1: the estimate / steady partials of the workgroup's share loaded in one round for every
// (head, dim) element of a thread before the attend and merged after it (more registers, for
// launches small enough to be resident at three workgroups per CU); else merged element by
// element before the attend.
template <int G, bool XM1, bool TIER>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(3))) void k_dec_retrieve(DecodeArgs a) {
  __shared__ float s_x[G][kPartStride];  // this workgroup's share of the earlier partials
  __shared__ int32_t l_ts[kWinR + 1], l_co[kWinR], l_id[kWinR];
  __shared__ int32_t d_src[kDecThreads];  // the current rows' descriptors (describe_rows)
  __shared__ __align__(16) float d_wgt[kDecThreads];
  __shared__ int32_t d_dst[TIER ? kDecThreads : 1];
  __shared__ int32_t t_blk[TIER ? kDecThreads : 1], t_res[TIER ? kDecThreads : 1];
  __shared__ RetLds<G> lds;
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv, w_item = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nB = a.nB, nSP = a.nEW + a.nSt;
  float* parts = a.part + (size_t)bh * a.nP * G * kPartStride;
  // ---- this workgroup's virtual rows [T0, T1) and listed clusters [r_lo, r_hi)
  const int4 info = reinterpret_cast<const int4*>(a.wg_info)[(size_t)bh * kMaxRetrieveWG + w_item];
  const int T0 = info.x, T1 = info.y, r_lo = info.z, r_hi = info.w;
  const int32_t* g_ts = a.sel_ts + (size_t)bh * (a.rcap + 1);
  // ---- the estimate / steady partials w_item, w_item + nB, ... merged into s_x. XM1: the
  // first XB of them are loaded here for every (head, dim) element of the thread and merged
  // after the attend, so that their round trip overlaps it.
  constexpr int IPT = XM1 ? (G * 128 + kDecThreads - 1) / kDecThreads : 1;
  constexpr int XB = 4;
  float xm[IPT][XB], xl[IPT][XB], xo[IPT][XB];
  // XM1: the next XB2 partials (w_item + (XB + k) nB) go to LDS by direct loads issued here,
  // in 16-byte chunks, one wave instruction per 64 chunks (the area is padded to whole
  // instructions); they land during the attend
  // (groups of at most four heads: the larger groups' registers and LDS are full already)
  constexpr int XB2 = XM1 && G <= 4 ? 2 : 0;
  constexpr int kPartChunks = G * kPartStride / 4;  // 16-byte chunks of one partial
  constexpr int kX2Chunks = XB2 > 0 ? (XB2 * kPartChunks + 63) / 64 * 64 : 1;
  __shared__ __align__(16) float s_x2[kX2Chunks * 4];
  if constexpr (XB2 > 0) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const int lane = tid & 63;
    for (int c0 = wave * 64; c0 < kX2Chunks; c0 += kDecThreads) {
      const int c = min(c0 + lane, XB2 * kPartChunks - 1);
      const int k = c / kPartChunks, pk = min(w_item + (XB + k) * nB, nSP - 1);
      __builtin_amdgcn_global_load_lds(parts + (size_t)pk * G * kPartStride + (c - k * kPartChunks) * 4,
                                       (lds_ptr)&s_x2[c0 * 4], 16, 0, 0);
    }
  }
  if constexpr (XM1) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = min(tid + i * kDecThreads, G * 128 - 1), h = idx >> 7, d = idx & 127;
#pragma unroll
      for (int k = 0; k < XB; ++k) {
        const int pk = w_item + k * nB;
        const float* pp = parts + ((size_t)pk * G + h) * kPartStride;
        xm[i][k] = pk < nSP ? pp[128] : kNegInf;
        xl[i][k] = pk < nSP ? pp[129] : 0.f;
        xo[i][k] = pk < nSP ? pp[d] : 0.f;
      }
    }
  } else {
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
  }
  // B operands of the logits: column c = lane % 16 holds query head c mod G for c < 2G (zero
  // beyond), dims 32 s + 8 (lane / 16)
  bf16x8 qb[4];
  {
    const int qc = lane & 15, kg = lane >> 4, qh = qc < G ? qc : qc - G;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      u32x4 v = {0, 0, 0, 0};
      if (qc < 2 * G)
        v = ld16(a.q + ((size_t)(b * a.Hq + g * G + qh) * kHeadDim + s4 * 32 + kg * 8));
      qb[s4] = __builtin_bit_cast(bf16x8, v);
    }
  }
  MfmaState st;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.acc[t] = MfmaState::floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.f;
  const size_t lb = (size_t)bh * a.rcap;
  for (int rw = r_lo; rw < r_hi; rw += kWinR) {
    const int cnt = min(kWinR, r_hi - rw);
    for (int i = tid; i <= cnt; i += kDecThreads) {
      l_ts[i] = g_ts[rw + i];
      if (i < cnt) {
        l_co[i] = a.sel_coff[lb + rw + i];
        l_id[i] = a.sel_id[lb + rw + i];
      }
    }
    __syncthreads();
    const int ts = max(T0, l_ts[0]), te = min(T1, l_ts[cnt]);
    for (int c0 = ts; c0 < te; c0 += kDecThreads) {
      const int nr = min(kDecThreads, te - c0);
      const int cls =
          describe_rows<TIER>(a, bh, c0, nr, l_ts, l_co, l_id, cnt, d_src, d_wgt, d_dst, t_blk,
                              t_res);
      if constexpr (TIER) {
        const int nc = __syncthreads_count(cls == 1), nh = __syncthreads_count(cls >= 2),
                  nw = __syncthreads_count(cls == 3);
        if (tid == 0) {
          if (nc) atomicAdd(a.tctr + kTcRowsCached, (uint32_t)nc);
          if (nh) atomicAdd(a.tctr + kTcRowsHost, (uint32_t)nh);
          if (nw) atomicAdd(a.tctr + kTcRowsWritten, (uint32_t)nw);
        }
      } else {
        __syncthreads();
      }
      attend_rows_mfma<G, TIER>(a, bh, qb, st, nr, d_src, d_wgt, d_dst, lds.w[wave]);
      __syncthreads();
    }
    __syncthreads();
  }
  if constexpr (XM1) {
    drain_vmem();  // (the staged partials have landed: every wave's own loads, then all)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = tid + i * kDecThreads;
      float M = kNegInf;
#pragma unroll
      for (int k = 0; k < XB; ++k) M = fmaxf(M, xm[i][k]);
      float Ls = 0.f, O = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int k = 0; k < XB; ++k) {
          const float f = fast_exp2(xm[i][k] - M);
          O += f * xo[i][k];
          Ls += f * xl[i][k];
        }
      }
      {
        const int h = min(idx, G * 128 - 1) >> 7, d = idx & 127;
#pragma unroll
        for (int k = 0; k < XB2; ++k) {  // the partials staged in LDS
          if (w_item + (XB + k) * nB < nSP) {
            const float* xp = &s_x2[(k * G + h) * kPartStride];
            float a1, a2, mn;
            lse_pair(M, xp[128], a1, a2, mn);
            O = a1 * O + a2 * xp[d];
            Ls = a1 * Ls + a2 * xp[129];
            M = mn;
          }
        }
      }
      if (w_item + (XB + XB2) * nB < nSP) {  // still more partials for this workgroup
        float M2, L2, O2, a1, a2, mn;
        merge_partials<false, 4>(parts, G, min(idx, G * 128 - 1), w_item + (XB + XB2) * nB, nB,
                                 nSP, M2, L2, O2);
        lse_pair(M, M2, a1, a2, mn);
        O = a1 * O + a2 * O2;
        Ls = a1 * Ls + a2 * L2;
        M = mn;
      }
      if (idx < G * 128) {
        const int h = idx >> 7, d = idx & 127;
        s_x[h][d] = O;
        if (d == 0) {
          s_x[h][128] = M;
          s_x[h][129] = Ls;
        }
      }
    }
  }
  // (the barriers inside make s_x visible before it is read)
  write_mfma_partial<G>(st, &s_x[0][0], parts + (size_t)(nSP + w_item) * G * kPartStride, lds);
  uint32_t* ctr = a.counter + (size_t)bh * kCtrStride;
  const int gsz = (nB + a.nG - 1) / a.nG;  // retrieve partials per merge group
  const int grp = w_item / gsz, g0 = grp * gsz, gn = min(gsz, nB - g0);
  if (!arrive_last(ctr + kCtrGroup + grp, (uint32_t)gn)) return;
  const int bq = b * a.Hq + g * G;
  const bool single = a.nG == 1;
  float* gp = parts + (size_t)(nSP + nB + grp) * G * kPartStride;
  auto write_out = [&](int h, int d4, float M, float L, float4 o) {
    float* op = a.out + (size_t)(bq + h) * kHeadDim + d4;
    const float r = 1.f / L;
    *reinterpret_cast<float4*>(op) = make_float4(o.x * r, o.y * r, o.z * r, o.w * r);
    if (d4 == 0 && a.lse) a.lse[bq + h] = (M + log2f(L)) * kLn2;
  };
  if (single) {
    merge_block<G, true, kMergeBatch>(parts, nSP + g0, 1, gn, lds.xh, write_out);
    return;
  }
  merge_block<G, true, kMergeBatch>(parts, nSP + g0, 1, gn, lds.xh,
                                    [&](int h, int d4, float M, float L, float4 o) {
    float* q = gp + h * kPartStride + d4;
    st_dev(q, o.x);
    st_dev(q + 1, o.y);
    st_dev(q + 2, o.z);
    st_dev(q + 3, o.w);
    if (d4 == 0) {
      st_dev(gp + h * kPartStride + 128, M);
      st_dev(gp + h * kPartStride + 129, L);
    }
  });
  if (!arrive_last(ctr + kCtrFinal, (uint32_t)a.nG)) return;
  merge_block<G, true, kMergeBatch>(parts, nSP + nB, 1, a.nG, lds.xh, write_out);
}

// ------------------------------------------------------------------------------------
// host-memory tier: step and reset
// ------------------------------------------------------------------------------------
// After the retrieve of a step: the next step begins, and the hand's position is noted (a
// step's claims go round the slots once at most).
__global__ void k_tier_step(DecodeArgs a) {
  if (threadIdx.x == 0) {
    a.tctr[kTcHandStart] = ld_dev(a.tctr + kTcHand);
    a.tctr[kTcStep] = ld_dev(a.tctr + kTcStep) + 1u;
  }
}

// Empty cache: no block cached, no slot owned (owner -1, step 0), step 1, counters zero.
__global__ __launch_bounds__(kDecThreads) void k_tier_reset(DecodeArgs a) {
  const size_t i0 = (size_t)blockIdx.x * kDecThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kDecThreads;
  const size_t ntab = (size_t)a.B * a.Hkv * a.nblk;
  for (size_t i = i0; i < ntab; i += stride) a.tab[i] = -1;
  for (size_t i = i0; i < (size_t)a.nslots; i += stride) {
    a.slotw[i] = 0xffffffffull;
    a.valid[i] = 0u;
  }
  if (i0 < (size_t)kTcWords) a.tctr[i0] = i0 == (size_t)kTcStep ? 1u : 0u;
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
  attend_rows<G>(a, a.k, a.v, (size_t)bh * a.Lcap, q, st, wb, we, [](int64_t t) { return t; });
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
// attention over the steady zone and listed cache rows (the vector-search retrieval zone):
// virtual rows [0, n_steady) are the steady zone, then rows_pos[bh][0 .. rows_n[bh]);
// split-K partials over nB workgroups per head, then the dense merge
// ------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kDecThreads) void k_listed_partial(DecodeArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv, g = bh % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  u32x4 q[G];
  load_q<G>(a, b, g, c, q);
  Online<G> st;
  st.init();
  const int64_t n_steady = (int64_t)a.n_sink + a.n_recent + (a.L - a.L0);
  const int32_t* pos = a.rows_pos + (size_t)bh * a.rows_k;
  const int64_t n = n_steady + min(max(a.rows_n[bh], 0), a.rows_k);
  const int nB = a.nB, w = blockIdx.x;
  const int64_t t0 = n * w / nB, t1 = n * (w + 1) / nB;
  const int64_t wb = t0 + (t1 - t0) * wave / 4, we = t0 + (t1 - t0) * (wave + 1) / 4;
  attend_rows<G>(a, a.k, a.v, (size_t)bh * a.Lcap, q, st, wb, we, [&](int64_t t) {
    return t < n_steady ? steady_row(a, t) : (int64_t)pos[t - n_steady];
  });
  write_block_partial<G>(st, nullptr, a.part + ((size_t)bh * nB + w) * G * kPartStride);
}

// ------------------------------------------------------------------------------------
template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_dec_score<G>, dim3(a.nSW, BH), dim3(kDecThreads), 0, s, a);
  if (e != hipSuccess) return e;
  if (a.hist_kernel) {
    e = launch(tr, k_dec_hist, dim3(a.nH, BH), dim3(kDecThreads), 0, s, a);
    if (e != hipSuccess) return e;
  }
  const dim3 ggrid((a.nH + a.nEW + a.nSt) * BH);
  e = a.hist_kernel ? launch(tr, k_dec_gather<G, true>, ggrid, dim3(kDecThreads), 0, s, a)
                    : launch(tr, k_dec_gather<G, false>, ggrid, dim3(kDecThreads), 0, s, a);
  if (e != hipSuccess) return e;
  if (a.tier) {
    e = a.nB * BH <= 3 * kCUs
            ? launch(tr, k_dec_retrieve<G, true, true>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a)
            : launch(tr, k_dec_retrieve<G, false, true>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
    if (e != hipSuccess) return e;
    return launch(tr, k_tier_step, dim3(1), dim3(64), 0, s, a);
  }
  if (a.nB * BH <= 3 * kCUs)
    return launch(tr, k_dec_retrieve<G, true, false>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
  return launch(tr, k_dec_retrieve<G, false, false>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
}

template <int G>
static hipError_t launch_dense_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_dense_partial<G>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
  if (e != hipSuccess) return e;
  return launch(tr, k_dense_merge<G>, dim3(BH), dim3(kDecThreads), 0, s, a);
}

template <int G>
static hipError_t launch_listed_g(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_listed_partial<G>, dim3(a.nB, BH), dim3(kDecThreads), 0, s, a);
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

// ------------------------------------------------------------------------------------
// scratch of the allocation-free decode entry point
// ------------------------------------------------------------------------------------
// One copy per GPU, allocated when the code object is loaded on that device and kept until
// the process ends. In host code the name stands for a host-side stand-in, not a device
// address: host code only ever uses the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  WAVE_DISPATCH_G(launch_decode_g, a, s, tr)
}
hipError_t launch_dense_decode(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  WAVE_DISPATCH_G(launch_dense_g, a, s, tr)
}
hipError_t launch_listed_attention(const DecodeArgs& a, hipStream_t s, Tracer* tr) {
  WAVE_DISPATCH_G(launch_listed_g, a, s, tr)
}
hipError_t tier_counters_copy(uint32_t* c, const void* state, hipStream_t s) {
  const hipError_t e = hipMemcpyAsync(c, state, kTcWords * sizeof(uint32_t),
                                      hipMemcpyDeviceToHost, s);
  return e != hipSuccess ? e : hipStreamSynchronize(s);
}
hipError_t launch_tier_reset(const DecodeArgs& a, hipStream_t s) {
  const size_t n = std::max((size_t)a.B * a.Hkv * a.nblk, (size_t)a.nslots);
  const int nb = (int)std::min<size_t>((n + kDecThreads - 1) / kDecThreads, 4096);
  return launch(nullptr, k_tier_reset, dim3(std::max(nb, 1)), dim3(kDecThreads), 0, s, a);
}

}  // namespace wave
