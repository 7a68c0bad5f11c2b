// Wave-index build: segmented spherical k-means over each KV head's keys (gfx950).
//
// The summaries of RetroInfer build the index during prefill by clustering the keys of each
// segment of the context locally (gist.science de/fr/zh, section 2A "segmented
// clustering"; the zh summary ties it to RoPE's positional locality), with spherical
// k-means (fr, section 2A), and keep per-cluster centroids and precomputed value sums for
// the estimation zone (zh, section 2A).
//
// Per (b, kv-head, segment), T passes of
//   assign: a_i = argmax_j k_i . mu_j  (the positive factor 1/||k_i|| of the cosine does not
//           change the argmax, so the contraction runs on the raw bf16 keys) -- a dense
//           [points x 128] x [128 x k_seg] product on bf16 MFMA (v_mfma_f32_32x32x16_bf16)
//           with the argmax fused into the epilogue;
//   sort:   stable counting sort of the labels (one workgroup per segment, wave ballots
//           give each point its rank among equal labels) -- no atomics on data, so every
//           later sum runs in a fixed order and the build is bitwise reproducible;
//   update: mu_j = bf16(u_j / ||u_j||), u_j = sum of the members' unit keys, summed in
//           position order by 16 lanes per row, 16 member rows in flight at a time (empty
//           clusters keep mu_j).
// Then finalise: sizes, offsets, mean raw key and value sum per cluster, and the
// cluster-contiguous permutation of K and V (each row read once, written once), so that
// decode reads a retrieved cluster as one contiguous run of rows.
#include <algorithm>
#include <cfloat>

#include "wave_common.h"
#include "wave_kernels.h"

namespace wave {

struct Seg {
  int64_t lo, hi;  // indexed positions [lo, hi) of the segment
};

__device__ __forceinline__ Seg seg_range(const BuildArgs& a, int s) {
  int64_t lo = max((int64_t)s * a.S, a.idx_lo);
  int64_t hi = min((int64_t)(s + 1) * a.S, a.idx_hi);
  if (hi < lo) hi = lo;
  return {lo, hi};
}

// usable clusters of a segment with n points: all k_seg, or one per point if fewer
__device__ __forceinline__ int n_valid_clusters(const BuildArgs& a, int64_t n) {
  return n >= a.kseg ? a.kseg : (int)n;
}

// ------------------------------------------------------------------------------------
// norms of the indexed keys: inv_norm = 1/||k|| (0 for a zero key)
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_norms(BuildArgs a) {
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, grp = (threadIdx.x >> 4), c = lane & 15;
  const int64_t lo = max(a.idx_lo, (int64_t)a.seg0 * a.S), n = a.idx_hi - lo;
  for (int64_t i = (int64_t)blockIdx.x * 16 + grp; i < n; i += (int64_t)gridDim.x * 16) {
    const int64_t p = lo + i;
    const u32x4 kr = ld16(a.k + ((size_t)bh * a.Lcap + p) * kHeadDim + c * 8);
    float ss = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float x0 = bf_lo(kr[d]), x1 = bf_hi(kr[d]);
      ss += x0 * x0 + x1 * x1;
    }
    ss = sum16(ss);
    if (c == 0) a.inv_norm[(size_t)bh * a.L0 + p] = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
  }
}

// ------------------------------------------------------------------------------------
// seeds: mu_j = bf16(unit key of local point j * floor(n_s / k_seg)); first n_s points
// if the segment is short, zero rows for the clusters that stay empty
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_seeds(BuildArgs a, uint16_t* __restrict__ mu) {
  const int s = a.seg0 + blockIdx.y, bh = blockIdx.z;
  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const Seg sg = seg_range(a, s);
  const int64_t n = sg.hi - sg.lo;
  const int j = blockIdx.x * 16 + grp;
  if (j >= a.kseg) return;
  u32x4 out = {0, 0, 0, 0};
  int64_t p = -1;
  if (n >= a.kseg) p = sg.lo + (int64_t)j * (n / a.kseg);
  else if (j < n) p = sg.lo + j;
  if (p >= 0) {
    const u32x4 kr = ld16(a.k + ((size_t)bh * a.Lcap + p) * kHeadDim + c * 8);
    const float inv = a.inv_norm[(size_t)bh * a.L0 + p];
#pragma unroll
    for (int d = 0; d < 4; ++d) out[d] = pack_bf2(bf_lo(kr[d]) * inv, bf_hi(kr[d]) * inv);
  }
  st16(mu + ((size_t)bh * a.C + (size_t)s * a.kseg + j) * kHeadDim + c * 8, out);
}

// ------------------------------------------------------------------------------------
// assignment on MFMA
// ------------------------------------------------------------------------------------
constexpr int kAsgWaves = 4;
constexpr int kAsgNB = 2;                                  // 32-point column blocks per wave
constexpr int kAsgPoints = kAsgWaves * kAsgNB * 32;        // points per workgroup
constexpr int kAsgTile = 128;                              // centroids per LDS tile
constexpr int kAsgLdsStride = kRowBytes + 16;              // padded row: no bank conflicts

__global__ __launch_bounds__(256) void k_assign(BuildArgs a, const uint16_t* __restrict__ mu) {
  const int blk = blockIdx.x, s = a.seg0 + blockIdx.y, bh = blockIdx.z;
  const Seg sg = seg_range(a, s);
  const int64_t n = sg.hi - sg.lo;
  if ((int64_t)blk * kAsgPoints >= n) return;
  const int nvalid = n_valid_clusters(a, n);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  __shared__ __attribute__((aligned(16))) unsigned char s_mu[kAsgTile * kAsgLdsStride];

  // B operands: this wave's points, 32 per column block. Lane holds elements
  // k = 16*kk + 8*half + [0, 8) of point (col) for every 16-wide k step kk.
  bf16x8 bq[kAsgNB][8];
  int64_t pidx[kAsgNB];
#pragma unroll
  for (int nb = 0; nb < kAsgNB; ++nb) {
    pidx[nb] = (int64_t)blk * kAsgPoints + wave * (kAsgNB * 32) + nb * 32 + col;
    const bool ok = pidx[nb] < n;
    const uint16_t* row = a.k + ((size_t)bh * a.Lcap + sg.lo + (ok ? pidx[nb] : 0)) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = ok ? ld16(row + kk * 16 + half * 8) : u32x4{0, 0, 0, 0};
      bq[nb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float best[kAsgNB];
  int bidx[kAsgNB];
#pragma unroll
  for (int nb = 0; nb < kAsgNB; ++nb) {
    best[nb] = kNegInf;
    bidx[nb] = 0;
  }

  const uint16_t* mus = mu + ((size_t)bh * a.C + (size_t)s * a.kseg) * kHeadDim;
  for (int t0 = 0; t0 < nvalid; t0 += kAsgTile) {
    __syncthreads();
    // stage centroids [t0, t0 + 128) (zero rows past k_seg)
    for (int q = tid; q < kAsgTile * 16; q += 256) {
      const int r = q >> 4, ch = q & 15;
      u32x4 v = {0, 0, 0, 0};
      if (t0 + r < a.kseg) v = ld16(mus + (size_t)(t0 + r) * kHeadDim + ch * 8);
      *reinterpret_cast<u32x4*>(s_mu + r * kAsgLdsStride + ch * 16) = v;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kAsgTile / 32; ++rb) {
      const int m0 = t0 + rb * 32;
      if (m0 >= nvalid) break;
      floatx16 acc[kAsgNB];
#pragma unroll
      for (int nb = 0; nb < kAsgNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        // A operand: centroid row (m0 + col), elements 16*kk + 8*half + [0, 8)
        const bf16x8 am = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(s_mu + (rb * 32 + col) * kAsgLdsStride +
                                                     (kk * 2 + half) * 16));
#pragma unroll
        for (int nb = 0; nb < kAsgNB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bq[nb][kk], acc[nb], 0, 0, 0);
      }
      // D[m][n]: lane holds column n = col and rows m = 8*(i/4) + 4*half + i%4 (increasing
      // in i), so a strict '>' keeps the lowest centroid id among equal scores
#pragma unroll
      for (int nb = 0; nb < kAsgNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + 8 * (i >> 2) + 4 * half + (i & 3);
          const float v = acc[nb][i];
          if (m < nvalid && v > best[nb]) {
            best[nb] = v;
            bidx[nb] = m;
          }
        }
    }
  }
  // the two half-waves hold disjoint centroid rows of the same points
#pragma unroll
  for (int nb = 0; nb < kAsgNB; ++nb) {
    const float ov = __shfl_xor(best[nb], 32);
    const int oi = __shfl_xor(bidx[nb], 32);
    if (ov > best[nb] || (ov == best[nb] && oi < bidx[nb])) {
      best[nb] = ov;
      bidx[nb] = oi;
    }
    if (half == 0 && pidx[nb] < n) a.lab[(size_t)bh * a.L0 + sg.lo + pidx[nb]] = bidx[nb];
  }
}

// Segment-resident variant (k_seg <= kA2MaxK): a 512-thread workgroup stages all centroids
// of its segment in LDS once (k_seg x 272 B) and each wave loops over 64-point blocks of its
// share of the segment's points. Per 32-centroid row block the argmax takes a max3 tree of
// the 16 scores a lane holds, each carrying its row in its low mantissa bits, and keeps it
// when it beats the running best (rows in increasing id order, so a strict '>' keeps the
// earlier block on equal keys).
constexpr int kA2Threads = 512;
constexpr int kA2Waves = kA2Threads / 64;
constexpr int kA2MaxK = 512;

__global__ __launch_bounds__(kA2Threads) void k_assign_seg(BuildArgs a, const uint16_t* __restrict__ mu,
                                                           int nsplit) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_mu2[];
  const int split = blockIdx.x, s = a.seg0 + blockIdx.y, bh = blockIdx.z;
  const Seg sg = seg_range(a, s);
  const int64_t n = sg.hi - sg.lo;
  if (n <= 0) return;
  const int nvalid = n_valid_clusters(a, n);
  const int kpad = (nvalid + 31) & ~31;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const uint16_t* mus = mu + ((size_t)bh * a.C + (size_t)s * a.kseg) * kHeadDim;
  // this split's points, in 64-point blocks (loads clamp to the last point: columns past the
  // segment are scored but never written)
  const int64_t nblk = (n + 63) / 64;
  const int64_t b0 = nblk * split / nsplit, b1 = nblk * (split + 1) / nsplit;
  auto load_block = [&](int64_t blk, bf16x8 (&bq)[2][8]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t p = min(blk * 64 + nb * 32 + col, n - 1);
      const uint16_t* row = a.k + ((size_t)bh * a.Lcap + sg.lo + p) * kHeadDim;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        bq[nb][kk] = __builtin_bit_cast(bf16x8, ld16_stream(row + kk * 16 + half * 8));
    }
  };
  // the wave's first key block is loaded before the centroids are staged, so that both
  // take one memory round trip
  int64_t blk = b0 + wave;
  bf16x8 bq[2][8];
  if (blk < b1) load_block(blk, bq);
  // the centroids: 16-byte chunks, up to 16 per thread with all their loads in flight
  // together (rows clamp to the last valid one, padding rows are written as zero)
  for (int q0 = 0; q0 < kpad * 16; q0 += 16 * kA2Threads) {
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = q0 + j * kA2Threads + tid, r = min(q >> 4, kpad - 1), ch = q & 15;
      v[j] = ld16(mus + (size_t)min(r, nvalid - 1) * kHeadDim + ch * 8);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = q0 + j * kA2Threads + tid, r = q >> 4, ch = q & 15;
      if (r >= nvalid) v[j] = u32x4{0, 0, 0, 0};
      if (q < kpad * 16) *reinterpret_cast<u32x4*>(s_mu2 + r * kAsgLdsStride + ch * 16) = v[j];
    }
  }
  int* s_next = reinterpret_cast<int*>(s_mu2 + kpad * kAsgLdsStride);
  if (tid == 0) *s_next = (int)(b0 + kA2Waves);
  __syncthreads();
  // row of the A operand (centroids) that this lane supplies for row block m0 and k step kk
  // (rows clamp to the last padded one, so reads need no branch)
  auto a_row = [&](int m0, int kk) {
    const unsigned char* r = s_mu2 + min(m0 + col, kpad - 1) * kAsgLdsStride + half * 16;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(r + kk * 32));
  };
  // The low 4 mantissa bits of each score are replaced by 15 - i for accumulator element i
  // (rows ascend with i), and a float max over a point's scores then picks its best row.
  // Whatever the sign of the best score, the replaced bits move a score by under 16 ulps, so
  // the winner's score is within 16 ulps of the best one (a relative 2^-19, far below the
  // bf16 rounding of the operands); only which of such near-equal centroids wins can change
  // (among exactly equal positive scores, the lowest row).
  auto score_block = [&](int64_t blk, const bf16x8 (&bq)[2][8]) {
    float best[2] = {kNegInf, kNegInf};
    int bblk[2] = {0, 0};
    bf16x8 am[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) am[kk] = a_row(0, kk);
    // products of row block m0; each A operand is refilled with the next row block's once
    // its products are issued
    auto products = [&](int m0, floatx16 (&acc)[2]) {
      const floatx16 zero = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[kk], bq[nb][kk],
                                                            kk == 0 ? zero : acc[nb], 0, 0, 0);
        am[kk] = a_row(m0 + 32, kk);
      }
    };
    // best row of row block m0 per point; element i holds row m0 + 8 * (i / 4) + 4 * half +
    // i % 4, and in the last block rows >= nvalid get -FLT_MAX, below every score
    auto pick = [&](int m0, const floatx16 (&acc)[2], bool last) {
      const int lim = nvalid - m0 - 4 * half;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float key[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          key[i] = __uint_as_float((__float_as_uint(acc[nb][i]) & ~15u) | (15u - i));
        if (last) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + (i & 3) >= lim) key[i] = -FLT_MAX;
        }
        float bm = fmaxf(fmaxf(key[0], key[1]), key[2]);
        bm = fmaxf(fmaxf(bm, key[3]), key[4]);
        bm = fmaxf(fmaxf(bm, key[5]), key[6]);
        bm = fmaxf(fmaxf(bm, key[7]), key[8]);
        bm = fmaxf(fmaxf(bm, key[9]), key[10]);
        bm = fmaxf(fmaxf(bm, key[11]), key[12]);
        bm = fmaxf(fmaxf(bm, key[13]), key[14]);
        bm = fmaxf(bm, key[15]);
        // strict: an equal key in a later block has a higher row
        if (bm > best[nb]) {
          best[nb] = bm;
          bblk[nb] = m0;
        }
      }
    };
    // software pipeline over the row blocks: the products of block r are issued before the
    // scores of block r - 1 are reduced, so the matrix core and the vector ALU overlap
    const int nrb = kpad / 32;
    // (each products + pick pair is one scheduling region, the compiler interleaving the
    // reduction's ALU work between the 16 matrix products)
    floatx16 acc0[2], acc1[2];
    products(0, acc0);
    int r = 1;
    for (; r + 1 < nrb; r += 2) {
      __builtin_amdgcn_sched_barrier(0);
      products(32 * r, acc1);
      pick(32 * (r - 1), acc0, false);
      __builtin_amdgcn_sched_barrier(0);
      products(32 * (r + 1), acc0);
      pick(32 * r, acc1, false);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (r < nrb) {
      products(32 * r, acc1);
      pick(32 * (r - 1), acc0, false);
      pick(32 * r, acc1, true);
    } else {
      pick(32 * (r - 1), acc0, true);
    }
    // the two half-waves hold disjoint centroid rows of the same points
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t bb = __float_as_uint(best[nb]);
      const int i = 15 - (int)(bb & 15u);
      const float tv = __uint_as_float(bb & ~15u);
      const int idx = bblk[nb] + 8 * (i >> 2) + 4 * half + (i & 3);
      const float ov = __shfl_xor(tv, 32);
      const int oi = __shfl_xor(idx, 32);
      const int pick = (ov > tv || (ov == tv && oi < idx)) ? oi : idx;
      const int64_t p = blk * 64 + nb * 32 + col;
      if (half == 0 && p < n) a.lab[(size_t)bh * a.L0 + sg.lo + p] = pick;
    }
  };
  // Blocks b0 + wave go to the waves first; every later block goes to whichever wave asks
  // next (a counter in LDS), so the waves of the workgroup, and with them the SIMDs, stay
  // busy until its last block. A wave claims its next block when it starts the current one.
  // (Its keys are loaded after the current block is scored: the other wave on the SIMD keeps
  // the matrix core busy meanwhile.)
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(s_next, 1);
    return (int64_t)__shfl(v, 0);
  };
  while (blk < b1) {
    const int64_t nxt = claim();
    score_block(blk, bq);
    blk = nxt;
    if (blk < b1) load_block(blk, bq);
  }
}

// ------------------------------------------------------------------------------------
// stable counting sort of a segment's labels: order = local point ids by (label, position)
// ------------------------------------------------------------------------------------
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kMaxSeg = 16384;
constexpr int kMaxKseg = 2048;

__device__ __forceinline__ uint32_t scan1024_excl(uint32_t x, uint32_t* s_tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = lane < kSortWaves ? s_tmp[lane] : 0u;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < kSortWaves) s_tmp[lane] = t;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? s_tmp[wave - 1] : 0u;
  total = s_tmp[kSortWaves - 1];
  __syncthreads();
  return v - x + before;
}

// Wave w ranks the points of its contiguous chunk [w cs, (w + 1) cs) of the segment, 64 at a
// time in position order: lanes holding the same label find each other by ballots over the
// label bits, and the wave's running count of each label (a row of s_cnt, read by every lane
// and then advanced by the label's first lane: one wave's LDS operations complete in order)
// gives each point its rank among the chunk's points of that label. The counts then become,
// label by label, the number of points of that label in earlier chunks, and the scan of the
// label totals gives each label's first slot, so that a point's slot is its label's first
// slot + its chunk's base + its rank: the stable order by (label, position), with three
// workgroup barriers besides the scan's.
constexpr int kSortBlocks = kMaxSeg / kSortWaves / 64;  // 64-point blocks per chunk, at most

__global__ __launch_bounds__(kSortThreads) void k_sort(BuildArgs a) {
  const int s = a.seg0 + blockIdx.x, bh = blockIdx.y;
  const Seg sg = seg_range(a, s);
  const int n = (int)(sg.hi - sg.lo);
  const int K = a.kseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint16_t s_lab[kMaxSeg];
  __shared__ uint16_t s_cnt[kSortWaves][kMaxKseg];  // per chunk: running count, then base
  __shared__ uint32_t s_start[kMaxKseg + 1];
  __shared__ uint32_t s_tmp[32];

  const int32_t* lab = a.lab + (size_t)bh * a.L0 + sg.lo;
  {
    // every label load issued before the first LDS write (one round trip, not one per
    // 1024 labels)
    constexpr int kL = kMaxSeg / kSortThreads;
    uint32_t lv[kL];
#pragma unroll
    for (int k = 0; k < kL; ++k)
      if (k * kSortThreads < n) lv[k] = (uint32_t)lab[min(k * kSortThreads + tid, n - 1)];
#pragma unroll
    for (int k = 0; k < kL; ++k) {
      const int i = k * kSortThreads + tid;
      if (k * kSortThreads < n && i < n) s_lab[i] = (uint16_t)lv[k];
    }
  }
  {
    uint32_t* z = reinterpret_cast<uint32_t*>(&s_cnt[0][0]);
    for (int q = tid; q < kSortWaves * kMaxKseg / 2; q += kSortThreads) z[q] = 0u;
  }
  __syncthreads();
  // ---- ranks within the wave's chunk (no workgroup barrier)
  const int cs = (n + 64 * kSortWaves - 1) / (64 * kSortWaves) * 64;  // chunk length
  const int nblk = cs / 64;
  const int nbits = 32 - __clz(max(K - 1, 1));
  uint32_t packed[kSortBlocks];  // label | rank in the chunk << 16 (all ones: no point)
  uint16_t* cnt = &s_cnt[wave][0];
#pragma unroll
  for (int k = 0; k < kSortBlocks; ++k) {
    packed[k] = 0xffffffffu;
    if (k < nblk) {
      const int i = wave * cs + 64 * k + lane;
      const bool ok = i < n;
      const uint32_t l = ok ? s_lab[i] : 0u;
      uint64_t peers = __ballot(ok);
      for (int bit = 0; bit < nbits; ++bit) {
        const uint64_t bb = __ballot(ok && ((l >> bit) & 1u));
        peers &= ((l >> bit) & 1u) ? bb : ~bb;
      }
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(peers >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)peers, 0u));
      const uint32_t prev = ok ? cnt[l] : 0u;
      if (ok && rank == 0) cnt[l] = (uint16_t)(prev + (uint32_t)__popcll(peers));
      if (ok) packed[k] = l | ((prev + rank) << 16);
    }
    __builtin_amdgcn_wave_barrier();  // (the next block's reads stay after this write)
  }
  __syncthreads();
  // ---- per label: counts -> bases of the chunks, totals -> first slots; thread t owns
  // labels [t per, (t + 1) per)
  {
    const int per = (K + kSortThreads - 1) / kSortThreads;
    const int j0 = min(K, tid * per), j1 = min(K, j0 + per);
    uint32_t loc = 0;
    for (int j = j0; j < j1; ++j) {
      uint32_t run = 0;
#pragma unroll
      for (int w = 0; w < kSortWaves; ++w) {
        const uint32_t c = s_cnt[w][j];
        s_cnt[w][j] = (uint16_t)run;
        run += c;
      }
      s_start[j] = run;
      loc += run;
    }
    uint32_t total;
    uint32_t run = scan1024_excl(loc, s_tmp, total);
    for (int j = j0; j < j1; ++j) {
      const uint32_t c = s_start[j];
      s_start[j] = run;
      run += c;
    }
    if (tid == 0) s_start[K] = total;
  }
  __syncthreads();
  int32_t* cst = a.cstart + ((size_t)bh * a.nseg + s) * (K + 1);
  for (int j = tid; j <= K; j += kSortThreads) cst[j] = (int32_t)s_start[j];
  int32_t* order = a.order + (size_t)bh * a.L0 + sg.lo;
#pragma unroll
  for (int k = 0; k < kSortBlocks; ++k) {
    if (packed[k] != 0xffffffffu) {
      const uint32_t l = packed[k] & 0xffffu;
      order[s_start[l] + s_cnt[wave][l] + (packed[k] >> 16)] = wave * cs + 64 * k + lane;
    }
  }
}

// ------------------------------------------------------------------------------------
// update: mu_j = bf16(u_j / ||u_j||), u_j = sum of member unit keys (position order)
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_update(BuildArgs a, const uint16_t* __restrict__ mu_in,
                                                uint16_t* __restrict__ mu_out) {
  const int s = a.seg0 + blockIdx.y, bh = blockIdx.z;
  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int j = blockIdx.x * 16 + grp;
  if (j >= a.kseg) return;
  const Seg sg = seg_range(a, s);
  const int32_t* cst = a.cstart + ((size_t)bh * a.nseg + s) * (a.kseg + 1);
  const int cs = cst[j], ce = cst[j + 1];
  const int32_t* order = a.order + (size_t)bh * a.L0 + sg.lo;
  const size_t krow0 = (size_t)bh * a.Lcap;
  const float* inv = a.inv_norm + (size_t)bh * a.L0;
  float u[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) u[d] = 0.f;
  // members in batches of 16: lane c of the group loads the batch's c-th member index, and
  // then all 16 rows are loaded at once (a batch past the last member repeats it with
  // weight 0), so a batch costs two dependent memory round trips
  for (int r = cs; r < ce; r += 16) {
    const int nm = min(16, ce - r);
    const int mine = order[r + min(c, nm - 1)];
    u32x4 kr[16];
    float iv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t p = sg.lo + __shfl(mine, min(e, nm - 1), 16);
      kr[e] = ld16(a.k + (krow0 + p) * kHeadDim + c * 8);
      iv[e] = e < nm ? inv[p] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u[2 * d] += bf_lo(kr[e][d]) * iv[e];
        u[2 * d + 1] += bf_hi(kr[e][d]) * iv[e];
      }
  }
  const size_t mrow = ((size_t)bh * a.C + (size_t)s * a.kseg + j) * kHeadDim + c * 8;
  u32x4 out;
  if (ce > cs) {
    float ss = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) ss += u[d] * u[d];
    ss = sum16(ss);
    const float nrm = sqrtf(ss);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      out[d] = nrm > 0.f ? pack_bf2(u[2 * d] / nrm, u[2 * d + 1] / nrm) : 0u;
  } else {
    out = ld16(mu_in + mrow);
  }
  st16(mu_out + mrow, out);
}

// ------------------------------------------------------------------------------------
// finalise: sizes, offsets, mean key, value sum, permuted K/V rows, labels, perm
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_finalise(BuildArgs a) {
  const int s = a.seg0 + blockIdx.y, bh = blockIdx.z;
  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int j = blockIdx.x * 16 + grp;
  if (j >= a.kseg) return;
  const Seg sg = seg_range(a, s);
  const int32_t* cst = a.cstart + ((size_t)bh * a.nseg + s) * (a.kseg + 1);
  const int cs = cst[j], ce = cst[j + 1];
  const int32_t* order = a.order + (size_t)bh * a.L0 + sg.lo;
  const size_t row0 = (size_t)bh * a.Lcap;
  const float* inv = a.inv_norm + (size_t)bh * a.L0;
  const int gid = s * a.kseg + j;
  float uk[8], ux[8], uv[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) uk[d] = ux[d] = uv[d] = 0.f;
  // members in batches of 8, as in the update: the batch's member indices in one load,
  // then all its key and value rows at once (a batch past the last member repeats it, and
  // the repeats are skipped)
  for (int r = cs; r < ce; r += 8) {
    const int nm = min(8, ce - r);
    const int mine = order[r + min(c & 7, nm - 1)];
    u32x4 kr[8], vr[8];
    float iv[8];
    int64_t pp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pp[e] = sg.lo + __shfl(mine, min(e, nm - 1), 16);
      kr[e] = ld16(a.k + (row0 + pp[e]) * kHeadDim + c * 8);
      vr[e] = ld16(a.v + (row0 + pp[e]) * kHeadDim + c * 8);
      iv[e] = inv[pp[e]];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= nm) continue;
      const int64_t slot = sg.lo + r + e;
      st16(a.k_out + (row0 + slot) * kHeadDim + c * 8, kr[e]);
      st16(a.v_out + (row0 + slot) * kHeadDim + c * 8, vr[e]);
      if (c == 0 && a.perm) a.perm[(size_t)bh * a.L0 + slot] = (int32_t)pp[e];
      if (c == 1 && a.labels) a.labels[(size_t)bh * a.L0 + pp[e]] = gid;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float k0 = bf_lo(kr[e][d]), k1 = bf_hi(kr[e][d]);
        uk[2 * d] += k0;
        uk[2 * d + 1] += k1;
        ux[2 * d] += k0 * iv[e];
        ux[2 * d + 1] += k1 * iv[e];
        uv[2 * d] += bf_lo(vr[e][d]);
        uv[2 * d + 1] += bf_hi(vr[e][d]);
      }
    }
  }
  const int cnt = ce - cs;
  const size_t crow = ((size_t)bh * a.C + gid) * kHeadDim + c * 8;
  u32x4 cm = {0, 0, 0, 0}, vs = {0, 0, 0, 0};
  if (cnt > 0) {
    const float fn = (float)cnt;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      cm[d] = pack_bf2(uk[2 * d] / fn, uk[2 * d + 1] / fn);
      vs[d] = pack_bf2(uv[2 * d], uv[2 * d + 1]);
    }
  }
  st16(a.cmean + crow, cm);
  st16(a.vsum + crow, vs);
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) ss += ux[d] * ux[d];
  ss = sum16(ss);
  if (c == 0) {
    a.csize[(size_t)bh * a.C + gid] = cnt;
    a.coff[(size_t)bh * a.C + gid] = (int32_t)(sg.lo + cs);
    a.cnorm[(size_t)bh * a.C + gid] = sqrtf(ss);
  }
}

// steady rows stay in place: copy them, label -1, perm = identity. An extension leaves the
// sink rows of k_out / v_out as the earlier build wrote them (and does not read them from k,
// v), and still writes their labels and perm.
__global__ __launch_bounds__(256) void k_steady(BuildArgs a) {
  const int bh = blockIdx.y;
  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int64_t n = (int64_t)a.n_sink + a.n_recent;
  for (int64_t t = (int64_t)blockIdx.x * 16 + grp; t < n; t += (int64_t)gridDim.x * 16) {
    const int64_t p = t < a.n_sink ? t : a.L0 - a.n_recent + (t - a.n_sink);
    const size_t row = ((size_t)bh * a.Lcap + p) * kHeadDim + c * 8;
    if (!(a.extend && t < a.n_sink)) {
      st16(a.k_out + row, ld16(a.k + row));
      st16(a.v_out + row, ld16(a.v + row));
    }
    if (c == 0 && a.perm) a.perm[(size_t)bh * a.L0 + p] = (int32_t)p;
    if (c == 1 && a.labels) a.labels[(size_t)bh * a.L0 + p] = -1;
  }
}

// objective J = sum over clusters of ||u_j|| (fixed summation order)
__global__ __launch_bounds__(256) void k_objective(BuildArgs a) {
  const int bh = blockIdx.x;
  __shared__ float s_part[256];
  float acc = 0.f;
  for (int j = threadIdx.x; j < a.C; j += 256) acc += a.cnorm[(size_t)bh * a.C + j];
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s_part[threadIdx.x] += s_part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.objective[bh] = s_part[0];
}

// blocks of an earlier index copied into a larger one: blockIdx.y = (b, kv-head), z = block
__global__ __launch_bounds__(256) void k_copy_blocks(CopyArgs c) {
  const CopyBlock& b = c.blk[blockIdx.z];
  const int bh = blockIdx.y;
  const uint32_t* src = b.src + (size_t)bh * b.src_stride;
  uint32_t* dst = b.dst + (size_t)bh * b.dst_stride;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < b.words;
       i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy_blocks(const CopyArgs& c, hipStream_t st, Tracer* tr) {
  if (c.n <= 0) return hipSuccess;
  int64_t most = 0;
  for (int i = 0; i < c.n; ++i) most = std::max(most, c.blk[i].words);
  const int nx = (int)std::max<int64_t>(1, std::min<int64_t>((most + 255) / 256, 1024));
  return launch(tr, k_copy_blocks, dim3(nx, c.BH, c.n), dim3(256), 0, st, c);
}

// ------------------------------------------------------------------------------------
hipError_t launch_build(const BuildArgs& a, hipStream_t st, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  // segments [seg0, nseg) are built (seg0 > 0: an extension of an earlier index)
  const int nsb = a.nseg - a.seg0;
  const int64_t nidx = a.idx_hi - std::max(a.idx_lo, (int64_t)a.seg0 * a.S);
  const dim3 gseg((a.kseg + 15) / 16, nsb, BH);
  hipError_t e;
#define WAVE_TRY(X)                 \
  do {                              \
    e = (X);                        \
    if (e != hipSuccess) return e;  \
  } while (0)
  // an extension by nothing (n_recent = 0 and an unchanged length that ends a segment)
  // builds no segment: only the steady rows' labels and perm below
  if (nsb > 0) {
  if (nidx > 0) {
    const int nb = (int)std::min<int64_t>((nidx + 15) / 16, 4096);
    WAVE_TRY(launch(tr, k_norms, dim3(nb, BH), dim3(256), 0, st, a));
  }
  WAVE_TRY(launch(tr, k_seeds, gseg, dim3(256), 0, st, a, a.mu[0]));
  const dim3 gasg((a.S + kAsgPoints - 1) / kAsgPoints, nsb, BH);
  // segment-resident assignment when a segment's centroids fit in LDS; enough splits of
  // each segment to give every CU a workgroup
  const bool seg_res = a.kseg <= kA2MaxK;
  const int nsplit = std::max(1, std::min((a.S + 63) / 64, (256 + nsb * BH - 1) / (nsb * BH)));
  // centroid rows, then the block counter
  const size_t lds2 = (size_t)((std::min(a.kseg, a.S) + 31) & ~31) * kAsgLdsStride + 16;
  if (seg_res) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&k_assign_seg), hipFuncAttributeMaxDynamicSharedMemorySize,
        kA2MaxK * kAsgLdsStride + 16);
    if (attr != hipSuccess) return attr;
  }
  for (int t = 1; t <= a.T; ++t) {
    const uint16_t* cur = a.mu[(t - 1) & 1];
    if (seg_res)
      WAVE_TRY(launch(tr, k_assign_seg, dim3(nsplit, nsb, BH), dim3(kA2Threads),
                      (uint32_t)lds2, st, a, cur, nsplit));
    else
      WAVE_TRY(launch(tr, k_assign, gasg, dim3(256), 0, st, a, cur));
    WAVE_TRY(launch(tr, k_sort, dim3(nsb, BH), dim3(kSortThreads), 0, st, a));
    if (t < a.T) WAVE_TRY(launch(tr, k_update, gseg, dim3(256), 0, st, a, cur, a.mu[t & 1]));
  }
  WAVE_TRY(launch(tr, k_finalise, gseg, dim3(256), 0, st, a));
  }
  if (a.n_sink + a.n_recent > 0) {
    const int nb = (int)std::min<int64_t>(((int64_t)a.n_sink + a.n_recent + 15) / 16, 1024);
    WAVE_TRY(launch(tr, k_steady, dim3(nb, BH), dim3(256), 0, st, a));
  }
  if (a.objective) WAVE_TRY(launch(tr, k_objective, dim3(BH), dim3(256), 0, st, a));
  if (a.last_mu && nsb > 0) {
    // clusters [seg0 k_seg, C) of every (b, kv-head): the ones this call built
    const size_t row = kHeadDim * sizeof(uint16_t), c0 = (size_t)a.seg0 * a.kseg;
    WAVE_TRY(hipMemcpy2DAsync(a.last_mu + c0 * kHeadDim, (size_t)a.C * row,
                              a.mu[(a.T - 1) & 1] + c0 * kHeadDim, (size_t)a.C * row,
                              (a.C - c0) * row, BH, hipMemcpyDeviceToDevice, st));
  }
#undef WAVE_TRY
  return hipSuccess;
}

}  // namespace wave
