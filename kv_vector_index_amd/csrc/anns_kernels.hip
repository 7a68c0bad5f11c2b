// Attention-aware vector search for gfx950: the graph built from training queries and the
// beam search of a decode step (the retrieval of the RetrievalAttention abstract, jarxiv.com:
// an index over the KV vectors, searched per decode step, whose structure follows the
// distribution of the queries rather than of the keys).
//
// Build, per (b, kv-head), over the N keys of the indexed zone (node x = position n_sink + x):
//   1. k_anns_lists: each training query's M best nodes by inner product, best first (ties
//      to the lower id). The scores come from v_mfma_f32_16x16x32_bf16 (keys as A rows,
//      64 training queries as four B column tiles, 128 nodes per batch with the next batch's
//      loads in flight, last position first); every training query keeps its candidates
//      that reach its current M-th score in LDS and sorts them down to M when the buffer
//      fills.
//   2. k_anns_count / k_anns_scan / k_anns_scatter: the postings of every node (its place in
//      each list that holds it, with the list), grouped by node.
//   3. k_anns_link: each node's neighbours, at most R without repeats, in the order of its
//      postings by (place, list): where it heads a list, the list's other nodes in list
//      order, else the list's head. Each list's head is also the training query's entry.
// Search, one 1024-thread workgroup per (b, kv-head) (k_anns_search): the search vector is
// the fp32 sum of the group's query rows; every score is an fp32 dot product in a fixed order
// (blocks of 8 dims in order, then a pairwise tree of the block sums) without fused
// multiply-adds, so that each decision is reproducible exactly. The pool starts from the entries of the n_entry training queries nearest the
// search vector and each round expands the W best unexpanded pool entries: their unvisited
// neighbours are scored, sorted and merged into the pool, which keeps its ef best entries.
#include "wave_common.h"

#include <limits.h>

namespace wave {
namespace {

constexpr int kAnnsListSortN = 128;    // a training query's candidates sort as 128 entries

// best-first order: higher score, then lower id (no short-circuit: both operands are
// evaluated, so the compiler keeps the comparisons free of branches)
__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
  return (sa > sb) | ((sa == sb) & (ia < ib));
}

// ------------------------------------------------------------------------------------
// 1. training lists: one wave per 64 training queries
// ------------------------------------------------------------------------------------
struct ListLds {
  float s[kAnnsListQueries][kAnnsListCap];
  int32_t id[kAnnsListQueries][kAnnsListCap];
  int32_t cnt[kAnnsListQueries];
  float theta[kAnnsListQueries];       // the M-th best score so far (-inf until M are held)
};
static_assert(kAnnsListCap <= kAnnsListSortN && kAnnsListSortN == 128, "list sort size");
static_assert(kAnnsMaxList <= 64, "a list fits one entry per lane");

// Sort training query qq's candidates best first and keep the first M; the M-th score
// becomes its threshold. Called by the whole wave.
__device__ void compact_list(ListLds& L, int qq, int M) {
  const int lane = threadIdx.x;
  const int cnt = L.cnt[qq];
  float s[2];
  int id[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = lane + 64 * h;
    s[h] = p < cnt ? L.s[qq][p] : kNegInf;
    id[h] = p < cnt ? L.id[qq][p] : INT_MAX;
  }
  // bitonic sort of the 128 positions p = lane (h = 0) and lane + 64 (h = 1)
#pragma unroll
  for (int k = 2; k <= kAnnsListSortN; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j == 64) {   // (k = 128: one ascending block) partner = the lane's other entry
        if (better(s[1], id[1], s[0], id[0])) {
          const float ts = s[0]; s[0] = s[1]; s[1] = ts;
          const int ti = id[0]; id[0] = id[1]; id[1] = ti;
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int p = lane + 64 * h;
          const float ps = __shfl_xor(s[h], j);
          const int pi = __shfl_xor(id[h], j);
          const bool lower = (p & j) == 0, up = (p & k) == 0;
          // the lower position of an ascending block keeps the better entry
          if ((lower == up) != better(s[h], id[h], ps, pi)) {
            s[h] = ps;
            id[h] = pi;
          }
        }
      }
    }
  }
  const int keep = min(cnt, M);
  const float th = __shfl(s[0], max(M - 1, 0));
  __syncthreads();
  if (lane < keep) {
    L.s[qq][lane] = s[0];
    L.id[qq][lane] = id[0];
  }
  if (lane == 0) {
    L.cnt[qq] = keep;
    L.theta[qq] = keep == M ? th : kNegInf;
  }
  __syncthreads();
}

__global__ __launch_bounds__(64) void k_anns_lists(AnnsArgs a) {
  typedef __attribute__((ext_vector_type(4))) float floatx4;
  __shared__ ListLds L;
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  // (workgroups are dealt to the eight XCDs in turn: with bh = index mod BH, the workgroups
  // of one (b, kv-head) share an XCD and its L2 while they stream the same keys)
  const int BH = a.B * a.Hkv;
  const int bh = blockIdx.x % BH;
  const int t0 = (blockIdx.x / BH) * kAnnsListQueries;
  const int N = a.N, M = a.M;
  // B operands: training query t0 + 16 c + n, dims 32 s4 + 8 g .. + 7
  bf16x8 qb[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = t0 + 16 * c + n;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      qb[c][s4] = __builtin_bit_cast(
          bf16x8, t < a.n_t ? ld16(a.train + ((size_t)bh * a.n_t + t) * kHeadDim + s4 * 32 + g * 8)
                            : u32x4{0, 0, 0, 0});
  }
  // (a column past the last training query never takes a candidate)
  L.cnt[lane] = 0;
  L.theta[lane] = t0 + lane < a.n_t ? kNegInf : __builtin_huge_valf();
  __syncthreads();
  float th[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) th[c] = L.theta[16 * c + n];
  const uint16_t* kb = a.k + ((size_t)bh * a.Lcap + a.n_sink) * kHeadDim;
  // A operands: node N - 1 - (base + n), dims 32 s4 + 8 g .. + 7, in batches of TB tiles of
  // 16 nodes; the next batch's loads are in flight while a batch is scored. The nodes stream
  // from the last position back (the training queries' best keys tend to lie near their own
  // positions at the end, so the thresholds rise early); every new node then has a lower id
  // than the nodes held, so it enters exactly when its score reaches the threshold.
  constexpr int TB = 8;
  u32x4 ka[TB][4], kn[TB][4];
  auto load_batch = [&](int base, u32x4 (&dst)[TB][4]) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int xr = base + 16 * j + n;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        dst[j][s4] = xr < N ? ld16(kb + (size_t)(N - 1 - xr) * kHeadDim + s4 * 32 + g * 8)
                            : u32x4{0, 0, 0, 0};
    }
  };
  load_batch(0, ka);
  for (int base = 0; base < N; base += 16 * TB) {
    load_batch(base + 16 * TB, kn);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int tb = base + 16 * j;
      if (tb >= N) break;
      floatx4 d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          d[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[j][s4]),
                                                         qb[c][s4], d[c], 0, 0, 0);
      }
      // lane (g, n) holds nodes N - 1 - (tb + 4 g + i) against training queries 16 c + n;
      // once the lists are full most tiles reach no threshold and skip the bookkeeping
      bool hit = false;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) hit |= tb + 4 * g + i < N && d[c][i] >= th[c];
      if (!__ballot(hit)) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int xr = tb + 4 * g + i;
          if (xr < N && d[c][i] >= th[c]) {
            const int qq = 16 * c + n;
            const int p = atomicAdd(&L.cnt[qq], 1);
            L.s[qq][p] = d[c][i];
            L.id[qq][p] = N - 1 - xr;
          }
        }
      __syncthreads();
      // a buffer that might not take the next tile's 16 is sorted down to M
      uint64_t need = __ballot(L.cnt[lane] > kAnnsListCap - 16);
      if (need) {
        while (need) {
          const int qq = __builtin_ctzll(need);
          need &= need - 1;
          compact_list(L, qq, M);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) th[c] = L.theta[16 * c + n];
      }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) ka[j][s4] = kn[j][s4];
  }
  for (int qq = 0; qq < kAnnsListQueries && t0 + qq < a.n_t; ++qq) {
    compact_list(L, qq, M);
    const int t = t0 + qq;
    if (lane < M)
      a.lists[((size_t)bh * a.n_t + t) * M + lane] = lane < L.cnt[qq] ? L.id[qq][lane] : -1;
  }
}

// ------------------------------------------------------------------------------------
// 2. postings grouped by node, 3. links
// ------------------------------------------------------------------------------------
__global__ void k_anns_zero(AnnsArgs a) {
  const size_t n = (size_t)a.B * a.Hkv * a.N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    a.cnt[i] = 0;
}

// one thread per list entry: the node's posting count; a list's first entry is its entry
__global__ void k_anns_count(AnnsArgs a) {
  const size_t per = (size_t)a.n_t * a.M;
  const size_t n = (size_t)a.B * a.Hkv * per;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int bh = (int)(e / per);
  const int rem = (int)(e - (size_t)bh * per), t = rem / a.M, r = rem - t * a.M;
  const int x = a.lists[e];
  if (r == 0) a.entry[(size_t)bh * a.n_t + t] = x;
  if (x >= 0 && x < a.N) atomicAdd(&a.cnt[(size_t)bh * a.N + x], 1);
}

// one workgroup per (b, kv-head): off = exclusive scan of the counts (off[N] = total); the
// counts go back to zero for the scatter's cursors
__global__ __launch_bounds__(1024) void k_anns_scan(AnnsArgs a) {
  __shared__ ScanTmp<1024> tmp;
  const int bh = blockIdx.x, tid = threadIdx.x;
  int32_t* cnt = a.cnt + (size_t)bh * a.N;
  int32_t* off = a.off + (size_t)bh * (a.N + 1);
  uint32_t carry = 0;
  for (int base = 0; base < a.N; base += 4 * 1024) {
    uint32_t v[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + 4 * tid + j;
      v[j] = i < a.N ? (uint32_t)cnt[i] : 0u;
      sum += v[j];
    }
    uint32_t total;
    uint32_t run = carry + scan_excl<1024>(sum, tmp, &total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + 4 * tid + j;
      if (i < a.N) {
        off[i] = (int32_t)run;
        cnt[i] = 0;
      }
      run += v[j];
    }
    carry += total;
  }
  if (tid == 0) off[a.N] = (int32_t)carry;
}

__global__ void k_anns_scatter(AnnsArgs a) {
  const size_t per = (size_t)a.n_t * a.M;
  const size_t n = (size_t)a.B * a.Hkv * per;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int bh = (int)(e / per);
  const int rem = (int)(e - (size_t)bh * per), t = rem / a.M, r = rem - t * a.M;
  const int x = a.lists[e];
  if (x < 0 || x >= a.N) return;
  const int p = a.off[(size_t)bh * (a.N + 1) + x] + atomicAdd(&a.cnt[(size_t)bh * a.N + x], 1);
  a.post[(size_t)bh * per + p] = (r << kAnnsPlaceShift) | t;
}

// one thread per node: take its postings in (place, list) order (the smallest key above the
// last one taken, by a scan of the node's postings) until R neighbours are held
__global__ void k_anns_link(AnnsArgs a) {
  const size_t n = (size_t)a.B * a.Hkv * a.N;
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int bh = (int)(e / a.N), x = (int)(e - (size_t)bh * a.N);
  const int32_t* off = a.off + (size_t)bh * (a.N + 1);
  const int32_t* post = a.post + (size_t)bh * a.n_t * a.M;
  const int32_t* lists = a.lists + (size_t)bh * a.n_t * a.M;
  int32_t* row = a.graph + e * a.R;
  const int p0 = off[x], p1 = off[x + 1];
  int taken = 0, last = -1;
  auto add = [&](int y) {
    if (y < 0) return;
    for (int j = 0; j < taken; ++j)
      if (row[j] == y) return;
    row[taken++] = y;
  };
  while (taken < a.R) {
    int key = INT_MAX;
    for (int p = p0; p < p1; ++p) {
      const int v = post[p];
      if (v > last && v < key) key = v;
    }
    if (key == INT_MAX) break;
    last = key;
    const int r = key >> kAnnsPlaceShift, t = key & ((1 << kAnnsPlaceShift) - 1);
    const int32_t* lt = lists + (size_t)t * a.M;
    if (r == 0) {
      for (int j = 1; j < a.M && taken < a.R; ++j) add(lt[j]);
    } else {
      add(lt[0]);
    }
  }
  for (int j = taken; j < a.R; ++j) row[j] = -1;
}

// ------------------------------------------------------------------------------------
// search
// ------------------------------------------------------------------------------------
// Dot product of u with a bf16 row by the 16 lanes of a DPP row: lane j holds u's dims
// 8 j .. 8 j + 7 (uj) and the row's 16 bytes at the same dims (r). Its 8 products are summed
// in dim order, then the 16 block sums pairwise, neighbours first (lane ^ 1, lane ^ 2, then the
// half-row and row mirrors); every product and sum is rounded to fp32 (no fused
// multiply-add), and every lane of the row receives the score.
__device__ __forceinline__ float group_dot(const float (&uj)[8], const u32x4& r) {
#pragma clang fp contract(off)
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p0 = uj[2 * e] * bf_lo(w[e]);
    acc = acc + p0;
    const float p1 = uj[2 * e + 1] * bf_hi(w[e]);
    acc = acc + p1;
  }
  return sum16(acc);
}

// Scores of the rows base + ids[c] * d for c < n into sc[c], by the 16-lane groups of the
// workgroup, U rows per group at a time (their loads in flight together). With adj, each
// node's neighbour list (R entries from adj + id * R) is read too, so that it is in the
// cache if the node is expanded in a later round; the values fold into *sink.
template <int NT, int U>
__device__ __forceinline__ void score_rows(const float (&uj)[8], const uint16_t* base,
                                           const int32_t* ids, float* sc, int n,
                                           const int32_t* adj = nullptr, int R = 0,
                                           int32_t* sink = nullptr) {
  constexpr int kG = NT / 16;
  const int grp = threadIdx.x >> 4, j = threadIdx.x & 15;
  for (int c0 = grp; c0 < n; c0 += U * kG) {
    u32x4 r[U];
    int32_t nb[U];
#pragma unroll
    for (int m = 0; m < U; ++m) {
      const int c = c0 + m * kG;
      const int id = c < n ? (ids ? ids[c] : c) : 0;
      r[m] = c < n ? ld16(base + (size_t)id * kHeadDim + 8 * j) : u32x4{0, 0, 0, 0};
      nb[m] = adj && c < n ? adj[(size_t)id * R + min(4 * j, R - 1)] : 0;
    }
    if (adj) {
#pragma unroll
      for (int m = 0; m < U; ++m) *sink ^= nb[m];
    }
#pragma unroll
    for (int m = 0; m < U; ++m) {
      const int c = c0 + m * kG;
      if (c < n) {
        const float v = group_dot(uj, r[m]);
        if (j == 0) sc[c] = v;
      }
    }
  }
}

// Sort entries [c0, c0 + 64) of (es, ei) best first across the lanes of one wave (entries
// from n on count as worst and stay unwritten): a bitonic network over lane exchanges.
__device__ __forceinline__ void wave_sort64(float* es, int32_t* ei, int c0, int n) {
  const int lane = threadIdx.x & 63, p = c0 + lane;
  float v = p < n ? es[p] : kNegInf;
  int i = p < n ? ei[p] : INT_MAX;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float pv = __shfl_xor(v, j);
      const int pi = __shfl_xor(i, j);
      const bool lower = (lane & j) == 0, up = (lane & k) == 0;
      // the lower lane of an ascending block keeps the better entry
      if ((lower == up) != better(v, i, pv, pi)) {
        v = pv;
        i = pi;
      }
    }
  }
  if (p < n) {
    es[p] = v;
    ei[p] = i;
  }
}

// The number of entries of the sorted run (es, ei)[c0, c0 + m) better than (s, id).
__device__ __forceinline__ int count_better_sorted(const float* es, const int32_t* ei, int c0,
                                                   int m, float s, int id) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (better(es[c0 + mid], ei[c0 + mid], s, id)) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// The entries among (es, ei)[0, n) (in any order) better than (s, id): four per LDS read.
__device__ __forceinline__ int count_better_all(const float* es, const int32_t* ei, int n,
                                                float s, int id) {
  int cnt = 0, c = 0;
#pragma unroll 4
  for (; c + 4 <= n; c += 4) {
    const float4 s4 = *reinterpret_cast<const float4*>(es + c);
    const int4 i4 = *reinterpret_cast<const int4*>(ei + c);
    cnt += (int)better(s4.x, i4.x, s, id) + (int)better(s4.y, i4.y, s, id) +
           (int)better(s4.z, i4.z, s, id) + (int)better(s4.w, i4.w, s, id);
  }
  for (; c < n; ++c) cnt += (int)better(es[c], ei[c], s, id);
  return cnt;
}

// The entries of (es, ei)[0, n), made of sorted runs of `run` entries, better than (s, id),
// leaving out the run that starts at `skip` (none when skip < 0).
__device__ __forceinline__ int count_better_runs(const float* es, const int32_t* ei, int n,
                                                 int run, int skip, float s, int id) {
  int cnt = 0;
  for (int c0 = 0; c0 < n; c0 += run)
    if (c0 != skip) cnt += count_better_sorted(es, ei, c0, min(run, n - c0), s, id);
  return cnt;
}

// The rank of entry e of (es, ei)[0, n), made of sorted runs of `run` entries: its place in
// its own run plus the entries better than it in each other run.
__device__ __forceinline__ int rank_in_runs(const float* es, const int32_t* ei, int n, int run,
                                            int e) {
  return e % run + count_better_runs(es, ei, n, run, e - e % run, es[e], ei[e]);
}

// the search vector u of (b, kv-head): the group's query rows summed in fp32, head by head;
// this lane's 8 dims (8 (lane & 15) ..) into uj. Needs 128 floats of LDS and a barrier.
__device__ __forceinline__ void search_vector(const AnnsArgs& a, int bh, float* u,
                                              float (&uj)[8]) {
  const int b = bh / a.Hkv, g = bh % a.Hkv;
  if (threadIdx.x < kHeadDim) {
    const uint16_t* q = a.q + (size_t)(b * a.Hq + g * a.G) * kHeadDim + threadIdx.x;
    float v = __uint_as_float((uint32_t)q[0] << 16);
    for (int h = 1; h < a.G; ++h) v = v + __uint_as_float((uint32_t)q[(size_t)h * kHeadDim] << 16);
    u[threadIdx.x] = v;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) uj[e] = u[8 * (threadIdx.x & 15) + e];
}

// ---- seeds: workgroup x of (b, kv-head) scores training queries [x chunk, (x + 1) chunk)
// and keeps its n_entry best, best first (score descending, id ascending; -inf / INT_MAX
// pads)
constexpr int kSeedThreads = 256;
__global__ __launch_bounds__(kSeedThreads) void k_anns_seed(AnnsArgs a) {
  __shared__ float u[kHeadDim];
  __shared__ float sc[kAnnsMaxTrain / kAnnsMaxSeedWG];
  __shared__ int32_t sid[kAnnsMaxTrain / kAnnsMaxSeedWG];
  const int bh = blockIdx.y, x = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float uj[8];
  search_vector(a, bh, u, uj);
  const int t0 = x * a.seed_chunk, n = max(0, min(a.n_t - t0, a.seed_chunk));
  score_rows<kSeedThreads, 8>(uj, a.train + ((size_t)bh * a.n_t + t0) * kHeadDim, nullptr, sc,
                              n);
  for (int c = threadIdx.x; c < n; c += kSeedThreads) sid[c] = t0 + c;
  __syncthreads();
  for (int c0 = 64 * wave; c0 < n; c0 += kSeedThreads) wave_sort64(sc, sid, c0, n);
  __syncthreads();
  // the n_entry best by rank among the sorted runs of 64; padding where n < n_entry
  float* out_s = a.seed_s + ((size_t)bh * kAnnsMaxSeedWG + x) * a.n_entry;
  int32_t* out_i = a.seed_i + ((size_t)bh * kAnnsMaxSeedWG + x) * a.n_entry;
  for (int c = threadIdx.x; c < n; c += kSeedThreads) {
    const int r = rank_in_runs(sc, sid, n, 64, c);
    if (r < a.n_entry) {
      out_s[r] = sc[c];
      out_i[r] = sid[c];
    }
  }
  for (int r = n + threadIdx.x; r < a.n_entry; r += kSeedThreads) {
    out_s[r] = kNegInf;
    out_i[r] = INT_MAX;
  }
  (void)lane;
}

constexpr int32_t kExpanded = (int32_t)0x80000000;   // pool id flag: expanded
constexpr int kCtrCand = 0, kCtrVisited = 1, kCtrScan = 16;   // LDS counters

__global__ __launch_bounds__(kAnnsSearchThreads) void k_anns_search(AnnsArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  float* u = reinterpret_cast<float*>(lds);
  int32_t* sel = reinterpret_cast<int32_t*>(lds + kHeadDim * 4);
  int32_t* ctr = sel + kAnnsMaxExpand;
  ScanTmp<kAnnsSearchThreads>& scan = *reinterpret_cast<ScanTmp<kAnnsSearchThreads>*>(ctr + kCtrScan);
  float* cs = reinterpret_cast<float*>(ctr + 32);
  int32_t* ci = reinterpret_cast<int32_t*>(cs + kAnnsMaxCand);
  const uint32_t ps = anns_pool_stride(a.ef);
  float* pS[2] = {reinterpret_cast<float*>(lds + kAnnsLdsFixed),
                  reinterpret_cast<float*>(lds + kAnnsLdsFixed + 8 * ps)};
  int32_t* pI[2] = {reinterpret_cast<int32_t*>(lds + kAnnsLdsFixed + 4 * ps),
                    reinterpret_cast<int32_t*>(lds + kAnnsLdsFixed + 12 * ps)};
  uint32_t* vis = reinterpret_cast<uint32_t*>(lds + kAnnsLdsFixed + 16 * ps);
  static_assert(kAnnsSearchThreads / 64 <= 16, "scan words fit the counters");
  static_assert(kAnnsMaxSeedWG * kAnnsMaxEntry <= kAnnsMaxCand, "seed candidates fit");

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int N = a.N, E = a.n_entry;
  const uint16_t* kb = a.k + ((size_t)bh * a.Lcap + a.n_sink) * kHeadDim;

  for (int i = tid; i < (N + 31) / 32; i += kAnnsSearchThreads) vis[i] = 0u;
  if (tid < kCtrScan) ctr[tid] = 0;
  // the seed workgroups' candidates
  const int ns = a.nseed * E;
  for (int i = tid; i < ns; i += kAnnsSearchThreads) {
    const int w = i / E, e = i - w * E;
    cs[i] = a.seed_s[((size_t)bh * kAnnsMaxSeedWG + w) * E + e];
    ci[i] = a.seed_i[((size_t)bh * kAnnsMaxSeedWG + w) * E + e];
  }
  float uj[8];
  search_vector(a, bh, u, uj);          // (its barrier also publishes the candidates)
  // ---- seeds: the entries of the n_entry best training queries (rank among the candidates)
  int seed_t = INT_MAX;
  if (tid < ns) {   // (each seed workgroup's list is a sorted run of E)
    if (rank_in_runs(cs, ci, ns, E, tid) < E) seed_t = ci[tid];
  }
  __syncthreads();
  if (seed_t < a.n_t) {
    const int x = a.entry[(size_t)bh * a.n_t + seed_t];
    if (x >= 0 && x < N) {
      const uint32_t bit = 1u << (x & 31);
      if (!(atomicOr(&vis[x >> 5], bit) & bit)) ci[atomicAdd(&ctr[kCtrCand], 1)] = x;
    }
  }
  __syncthreads();

  int cur = 0, psize = 0, rounds = 0;
  int32_t sink = 0;
  for (;;) {
    // ---- the listed new nodes ci[0, nc): scored, sorted in runs of 64 (one wave each), then
    // merged into the pool by rank (a pool entry moves down by the new nodes better than it;
    // a new node lands after the pool entries and the new nodes better than it); the pool
    // keeps its ef best
    const int nv = ctr[kCtrCand];   // nodes scored this round
    int nc = nv;
    if (nv > 0) {
      score_rows<kAnnsSearchThreads, 4>(uj, kb, ci, cs, nv, a.graph + (size_t)bh * N * a.R,
                                        a.R, &sink);
      __syncthreads();
      if (psize == a.ef) {
        // a full pool keeps only nodes better than its last entry: the others are dropped
        // before the sort (they stay visited)
        const float ws = pS[cur][a.ef - 1];
        const int wid = pI[cur][a.ef - 1] & INT_MAX;
        float v0 = kNegInf, v1 = kNegInf;
        int i0 = 0, i1 = 0;
        uint32_t f0 = 0, f1 = 0;
        if (tid < nv) {
          v0 = cs[tid];
          i0 = ci[tid];
          f0 = better(v0, i0, ws, wid) ? 1u : 0u;
        }
        if (tid + kAnnsSearchThreads < nv) {
          v1 = cs[tid + kAnnsSearchThreads];
          i1 = ci[tid + kAnnsSearchThreads];
          f1 = better(v1, i1, ws, wid) ? 1u : 0u;
        }
        uint32_t total;
        const uint32_t at = scan_excl<kAnnsSearchThreads>(f0 + f1, scan, &total);
        if (f0) {
          cs[at] = v0;
          ci[at] = i0;
        }
        if (f1) {
          cs[at + f0] = v1;
          ci[at + f0] = i1;
        }
        nc = (int)total;
        __syncthreads();
      }
    }
    if (nc > 0) {
      // more than 64 new nodes: sorted runs of 64 and binary searches; else plain counts
      const bool runs = nc > 64;
      if (runs) {
        for (int c0 = 64 * (tid >> 6); c0 < nc; c0 += kAnnsSearchThreads)
          wave_sort64(cs, ci, c0, nc);
        __syncthreads();
      }
      const float* S = pS[cur];
      const int32_t* I = pI[cur];
      float* S2 = pS[cur ^ 1];
      int32_t* I2 = pI[cur ^ 1];
      for (int e = tid; e < psize + nc; e += kAnnsSearchThreads) {
        float sv;
        int32_t iv, id;
        int rank;
        if (e < psize) {
          sv = S[e];
          iv = I[e];
          id = iv & INT_MAX;
          rank = e;
        } else {
          sv = cs[e - psize];
          iv = id = ci[e - psize];
          int lo = 0, hi = psize;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (better(S[mid], I[mid] & INT_MAX, sv, id)) lo = mid + 1;
            else hi = mid;
          }
          rank = lo;
        }
        // the new nodes better than it (sorted runs of 64: its own run gives its place)
        rank += !runs ? count_better_all(cs, ci, nc, sv, id)
                      : count_better_runs(cs, ci, nc, 64, e < psize ? -1 : (e - psize) & ~63,
                                          sv, id) + (e < psize ? 0 : (e - psize) & 63);
        if (rank < a.ef) {
          S2[rank] = sv;
          I2[rank] = iv;
        }
      }
      cur ^= 1;
      psize = min(a.ef, psize + nc);
    }
    if (tid == 0) ctr[kCtrVisited] += nv;
    __syncthreads();
    if (rounds >= a.max_rounds) break;
    // ---- the W best unexpanded pool entries, in pool order
    const int32_t pid = tid < psize ? pI[cur][tid] : kExpanded;
    const uint32_t flag = pid >= 0 ? 1u : 0u;
    uint32_t total;
    const uint32_t rank = scan_excl<kAnnsSearchThreads>(flag, scan, &total);
    if (flag && rank < (uint32_t)a.W) {
      sel[rank] = pid;
      pI[cur][tid] = pid | kExpanded;
    }
    const int nsel = min((int)total, a.W);
    if (tid == 0) ctr[kCtrCand] = 0;
    __syncthreads();
    if (nsel == 0) break;
    ++rounds;
    // ---- their unvisited neighbours, listed
    for (int s = tid; s < nsel * a.R; s += kAnnsSearchThreads) {
      const int src = sel[s / a.R];
      const int y = a.graph[((size_t)bh * N + src) * a.R + s % a.R];
      if (y < 0 || y >= N) continue;
      const uint32_t bit = 1u << (y & 31);
      if (atomicOr(&vis[y >> 5], bit) & bit) continue;
      ci[atomicAdd(&ctr[kCtrCand], 1)] = y;
    }
    __syncthreads();
  }
  // ---- the k best pool entries
  for (int o = tid; o < a.n_ret; o += kAnnsSearchThreads)
    a.found_pos[(size_t)bh * a.n_ret + o] = o < psize ? (pI[cur][o] & INT_MAX) + a.n_sink : -1;
  atomicXor(&ctr[kCtrScan - 1], sink);   // (keeps every thread's neighbour-list reads)
  if (tid == 0) {
    a.found_n[bh] = min(a.n_ret, psize);
    if (a.stats) {
      a.stats[2 * bh] = rounds;
      a.stats[2 * bh + 1] = ctr[kCtrVisited];
    }
  }
}

}  // namespace

hipError_t launch_anns_build(const AnnsArgs& a, hipStream_t s, Tracer* tr) {
  const int BH = a.B * a.Hkv;
  hipError_t e = launch(tr, k_anns_lists,
                        dim3((a.n_t + kAnnsListQueries - 1) / kAnnsListQueries * BH), dim3(64), 0,
                        s, a);
  if (e != hipSuccess) return e;
  const size_t nodes = (size_t)BH * a.N, entries = (size_t)BH * a.n_t * a.M;
  const int nt = 256;
  if (nodes) {
    e = launch(tr, k_anns_zero, dim3((unsigned)std::min<size_t>((nodes + nt - 1) / nt, 4096)),
               dim3(nt), 0, s, a);
    if (e != hipSuccess) return e;
  }
  e = launch(tr, k_anns_count, dim3((unsigned)((entries + nt - 1) / nt)), dim3(nt), 0, s, a);
  if (e != hipSuccess || !nodes) return e;
  e = launch(tr, k_anns_scan, dim3(BH), dim3(1024), 0, s, a);
  if (e != hipSuccess) return e;
  e = launch(tr, k_anns_scatter, dim3((unsigned)((entries + nt - 1) / nt)), dim3(nt), 0, s, a);
  if (e != hipSuccess) return e;
  return launch(tr, k_anns_link, dim3((unsigned)((nodes + nt - 1) / nt)), dim3(nt), 0, s, a);
}

hipError_t launch_anns_search(const AnnsArgs& a, hipStream_t s, Tracer* tr) {
  hipError_t e = launch(tr, k_anns_seed, dim3(a.nseed, a.B * a.Hkv), dim3(kSeedThreads), 0, s,
                        a);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_anns_search),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)a.search_lds);
  if (e != hipSuccess) return e;
  return launch(tr, k_anns_search, dim3(a.B * a.Hkv), dim3(kAnnsSearchThreads), a.search_lds,
                s, a);
}

}  // namespace wave
