// Attention-aware vector search for gfx950: the graph built from training queries and the
// beam search of a decode step (the retrieval of the RetrievalAttention abstract, jarxiv.com:
// an index over the KV vectors, searched per decode step, whose structure follows the
// distribution of the queries rather than of the keys).
//
// Build, per (b, kv-head), over the N keys of the indexed zone (node x = position n_sink + x):
//   1. k_anns_lists: each training query's M best nodes by inner product, best first (ties
//      to the lower id). The scores come from v_mfma_f32_16x16x32_bf16 (keys as A rows,
//      64 training queries as four B column tiles); every training query keeps its candidates
//      above its current M-th score in LDS and sorts them down to M when the buffer fills.
//   2. k_anns_count / k_anns_scan / k_anns_scatter: the postings of every node (its place in
//      each list that holds it, with the list), grouped by node.
//   3. k_anns_link: each node's neighbours, at most R without repeats, in the order of its
//      postings by (place, list): where it heads a list, the list's other nodes in list
//      order, else the list's head. Each list's head is also the training query's entry.
// Search, one 1024-thread workgroup per (b, kv-head) (k_anns_search): the search vector is
// the fp32 sum of the group's query rows; every score is an fp32 dot product accumulated over
// the dims in order without fused multiply-adds, so that each decision is reproducible
// exactly. The pool starts from the entries of the n_entry training queries nearest the
// search vector and each round expands the W best unexpanded pool entries: their unvisited
// neighbours are scored, sorted and merged into the pool, which keeps its ef best entries.
#include "wave_common.h"

#include <limits.h>

namespace wave {
namespace {

constexpr int kAnnsListSortN = 128;    // a training query's candidates sort as 128 entries

// best-first order: higher score, then lower id
__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
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
  const int bh = blockIdx.y;
  const int t0 = blockIdx.x * kAnnsListQueries;
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
  L.cnt[lane] = 0;
  L.theta[lane] = kNegInf;
  __syncthreads();
  float th[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
  const uint16_t* kb = a.k + ((size_t)bh * a.Lcap + a.n_sink) * kHeadDim;
  // A operands: node base + n, dims 32 s4 + 8 g .. + 7 (one tile of 16 nodes, loaded a tile
  // ahead)
  u32x4 ka[4], kn[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
    ka[s4] = n < N ? ld16(kb + (size_t)n * kHeadDim + s4 * 32 + g * 8) : u32x4{0, 0, 0, 0};
  for (int base = 0; base < N; base += 16) {
    const int xn = base + 16 + n;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      kn[s4] = xn < N ? ld16(kb + (size_t)xn * kHeadDim + s4 * 32 + g * 8) : u32x4{0, 0, 0, 0};
    floatx4 d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        d[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[s4]),
                                                       qb[c][s4], d[c], 0, 0, 0);
    }
    // lane (g, n) holds nodes base + 4 g + i against training queries 16 c + n
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = base + 4 * g + i;
        if (x < N && t0 + 16 * c + n < a.n_t && d[c][i] > th[c]) {
          const int qq = 16 * c + n;
          const int p = atomicAdd(&L.cnt[qq], 1);
          L.s[qq][p] = d[c][i];
          L.id[qq][p] = x;
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
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) ka[s4] = kn[s4];
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
// fp32 dot product of u (d floats in LDS) with a bf16 row: products and sums rounded to
// fp32 one at a time, over the dims in order
__device__ __noinline__ float seq_dot(const float* u, const uint16_t* row) {
#pragma clang fp contract(off)
  u32x4 r[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) r[c] = ld16(row + c * 8);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint32_t w[4] = {r[c].x, r[c].y, r[c].z, r[c].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = u[c * 8 + 2 * e] * bf_lo(w[e]);
      acc = acc + p0;
      const float p1 = u[c * 8 + 2 * e + 1] * bf_hi(w[e]);
      acc = acc + p1;
    }
  }
  return acc;
}

// bitonic sort of (s, id)[0, n) best first, n padded to a power of two P with worst entries
// (whole workgroup)
__device__ void block_sort(float* s, int32_t* id, int n) {
  int P = 2;
  while (P < n) P <<= 1;
  for (int i = n + threadIdx.x; i < P; i += blockDim.x) {
    s[i] = kNegInf;
    id[i] = INT_MAX;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int pi = threadIdx.x; pi < P / 2; pi += blockDim.x) {
        const int lo = 2 * pi - (pi & (j - 1)), hi = lo + j;
        const bool up = (lo & k) == 0;   // an ascending block: the lower position is better
        const float sl = s[lo], sh = s[hi];
        const int il = id[lo], ih = id[hi];
        if (better(sh, ih, sl, il) == up) {
          s[lo] = sh; s[hi] = sl;
          id[lo] = ih; id[hi] = il;
        }
      }
      __syncthreads();
    }
  }
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x, b = bh / a.Hkv, g = bh % a.Hkv;
  const int N = a.N;
  const uint16_t* kb = a.k + ((size_t)bh * a.Lcap + a.n_sink) * kHeadDim;

  // search vector: the group's query rows summed in fp32, head by head
  if (tid < kHeadDim) {
    const uint16_t* q = a.q + (size_t)(b * a.Hq + g * a.G) * kHeadDim + tid;
    float v = __uint_as_float((uint32_t)q[0] << 16);
    for (int h = 1; h < a.G; ++h) v = v + __uint_as_float((uint32_t)q[(size_t)h * kHeadDim] << 16);
    u[tid] = v;
  }
  for (int i = tid; i < (N + 31) / 32; i += kAnnsSearchThreads) vis[i] = 0u;
  if (tid < kCtrScan) ctr[tid] = 0;
  __syncthreads();

  // ---- seeds: each wave's n_entry nearest training queries by repeated wave argmax, then
  // the best n_entry of those; their entries are scored
  constexpr int kTPT = kAnnsMaxTrain / kAnnsSearchThreads;   // training queries per thread
  const int E = a.n_entry;
  {
    float ts[kTPT];
#pragma unroll
    for (int j = 0; j < kTPT; ++j) {
      const int t = tid + j * kAnnsSearchThreads;
      ts[j] = t < a.n_t ? seq_dot(u, a.train + ((size_t)bh * a.n_t + t) * kHeadDim) : kNegInf;
    }
    uint32_t used = 0;
    for (int e = 0; e < E; ++e) {
      float bs = kNegInf;
      int bi = INT_MAX, bj = -1;
#pragma unroll
      for (int j = 0; j < kTPT; ++j) {
        const int t = tid + j * kAnnsSearchThreads;
        if (!((used >> j) & 1u) && t < a.n_t && better(ts[j], t, bs, bi)) {
          bs = ts[j];
          bi = t;
          bj = j;
        }
      }
      float ws = bs;
      int wi = bi;
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) {
        const float os = __shfl_xor(ws, m);
        const int oi = __shfl_xor(wi, m);
        if (better(os, oi, ws, wi)) {
          ws = os;
          wi = oi;
        }
      }
      if (bj >= 0 && bi == wi) used |= 1u << bj;
      if (lane == 0) {
        cs[wave * E + e] = ws;
        ci[wave * E + e] = wi;
      }
    }
  }
  __syncthreads();
  block_sort(cs, ci, (kAnnsSearchThreads / 64) * E);
  const int tseed = tid < E ? ci[tid] : INT_MAX;
  __syncthreads();
  if (tid < E && tseed < a.n_t) {
    const int x = a.entry[(size_t)bh * a.n_t + tseed];
    if (x >= 0 && x < N) {
      const uint32_t bit = 1u << (x & 31);
      if (!(atomicOr(&vis[x >> 5], bit) & bit)) {
        const float sc = seq_dot(u, kb + (size_t)x * kHeadDim);
        const int p = atomicAdd(&ctr[kCtrCand], 1);
        cs[p] = sc;
        ci[p] = x;
      }
    }
  }
  __syncthreads();

  int cur = 0, psize = 0, rounds = 0;
  for (;;) {
    // ---- the round's new nodes (ctr[kCtrCand] of them in cs, ci): sort, merge into the pool
    const int nc = ctr[kCtrCand];
    if (nc > 0) {
      block_sort(cs, ci, nc);
      const int out = min(a.ef, psize + nc);
      const float* S = pS[cur];
      const int32_t* I = pI[cur];
      for (int o = tid; o < out; o += kAnnsSearchThreads) {
        // co-rank: i pool entries and o - i new nodes precede output o
        int lo = max(0, o - nc), hi = min(o, psize);
        while (lo < hi) {
          const int mid = (lo + hi) >> 1, j = o - mid;
          if (better(S[mid], I[mid] & INT_MAX, cs[j - 1], ci[j - 1])) lo = mid + 1;
          else hi = mid;
        }
        const int i = lo, j = o - lo;
        const bool from_pool = i < psize && (j >= nc || better(S[i], I[i] & INT_MAX, cs[j], ci[j]));
        pS[cur ^ 1][o] = from_pool ? S[i] : cs[j];
        pI[cur ^ 1][o] = from_pool ? I[i] : ci[j];
      }
      cur ^= 1;
      psize = out;
    }
    if (tid == 0) ctr[kCtrVisited] += nc;
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
    // ---- their unvisited neighbours, scored
    for (int s = tid; s < nsel * a.R; s += kAnnsSearchThreads) {
      const int src = sel[s / a.R];
      const int y = a.graph[((size_t)bh * N + src) * a.R + s % a.R];
      if (y < 0 || y >= N) continue;
      const uint32_t bit = 1u << (y & 31);
      if (atomicOr(&vis[y >> 5], bit) & bit) continue;
      const float sc = seq_dot(u, kb + (size_t)y * kHeadDim);
      const int p = atomicAdd(&ctr[kCtrCand], 1);
      cs[p] = sc;
      ci[p] = y;
    }
    __syncthreads();
  }
  // ---- the k best pool entries
  for (int o = tid; o < a.n_ret; o += kAnnsSearchThreads)
    a.found_pos[(size_t)bh * a.n_ret + o] = o < psize ? (pI[cur][o] & INT_MAX) + a.n_sink : -1;
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
                        dim3((a.n_t + kAnnsListQueries - 1) / kAnnsListQueries, BH), dim3(64), 0,
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
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_anns_search),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)a.search_lds);
  if (e != hipSuccess) return e;
  return launch(tr, k_anns_search, dim3(a.B * a.Hkv), dim3(kAnnsSearchThreads), a.search_lds,
                s, a);
}

}  // namespace wave
