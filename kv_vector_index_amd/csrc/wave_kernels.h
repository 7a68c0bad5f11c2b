// Internal interface between the host API (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace wave {

constexpr int kHeadDim = 128;      // d
constexpr int kRowBytes = 256;     // one bf16 row of d = 128
constexpr int kMaxGroup = 8;       // largest GQA group (query heads per KV head)
constexpr float kLog2eHost = 1.4426950408889634f;

// Optional per-kernel timing events: the launch helper (wave_common.h) hands the next two
// caller-provided events to hipExtLaunchKernel, which records them at the start and the end
// of that kernel's execution.
struct Tracer {
  hipEvent_t* ev;
  int cap, n;
};

// ---------------------------------------------------------------- decode
constexpr int kDecThreads = 256;      // every decode workgroup: 4 waves
constexpr int kChunk = 128;           // clusters per score / estimate workgroup (32 per wave)
constexpr int kTokChunk = 128;        // steady tokens per steady workgroup
constexpr int kEstChunks = 1;         // chunks of 128 clusters per estimate workgroup
constexpr int kPartStride = 132;      // floats per (partial, head): o[128], m, l, 2 pad
constexpr int kSelSpan = 2048;        // group scores listed per selection workgroup
constexpr int kHistBins = 4096;       // value-range histogram of the group scores
// heads of at most this many clusters are selected by one workgroup holding all their
// scores in registers; larger heads get the histogram kernel and one selection workgroup
// per kSelSpan scores
constexpr int kLocalSelectMax = 8192;
constexpr int kNarrowBins = 1024;     // histogram of a crowded cut bin's scores
constexpr int kCand = 256;            // scores ranked exactly in LDS
constexpr int kMaxClusters = 65536;   // clusters per (b, kv-head) supported by the decode
constexpr int kMaxRetrieveWG = 256;   // retrieve workgroups per (b, kv-head)
constexpr int kMergeGroup = 16;       // retrieve partials per first-level merge (about)
constexpr int kMergeBatch = 14;       // partials per half-workgroup and round of loads in a merge
constexpr int kWinR = 256;            // listed clusters staged per LDS window of a retrieve WG
constexpr int kRetBlock = 32;         // virtual rows per retrieve wave and step (one K step)
constexpr int kRowsPerItem = 128;     // retrieved rows per retrieve workgroup (target)
constexpr int kCUs = 256;              // compute units of an MI355X
constexpr int kRetrieveWGPerCall = 768;   // retrieve workgroups of one call (at most, about)
// per (b, kv-head) counters, cleared by the score kernel in every call
constexpr int kCtrStride = 32;
constexpr int kCtrGather = 1;         // select workgroups of the gather kernel arrived
constexpr int kCtrSure = 2;           // clusters above the cut bin listed so far
constexpr int kCtrTie = 3;            // clusters in the cut bin listed so far
constexpr int kCtrFinal = 4;          // first-level merges arrived
constexpr int kCtrGroup = 8;          // + group: retrieve workgroups of that group arrived

// A retrieved cluster j of size n_j occupies n_j + 1 consecutive "virtual rows": its n_j
// tokens, then one row that removes its centroid estimate (logit s_j, weight -n_j, value
// -V_j) from the estimate over all clusters.
struct DecodeArgs {
  // inputs
  const uint16_t* q;       // [B, Hq, d]
  const uint16_t* k;       // [B, Hkv, Lcap, d]
  const uint16_t* v;
  const uint16_t* cmean;   // [B, Hkv, C, d]
  const uint16_t* vsum;
  const int32_t* csize;    // [B, Hkv, C]
  const int32_t* coff;
  // outputs
  float* out;              // [B, Hq, d]
  float* lse;              // [B, Hq] or null
  int32_t* selected;       // [B, Hkv, n_retrieve] or null
  // workspace
  uint32_t* counter;       // [BH, kCtrStride]
  float* smm;              // [BH, nSW, 2] min and max finite group score per score WG
  uint32_t* hist;          // [BH, kHistBins] histogram of the group scores (large heads)
  int32_t* sure;           // [BH, rcap] clusters above the cut bin (arrival order)
  float* tie_key;          // [BH, C] clusters in the cut bin (arrival order): score, id
  int32_t* tie_id;
  float* scores;           // [BH, C, G] log2-domain centroid logits of each query head
  float* shat;             // [BH, Cp] group-mean logits (natural units; -inf: empty / pad)
  int32_t* sel_id;         // [BH, rcap] the selection (ascending ids)
  int32_t* sel_ts;         // [BH, rcap + 1] first virtual row of each cluster, then total
  int32_t* sel_coff;       // [BH, rcap] first cache row of each cluster
  int32_t* sel_n;          // [BH]
  int32_t* wg_info;        // [BH, kMaxRetrieveWG, 4] per retrieve workgroup: T0, T1, r_lo, r_hi
  float* part;             // [BH, nP, G, kPartStride] partial softmax states
  // shape
  int B, Hq, Hkv, G;
  int64_t L, L0, Lcap;
  int C, Cp, n_sink, n_recent, n_retrieve, rcap;
  // per (b, kv-head): chunks of 128 clusters, score workgroups, estimate workgroups (one per
  // chunk), steady workgroups, selection workgroups, retrieve workgroups, their
  // merge groups, partial slots (estimate, steady, retrieve, merge)
  int nS, nSW, nEW, nSt, nH, nB, nG, nP;
  float scale, scale_log2;
  int hist_kernel;         // 1: the histogram kernel runs (Cp > kLocalSelectMax)
  // host-memory tier (tier != 0): the cache's rows live in host memory (hk, hv, the same
  // layout as k, v), the steady zone in a compact device buffer (sk, sv: [BH, Ls, d], rows
  // [0, n_sink) then [L0 - n_recent, Lcap)), and a device block cache of nslots slots of
  // kTierBlock K rows then kTierBlock V rows holds rows of recently retrieved blocks of
  // kTierBlock consecutive cache rows
  int tier;
  const uint16_t* hk;
  const uint16_t* hv;
  const uint16_t* sk;
  const uint16_t* sv;
  int64_t Ls;
  uint16_t* cache;         // [nslots, 2, kTierBlock, d]
  int32_t* tab;            // [BH, nblk] slot of each block, -1 none, -2 being claimed
  uint64_t* slotw;         // [nslots] owner block (bh * nblk + block; low half, -1 none) and
                           //   2 * (last step that pinned or claimed it) + claimed (high half)
  uint32_t* valid;         // [nslots] rows of the owner block held (bit r: row r of the block)
  uint32_t* tctr;          // kTc* counters
  int nslots, nblk;
  // attention over the steady zone and listed rows (the vector-search retrieval zone):
  // rows_pos [BH, rows_k] cache rows (-1 padded after rows_n[bh] entries)
  const int32_t* rows_pos;
  const int32_t* rows_n;
  int rows_k;
};

// host-memory tier
constexpr int kTierBlock = 32;        // cache rows per block (one slot)
constexpr int kTcStep = 0;            // the current step (from 1; stamps below it are older)
constexpr int kTcHand = 1;            // replacement hand (slots are tried in its order)
constexpr int kTcRowsWritten = 2;     // rows read over the bus and written into a slot (total)
constexpr int kTcRowsCached = 4;      // retrieved token rows read from the block cache (total)
constexpr int kTcRowsHost = 5;        // retrieved token rows read from host memory (total)
constexpr int kTcAdmitted = 6;        // slots claimed for a block (total)
constexpr int kTcRefused = 7;         // claims that found no slot (total)
constexpr int kTcHandStart = 8;       // the hand when this step began
constexpr int kTcWords = 16;

// Enqueue one tripartite decode step (score, histogram for large heads, gather, retrieve
// kernels; with the host-memory tier, then the step kernel). Returns the first launch error.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, Tracer* tr);
// Empty the host-memory tier's block cache (table, owners, stamps, counters).
hipError_t launch_tier_reset(const DecodeArgs& a, hipStream_t stream);
// Copy the tier's kTcWords counters (the start of its state) to host memory c, synchronously.
hipError_t tier_counters_copy(uint32_t* c, const void* state, hipStream_t stream);
// Enqueue dense decode over [0, L): split-K partials (part, nB per head) + merge.
hipError_t launch_dense_decode(const DecodeArgs& a, hipStream_t stream, Tracer* tr);
// Enqueue attention over the steady zone and the rows listed in rows_pos / rows_n:
// split-K partials (part, nB per head) + merge.
hipError_t launch_listed_attention(const DecodeArgs& a, hipStream_t stream, Tracer* tr);

// The library's own decode scratch on the current device (a static device array, one copy
// per GPU, kept until the process ends), for callers that cannot allocate: its address,
// looked up once per device. Calls that use it on one GPU must not overlap.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// ---------------------------------------------------------------- build
struct BuildArgs {
  const uint16_t* k;       // [B, Hkv, Lcap, d]
  const uint16_t* v;
  uint16_t* k_out;
  uint16_t* v_out;
  uint16_t* cmean;         // [B, Hkv, C, d]
  uint16_t* vsum;
  int32_t* csize;          // [B, Hkv, C]
  int32_t* coff;
  int32_t* labels;         // [B, Hkv, L0] or null
  int32_t* perm;           // [B, Hkv, L0] or null
  uint16_t* last_mu;       // [B, Hkv, C, d] or null
  float* objective;        // [B, Hkv] or null
  // workspace
  float* inv_norm;         // [BH, L0]
  uint16_t* mu[2];         // [BH, C, d] ping-pong unit centroids
  int32_t* lab;            // [BH, L0] local label per position (indexed positions only)
  int32_t* order;          // [BH, L0] per segment: local point ids sorted by (label, position)
  int32_t* cstart;         // [BH, nseg, k_seg + 1] cluster starts in sorted order
  float* cnorm;            // [BH, C] ||sum of unit points|| of each cluster
  // shape
  int B, Hkv;
  int64_t L0, Lcap;
  int S, kseg, nseg, C, T, n_sink, n_recent;
  int64_t idx_lo, idx_hi;  // indexed positions [idx_lo, idx_hi)
  int seg0;                // first segment built (an extension keeps the segments before it)
  int extend;              // 1: an extension (the sink rows of k_out are already in place)
};

// One contiguous block of 4-byte words per (b, kv-head) copied from an earlier index into
// a larger one (src and dst strides in words per head).
struct CopyBlock {
  const uint32_t* src;
  uint32_t* dst;
  int64_t words, src_stride, dst_stride;
};
constexpr int kMaxCopyBlocks = 8;
struct CopyArgs {
  CopyBlock blk[kMaxCopyBlocks];
  int n, BH;
};
// Enqueue the copy of the blocks (one kernel).
hipError_t launch_copy_blocks(const CopyArgs& c, hipStream_t stream, Tracer* tr);

hipError_t launch_build(const BuildArgs& a, hipStream_t stream, Tracer* tr);

// ---------------------------------------------------------------- attention-aware vector search
constexpr int kAnnsListQueries = 64;   // training queries per list workgroup (one wave)
constexpr int kAnnsListCap = 96;       // candidate entries per training query in LDS
constexpr int kAnnsMaxList = 64;       // M
constexpr int kAnnsMaxDegree = 64;     // R
constexpr int kAnnsSearchThreads = 1024;
constexpr int kAnnsMaxPool = 1024;     // ef
constexpr int kAnnsMaxCand = 2048;     // W * R (neighbours examined per round)
constexpr int kAnnsMaxExpand = 64;     // W
constexpr int kAnnsMaxEntry = 64;      // n_entry
constexpr int kAnnsMaxTrain = 16384;   // training queries per (b, kv-head)
constexpr int kAnnsMaxSeedWG = 16;     // seed workgroups per (b, kv-head)
constexpr int kAnnsPlaceShift = 24;    // posting key: place << 24 | list
constexpr uint32_t kAnnsMaxLds = 160u * 1024u;   // LDS of one workgroup

struct AnnsArgs {
  const uint16_t* k;       // [B, Hkv, Lcap, d] the cache (positions)
  const uint16_t* train;   // [B, Hkv, n_t, d] training queries
  const uint16_t* q;       // [B, Hq, d] decode queries
  int32_t* graph;          // [BH, N, R] neighbours, -1 padded
  int32_t* entry;          // [BH, n_t] each training query's first node
  int32_t* lists;          // [BH, n_t, M] training lists (node ids, -1 padded)
  // build workspace
  int32_t* cnt;            // [BH, N] postings per node, then the scatter cursor
  int32_t* off;            // [BH, N + 1] first posting of each node
  int32_t* post;           // [BH, n_t * M] postings: place << 24 | list
  // search outputs
  int32_t* found_pos;      // [BH, n_ret] retrieved cache rows, best first, -1 padded
  int32_t* found_n;        // [BH]
  int32_t* stats;          // [BH, 2] rounds, nodes scored (or null)
  float* seed_s;           // [BH, kAnnsMaxSeedWG, n_entry] each seed workgroup's best training
  int32_t* seed_i;         //   queries: scores and indices
  int nseed, seed_chunk;   // seed workgroups per (b, kv-head), training queries per one
  int B, Hq, Hkv, G;
  int64_t Lcap, L0;
  int n_sink, n_recent, N;
  int n_t, M, R, n_entry, ef, W, n_ret, max_rounds;   // n_ret: k, the nodes retrieved
  uint32_t search_lds;     // dynamic LDS bytes of the search workgroup
};
// LDS of the search workgroup, in this order: the search vector (d floats), the expanded
// nodes (kAnnsMaxExpand), 32 counters, the round's new nodes (scores, then ids), two pools
// of ef entries (scores, then ids, each), the visited bitmap (one bit per node).
constexpr uint32_t kAnnsLdsFixed = kHeadDim * 4 + kAnnsMaxExpand * 4 + 32 * 4 + kAnnsMaxCand * 8;
constexpr uint32_t anns_pool_stride(int n) { return (uint32_t)((n + 3) / 4 * 4); }
constexpr uint64_t anns_search_lds(int64_t N, int ef) {
  return kAnnsLdsFixed + 16ull * anns_pool_stride(ef) + (uint64_t)((N + 127) / 128) * 16;
}
// Enqueue the graph build: training lists, postings, links, entries.
hipError_t launch_anns_build(const AnnsArgs& a, hipStream_t stream, Tracer* tr);
// Enqueue the search of one decode step: the seed kernel (nseed workgroups per head), then
// the search (found_pos, found_n, stats).
hipError_t launch_anns_search(const AnnsArgs& a, hipStream_t stream, Tracer* tr);

}  // namespace wave
