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

// Optional kernel-boundary events: mark() records the next caller-provided event on the
// stream right before each kernel launch, and once after the last one.
struct Tracer {
  hipEvent_t* ev;
  int cap, n;
  static void mark(Tracer* t, hipStream_t s) {
    if (t && t->ev && t->n < t->cap) hipEventRecord(t->ev[t->n++], s);
  }
};

// ---------------------------------------------------------------- decode
constexpr int kDecThreads = 256;      // streaming / retrieved / dense kernels
constexpr int kSelThreads = 1024;     // per-(b, kv-head) select kernel
constexpr int kEstChunk = 256;        // clusters per streaming workgroup
constexpr int kTokChunk = 256;        // tokens per steady / dense workgroup
constexpr int kPartStride = 132;      // floats per (partial, head): o[128], m, l, 2 pad
constexpr int kSelStageMax = 16384;   // group scores staged in LDS by the select kernel

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
  float* shat;             // [BH, C] group scores
  float* partA;            // [BH, nA, G, kPartStride]
  float* mergedA;          // [BH, G, kPartStride]
  float* partB;            // [BH, nB, G, kPartStride]
  int32_t* sel;            // [BH, rcap] retrieved ids, ascending
  int32_t* slots;          // [BH, L0] cache rows of the retrieved tokens
  int32_t* nsel;           // [BH]
  int32_t* ntok;           // [BH]
  uint32_t* counter;       // [BH]
  // shape
  int B, Hq, Hkv, G;
  int64_t L, L0, Lcap;
  int C, n_sink, n_recent, n_retrieve, rcap;
  int nEst, nSteady, nA, nB;
  float scale, scale_log2;
};

// Enqueue the tripartite decode (three kernels). Returns the first launch error.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, Tracer* tr);
// Enqueue dense decode over [0, L): partial kernel over nB splits (partB) + merge.
hipError_t launch_dense_decode(const DecodeArgs& a, hipStream_t stream, Tracer* tr);

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
};

hipError_t launch_build(const BuildArgs& a, hipStream_t stream, Tracer* tr);

}  // namespace wave
