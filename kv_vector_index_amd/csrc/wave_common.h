// Device helpers shared by the wave-index kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wave_kernels.h"

namespace wave {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float floatx16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// streaming load: data read once per call, do not keep it in the caches
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// bf16 pair packed in a uint32 -> two floats (exact)
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
// dot of 8 bf16 (16 bytes) with 8 bf16, fp32 accumulation
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b) {
  float s = dot2(a.x, b.x, 0.f);
  s = dot2(a.y, b.y, s);
  s = dot2(a.z, b.z, s);
  return dot2(a.w, b.w, s);
}

// DPP lane permutations inside a row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of a DPP row; every lane receives the total (fixed order)
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Data exchanged between workgroups of one kernel: device-coherent (sc1) loads and stores,
// seen consistently by every XCD without writing back or invalidating whole L2 caches.
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's earlier vector-memory operations have completed (device-coherent
// stores acknowledged); also a compiler barrier for memory accesses.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- block-wide scans for NT-thread workgroups
template <int NT>
struct ScanTmp {
  uint32_t w[NT / 64];
};

// Inclusive scan over the 64 lanes of a wave: four DPP row shifts (lanes shifted in from
// outside the 16-lane row read 0) scan each row, then the three lower rows' totals are read
// back as scalars and added to the rows above them.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  auto shr = [](uint32_t v, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, decltype(ctrl)::value, 0xF, 0xF,
                                                 true);
  };
  x += shr(x, std::integral_constant<int, 0x111>{});  // row_shr:1
  x += shr(x, std::integral_constant<int, 0x112>{});  // row_shr:2
  x += shr(x, std::integral_constant<int, 0x114>{});  // row_shr:4
  x += shr(x, std::integral_constant<int, 0x118>{});  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// exclusive scan over the block; *total = block sum
template <int NT>
__device__ __forceinline__ uint32_t scan_excl(uint32_t x, ScanTmp<NT>& tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t v = wave_scan_incl(x);
  if (lane == 63) tmp.w[wave] = v;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = tmp.w[w];
    before += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + v - x;
}

// Enqueue a kernel; with a tracer that has room, its next two events time this kernel
// (recorded at the start and the end of its execution). Returns the launch status.
template <typename F, typename... Args>
inline hipError_t launch(Tracer* tr, F kernel, dim3 grid, dim3 block, uint32_t lds,
                         hipStream_t s, Args... args) {
  if (tr && tr->ev && tr->n + 2 <= tr->cap) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, tr->ev[tr->n], tr->ev[tr->n + 1], 0u,
                          args...);
    tr->n += 2;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
  return hipGetLastError();
}

}  // namespace wave
