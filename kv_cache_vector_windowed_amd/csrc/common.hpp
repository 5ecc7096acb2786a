// Shared host/device plumbing of the gfx950 library: status handling, workspace carving,
// kernel launch with optional event timing, and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "a2ats.h"

namespace a2ats {

// ------------------------------------------------------------------ host side
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves aligned sub-buffers from the caller's workspace; `base == nullptr` only sizes.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    size_t off = used;
    used = align_up(used + count * sizeof(T));
    return base ? reinterpret_cast<T*>(base + off) : nullptr;
  }
};

inline bool ws_ok(const void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  if (!ws || have < need) return false;
  return (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0;
}

// Records start/stop events around a launch when profiling is on (see a2ats_profile_*).
void profile_begin(const char* name, hipStream_t s, int* slot);
void profile_end(int slot, hipStream_t s);

template <typename K, typename... Args>
inline int launch(const char* name, K kernel, dim3 grid, dim3 block, size_t shmem,
                  hipStream_t s, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return A2ATS_OK;
  int slot = -1;
  profile_begin(name, s, &slot);
  hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  hipError_t e = hipGetLastError();
  profile_end(slot, s);
  return e == hipSuccess ? A2ATS_OK : A2ATS_EHIP;
}

// Allows a kernel more than the default dynamic LDS (gfx950 has 160 KB per workgroup).
template <typename K>
inline int set_dynamic_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return A2ATS_OK;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return e == hipSuccess ? A2ATS_OK : A2ATS_EHIP;
}

#define A2ATS_TRY(expr)          \
  do {                           \
    int st_ = (expr);            \
    if (st_ != A2ATS_OK) return st_; \
  } while (0)

// Number of workgroups for a 1-D launch, capped to keep the grid size in range.
inline unsigned grid_for(int64_t items, int per_block, int64_t cap = (int64_t)1 << 30) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return (unsigned)(g < 0 ? 0 : g);
}

// ------------------------------------------------------------------ device side
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Loads element i of a key/query row stored as fp32 (dt == A2ATS_F32) or bf16.
__device__ __forceinline__ float load_elem(const void* p, int dt, int64_t i) {
  return dt == A2ATS_F32 ? static_cast<const float*>(p)[i]
                         : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Round an fp64 value to bf16 (nearest, ties to even) directly, without passing through
// fp32: keep 8 significant bits of the fp64 significand, then reinterpret.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  uint16_t s16 = (u >> 63) ? 0x8000 : 0;
  uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return s16 | 0x7FC0;  // NaN
  double ad = __longlong_as_double(static_cast<long long>(a));
  if (ad < 0x1p-126) {
    // bf16 subnormal range: spacing 2^-133; round ad / 2^-133 to an integer, ties to even
    double q = ad * 0x1p133;
    double fl = floor(q);
    double rem = q - fl;
    uint32_t m = static_cast<uint32_t>(fl);
    if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m += 1;
    return s16 | static_cast<uint16_t>(m);  // m == 128 is the smallest normal
  }
  // normal range: round the significand at fp64 bit 45 (52 - 7 stored bf16 bits)
  uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1ull)) & ~0x00001FFFFFFFFFFFull;
  double rd = __longlong_as_double(static_cast<long long>(r));
  if (rd >= 0x1p128) return s16 | 0x7F80;  // overflow to infinity
  float f = static_cast<float>(rd);         // exact: at most 8 significant bits
  return s16 | static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): the LDS address
// is the wave-uniform lds (in M0) plus 16 x the lane index.  Completion is counted by vmcnt.
// Written as inline assembly rather than the compiler builtin: while a builtin copy is in
// flight the compiler waits for all outstanding LDS reads (lgkmcnt(0)) before using any of
// them, which exposes the full LDS latency at every use in a loop that streams the next
// stage while reading the current one.  The compiler does not track this copy: the caller
// reads the destination only after lds_dma_barrier() (vmcnt(0)), and the "memory" clobber
// keeps the compiler from moving LDS accesses across it.
// `lds` is an LDS byte offset (lds_offset()), equal in every lane.
__device__ __forceinline__ void lds_dma16(const void* gsrc, unsigned lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gsrc),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// LDS byte offset of a __shared__ object (a constant for a named array).
__device__ __forceinline__ unsigned lds_offset(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Barrier after this wave's LDS loads (direct and DS) have completed.
__device__ __forceinline__ void lds_dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding global loads, so a
// prefetch issued before it stays in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace a2ats
