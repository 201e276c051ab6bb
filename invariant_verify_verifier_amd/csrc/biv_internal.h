// Internal helpers shared by the gfx950 kernels of libbiverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/biverify.h"

namespace biv {

// ---------------------------------------------------------------- errors

void set_error(const char* fmt, ...);

inline biv_status fail(biv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  set_error("%s", buf);
  return s;
}

// Status after a launch: picks up launch-configuration errors only.
inline biv_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BIV_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return BIV_OK;
}

#define BIV_REQUIRE(cond, ...)                              \
  do {                                                      \
    if (!(cond)) return ::biv::fail(BIV_EINVAL, __VA_ARGS__); \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dt(int d) { return d == BIV_F32 || d == BIV_BF16; }
inline size_t dt_size(int d) { return d == BIV_BF16 ? 2 : 4; }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int dt) {
  return dt == BIV_BF16 ? bf2f(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float v, int dt) {
  if (dt == BIV_BF16)
    static_cast<uint16_t*>(p)[i] = f2bf(v);
  else
    static_cast<float*>(p)[i] = v;
}

// Butterfly sum over the 64 lanes of a wave; every lane ends with the same
// bits (each step adds a pair in both orders, and fp32 addition commutes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// One gfx950 global_load_lds_dwordx4: lane i copies 16 bytes from
// sbase + voff_i (sbase wave-uniform) to LDS bytes 16i..16i+15 after `dst`
// (wave-uniform).  Issued as inline asm so that the compiler does not model
// the LDS write: its own hazard tracking would wait for every outstanding
// copy before any LDS read, which serialises the K/V pipeline.  Callers order
// the copies with explicit vmcnt waits; loads the compiler issues itself stay
// correct, since untracked copies only make its vmcnt waits stricter.  M0
// (the LDS base of the copy) is not used by anything else in these kernels.
// kStream: the copy carries the non-temporal hint, so that a stream read
// once (a weight) does not displace data that is read again (activations
// shared by every column block) from the L2.  Only cache placement changes.
template <bool kStream = false>
__device__ __forceinline__ void lds_dma16(const void* sbase, unsigned voff, void* dst) {
  const unsigned m0v =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)dst);
  // readfirstlane yields a signed int: widen each half through uint32_t so
  // the low half is zero-extended, never sign-extended into the high half
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)((uintptr_t)sbase >> 32));
  const uint64_t sb = (uint64_t)lo | ((uint64_t)hi << 32);
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sb), "s"(m0v) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(m0v) : "memory");
}

__device__ __forceinline__ void vm_wait0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Gumbel-max pair order: the larger score wins, equal scores go to the lower
// index, a NaN score never wins.  The order is associative and commutative,
// so any grouping of a row's entries yields the same pair.
__device__ __forceinline__ void take_better(float& bv, int& bi, float v, int i) {
  v = (v != v) ? -INFINITY : v;
  const bool better = (v > bv) | ((v == bv) & (i < bi));  // selects, no branch
  bv = better ? v : bv;
  bi = better ? i : bi;
}

// Second half of the fused lm_head + Gumbel verification: reduce the
// per-group (score bits, index) pairs `part` [M][groups] of each row to its
// target, then the accepted prefix and correction of each request
// (verify.hip).
biv_status launch_gumbel_finish(const uint2* part, int groups, const int32_t* cand, int R, int K,
                                int32_t* target, int32_t* accept_len, int32_t* next_token, hipStream_t s);

}  // namespace biv
