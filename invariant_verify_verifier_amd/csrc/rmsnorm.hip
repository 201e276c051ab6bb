// rmsnorm_bi: batch-invariant RMSNorm, with an optional fused residual add.
//
// LLM-42 post, paragraph 1: RMSNorm becomes batch invariant with a fixed
// split of the reduction over the hidden dimension, chosen independently of
// how many compute units are busy.  Here the split is fixed by H alone: one
// 256-lane workgroup per row; each lane accumulates the squares of the
// elements it owns in a fixed ascending order with fp32 fused multiply-adds,
// then a fixed butterfly over the 64 lanes of each wave, then waves 0..3
// summed in ascending order.  Which elements a lane owns depends on H only:
//  - H a multiple of 1024: lane t owns the 4-element groups 4t + 1024j,
//    j = 0, 1, ..., and adds group j's four elements in ascending order
//    before group j + 1;
//  - any other H: lane t owns x[t], x[t + 256], ...
// Two kernels implement this: a vector kernel (H of 1024, 2048, 4096 or 8192
// with 16-byte aligned rows, each lane loading its groups as vectors and
// keeping them in registers for the output pass) and a scalar kernel for
// everything else.  They own and add the same elements in the same order, so
// pointer alignment never changes a row's bits, and rows never share a
// reduction, so M and the other rows cannot change a row either.
//
// With a residual (the sublayer output x added to the residual stream r in
// the same pass): s = fl32(x + r) is rounded once to x's dtype, written back
// to r, and s is what gets normalised.
#include "biv_internal.h"

namespace biv {

constexpr int kNormThreads = 256;

// Element i of the row the lane reads: x alone, or x + r (rounded to XDT and
// stored back to r).  The same function serves both kernels' scalar loads.
template <int XDT, bool RES>
__device__ __forceinline__ float norm_input(const void* __restrict__ x, void* __restrict__ res, int64_t i) {
  const float v = load_as_f32(x, i, XDT);
  if constexpr (!RES) {
    return v;
  } else {
    const float s = __fadd_rn(v, load_as_f32(res, i, XDT));
    store_from_f32(res, i, s, XDT);
    return XDT == BIV_BF16 ? bf2f(f2bf(s)) : s;  // the stored (rounded) value
  }
}

// Scalar kernel: any H, any alignment.  G4 selects the grouped ownership
// (H a multiple of 1024).
template <int XDT, int YDT, bool RES, bool G4>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const void* __restrict__ x, void* __restrict__ res,
                                                               const void* __restrict__ gamma,
                                                               void* __restrict__ y, int H, float eps) {
  const int64_t base = (int64_t)blockIdx.x * H;
  const int t = threadIdx.x;
  float ss = 0.0f;
  if constexpr (G4) {
    for (int i0 = 4 * t; i0 < H; i0 += 4 * kNormThreads)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = norm_input<XDT, RES>(x, res, base + i0 + c);
        ss = __fmaf_rn(v, v, ss);
      }
  } else {
    for (int i = t; i < H; i += kNormThreads) {
      const float v = norm_input<XDT, RES>(x, res, base + i);
      ss = __fmaf_rn(v, v, ss);
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[kNormThreads / 64];
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot = __fadd_rn(tot, part[w]);
  const float mean = __fdiv_rn(tot, (float)H);
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(mean, eps)));
  // output pass: each lane rereads only elements it wrote (the residual case)
  // or only reads (x), so no synchronisation is needed between the passes
  const void* src = RES ? static_cast<const void*>(res) : x;
  auto out = [&](int i) {
    const float v = load_as_f32(src, base + i, XDT);
    const float g = load_as_f32(gamma, i, YDT);
    store_from_f32(y, base + i, __fmul_rn(__fmul_rn(v, inv), g), YDT);
  };
  if constexpr (G4) {
    for (int i0 = 4 * t; i0 < H; i0 += 4 * kNormThreads)
#pragma unroll
      for (int c = 0; c < 4; ++c) out(i0 + c);
  } else {
    for (int i = t; i < H; i += kNormThreads) out(i);
  }
}

// Four consecutive elements as fp32 (16-byte fp32 or 8-byte bf16 load).
template <int DT>
__device__ __forceinline__ void load4(const void* p, int64_t e, float* o) {
  if constexpr (DT == BIV_F32) {
    const f32x4 q = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + e);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = q[c];
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + e);
    o[0] = bf2f((uint16_t)(q.x & 0xffffu));
    o[1] = bf2f((uint16_t)(q.x >> 16));
    o[2] = bf2f((uint16_t)(q.y & 0xffffu));
    o[3] = bf2f((uint16_t)(q.y >> 16));
  }
}

// Four fp32 values rounded once to DT and stored; `o` becomes the stored values.
template <int DT>
__device__ __forceinline__ void store4(void* p, int64_t e, float* o) {
  if constexpr (DT == BIV_F32) {
    const f32x4 q = {o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + e) = q;
  } else {
    uint16_t b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      b[c] = f2bf(o[c]);
      o[c] = bf2f(b[c]);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + e) =
        make_uint2((uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16));
  }
}

// Vector kernel for H = 1024 * NV (the grouped ownership): lane t holds
// elements 4t + 1024j .. +3, j = 0..NV-1, and the same elements of gamma,
// read once.
template <int XDT, int YDT, bool RES, int NV>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_vec_kernel(const void* __restrict__ x, void* __restrict__ res,
                                                                   const void* __restrict__ gamma,
                                                                   void* __restrict__ y, float eps) {
  constexpr int H = 1024 * NV;
  const int64_t base = (int64_t)blockIdx.x * H;
  const int t = threadIdx.x;
  float v[NV][4];
#pragma unroll
  for (int j = 0; j < NV; ++j) load4<XDT>(x, base + 4 * t + 1024 * j, v[j]);
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float r[4];
      load4<XDT>(res, base + 4 * t + 1024 * j, r);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[j][c] = __fadd_rn(v[j][c], r[c]);
      store4<XDT>(res, base + 4 * t + 1024 * j, v[j]);  // v becomes the rounded s
    }
  }
  // gamma is loaded with x, so its latency hides behind the reduction
  float gm[NV][4];
#pragma unroll
  for (int j = 0; j < NV; ++j) load4<YDT>(gamma, 4 * t + 1024 * j, gm[j]);
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) ss = __fmaf_rn(v[j][c], v[j][c], ss);
  ss = wave_sum(ss);
  __shared__ float part[kNormThreads / 64];
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot = __fadd_rn(tot, part[w]);
  const float mean = __fdiv_rn(tot, (float)H);
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(mean, eps)));
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __fmul_rn(__fmul_rn(v[j][c], inv), gm[j][c]);
    store4<YDT>(y, base + 4 * t + 1024 * j, o);
  }
}

template <int XDT, int YDT, bool RES>
static void launch_norm(const void* x, void* res, const void* gamma, void* y, int64_t M, int64_t H, float eps,
                        hipStream_t s, bool vec) {
  dim3 grid((unsigned)M), block(kNormThreads);
  if (vec) {
    switch (H / 1024) {
      case 1: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, RES, 1>), grid, block, 0, s, x, res, gamma, y, eps); return;
      case 2: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, RES, 2>), grid, block, 0, s, x, res, gamma, y, eps); return;
      case 4: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, RES, 4>), grid, block, 0, s, x, res, gamma, y, eps); return;
      case 8: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, RES, 8>), grid, block, 0, s, x, res, gamma, y, eps); return;
      default: break;
    }
  }
  if (H % 1024 == 0)
    hipLaunchKernelGGL((rmsnorm_kernel<XDT, YDT, RES, true>), grid, block, 0, s, x, res, gamma, y, (int)H, eps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<XDT, YDT, RES, false>), grid, block, 0, s, x, res, gamma, y, (int)H, eps);
}

template <int XDT, int YDT>
static void launch_norm_res(const void* x, void* res, const void* gamma, void* y, int64_t M, int64_t H, float eps,
                            hipStream_t s, bool vec) {
  if (res)
    launch_norm<XDT, YDT, true>(x, res, gamma, y, M, H, eps, s, vec);
  else
    launch_norm<XDT, YDT, false>(x, nullptr, gamma, y, M, H, eps, s, vec);
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

}  // namespace biv

extern "C" biv_status rmsnorm_bi(const void* x, biv_dtype x_dt, void* residual, const void* gamma, void* y,
                                 biv_dtype y_dt, int64_t M, int64_t H, float eps, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(x_dt) && valid_dt(y_dt), "rmsnorm_bi: bad dtype");
  BIV_REQUIRE(M >= 0 && H >= 1 && H <= 65536, "rmsnorm_bi: bad sizes M=%lld H=%lld", (long long)M, (long long)H);
  BIV_REQUIRE(M <= 0x7fffffff, "rmsnorm_bi: M too large");
  BIV_REQUIRE(eps >= 0.0f, "rmsnorm_bi: eps must be >= 0");
  if (M == 0) return BIV_OK;
  BIV_REQUIRE(x && gamma && y, "rmsnorm_bi: NULL pointer");
  const size_t xb = (size_t)M * (size_t)H * dt_size(x_dt), yb = (size_t)M * (size_t)H * dt_size(y_dt);
  BIV_REQUIRE(!overlaps(x, xb, y, yb), "rmsnorm_bi: x and y overlap");
  if (residual) {
    BIV_REQUIRE(!overlaps(residual, xb, x, xb) && !overlaps(residual, xb, y, yb),
                "rmsnorm_bi: residual overlaps x or y");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // vector kernel: H of 1024, 2048, 4096 or 8192 and 16-byte aligned rows;
  // it adds the same elements in the same order as the scalar kernel, so the
  // choice never changes bits
  const bool vec = (H == 1024 || H == 2048 || H == 4096 || H == 8192) && aligned16(x) && aligned16(y) &&
                   aligned16(gamma) && (residual == nullptr || aligned16(residual));
  if (x_dt == BIV_F32 && y_dt == BIV_F32)
    launch_norm_res<BIV_F32, BIV_F32>(x, residual, gamma, y, M, H, eps, s, vec);
  else if (x_dt == BIV_F32 && y_dt == BIV_BF16)
    launch_norm_res<BIV_F32, BIV_BF16>(x, residual, gamma, y, M, H, eps, s, vec);
  else if (x_dt == BIV_BF16 && y_dt == BIV_BF16)
    launch_norm_res<BIV_BF16, BIV_BF16>(x, residual, gamma, y, M, H, eps, s, vec);
  else
    launch_norm_res<BIV_BF16, BIV_F32>(x, residual, gamma, y, M, H, eps, s, vec);
  return launched("rmsnorm_bi");
}
