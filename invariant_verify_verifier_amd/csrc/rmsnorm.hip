// rmsnorm_bi: batch-invariant RMSNorm.
//
// LLM-42 post, paragraph 1: RMSNorm becomes batch invariant with a fixed
// split of the reduction over the hidden dimension, chosen independently of
// how many compute units are busy.  Here the split is fixed by H alone: one
// 256-lane workgroup per row; each lane accumulates its own elements in a
// fixed ascending order with fp32 fused multiply-adds, then a fixed butterfly
// over the 64 lanes of each wave, then waves 0..3 summed in ascending order.
// When H is 1024, 2048, 4096 or 8192 lane t owns the 4-element groups
// 4t + 1024j (j ascending), loaded as vectors and kept in registers for the
// output pass; otherwise lane t owns x[t], x[t+256], ...  Rows never share a
// reduction, so M and the other rows cannot change a row.
#include "biv_internal.h"

namespace biv {

constexpr int kNormThreads = 256;

template <int XDT, int YDT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const void* __restrict__ x,
                                                               const void* __restrict__ gamma,
                                                               void* __restrict__ y, int H, float eps) {
  const int64_t row = blockIdx.x;
  const int64_t base = row * (int64_t)H;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += kNormThreads) {
    const float v = load_as_f32(x, base + i, XDT);
    ss = __fmaf_rn(v, v, ss);
  }
  ss = wave_sum(ss);
  __shared__ float part[kNormThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot = __fadd_rn(tot, part[w]);
  const float mean = __fdiv_rn(tot, (float)H);
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(mean, eps)));
  for (int i = threadIdx.x; i < H; i += kNormThreads) {
    const float v = load_as_f32(x, base + i, XDT);
    const float g = load_as_f32(gamma, i, YDT);
    store_from_f32(y, base + i, __fmul_rn(__fmul_rn(v, inv), g), YDT);
  }
}

// Vector path for H = 1024 * NV: lane t holds elements 4t + 1024j .. +3,
// j = 0..NV-1, and the same elements of gamma, read once.
template <int XDT, int YDT, int NV>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_vec_kernel(const void* __restrict__ x,
                                                                   const void* __restrict__ gamma,
                                                                   void* __restrict__ y, float eps) {
  constexpr int H = 1024 * NV;
  const int64_t base = (int64_t)blockIdx.x * H;
  const int t = threadIdx.x;
  float v[NV][4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t e = base + 4 * t + 1024 * j;
    if constexpr (XDT == BIV_F32) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[j][c] = q[c];
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + e);
      v[j][0] = bf2f((uint16_t)(q.x & 0xffffu));
      v[j][1] = bf2f((uint16_t)(q.x >> 16));
      v[j][2] = bf2f((uint16_t)(q.y & 0xffffu));
      v[j][3] = bf2f((uint16_t)(q.y >> 16));
    }
  }
  // gamma is loaded with x, so its latency hides behind the reduction
  float gm[NV][4];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i0 = 4 * t + 1024 * j;
    if constexpr (YDT == BIV_F32) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(static_cast<const float*>(gamma) + i0);
#pragma unroll
      for (int c = 0; c < 4; ++c) gm[j][c] = q[c];
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(gamma) + i0);
      gm[j][0] = bf2f((uint16_t)(q.x & 0xffffu));
      gm[j][1] = bf2f((uint16_t)(q.x >> 16));
      gm[j][2] = bf2f((uint16_t)(q.y & 0xffffu));
      gm[j][3] = bf2f((uint16_t)(q.y >> 16));
    }
  }
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
    const int i0 = 4 * t + 1024 * j;
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __fmul_rn(__fmul_rn(v[j][c], inv), gm[j][c]);
    if constexpr (YDT == BIV_F32) {
      const f32x4 q = {o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(static_cast<float*>(y) + base + i0) = q;
    } else {
      const uint2 q = make_uint2((uint32_t)f2bf(o[0]) | ((uint32_t)f2bf(o[1]) << 16),
                                 (uint32_t)f2bf(o[2]) | ((uint32_t)f2bf(o[3]) << 16));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + base + i0) = q;
    }
  }
}

template <int XDT, int YDT>
static void launch_norm(const void* x, const void* gamma, void* y, int64_t M, int64_t H, float eps,
                        hipStream_t s, bool vec) {
  dim3 grid((unsigned)M), block(kNormThreads);
  if (vec) {
    switch (H / 1024) {
      case 1: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, 1>), grid, block, 0, s, x, gamma, y, eps); return;
      case 2: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, 2>), grid, block, 0, s, x, gamma, y, eps); return;
      case 4: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, 4>), grid, block, 0, s, x, gamma, y, eps); return;
      case 8: hipLaunchKernelGGL((rmsnorm_vec_kernel<XDT, YDT, 8>), grid, block, 0, s, x, gamma, y, eps); return;
      default: break;
    }
  }
  hipLaunchKernelGGL((rmsnorm_kernel<XDT, YDT>), grid, block, 0, s, x, gamma, y, (int)H, eps);
}

}  // namespace biv

extern "C" biv_status rmsnorm_bi(const void* x, biv_dtype x_dt, const void* gamma, void* y, biv_dtype y_dt,
                                 int64_t M, int64_t H, float eps, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(x_dt) && valid_dt(y_dt), "rmsnorm_bi: bad dtype");
  BIV_REQUIRE(M >= 0 && H >= 1 && H <= 65536, "rmsnorm_bi: bad sizes M=%lld H=%lld", (long long)M, (long long)H);
  BIV_REQUIRE(M <= 0x7fffffff, "rmsnorm_bi: M too large");
  BIV_REQUIRE(eps >= 0.0f, "rmsnorm_bi: eps must be >= 0");
  if (M == 0) return BIV_OK;
  BIV_REQUIRE(x && gamma && y, "rmsnorm_bi: NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // vector path: H of 1024, 2048, 4096 or 8192 and 16-byte aligned rows (the
  // path is fixed by H and the pointers, never by M)
  const bool vec = (H == 1024 || H == 2048 || H == 4096 || H == 8192) && aligned16(x) && aligned16(y) &&
                   aligned16(gamma);
  if (x_dt == BIV_F32 && y_dt == BIV_F32)
    launch_norm<BIV_F32, BIV_F32>(x, gamma, y, M, H, eps, s, vec);
  else if (x_dt == BIV_F32 && y_dt == BIV_BF16)
    launch_norm<BIV_F32, BIV_BF16>(x, gamma, y, M, H, eps, s, vec);
  else if (x_dt == BIV_BF16 && y_dt == BIV_BF16)
    launch_norm<BIV_BF16, BIV_BF16>(x, gamma, y, M, H, eps, s, vec);
  else
    launch_norm<BIV_BF16, BIV_F32>(x, gamma, y, M, H, eps, s, vec);
  return launched("rmsnorm_bi");
}
