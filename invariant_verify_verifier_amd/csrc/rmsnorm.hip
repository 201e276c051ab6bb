// rmsnorm_bi: batch-invariant RMSNorm.
//
// LLM-42 post, paragraph 1: RMSNorm becomes batch invariant with a fixed
// split of the reduction over the hidden dimension, chosen independently of
// how many compute units are busy.  Here the split is fixed by H alone: one
// 256-lane workgroup per row, lane t accumulates x[t], x[t+256], ... in
// ascending order with fp32 fused multiply-adds, then a fixed butterfly over
// the 64 lanes of each wave, then waves 0..3 summed in ascending order.
// Rows never share a reduction, so M and the other rows cannot change a row.
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
  dim3 grid((unsigned)M), block(kNormThreads);
  if (x_dt == BIV_F32 && y_dt == BIV_F32)
    hipLaunchKernelGGL((rmsnorm_kernel<BIV_F32, BIV_F32>), grid, block, 0, s, x, gamma, y, (int)H, eps);
  else if (x_dt == BIV_F32 && y_dt == BIV_BF16)
    hipLaunchKernelGGL((rmsnorm_kernel<BIV_F32, BIV_BF16>), grid, block, 0, s, x, gamma, y, (int)H, eps);
  else if (x_dt == BIV_BF16 && y_dt == BIV_BF16)
    hipLaunchKernelGGL((rmsnorm_kernel<BIV_BF16, BIV_BF16>), grid, block, 0, s, x, gamma, y, (int)H, eps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<BIV_BF16, BIV_F32>), grid, block, 0, s, x, gamma, y, (int)H, eps);
  return launched("rmsnorm_bi");
}
