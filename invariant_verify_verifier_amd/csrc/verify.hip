// gumbel_verify: Gumbel-max coupled verification of K candidates per request.
//
// Reading-club post on Gumbel coupling: the Gumbel-max trick samples from the
// softmax as argmax(logits + g) with g ~ Gumbel(0,1) prepared in advance;
// with the same noise on both sides, verification reduces to comparing the
// draft's token with the target's token.
//
// Kernel 1 (one workgroup per row r*K + j): stream the row's logits and noise
// (HBM-bound, 8 bytes per vocab entry), s = fl32(l + g), keep the best
// (value, index) pair per lane, reduce across the workgroup.  The pair order
// "larger value wins, equal values go to the lower index" is associative and
// commutative, so the reduction order cannot change the result.
// Kernel 2 (one lane per request): first j with target != cand.
#include "biv_internal.h"

namespace biv {

constexpr int kVerifyThreads = 1024;

template <bool kVec4>
__global__ __launch_bounds__(kVerifyThreads) void gumbel_argmax_kernel(const float* __restrict__ logits,
                                                                       const float* __restrict__ noise,
                                                                       int V, int32_t* __restrict__ target) {
  const int64_t row = blockIdx.x;
  const float* lr = logits + row * (int64_t)V;
  const float* nr = noise + row * (int64_t)V;
  float bv = -INFINITY;
  int bi = V;  // loses every comparison with a real index
  if (kVec4) {
    const f32x4* l4 = reinterpret_cast<const f32x4*>(lr);
    const f32x4* n4 = reinterpret_cast<const f32x4*>(nr);
    const int V4 = V >> 2;
    int i = threadIdx.x;
    // four independent 32-byte pairs in flight per lane
    for (; i + 3 * kVerifyThreads < V4; i += 4 * kVerifyThreads) {
      f32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = __builtin_nontemporal_load(l4 + i + u * kVerifyThreads);
        b[u] = __builtin_nontemporal_load(n4 + i + u * kVerifyThreads);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int base = 4 * (i + u * kVerifyThreads);
        take_better(bv, bi, a[u].x + b[u].x, base + 0);
        take_better(bv, bi, a[u].y + b[u].y, base + 1);
        take_better(bv, bi, a[u].z + b[u].z, base + 2);
        take_better(bv, bi, a[u].w + b[u].w, base + 3);
      }
    }
    for (; i < V4; i += kVerifyThreads) {
      const f32x4 a = __builtin_nontemporal_load(l4 + i);
      const f32x4 b = __builtin_nontemporal_load(n4 + i);
      take_better(bv, bi, a.x + b.x, 4 * i + 0);
      take_better(bv, bi, a.y + b.y, 4 * i + 1);
      take_better(bv, bi, a.z + b.z, 4 * i + 2);
      take_better(bv, bi, a.w + b.w, 4 * i + 3);
    }
  } else {
    for (int i = threadIdx.x; i < V; i += kVerifyThreads) take_better(bv, bi, lr[i] + nr[i], i);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    take_better(bv, bi, ov, oi);
  }
  __shared__ float sv[kVerifyThreads / 64];
  __shared__ int si[kVerifyThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kVerifyThreads / 64; ++w) take_better(bv, bi, sv[w], si[w]);
    target[row] = bi;
  }
}

// One workgroup per row: fold the row's per-group best pairs (written by the
// lm_head GEMM's Gumbel epilogue) into its target.
__global__ __launch_bounds__(256) void gumbel_groups_kernel(const uint2* __restrict__ part, int groups,
                                                          int32_t* __restrict__ target) {
  const int64_t row = blockIdx.x;
  const uint2* pr = part + row * (int64_t)groups;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < groups; i += 256) {
    const uint2 p = pr[i];
    take_better(bv, bi, __uint_as_float(p.x), (int)p.y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    take_better(bv, bi, ov, oi);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) take_better(bv, bi, sv[w], si[w]);
    target[row] = bi;
  }
}

__global__ void verify_decide_kernel(const int32_t* __restrict__ target, const int32_t* __restrict__ cand,
                                     int R, int K, int32_t* __restrict__ accept_len,
                                     int32_t* __restrict__ next_token) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  int a = K, nx = -1;
  for (int j = 0; j < K; ++j) {
    const int t = target[(int64_t)r * K + j];
    if (t != cand[(int64_t)r * K + j]) {
      a = j;
      nx = t;
      break;
    }
  }
  accept_len[r] = a;
  next_token[r] = nx;
}

// Gumbel top-k (the Gumbel post's top-k sampling for free): the k largest
// s = fl32(l + g) of a row, in take_better's order (descending scores, equal
// scores by index, NaN as -inf).  One 1024-thread workgroup per row.  Each
// thread keeps its own best kTopMax entries, sorted, by insertion (only
// entries that beat its current last one are inserted); then k rounds each
// pick the best head among the threads' lists and pop it from its owner.
// Any element of the row's top k is within its own thread's top kTopMax, so
// the rounds find exactly the row's top k.
constexpr int kTopMax = 8;

__device__ __forceinline__ bool pair_better(float v, int i, float bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
}

// (tw, iw): an entry that at least kTopMax entries of the row beat or equal,
// so anything worse than it cannot be in the row's top kTopMax.
__device__ __forceinline__ void topk_insert(float* tv, int* ti, float v, int i, float tw, int iw) {
  v = (v != v) ? -INFINITY : v;
  if (!pair_better(v, i, tv[kTopMax - 1], ti[kTopMax - 1]) || !pair_better(v, i, tw, iw)) return;
#pragma unroll
  for (int j = 0; j < kTopMax; ++j) {  // bubble the new entry into place
    const bool b = pair_better(v, i, tv[j], ti[j]);
    const float ov = tv[j];
    const int oi = ti[j];
    tv[j] = b ? v : ov;
    ti[j] = b ? i : oi;
    v = b ? ov : v;
    i = b ? oi : i;
  }
}

template <bool kVec4>
__global__ __launch_bounds__(kVerifyThreads) void gumbel_topk_kernel(const float* __restrict__ logits,
                                                                     const float* __restrict__ noise, int V, int k,
                                                                     int32_t* __restrict__ idx,
                                                                     float* __restrict__ score) {
  const int64_t row = blockIdx.x;
  const float* lr = logits + row * (int64_t)V;
  const float* nr = noise + row * (int64_t)V;
  float tv[kTopMax];
  int ti[kTopMax];
#pragma unroll
  for (int j = 0; j < kTopMax; ++j) {
    tv[j] = -INFINITY;
    ti[j] = 0x7fffffff;
  }
  // Wave threshold: the best of the lanes' last kept entries.  The lane that
  // holds it keeps kTopMax entries at least as good, so every entry worse
  // than it is skipped without an insertion (refreshed every 8 steps of the
  // vector loop, every 32 of the scalar one).
  float tw = -INFINITY;
  int iw = 0x7fffffff;
  auto refresh = [&]() {
    tw = tv[kTopMax - 1];
    iw = ti[kTopMax - 1];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(tw, o, 64);
      const int oi = __shfl_xor(iw, o, 64);
      take_better(tw, iw, ov, oi);
    }
  };
  if (kVec4) {
    const f32x4* l4 = reinterpret_cast<const f32x4*>(lr);
    const f32x4* n4 = reinterpret_cast<const f32x4*>(nr);
    const int V4 = V >> 2;
    // iterations are wave-uniform (the loop bound is the same for every lane)
    for (int base = 0; base < V4; base += kVerifyThreads) {
      const int i = base + threadIdx.x;
      if (i < V4) {
        const f32x4 a = __builtin_nontemporal_load(l4 + i);
        const f32x4 b = __builtin_nontemporal_load(n4 + i);
        topk_insert(tv, ti, a.x + b.x, 4 * i + 0, tw, iw);
        topk_insert(tv, ti, a.y + b.y, 4 * i + 1, tw, iw);
        topk_insert(tv, ti, a.z + b.z, 4 * i + 2, tw, iw);
        topk_insert(tv, ti, a.w + b.w, 4 * i + 3, tw, iw);
      }
      if (((base / kVerifyThreads) & 7) == 7) refresh();
    }
  } else {
    for (int base = 0; base < V; base += kVerifyThreads) {
      const int i = base + threadIdx.x;
      if (i < V) topk_insert(tv, ti, lr[i] + nr[i], i, tw, iw);
      if (((base / kVerifyThreads) & 31) == 31) refresh();
    }
  }
  __shared__ float sv[kVerifyThreads / 64];
  __shared__ int si[kVerifyThreads / 64];
  __shared__ int win_i;
  const int wave = threadIdx.x >> 6;
  for (int t = 0; t < k; ++t) {
    float bv = tv[0];
    int bi = ti[0];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      take_better(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 63) == 0) {
      sv[wave] = bv;
      si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < kVerifyThreads / 64; ++w) take_better(bv, bi, sv[w], si[w]);
      win_i = bi;
      idx[row * k + t] = bi;
      if (score) score[row * k + t] = bv;
    }
    __syncthreads();
    if (ti[0] == win_i) {  // the owner pops its head (indices are unique in a row)
#pragma unroll
      for (int j = 0; j < kTopMax - 1; ++j) {
        tv[j] = tv[j + 1];
        ti[j] = ti[j + 1];
      }
      tv[kTopMax - 1] = -INFINITY;
      ti[kTopMax - 1] = 0x7fffffff;
    }
  }
}

biv_status launch_gumbel_finish(const uint2* part, int groups, const int32_t* cand, int R, int K,
                                int32_t* target, int32_t* accept_len, int32_t* next_token, hipStream_t s) {
  hipLaunchKernelGGL(gumbel_groups_kernel, dim3((unsigned)(R * K)), dim3(256), 0, s, part, groups, target);
  const biv_status st = launched("lm_head_gumbel_verify/groups");
  if (st != BIV_OK) return st;
  hipLaunchKernelGGL(verify_decide_kernel, dim3((R + 63) / 64), dim3(64), 0, s, target, cand, R, K, accept_len,
                     next_token);
  return launched("lm_head_gumbel_verify/decide");
}

}  // namespace biv

namespace biv {
// One thread per request: the branch with the longest accepted prefix, the
// lowest branch index among equals.
__global__ void tree_select_kernel(const int32_t* __restrict__ accept_len, const int32_t* __restrict__ next_token,
                                   int R, int B, int32_t* __restrict__ best, int32_t* __restrict__ accept_out,
                                   int32_t* __restrict__ next_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int32_t* a = accept_len + (int64_t)r * B;
  int bb = 0, ba = a[0];
  for (int b = 1; b < B; ++b) {
    if (a[b] > ba) {
      ba = a[b];
      bb = b;
    }
  }
  best[r] = bb;
  accept_out[r] = ba;
  next_out[r] = next_token[(int64_t)r * B + bb];
}
}  // namespace biv

extern "C" biv_status gumbel_verify(const float* logits, const float* noise, const int32_t* cand, int R,
                                    int K, int V, int32_t* target, int32_t* accept_len,
                                    int32_t* next_token, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(R >= 0 && K >= 1 && V >= 1, "gumbel_verify: need R >= 0, K >= 1, V >= 1 (R=%d K=%d V=%d)", R, K, V);
  BIV_REQUIRE((int64_t)R * K <= 0x7fffffff, "gumbel_verify: R*K too large");
  if (R == 0) return BIV_OK;
  BIV_REQUIRE(logits && noise && cand && target && accept_len && next_token, "gumbel_verify: NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = (V % 4 == 0) && aligned16(logits) && aligned16(noise);
  const unsigned rows = (unsigned)(R * K);
  if (vec)
    hipLaunchKernelGGL(gumbel_argmax_kernel<true>, dim3(rows), dim3(kVerifyThreads), 0, s, logits, noise, V, target);
  else
    hipLaunchKernelGGL(gumbel_argmax_kernel<false>, dim3(rows), dim3(kVerifyThreads), 0, s, logits, noise, V, target);
  biv_status st = launched("gumbel_verify/argmax");
  if (st != BIV_OK) return st;
  hipLaunchKernelGGL(verify_decide_kernel, dim3((R + 63) / 64), dim3(64), 0, s, target, cand, R, K, accept_len,
                     next_token);
  return launched("gumbel_verify/decide");
}

extern "C" biv_status gumbel_topk(const float* logits, const float* noise, int rows, int V, int k, int32_t* idx,
                                  float* score, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(rows >= 0 && V >= 1 && k >= 1 && k <= V, "gumbel_topk: need rows >= 0, 1 <= k <= V (k=%d V=%d)", k, V);
  if (k > kTopMax) return fail(BIV_EUNSUPPORTED, "gumbel_topk: k=%d > %d", k, kTopMax);
  if (rows == 0) return BIV_OK;
  BIV_REQUIRE(logits && noise && idx, "gumbel_topk: NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((V % 4 == 0) && aligned16(logits) && aligned16(noise))
    hipLaunchKernelGGL(gumbel_topk_kernel<true>, dim3((unsigned)rows), dim3(kVerifyThreads), 0, s, logits, noise, V, k,
                       idx, score);
  else
    hipLaunchKernelGGL(gumbel_topk_kernel<false>, dim3((unsigned)rows), dim3(kVerifyThreads), 0, s, logits, noise, V,
                       k, idx, score);
  return launched("gumbel_topk");
}

extern "C" biv_status tree_select(const int32_t* accept_len, const int32_t* next_token, int R, int B, int32_t* best,
                                  int32_t* accept_out, int32_t* next_out, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(R >= 0 && B >= 1, "tree_select: need R >= 0 and B >= 1 (R=%d B=%d)", R, B);
  BIV_REQUIRE((int64_t)R * B <= 0x7fffffff, "tree_select: too many branches");
  if (R == 0) return BIV_OK;
  BIV_REQUIRE(accept_len && next_token && best && accept_out && next_out, "tree_select: NULL pointer");
  hipLaunchKernelGGL(tree_select_kernel, dim3((unsigned)cdiv(R, 64)), dim3(64), 0, static_cast<hipStream_t>(stream),
                     accept_len, next_token, R, B, best, accept_out, next_out);
  return launched("tree_select");
}
