// kv_overwrite and the row-local elementwise helpers of the decoder forward.
//
// kv_overwrite follows the LLM-42 post, paragraph 3: the fast path's KV was
// computed at some other batch size and would pass its numerical drift on to
// later forwards, so every verification overwrites those slots with the
// verifier's values.  It is a bit copy into a paged cache
// [num_blocks, Hkv, 16, D]; one thread moves 16 bytes.
#include "biv_internal.h"

namespace biv {

// One 16-byte piece per thread: piece p of token t, head h.
__global__ void kv_overwrite_vec_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                        int64_t src_stride16, const int64_t* __restrict__ slot,
                                        uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int T,
                                        int Hkv, int row16, int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)Hkv * row16;
  if (gid >= (int64_t)T * per_tok) return;
  const int t = (int)(gid / per_tok);
  const int64_t rem = gid - (int64_t)t * per_tok;  // h * row16 + piece
  const int h = (int)(rem / row16);
  const int piece = (int)(rem - (int64_t)h * row16);
  const int64_t s = slot[t];
  if (s < 0 || s >= num_slots) return;
  const int64_t page = s >> 4, off = s & 15;
  const int64_t dst = ((page * Hkv + h) * 16 + off) * row16 + piece;
  const int64_t src = (int64_t)t * src_stride16 + rem;
  k_cache[dst] = k_new[src];
  v_cache[dst] = v_new[src];
}

// Element-wise fallback for unaligned rows.
template <typename E>
__global__ void kv_overwrite_elem_kernel(const E* __restrict__ k_new, const E* __restrict__ v_new,
                                         int64_t src_stride, const int64_t* __restrict__ slot,
                                         E* __restrict__ k_cache, E* __restrict__ v_cache, int T, int Hkv, int D,
                                         int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_tok = (int64_t)Hkv * D;
  if (gid >= (int64_t)T * per_tok) return;
  const int t = (int)(gid / per_tok);
  const int64_t rem = gid - (int64_t)t * per_tok;
  const int h = (int)(rem / D);
  const int d = (int)(rem - (int64_t)h * D);
  const int64_t s = slot[t];
  if (s < 0 || s >= num_slots) return;
  const int64_t dst = (((s >> 4) * Hkv + h) * 16 + (s & 15)) * D + d;
  k_cache[dst] = k_new[(int64_t)t * src_stride + rem];
  v_cache[dst] = v_new[(int64_t)t * src_stride + rem];
}

__global__ void embed_rows_kernel(const int32_t* __restrict__ ids, const void* __restrict__ table, int table_dt,
                                  void* __restrict__ out, int out_dt, int V, int H) {
  const int t = blockIdx.x;
  const int id = ids[t];
  const bool ok = id >= 0 && id < V;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float v = ok ? load_as_f32(table, (int64_t)id * H + i, table_dt) : 0.0f;
    store_from_f32(out, (int64_t)t * H + i, v, out_dt);
  }
}

// bf16 table, 16-byte pieces: one thread per 8 elements of a row (the same
// values as the element loop: bf16 -> fp32 is exact).
template <int OUT_DT>
__global__ void embed_rows_vec_kernel(const int32_t* __restrict__ ids, const uint16_t* __restrict__ table,
                                      void* __restrict__ out, int V, int H) {
  const int t = blockIdx.x;
  const int id = ids[t];
  const bool ok = id >= 0 && id < V;
  for (int i = 8 * threadIdx.x; i < H; i += 8 * blockDim.x) {
    uint4 q = make_uint4(0, 0, 0, 0);
    if (ok) q = *reinterpret_cast<const uint4*>(table + (int64_t)id * H + i);
    if constexpr (OUT_DT == BIV_BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (int64_t)t * H + i) = q;
    } else {
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
      float f[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f[2 * c] = bf2f((uint16_t)(w[c] & 0xffffu));
        f[2 * c + 1] = bf2f((uint16_t)(w[c] >> 16));
      }
      float* o = static_cast<float*>(out) + (int64_t)t * H + i;
      *reinterpret_cast<f32x4*>(o) = f32x4{f[0], f[1], f[2], f[3]};
      *reinterpret_cast<f32x4*>(o + 4) = f32x4{f[4], f[5], f[6], f[7]};
    }
  }
}

// One thread per (token, head, pair i < D/2).
__global__ void rope_apply_kernel(void* __restrict__ x, int64_t stride, const int32_t* __restrict__ pos,
                                  const float* __restrict__ cos_sin, int T, int n_heads, int D, int max_pos,
                                  int dt) {
  const int half = D >> 1;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * n_heads * half) return;
  const int t = (int)(gid / ((int64_t)n_heads * half));
  const int rem = (int)(gid - (int64_t)t * n_heads * half);
  const int h = rem / half, i = rem - h * half;
  const int p = pos[t];
  if (p < 0 || p >= max_pos) return;
  const float c = cos_sin[((int64_t)p * half + i) * 2 + 0];
  const float s = cos_sin[((int64_t)p * half + i) * 2 + 1];
  const int64_t ia = (int64_t)t * stride + (int64_t)h * D + i;
  const int64_t ib = ia + half;
  const float a = load_as_f32(x, ia, dt), b = load_as_f32(x, ib, dt);
  const float ra = __fsub_rn(__fmul_rn(a, c), __fmul_rn(b, s));
  const float rb = __fadd_rn(__fmul_rn(b, c), __fmul_rn(a, s));
  store_from_f32(x, ia, ra, dt);
  store_from_f32(x, ib, rb, dt);
}

// RoPE on the Q and K heads of a fused QKV row and the KV overwrite of its K
// and V heads in one pass over the row: the same fp32 rotation as
// rope_apply_kernel, rounded once to bf16; the rotated K goes both back to
// the row and to the cache slot, V is a bit copy.  bf16 only.  One thread per
// unit of a token: a group of 8 rotation pairs of a Q or K head (the 16 bytes
// at i0 and the 16 at i0 + D/2), or a 16-byte piece of a V head.
__global__ void rope_kv_vec_kernel(uint16_t* __restrict__ x, int64_t stride, const int32_t* __restrict__ pos,
                                   const float* __restrict__ cos_sin, const int64_t* __restrict__ slot,
                                   uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int T, int Hq, int Hkv,
                                   int D, int max_pos, int64_t num_slots) {
  const int half = D >> 1, groups = half >> 3, row16 = D >> 3;
  const int rot_units = (Hq + Hkv) * groups;
  const int per_tok = rot_units + Hkv * row16;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)T * per_tok) return;
  const int t = (int)(gid / per_tok);
  const int u = (int)(gid - (int64_t)t * per_tok);
  uint16_t* row = x + (int64_t)t * stride;
  const int64_t s = slot[t];
  const bool to_cache = s >= 0 && s < num_slots;
  const int64_t page = s >> 4, off = s & 15;
  if (u < rot_units) {
    const int h = u / groups, i0 = (u - h * groups) * 8;
    uint4* pa = reinterpret_cast<uint4*>(row + (int64_t)h * D + i0);
    uint4* pb = reinterpret_cast<uint4*>(row + (int64_t)h * D + half + i0);
    uint4 a = *pa, b = *pb;
    const int p = pos[t];
    if (p >= 0 && p < max_pos) {
      const float4* cs = reinterpret_cast<const float4*>(cos_sin + ((int64_t)p * half + i0) * 2);
      uint32_t* aw = reinterpret_cast<uint32_t*>(&a);
      uint32_t* bw = reinterpret_cast<uint32_t*>(&b);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 c2 = cs[q];  // (cos, sin) of pairs i0 + 2q and i0 + 2q + 1
        const float a0 = __uint_as_float(aw[q] << 16), a1 = __uint_as_float(aw[q] & 0xffff0000u);
        const float b0 = __uint_as_float(bw[q] << 16), b1 = __uint_as_float(bw[q] & 0xffff0000u);
        const float ra0 = __fsub_rn(__fmul_rn(a0, c2.x), __fmul_rn(b0, c2.y));
        const float rb0 = __fadd_rn(__fmul_rn(b0, c2.x), __fmul_rn(a0, c2.y));
        const float ra1 = __fsub_rn(__fmul_rn(a1, c2.z), __fmul_rn(b1, c2.w));
        const float rb1 = __fadd_rn(__fmul_rn(b1, c2.z), __fmul_rn(a1, c2.w));
        aw[q] = (uint32_t)f2bf(ra0) | ((uint32_t)f2bf(ra1) << 16);
        bw[q] = (uint32_t)f2bf(rb0) | ((uint32_t)f2bf(rb1) << 16);
      }
      *pa = a;
      *pb = b;
    }
    if (h >= Hq && to_cache) {
      uint4* dst = k_cache + ((page * Hkv + (h - Hq)) * 16 + off) * row16;
      dst[i0 >> 3] = a;
      dst[(half + i0) >> 3] = b;
    }
  } else if (to_cache) {
    const int v = u - rot_units;
    const int h = v / row16, piece = v - h * row16;
    const uint4* src = reinterpret_cast<const uint4*>(row + (int64_t)(Hq + Hkv + h) * D);
    v_cache[((page * Hkv + h) * 16 + off) * row16 + piece] = src[piece];
  }
}

__global__ void swiglu_kernel(const void* __restrict__ gu, void* __restrict__ out, int64_t M, int64_t N, int64_t block,
                              int dt) {
  const int64_t total = M * N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / N, n = e - m * N;
    // gate and up of output n: the two halves of the row, or the two halves
    // of its 2*block-column group
    const int64_t gi = block == 0 ? m * 2 * N + n : m * 2 * N + (n / block) * 2 * block + n % block;
    const int64_t ui = block == 0 ? gi + N : gi + block;
    const float g = load_as_f32(gu, gi, dt);
    const float u = load_as_f32(gu, ui, dt);
    const float act = __fdiv_rn(g, __fadd_rn(1.0f, expf(-g)));
    store_from_f32(out, e, __fmul_rn(act, u), dt);
  }
}

// Whole-page copies inside one layer's cache, one thread per 16 bytes of a
// page of K and the same 16 bytes of V.  Pairs with a page outside
// [0, num_blocks) or with src == dst are skipped.
__global__ void kv_copy_pages_kernel(const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                     uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int n, int64_t page16,
                                     int num_blocks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n * page16) return;
  const int i = (int)(gid / page16);
  const int64_t piece = gid - (int64_t)i * page16;
  const int sp = src[i], dp = dst[i];
  if (sp < 0 || sp >= num_blocks || dp < 0 || dp >= num_blocks || sp == dp) return;
  k_cache[(int64_t)dp * page16 + piece] = k_cache[(int64_t)sp * page16 + piece];
  v_cache[(int64_t)dp * page16 + piece] = v_cache[(int64_t)sp * page16 + piece];
}

}  // namespace biv

extern "C" biv_status kv_overwrite(const void* k_new, const void* v_new, int64_t src_stride, const int64_t* slot,
                                   void* k_cache, void* v_cache, int T, int Hkv, int D, int num_blocks,
                                   biv_dtype dt, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "kv_overwrite: bad dtype %d", (int)dt);
  BIV_REQUIRE(T >= 0 && Hkv >= 1 && D >= 1 && num_blocks >= 0, "kv_overwrite: bad sizes T=%d Hkv=%d D=%d", T, Hkv, D);
  BIV_REQUIRE(src_stride >= (int64_t)Hkv * D, "kv_overwrite: src_stride %lld < Hkv*D", (long long)src_stride);
  if (T == 0) return BIV_OK;
  BIV_REQUIRE(k_new && v_new && slot && k_cache && v_cache, "kv_overwrite: NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t es = dt_size(dt);
  const int64_t num_slots = (int64_t)num_blocks * 16;
  const bool vec = ((size_t)D * es) % 16 == 0 && ((size_t)src_stride * es) % 16 == 0 && aligned16(k_new) &&
                   aligned16(v_new) && aligned16(k_cache) && aligned16(v_cache);
  if (vec) {
    const int row16 = (int)((size_t)D * es / 16);
    const int64_t n = (int64_t)T * Hkv * row16;
    hipLaunchKernelGGL(kv_overwrite_vec_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                       static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                       (int64_t)((size_t)src_stride * es / 16), slot, static_cast<uint4*>(k_cache),
                       static_cast<uint4*>(v_cache), T, Hkv, row16, num_slots);
  } else {
    const int64_t n = (int64_t)T * Hkv * D;
    if (dt == BIV_BF16)
      hipLaunchKernelGGL(kv_overwrite_elem_kernel<uint16_t>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), src_stride, slot,
                         static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), T, Hkv, D, num_slots);
    else
      hipLaunchKernelGGL(kv_overwrite_elem_kernel<float>, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s,
                         static_cast<const float*>(k_new), static_cast<const float*>(v_new), src_stride, slot,
                         static_cast<float*>(k_cache), static_cast<float*>(v_cache), T, Hkv, D, num_slots);
  }
  return launched("kv_overwrite");
}

extern "C" biv_status embed_rows(const int32_t* ids, const void* table, biv_dtype table_dt, void* out,
                                 biv_dtype out_dt, int T, int V, int H, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(table_dt) && valid_dt(out_dt), "embed_rows: bad dtype");
  BIV_REQUIRE(T >= 0 && V >= 1 && H >= 1, "embed_rows: bad sizes");
  if (T == 0) return BIV_OK;
  BIV_REQUIRE(ids && table && out, "embed_rows: NULL pointer");
  if (table_dt == BIV_BF16 && H % 8 == 0 && aligned16(table) && aligned16(out)) {
    if (out_dt == BIV_BF16)
      hipLaunchKernelGGL(embed_rows_vec_kernel<BIV_BF16>, dim3(T), dim3(256), 0, static_cast<hipStream_t>(stream), ids,
                         static_cast<const uint16_t*>(table), out, V, H);
    else
      hipLaunchKernelGGL(embed_rows_vec_kernel<BIV_F32>, dim3(T), dim3(256), 0, static_cast<hipStream_t>(stream), ids,
                         static_cast<const uint16_t*>(table), out, V, H);
    return launched("embed_rows");
  }
  hipLaunchKernelGGL(embed_rows_kernel, dim3(T), dim3(256), 0, static_cast<hipStream_t>(stream), ids, table,
                     (int)table_dt, out, (int)out_dt, V, H);
  return launched("embed_rows");
}

extern "C" biv_status rope_apply(void* x, int64_t stride, const int32_t* pos, const float* cos_sin, int T,
                                 int n_heads, int D, int max_pos, biv_dtype dt, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "rope_apply: bad dtype");
  BIV_REQUIRE(T >= 0 && n_heads >= 1 && D >= 2 && D % 2 == 0 && max_pos >= 1, "rope_apply: bad sizes");
  BIV_REQUIRE(stride >= (int64_t)n_heads * D, "rope_apply: stride < n_heads*D");
  if (T == 0) return BIV_OK;
  BIV_REQUIRE(x && pos && cos_sin, "rope_apply: NULL pointer");
  const int64_t n = (int64_t)T * n_heads * (D / 2);
  hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), x, stride, pos, cos_sin, T, n_heads, D, max_pos, (int)dt);
  return launched("rope_apply");
}

extern "C" biv_status rope_kv_overwrite(void* qkv, int64_t stride, const int32_t* pos, const float* cos_sin,
                                        const int64_t* slot, void* k_cache, void* v_cache, int T, int Hq, int Hkv,
                                        int D, int max_pos, int num_blocks, biv_dtype dt, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "rope_kv_overwrite: bad dtype");
  BIV_REQUIRE(T >= 0 && Hq >= 1 && Hkv >= 1 && D >= 2 && D % 2 == 0 && max_pos >= 1 && num_blocks >= 0,
              "rope_kv_overwrite: bad sizes T=%d Hq=%d Hkv=%d D=%d", T, Hq, Hkv, D);
  BIV_REQUIRE(stride >= (int64_t)(Hq + 2 * Hkv) * D, "rope_kv_overwrite: stride %lld < (Hq+2*Hkv)*D",
              (long long)stride);
  if (T == 0) return BIV_OK;
  BIV_REQUIRE(qkv && pos && cos_sin && slot && k_cache && v_cache, "rope_kv_overwrite: NULL pointer");
  const bool vec = dt == BIV_BF16 && D % 16 == 0 && stride % 8 == 0 && aligned16(qkv) && aligned16(cos_sin) &&
                   aligned16(k_cache) && aligned16(v_cache);
  if (!vec) {
    // the two separate passes, same results
    const biv_status r = rope_apply(qkv, stride, pos, cos_sin, T, Hq + Hkv, D, max_pos, dt, stream);
    if (r != BIV_OK) return r;
    const size_t es = dt_size(dt);
    const char* base = static_cast<const char*>(qkv);
    return kv_overwrite(base + (size_t)Hq * D * es, base + (size_t)(Hq + Hkv) * D * es, stride, slot, k_cache,
                        v_cache, T, Hkv, D, num_blocks, dt, stream);
  }
  const int64_t per_tok = (int64_t)(Hq + Hkv) * (D / 16) + (int64_t)Hkv * (D / 8);
  const int64_t n = (int64_t)T * per_tok;
  hipLaunchKernelGGL(rope_kv_vec_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint16_t*>(qkv), stride, pos, cos_sin, slot,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), T, Hq, Hkv, D, max_pos,
                     (int64_t)num_blocks * 16);
  return launched("rope_kv_overwrite");
}

extern "C" biv_status swiglu(const void* gu, void* out, int64_t M, int64_t N, int64_t block, biv_dtype dt,
                              biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "swiglu: bad dtype");
  BIV_REQUIRE(M >= 0 && N >= 1, "swiglu: bad sizes");
  BIV_REQUIRE(block == 0 || (block >= 1 && N % block == 0), "swiglu: block %lld must be 0 or divide N=%lld",
              (long long)block, (long long)N);
  if (M == 0) return BIV_OK;
  BIV_REQUIRE(gu && out, "swiglu: NULL pointer");
  const int64_t n = M * N;
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(n, 256), 8192);
  hipLaunchKernelGGL(swiglu_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), gu, out, M, N,
                     block, (int)dt);
  return launched("swiglu");
}

extern "C" biv_status kv_copy_pages(const int32_t* src_page, const int32_t* dst_page, int n, void* k_cache,
                                    void* v_cache, int num_blocks, int Hkv, int D, biv_dtype dt, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "kv_copy_pages: bad dtype");
  BIV_REQUIRE(n >= 0 && num_blocks >= 1 && Hkv >= 1 && D >= 1, "kv_copy_pages: bad sizes");
  if (n == 0) return BIV_OK;
  BIV_REQUIRE(src_page && dst_page && k_cache && v_cache, "kv_copy_pages: NULL pointer");
  BIV_REQUIRE(aligned16(k_cache) && aligned16(v_cache), "kv_copy_pages: caches must be 16-byte aligned");
  const int64_t page16 = (int64_t)Hkv * 16 * D * (int64_t)dt_size(dt) / 16;  // a page is 16 tokens: whole 16-byte pieces
  const int64_t total = (int64_t)n * page16;
  BIV_REQUIRE(cdiv(total, 256) <= 0x7fffffff, "kv_copy_pages: too many pages");
  hipLaunchKernelGGL(kv_copy_pages_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), src_page, dst_page, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), n, page16, num_blocks);
  return launched("kv_copy_pages");
}
