// attn_decode_bi: batch-invariant paged decode/verify attention, and
// attn_decode_adaptive, its non-invariant counterpart.
//
// LLM-42 post, paragraph 1: batch-invariant attention uses a fixed KV-split
// size, with no adaptation to sequence length or to how busy the GPU is.
// Paragraphs 3-4: the verifier runs K query rows for each of N requests; row
// (r, j) is the token at position ctx[r] + j and attends to positions
// 0 .. ctx[r] + j.
//
// bf16 path.  The keys of a request are cut at fixed absolute positions:
//   sub-tile = 32 keys (one MFMA block), chunk = 256 keys (the KV split),
//   segment  = seg_tokens keys (1024 for the invariant kernel).
// One workgroup of four waves per (segment, KV head, request).  Each wave
// computes the partial (m, l, o) of one chunk for all rows of the KV head:
// S^T = K Q^T and O^T = V^T P^T on the 32x32x16 bf16 MFMA, softmax statistics
// in fp32 (log2 domain), rescaled sub-tile by sub-tile in ascending order.
// The four chunk partials meet in LDS and are left-folded in ascending chunk
// order into the segment result (each thread folds 16 of the 32 x 128
// outputs); a segment longer than four chunks repeats this in rounds.
// Segment results go to the workspace; a second, small kernel left-folds
// them in ascending order and writes the output (a request with a single
// segment is written directly).  A kernel boundary, not a device-wide fence,
// makes the segment results visible: on gfx950 such a fence writes back and
// invalidates the whole L2 of an XCD, once per workgroup.  The rows of one KV head (q_len positions x G query heads <= 32)
// share one 32-row MFMA block, so the K/V of a page is read once for all of
// them (the pages' tile rule: G x (1+D) rows per KV head, here G x K <= 32).
// K/V pages move from HBM straight into LDS (gfx950 global_load_lds_dwordx4).
//
// Every boundary is an absolute position and every fold runs in ascending
// order, so a row's bits depend only on its own query, its own request's KV
// and its position -- not on the batch, the other rows or the grid.  A chunk
// or segment with no visible key for a row folds as an exact no-op.
#include <algorithm>

#include "biv_internal.h"

namespace biv {

constexpr int kHD = 128;                 // head dim of the MFMA path
constexpr int kSub = 32;                 // keys per sub-tile
constexpr int kChunk = BIV_ATTN_CHUNK_TOKENS;
constexpr int kSubsPerChunk = kChunk / kSub;
constexpr int kWaves = 4;                // waves per workgroup = chunks per round
constexpr int kStage = kSub * kHD * 2 * 2;  // 16 KiB: K and V of one sub-tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int kv_swz(int key, int chunk) { return key * 256 + ((chunk ^ (key & 7)) << 4); }

struct AttnWs {
  float* part_o;   // [slot][4096]: element t + 256 k of thread t
  float* part_ml;  // [slot][64 lanes][2]
};

// (M, L, O) <- fold((M, L, O), (m, l, o)) for the 16 outputs a thread owns.
__device__ __forceinline__ void fold16(float& M, float& L, float (&O)[16], float m, float l, const float (&o)[16]) {
  const float mn = fmaxf(M, m);
  if (mn == -INFINITY) return;  // both empty
  const float a = exp2f(M - mn);  // 0 when M == -inf, exactly 1 when M == mn
  const float b = exp2f(m - mn);
  L = __fadd_rn(__fmul_rn(L, a), __fmul_rn(l, b));
#pragma unroll
  for (int k = 0; k < 16; ++k) O[k] = __fadd_rn(__fmul_rn(O[k], a), __fmul_rn(o[k], b));
  M = mn;
}

__global__ __launch_bounds__(64 * kWaves, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx,
    uint16_t* __restrict__ out, int q_len, int Hq, int Hkv, int max_blocks, int num_blocks, float scale_log2,
    int seg_tokens, int nseg_max, AttnWs ws) {
  // per wave: staging of one sub-tile's K and V (separate arrays, so the
  // compiler tracks the direct-to-LDS loads of each apart), reused for the
  // wave's chunk partial
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[kWaves][kStage / 2];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v[kWaves][kStage / 2];
  __shared__ float lds_ml[kWaves][64][2];
  const int seg = blockIdx.x, kvh = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int G = Hq / Hkv, nrows = q_len * G;
  const int L = ctx[r];
  const int n_tok = min(L + q_len, max_blocks * 16);
  const int nseg = (n_tok + seg_tokens - 1) / seg_tokens;
  if (seg >= nseg) return;
  const int tok_begin = seg * seg_tokens;
  const int tok_end = min(tok_begin + seg_tokens, n_tok);
  const int32_t* bt = block_table + (int64_t)r * max_blocks;

  // this lane's query row (MFMA column li) and its last visible key
  const int rho = li;
  const bool row_ok = rho < nrows;
  const int jq = row_ok ? rho / G : 0;
  const int hq = kvh * G + (row_ok ? rho % G : 0);
  const int last_key = row_ok ? L + jq : -1;
  const int64_t qtok = (int64_t)r * q_len + jq;

  bf16x8 bq[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (row_ok) {
      bq[t] = *reinterpret_cast<const bf16x8*>(q + qtok * q_stride + (int64_t)hq * kHD + 8 * (2 * t + g));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bq[t][e] = (__bf16)0.0f;
    }
  }

  unsigned char* Ks = lds_k[wave];
  unsigned char* Vs = lds_v[wave];
  const int n_pages = (n_tok + 15) >> 4;
  // Staging of 32 keys of K (or V) straight from HBM into LDS (gfx950
  // global_load_lds_dwordx4: no registers, lane i writes bytes 16i..16i+15 of
  // the instruction's 1 KiB window).  Instruction i covers keys 4i..4i+3, all
  // in one page; the XOR swizzle of the LDS layout is applied by choosing
  // which 16-byte chunk of its key each lane fetches.  Keys of a missing page
  // are fetched from page 0 (in bounds); their values, and those of positions
  // past the request's last one, are zeroed after landing: a masked key must
  // contribute exactly nothing, whatever its slot holds.  Each call issues 8
  // loads, counted by vmcnt in issue order.
  // byte offset of lane's 16-byte piece within a 4-key, 1 KiB window of a
  // page: key 4i + lane/16 (row), 16-byte chunk (lane%16) ^ (key%8) (the
  // swizzle); key%8 = 4(i%2) + lane/16, so two variants cover every i
  const unsigned voff_even = 256u * (lane >> 4) + 16u * ((lane & 15) ^ (lane >> 4));
  const unsigned voff_odd = 256u * (lane >> 4) + 16u * ((lane & 15) ^ (4 + (lane >> 4)));
  auto dma = [&](const uint16_t* cache, unsigned char* dst, int p0, int p1) {
    const uint16_t* b0 = cache + ((int64_t)(p0 >= 0 ? p0 : 0) * Hkv + kvh) * 16 * kHD;
    const uint16_t* b1 = cache + ((int64_t)(p1 >= 0 ? p1 : 0) * Hkv + kvh) * 16 * kHD;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned char* base = reinterpret_cast<const unsigned char*>(i < 4 ? b0 : b1) + 1024 * (i & 3);
      lds_dma16(base, (i & 1) ? voff_odd : voff_even, dst + 1024 * i);
    }
  };
  auto zero_missing = [&](int sub_base, int p0, int p1) {
    if (p0 >= 0 && p1 >= 0 && sub_base + kSub <= n_tok) return;  // wave-uniform
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 4 * i + (lane >> 4);
      const bool ok = (i < 4 ? p0 : p1) >= 0 && sub_base + key < n_tok;
      if (!ok) *reinterpret_cast<u32x4*>(Vs + 1024 * i + 16 * lane) = zero;  // row of key 4i + lane/16
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Segment result for the 16 outputs this thread owns: lane `lane`'s
  // accumulator values v = wave + 4k, k = 0..15 (row li).  It is only live
  // between rounds; a segment of more than one round (more than four chunks)
  // parks it in its workspace slot while the next round's chunks run.
  float Ms = -INFINITY, Ls = 0.0f, Os[16];
  const int64_t slot = ((int64_t)r * Hkv + kvh) * nseg_max + seg;
  float* slot_o = ws.part_o + slot * 4096;
  float* slot_ml = ws.part_ml + slot * 128;

  const int first_chunk = tok_begin / kChunk;
  const int end_chunk = (tok_end + kChunk - 1) / kChunk;
  for (int c0 = first_chunk; c0 < end_chunk; c0 += kWaves) {
    const int c = c0 + wave;
    float mc = -INFINITY, lc = 0.0f;
    f32x16 oc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) oc[d][v] = 0.0f;
    if (c < end_chunk) {
      // the chunk's 16 pages, one per lane 0..15, then read with readlane
      int mypage = -1;
      {
        const int lp = c * 16 + lane;
        if (lane < 16 && lp < n_pages) {
          const int p = bt[lp];
          mypage = (p >= 0 && p < num_blocks) ? p : -1;
        }
      }
      auto page = [&](int i) { return __builtin_amdgcn_readlane(mypage, i); };
      const int base0 = c * kChunk;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier LDS reads of the buffers are done
      dma(k_cache, Ks, page(0), page(1));
      dma(v_cache, Vs, page(0), page(1));
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // K of sub-tile 0 has landed
      for (int st = 0; st < kSubsPerChunk; ++st) {
        const int sub_base = base0 + st * kSub;
        const int p0 = page(2 * st), p1 = page(2 * st + 1);
        const bool more = st + 1 < kSubsPerChunk;
        // S^T[key][row] for the 32 keys of this sub-tile
        f32x16 s;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + kv_swz(li, 2 * t + g));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[t], s, 0, 0, 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K reads done: refill the K buffer
        if (more) dma(k_cache, Ks, page(2 * st + 2), page(2 * st + 3));
        // every row sees every key of the sub-tile: no per-score mask
        const bool all_visible = p0 >= 0 && p1 >= 0 && sub_base + kSub - 1 <= L;
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 8 * (v >> 2) + 4 * g + (v & 3);
          const bool ok = all_visible || (sub_base + kk <= last_key && (kk < 16 ? p0 : p1) >= 0);
          x[v] = ok ? __fmul_rn(s[v], scale_log2) : -INFINITY;
          tmax = fmaxf(tmax, x[v]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(mc, tmax);
        float alpha = 1.0f, lsum = 0.0f;
        bf16x8 pb[2];
        if (mn == -INFINITY) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[0][e] = (__bf16)0.0f;
            pb[1][e] = (__bf16)0.0f;
          }
        } else {
          alpha = exp2f(mc - mn);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = x[v] == -INFINITY ? 0.0f : exp2f(x[v] - mn);
            lsum = __fadd_rn(lsum, p);
            pb[v >> 3][v & 7] = (__bf16)p;
          }
        }
        lsum = __fadd_rn(lsum, __shfl_xor(lsum, 32, 64));
        lc = __fadd_rn(__fmul_rn(lc, alpha), lsum);
        mc = mn;
        // V of this sub-tile has landed (the K refill, if any, is newer)
        if (more)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        zero_missing(sub_base, p0, p1);
        const bool rescale = __any(alpha != 1.0f);  // wave-uniform; x * 1 == x exactly
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if (rescale) {
#pragma unroll
            for (int v = 0; v < 16; ++v) oc[d][v] = __fmul_rn(oc[d][v], alpha);
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            // V^T fragment: dim 32d + li, keys matching the lane group's P values
            bf16x8 va;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kk = 16 * h + (e < 4 ? 4 * g + e : 8 + 4 * g + (e - 4));
              const int dim = 32 * d + li;
              const uint16_t bits = *reinterpret_cast<const uint16_t*>(Vs + kv_swz(kk, dim >> 3) + 2 * (dim & 7));
              va[e] = __builtin_bit_cast(__bf16, bits);
            }
            oc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[h], oc[d], 0, 0, 0);
          }
        }
        if (more) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V reads done: refill the V buffer
          dma(v_cache, Vs, page(2 * st + 2), page(2 * st + 3));
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // K of the next sub-tile has landed
        }
      }
    }
    // chunk partials meet in LDS (the staging buffer of each wave)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // values 0..31 of each lane go to the K buffer, 32..63 to the V buffer
    float* pk = reinterpret_cast<float*>(lds_k[wave]);
    float* pv = reinterpret_cast<float*>(lds_v[wave]);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) (d < 2 ? pk : pv)[((d & 1) * 16 + v) * 64 + lane] = oc[d][v];
    lds_ml[wave][lane][0] = mc;
    lds_ml[wave][lane][1] = lc;
    __syncthreads();
    if (c0 == first_chunk) {
      Ms = -INFINITY;
      Ls = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) Os[k] = 0.0f;
    } else {  // resume the segment result parked after the previous round
      Ms = slot_ml[lane * 2 + 0];
      Ls = slot_ml[lane * 2 + 1];
#pragma unroll
      for (int k = 0; k < 16; ++k) Os[k] = slot_o[tid + 256 * k];
    }
    for (int w = 0; w < kWaves; ++w) {  // ascending chunk order
      const float* qk = reinterpret_cast<const float*>(lds_k[w]);
      const float* qv = reinterpret_cast<const float*>(lds_v[w]);
      float o[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int v = wave + 4 * k;
        o[k] = (v < 32 ? qk : qv)[(v & 31) * 64 + lane];
      }
      fold16(Ms, Ls, Os, lds_ml[w][lane][0], lds_ml[w][lane][1], o);
    }
    if (c0 + kWaves < end_chunk) {  // park for the next round (each thread reads back only its own values)
#pragma unroll
      for (int k = 0; k < 16; ++k) slot_o[tid + 256 * k] = Os[k];
      if (wave == 0) {
        slot_ml[lane * 2 + 0] = Ms;
        slot_ml[lane * 2 + 1] = Ls;
      }
    }
    __syncthreads();
  }

  // output element of value v = wave + 4k of lane `lane`
  auto write_out = [&](float Lsum, const float (&O)[16]) {
    if (!row_ok) return;
    const float inv = Lsum > 0.0f ? __fdiv_rn(1.0f, Lsum) : 0.0f;
    uint16_t* orow = out + (qtok * Hq + hq) * kHD;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int v = wave + 4 * k;
      const int vv = v & 15;
      const int dim = 32 * (v >> 4) + 8 * (vv >> 2) + 4 * g + (vv & 3);
      orow[dim] = f2bf(__fmul_rn(O[k], inv));
    }
  };

  if (nseg == 1) {
    write_out(Ls, Os);
    return;
  }
  // segment result -> workspace; attn_combine_kernel folds the segments
#pragma unroll
  for (int k = 0; k < 16; ++k) slot_o[tid + 256 * k] = Os[k];
  if (wave == 0) {
    slot_ml[lane * 2 + 0] = Ms;
    slot_ml[lane * 2 + 1] = Ls;
  }
}

// Second pass for requests with more than one segment: left-fold the segment
// results in ascending order (the same fold as above, element by element) and
// write the output.  One workgroup per (KV head, request); thread t owns the
// same 16 outputs as thread t of the first pass.
__global__ __launch_bounds__(256) void attn_combine_kernel(const int32_t* __restrict__ ctx,
                                                           uint16_t* __restrict__ out, int q_len, int Hq,
                                                           int Hkv, int max_blocks, int seg_tokens, int nseg_max,
                                                           AttnWs ws) {
  const int kvh = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int G = Hq / Hkv, nrows = q_len * G;
  const int n_tok = min(ctx[r] + q_len, max_blocks * 16);
  const int nseg = (n_tok + seg_tokens - 1) / seg_tokens;
  if (nseg <= 1 || li >= nrows) return;  // single segment: written by the first pass
  const int jq = li / G, hq = kvh * G + li % G;
  float M = -INFINITY, Lt = 0.0f, O[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) O[k] = 0.0f;
  for (int s2 = 0; s2 < nseg; ++s2) {
    const int64_t sl = ((int64_t)r * Hkv + kvh) * nseg_max + s2;
    float o2[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) o2[k] = __builtin_nontemporal_load(ws.part_o + sl * 4096 + tid + 256 * k);
    const float m2 = ws.part_ml[sl * 128 + lane * 2 + 0];
    const float l2 = ws.part_ml[sl * 128 + lane * 2 + 1];
    fold16(M, Lt, O, m2, l2, o2);
  }
  const float inv = Lt > 0.0f ? __fdiv_rn(1.0f, Lt) : 0.0f;
  uint16_t* orow = out + (((int64_t)r * q_len + jq) * Hq + hq) * kHD;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int v = wave + 4 * k;
    const int vv = v & 15;
    orow[32 * (v >> 4) + 8 * (vv >> 2) + 4 * g + (vv & 3)] = f2bf(__fmul_rn(O[k], inv));
  }
}

// fp32 path: one wave per (query row, query head, request).  Same chunking:
// 256-key chunks at absolute positions, chunk partials (natural-exp domain)
// left-folded in ascending order.  Lanes own keys for the scores and
// dimensions for the weighted sum; every sum runs in a fixed order.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, int64_t q_stride,
                                                      const float* __restrict__ k_cache,
                                                      const float* __restrict__ v_cache,
                                                      const int32_t* __restrict__ block_table,
                                                      const int32_t* __restrict__ ctx, float* __restrict__ out,
                                                      int q_len, int Hq, int Hkv, int D, int max_blocks,
                                                      int num_blocks, float scale) {
  __shared__ float qs[128];
  __shared__ float ps[kChunk];
  const int j = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x;
  const int G = Hq / Hkv, kvh = h / G;
  const int L = ctx[r];
  const int n_keys = min(L + j + 1, max_blocks * 16);
  const int32_t* bt = block_table + (int64_t)r * max_blocks;
  const int64_t qtok = (int64_t)r * q_len + j;
  const int64_t qrow = qtok * Hq + h;
  for (int d = lane; d < D; d += 64) qs[d] = q[qtok * q_stride + (int64_t)h * D + d];
  __syncthreads();
  float M = -INFINITY, Ls = 0.0f, O0 = 0.0f, O1 = 0.0f;
  for (int cb = 0; cb < n_keys; cb += kChunk) {
    const int ce = min(cb + kChunk, n_keys);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = cb + lane + 64 * u;
      float s = -INFINITY;
      if (key < ce) {
        const int page = bt[key >> 4];
        if (page >= 0 && page < num_blocks) {
          const float* kp = k_cache + (((int64_t)page * Hkv + kvh) * 16 + (key & 15)) * D;
          float acc = 0.0f;
          for (int d = 0; d < D; ++d) acc = __fmaf_rn(qs[d], kp[d], acc);
          s = __fmul_rn(acc, scale);
        }
      }
      sv[u] = s;
      mx = fmaxf(mx, s);
    }
    const float mc = wave_max(mx);
    float lsum = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p = (sv[u] == -INFINITY) ? 0.0f : expf(__fsub_rn(sv[u], mc));
      ps[lane + 64 * u] = p;
      lsum = __fadd_rn(lsum, p);
    }
    const float lc = wave_sum(lsum);
    __syncthreads();
    float o0 = 0.0f, o1 = 0.0f;
    for (int key = cb; key < ce; ++key) {
      const int page = bt[key >> 4];
      if (page < 0 || page >= num_blocks) continue;
      const float p = ps[key - cb];
      const float* vp = v_cache + (((int64_t)page * Hkv + kvh) * 16 + (key & 15)) * D;
      o0 = __fmaf_rn(p, vp[lane], o0);
      if (D > 64) o1 = __fmaf_rn(p, vp[lane + 64], o1);
    }
    __syncthreads();
    const float mn = fmaxf(M, mc);
    if (mn != -INFINITY) {
      const float a = expf(__fsub_rn(M, mn)), b = expf(__fsub_rn(mc, mn));
      Ls = __fadd_rn(__fmul_rn(Ls, a), __fmul_rn(lc, b));
      O0 = __fadd_rn(__fmul_rn(O0, a), __fmul_rn(o0, b));
      O1 = __fadd_rn(__fmul_rn(O1, a), __fmul_rn(o1, b));
      M = mn;
    }
  }
  const float inv = Ls > 0.0f ? __fdiv_rn(1.0f, Ls) : 0.0f;
  out[qrow * D + lane] = __fmul_rn(O0, inv);
  if (D > 64) out[qrow * D + lane + 64] = __fmul_rn(O1, inv);
}

static biv_status check_attn(const char* who, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* ctx, void* out, int R, int q_len, int Hq,
                             int Hkv, int D, int max_blocks, int num_blocks) {
  BIV_REQUIRE(R >= 0 && q_len >= 1 && Hq >= 1 && Hkv >= 1 && max_blocks >= 1 && num_blocks >= 1,
              "%s: bad sizes R=%d q_len=%d Hq=%d Hkv=%d max_blocks=%d num_blocks=%d", who, R, q_len, Hq, Hkv,
              max_blocks, num_blocks);
  BIV_REQUIRE(Hq % Hkv == 0, "%s: Hq=%d not a multiple of Hkv=%d", who, Hq, Hkv);
  BIV_REQUIRE(q_stride >= (int64_t)Hq * D, "%s: q_stride %lld < Hq*D", who, (long long)q_stride);
  BIV_REQUIRE((int64_t)max_blocks * 16 <= (1 << 30), "%s: max_blocks too large", who);
  BIV_REQUIRE(R <= 65535 && Hkv <= 65535 && q_len <= 65535 && Hq <= 65535, "%s: grid dimension too large", who);
  if (R > 0) BIV_REQUIRE(q && k_cache && v_cache && block_table && ctx && out, "%s: NULL pointer", who);
  (void)D;
  return BIV_OK;
}

static biv_status launch_attn_bf16(const char* who, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* ctx, void* out, int R, int q_len,
                                   int Hq, int Hkv, int max_blocks, int num_blocks, float scale, int seg_tokens,
                                   void* workspace, size_t workspace_bytes, hipStream_t s) {
  BIV_REQUIRE(q_len * (Hq / Hkv) <= 32, "%s: bf16 path needs q_len*Hq/Hkv <= 32 (got %d)", who, q_len * (Hq / Hkv));
  BIV_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && q_stride % 8 == 0,
              "%s: q (and its row stride) and the caches must be 16-byte aligned", who);
  const size_t need = biv_attn_workspace_bytes(R, Hkv, max_blocks, seg_tokens);
  BIV_REQUIRE(workspace != nullptr && workspace_bytes >= need, "%s: workspace needs %zu bytes (got %zu)", who, need,
              workspace_bytes);
  BIV_REQUIRE(aligned16(workspace), "%s: workspace must be 16-byte aligned", who);
  const int nseg_max = (int)cdiv((int64_t)max_blocks * 16, seg_tokens);
  BIV_REQUIRE(nseg_max <= 0x7fffffff, "%s: too many segments", who);
  AttnWs ws;
  ws.part_o = static_cast<float*>(workspace);
  ws.part_ml = ws.part_o + (size_t)R * Hkv * nseg_max * 4096;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(nseg_max, Hkv, R), dim3(64 * kWaves), 0, s, static_cast<const uint16_t*>(q), q_stride,
                     static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table, ctx,
                     static_cast<uint16_t*>(out), q_len, Hq, Hkv, max_blocks, num_blocks, scale * kLog2e,
                     seg_tokens, nseg_max, ws);
  biv_status st = launched(who);
  if (st != BIV_OK || nseg_max <= 1) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hkv, R), dim3(256), 0, s, ctx, static_cast<uint16_t*>(out), q_len,
                     Hq, Hkv, max_blocks, seg_tokens, nseg_max, ws);
  return launched(who);
}

}  // namespace biv

extern "C" size_t biv_attn_workspace_bytes(int R, int Hkv, int max_blocks, int seg_tokens) {
  using namespace biv;
  if (R <= 0 || Hkv <= 0 || max_blocks <= 0 || seg_tokens <= 0) return 0;
  const size_t nseg = (size_t)cdiv((int64_t)max_blocks * 16, seg_tokens);
  return (size_t)R * Hkv * nseg * (4096 + 128) * sizeof(float);
}

extern "C" biv_status attn_decode_bi(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx, void* out, int R, int q_len,
                                     int Hq, int Hkv, int D, int max_blocks, int num_blocks, float scale,
                                     biv_dtype dt, void* workspace, size_t workspace_bytes, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "attn_decode_bi: bad dtype");
  biv_status st = check_attn("attn_decode_bi", q, q_stride, k_cache, v_cache, block_table, ctx, out, R, q_len, Hq, Hkv, D,
                             max_blocks, num_blocks);
  if (st != BIV_OK) return st;
  if (R == 0) return BIV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == BIV_BF16) {
    if (D != kHD) return fail(BIV_EUNSUPPORTED, "attn_decode_bi: bf16 path supports D == 128 only (D=%d)", D);
    if (q_len * (Hq / Hkv) > 32)
      return fail(BIV_EUNSUPPORTED, "attn_decode_bi: bf16 path needs q_len*Hq/Hkv <= 32 (got %d)", q_len * (Hq / Hkv));
    return launch_attn_bf16("attn_decode_bi", q, q_stride, k_cache, v_cache, block_table, ctx, out, R, q_len, Hq, Hkv,
                            max_blocks, num_blocks, scale, BIV_ATTN_SEG_TOKENS, workspace, workspace_bytes, s);
  }
  if (D != 64 && D != 128) return fail(BIV_EUNSUPPORTED, "attn_decode_bi: fp32 path supports D in {64,128} (D=%d)", D);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(q_len, Hq, R), dim3(64), 0, s, static_cast<const float*>(q), q_stride,
                     static_cast<const float*>(k_cache), static_cast<const float*>(v_cache), block_table, ctx,
                     static_cast<float*>(out), q_len, Hq, Hkv, D, max_blocks, num_blocks, scale);
  return launched("attn_decode_bi/f32");
}

extern "C" int biv_attn_adaptive_split(int R, int Hkv, int max_blocks) {
  using namespace biv;
  if (R <= 0 || Hkv <= 0 || max_blocks <= 0) return kChunk;
  const int64_t cap = (int64_t)max_blocks * 16;
  const int64_t want = cdiv(1024, (int64_t)R * Hkv);  // segments per (request, head) for 4 waves per CU
  int64_t split = cdiv(cdiv(cap, want), kChunk) * kChunk;
  return (int)std::max<int64_t>(kChunk, split);
}

extern "C" biv_status attn_decode_adaptive(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                           const int32_t* block_table, const int32_t* ctx, void* out, int R,
                                           int q_len, int Hq, int Hkv, int D, int max_blocks, int num_blocks,
                                           float scale, int split_tokens, void* workspace, size_t workspace_bytes,
                                           biv_stream stream) {
  using namespace biv;
  biv_status st = check_attn("attn_decode_adaptive", q, q_stride, k_cache, v_cache, block_table, ctx, out, R, q_len, Hq, Hkv,
                             D, max_blocks, num_blocks);
  if (st != BIV_OK) return st;
  if (R == 0) return BIV_OK;
  if (D != kHD) return fail(BIV_EUNSUPPORTED, "attn_decode_adaptive: supports D == 128 only (D=%d)", D);
  if (q_len * (Hq / Hkv) > 32) return fail(BIV_EUNSUPPORTED, "attn_decode_adaptive: needs q_len*Hq/Hkv <= 32");
  BIV_REQUIRE(split_tokens >= 0 && split_tokens % kChunk == 0, "attn_decode_adaptive: split_tokens must be a multiple of %d", kChunk);
  const int split = split_tokens == 0 ? biv_attn_adaptive_split(R, Hkv, max_blocks) : split_tokens;
  return launch_attn_bf16("attn_decode_adaptive", q, q_stride, k_cache, v_cache, block_table, ctx, out, R, q_len, Hq, Hkv,
                          max_blocks, num_blocks, scale, split, workspace, workspace_bytes,
                          static_cast<hipStream_t>(stream));
}
