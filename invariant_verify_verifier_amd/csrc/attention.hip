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
//   segment  = seg_tokens keys (4096 for the invariant kernel), taken by one
//              wave, or split over several at small batch (see the kernel).
// One 64-lane wave per (segment, KV head, row block) -- or per part of a
// segment where the grid holds few segments -- four per CU.  The rows
// of one KV head in a row block (32/G positions x G query heads) share one
// 32-row MFMA block, so the K/V of a page is read once for all of them (the
// pages' tile rule: G x (1+D) rows per KV head, here G x K <= 32: a verify
// step of K <= 8 positions is one block per request; a longer q_len, e.g. a
// prefill, takes several blocks, each with the keys up to its last row).  The wave streams
// its segment's K and V sub-tiles from HBM straight into a ring of LDS slots
// (gfx950 global_load_lds_dwordx4) and computes S^T = K Q^T and O^T = V^T P^T
// on the 32x32x16 bf16 MFMA, softmax statistics in fp32 (log2 domain),
// sub-tile by sub-tile in ascending order; each finished chunk's partial
// (m, l, o) is left-folded into the segment result in registers (in the
// later parts of a split segment it is stored instead).  Segment results
// (and stored chunk partials) go to the workspace; where segments were
// split, a small kernel completes each split segment's fold (all segments
// of a request at once), and a second small kernel left-folds the segments
// in ascending order and writes the output (a request with a single,
// unsplit segment is written directly).  Kernel boundaries, not device-wide
// fences, make the partials visible: on gfx950 such a fence writes back and
// invalidates the whole L2 of an XCD.
//
// Every boundary is an absolute position and every fold runs in ascending
// order, so a row's bits depend only on its own query, its own request's KV
// and its position -- not on the batch, the other rows or the grid.  A chunk
// or segment with no visible key for a row folds as an exact no-op.
#include <algorithm>
#include <mutex>

#include "biv_internal.h"

namespace biv {

constexpr int kHD = 128;                 // head dim of the MFMA path
constexpr int kSub = 32;                 // keys per sub-tile
constexpr int kChunk = BIV_ATTN_CHUNK_TOKENS;
// The non-invariant comparison path's chunk: it cuts its segments at any
// multiple of it (its fold tree may vary with the split; that is what it is
// for).
constexpr int kAdaptiveChunk = 256;
static_assert(kChunk % kSub == 0 && kAdaptiveChunk % kSub == 0 && kChunk % kAdaptiveChunk == 0, "chunk sizes");
constexpr int kF32Chunk = 256;  // the fp32 path's chunk: four keys per lane
static_assert(kF32Chunk == kChunk, "both paths cut the keys at the same chunk boundaries");
constexpr int kSlot = kSub * kHD * 2;    // 8 KiB: K or V of one sub-tile
constexpr int kRing = 5;                 // LDS slots per wave (40 KiB: four waves fill a CU's 160 KiB)
static_assert(kRing == 5, "wait_ring: a full ring leaves four loads (32 copies) in flight");
constexpr int kPagesPerWin = 64;         // page ids held in one register (lane i: page i of the window)
constexpr int kPreWin = 4;               // page windows loaded at a wave's start (4096 tokens)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;            // max drift (log2) before the accumulators are rescaled

// 2^x with the hardware instruction (v_exp_f32): exact at 0 and -inf; a
// result below the normal range is flushed to zero.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of 16-byte piece c of key row k (256 bytes) in LDS is c ^ kv_swz(k).
// K reads (16 lanes = 16 consecutive keys, one piece each) and V transpose
// reads (4 consecutive keys x 4 consecutive pieces per 32 lanes) both land on
// distinct bank groups.
__device__ __forceinline__ int kv_swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }

__device__ __forceinline__ int pick_window(int w, int w0, int w1, int w2, int w3, int wx) {
  return w == 0 ? w0 : (w == 1 ? w1 : (w == 2 ? w2 : (w == 3 ? w3 : wx)));
}

// Rows of request r: q_len_r = q_off[r+1] - q_off[r] (clamped to [0, q_len])
// starting at row q_off[r], or q_len rows from row r*q_len without q_off.
struct ReqRows {
  int64_t first;  // row of position ctx[r] + 0
  int n;          // rows (0: the request has none)
};
__device__ __forceinline__ ReqRows req_rows(const int32_t* __restrict__ q_off, int r, int q_len) {
  if (q_off == nullptr) return {(int64_t)r * q_len, q_len};
  const int a = q_off[r], b = q_off[r + 1];
  return {(int64_t)a, a < 0 ? 0 : min(max(b - a, 0), q_len)};
}

struct AttnWs {
  float* part_o;   // [slot][16 groups][64 lanes][4]: values 4q .. 4q+3 of a lane in group q
  float* part_ml;  // [slot][64 lanes][2]
  float* chunk_o;  // chunk partials of split segments, same layout, slot (v, KV head, chunk)
  float* chunk_ml;
};

// Partial (m, l, o[64]) of a lane -> slot `slot` of (po, pml): sixteen 1 KiB
// stores of four values each, with the non-temporal hint when kStream, then
// m and l.
// Lanes of rows past the row block's last (live false) store nothing: the
// combine never reads them, and at one query position per request only 4 of
// the 32 rows are real.
template <bool kStream>
__device__ __forceinline__ void store_partial(float* po, float* pml, int64_t slot, int lane, bool live, float m,
                                              float l, const float* o) {
  if (!live) return;
  float* so = po + slot * 4096;
#pragma unroll
  for (int qg = 0; qg < 16; ++qg) {
    const f32x4 w = {o[4 * qg + 0], o[4 * qg + 1], o[4 * qg + 2], o[4 * qg + 3]};
    f32x4* dst = reinterpret_cast<f32x4*>(so + (qg * 64 + lane) * 4);
    if constexpr (kStream)
      __builtin_nontemporal_store(w, dst);
    else
      *dst = w;
  }
  pml[slot * 128 + lane * 2 + 0] = m;
  pml[slot * 128 + lane * 2 + 1] = l;
}

// A wave-uniform 64-bit value in SGPRs.  readfirstlane returns int: each
// half goes through uint32_t so that the low half is zero-extended, not
// sign-extended, when the two are put together.
__device__ __forceinline__ uint64_t wave_uniform_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// One ring slot's copies: two 16-token pages (K or V of one KV head) of
// 4 KiB each, eight gfx950 global_load_lds_dwordx4.  Lane i of copy c of
// page q reads 16 bytes at base_q + voff_c(i) + 1024c and writes them to LDS
// bytes m0_q + 1024c + 16i .. +15: the instruction's offset field moves the
// global address and the LDS address alike, so one M0 serves a page.
// base_q (64-bit) and m0_q are wave-uniform; m0_q is an LDS byte address.
// The copies carry the non-temporal hint: the K/V stream is read once per
// call, and keeping it from allocating in the caches made the 8B-shaped
// pass's attention 10% faster (279 -> 252 us) with the same bits.
// Issued as inline asm so that the compiler does not model the LDS writes
// (it would wait for every outstanding copy before any LDS read); the
// kernel orders the copies with explicit vmcnt waits.  The compiler cannot
// see into the block, so it carries its own wait states: 5 before the first
// load (an SGPR operand last written by a VALU instruction, such as
// readfirstlane, needs 5 before a memory instruction reads it; an M0 write
// needs 1 before an LDS DMA) and 1 after the second M0 write.  The bf16
// kernel has no other reader of M0 (the compiler sets M0 immediately before
// each instruction of its own that reads it).
__device__ __forceinline__ void lds_copy_slot(uint64_t base0, uint64_t base1, unsigned m00, unsigned m01,
                                              unsigned voff0, unsigned voff1, unsigned voff2, unsigned voff3) {
  const uint64_t b0 = wave_uniform_u64(base0), b1 = wave_uniform_u64(base1);
  const unsigned m0a = (uint32_t)__builtin_amdgcn_readfirstlane(m00);
  const unsigned m0b = (uint32_t)__builtin_amdgcn_readfirstlane(m01);
  asm volatile(
      "s_mov_b32 m0, %6\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %4 offset:0 nt\n\t"
      "global_load_lds_dwordx4 %1, %4 offset:1024 nt\n\t"
      "global_load_lds_dwordx4 %2, %4 offset:2048 nt\n\t"
      "global_load_lds_dwordx4 %3, %4 offset:3072 nt\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %5 offset:0 nt\n\t"
      "global_load_lds_dwordx4 %1, %5 offset:1024 nt\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:2048 nt\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:3072 nt" ::"v"(voff0),
      "v"(voff1), "v"(voff2), "v"(voff3), "s"(b0), "s"(b1), "s"(m0a), "s"(m0b)
      : "memory");
}

// Wait until at most 8n direct-to-LDS copies (n loads) are outstanding.
__device__ __forceinline__ void wait_loads_after(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
  }
}

// The same, with the common case (a full ring: n >= 4) as one wait.
__device__ __forceinline__ void wait_ring(int n) {
  if (n >= 4)
    asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else
    wait_loads_after(n);
}

// fp32 value of lane l ^ 32 combined with lane l's own: permlane32 swap
// exchanges the two 32-lane halves of a copy of x, so for every lane the two
// results are {x[l], x[l ^ 32]} in some order.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));  // x[l] + x[l ^ 32]: fp32 add commutes
}

// (M, L, O) <- fold((M, L, O), (m, l, o)) over N outputs.  The products
// and sums are written as one explicit fused multiply-add of a rounded
// product (o*b + round(O*a)), which the compiler cannot fuse differently
// from one kernel to the other: the fold gives the same bits in both
// kernels that run it (a chunk is folded in the first pass, or, in a split
// segment, in the second).
template <int N>
__device__ __forceinline__ void fold_into(float& M, float& L, float* O, float m, float l, const float* o) {
  const float mn = fmaxf(M, m);
  if (mn == -INFINITY) return;  // both empty
  const float a = exp2f(M - mn);  // 0 when M == -inf, exactly 1 when M == mn
  const float b = exp2f(m - mn);
  L = fmaf(l, b, L * a);
#pragma unroll
  for (int k = 0; k < N; ++k) O[k] = fmaf(o[k], b, O[k] * a);
  M = mn;
}

// One wave per (segment, KV head, request).  The wave streams the K and V
// sub-tiles of its segment through a ring of kRing 8 KiB LDS slots in the
// order K0 V0 K1 V1 ...; a slot is refilled with the load kRing places later
// as soon as it has been read, so up to kRing loads are in flight at once.
// Lane (li, g) owns query row li of the KV head's 32-row block: it computes
// S^T = K Q^T and O^T = V^T P^T with the 32x32x16 bf16 MFMA (its column),
// keeps the chunk partial (m, l, o) and the segment result (M, L, O) of its
// row in registers, and folds each finished chunk into the segment result.
template <bool kParts>
__global__ __launch_bounds__(64, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ q_off, uint16_t* __restrict__ out, int q_len, int Hq, int Hkv, int max_blocks,
    int num_blocks, float scale_log2,
    int seg_tokens, int nseg_max, AttnWs ws, const int32_t* __restrict__ items, int blk_pos, int n_rb, int parts,
    int head_fastest, int subs_per_chunk) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing * kSlot];
  // grid: (segment part, KV head, row block); (KV head, segment part, row
  // block) when head_fastest (no work list); or with a work list (parts
  // == 1) a 1-D grid of (list entry, KV head), KV head fastest; an entry is
  // v * nseg_max + seg.  Row block v = r * n_rb + b holds query positions
  // b*blk_pos .. +blk_pos-1 of request r (one block, v = r, whenever
  // q_len * G <= 32).  A segment is taken by `parts` waves, each over
  // seg_tokens / parts consecutive tokens: the first folds its chunks into
  // the segment's partial (the segment result when it is the only part
  // with keys); each later one writes its chunks' partials, which the
  // second kernel folds on in the same ascending order -- the same fold, so
  // the same bits, for any number of parts.
  int seg, kvh, v, part = 0;
  if (items != nullptr) {
    kvh = (int)(blockIdx.x % (unsigned)Hkv);
    const int e = items[blockIdx.x / (unsigned)Hkv];
    if (e < 0) return;
    v = e / nseg_max;
    seg = e - v * nseg_max;
  } else {
    const unsigned sx = head_fastest ? blockIdx.y : blockIdx.x;  // the segment (and part)
    if constexpr (kParts) {
      seg = (int)(sx / (unsigned)parts);
      part = (int)sx - seg * parts;
    } else {
      seg = (int)sx;
    }
    kvh = head_fastest ? blockIdx.x : blockIdx.y;
    v = blockIdx.z;
  }
  const int part_tok = kParts ? seg_tokens / parts : seg_tokens;
  const int tok_begin = seg * seg_tokens + part * part_tok;  // a multiple of kChunk
  const int r = v / n_rb, j0 = (v - r * n_rb) * blk_pos;  // request, first query position of the block
  const int lane = threadIdx.x, g = lane >> 5, li = lane & 31;
  const ReqRows rr = req_rows(q_off, r, q_len);
  const int G = Hq / Hkv, jn = min(blk_pos, rr.n - j0), nrows = jn * G;
  if (jn <= 0) return;  // a row block past the request's rows
  const int32_t* bt = block_table + (int64_t)r * max_blocks;
  const int page0 = tok_begin >> 4;  // first page of the part

  // The context length, the part's first page windows and the queries are
  // loaded together: none depends on another, and the copies of the first
  // sub-tiles can only start once all three have landed.
  const int L = ctx[r];
  int bt_w[kPreWin];  // the part's first kPreWin 64-page windows
#pragma unroll
  for (int w = 0; w < kPreWin; ++w) {
    const int lp = page0 + kPagesPerWin * w + lane;
    bt_w[w] = (part_tok > kPagesPerWin * 16 * w && lp < max_blocks) ? bt[lp] : -1;
  }
  // this lane's query row (MFMA column li)
  const bool row_ok = li < nrows;
  const int jq = j0 + (row_ok ? li / G : 0);
  const int hq = kvh * G + (row_ok ? li % G : 0);
  const int64_t qtok = rr.first + jq;
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

  const int n_tok = min(L + j0 + jn, max_blocks * 16);  // keys of the block's last row
  const int nseg = (n_tok + seg_tokens - 1) / seg_tokens;
  if (seg >= nseg) return;
  const int seg_end = min((seg + 1) * seg_tokens, n_tok);  // keys of this segment end here
  if (tok_begin >= seg_end) return;                        // a part with no keys
  const int tok_end = min(tok_begin + part_tok, seg_end);
  const bool split = kParts && seg_end - seg * seg_tokens > part_tok;  // the segment spans several parts
  const bool first_part = !kParts || part == 0;
  const int nsub = (tok_end - tok_begin + kSub - 1) / kSub;
  const int total = 2 * nsub;  // loads: K(s) = 2s, V(s) = 2s + 1
  const int n_pages = (n_tok + 15) >> 4;
  const int last_key = row_ok ? L + jq : -1;  // this row's last visible key

  // page ids of a 64-page window of the segment (-1: missing or out of range)
  auto window_ids = [&](int w, int raw) {
    const int lp = page0 + kPagesPerWin * w + lane;
    return (lp < n_pages && raw >= 0 && raw < num_blocks) ? raw : -1;
  };
  auto load_window = [&](int w) {
    const int lp = page0 + kPagesPerWin * w + lane;
    return window_ids(w, lp < n_pages ? bt[lp] : -1);
  };
  // windows 0 .. kPreWin-1 are loaded at the start; a later window (parts
  // longer than 4096 tokens) is loaded when the copies enter it
  const int pw0 = window_ids(0, bt_w[0]), pw1 = window_ids(1, bt_w[1]);
  const int pw2 = window_ids(2, bt_w[2]), pw3 = window_ids(3, bt_w[3]);
  int pwx = -1, winx = kPreWin - 1;
  uint32_t valid_q = 0;  // bits 2(s%16), 2(s%16)+1: pages of sub-tile s present

  // Direct-to-LDS copy of one sub-tile (32 keys) of K or V: 8 copies of
  // 4 keys (1 KiB) each; lane i writes LDS bytes 16i..16i+15 of its copy's
  // window, i.e. row 4c + i/16, position i%16, so it fetches piece
  // (i%16) ^ kv_swz(row) of that key.  kv_swz(4c + i/16) = 4(i/16) + c%4.
  const unsigned voff0 = 256u * (lane >> 4) + 16u * ((lane & 15) ^ (4 * (lane >> 4)));
  // copy c of a page (keys 4c .. 4c+3) reads piece (i%16) ^ kv_swz(4c + i/16):
  // the lane offset voff0 ^ 16c, and 1024c bytes into the page (the
  // instruction's offset field)
  const unsigned voff1 = voff0 ^ 16u, voff2 = voff0 ^ 32u, voff3 = voff0 ^ 48u;
  // LDS byte address of the ring (wave-uniform), once
  const unsigned ring_lds =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring);
  const uint64_t page_bytes = (uint64_t)Hkv * 16 * kHD * 2, head_bytes = (uint64_t)kvh * 16 * kHD * 2;
  // the window holding load j's pages (its register is passed by value to
  // the copy: selecting between captured variables inside the lambda would
  // force them into private memory)
  auto window_for = [&](int j) {
    const int w = (j >> 1) >> 5;
    if (!(j & 1) && w > winx) {  // K of the first sub-tile of window w >= kPreWin
      winx = w;
      pwx = load_window(w);
    }
    return w;
  };
  auto issue = [&](int j, int slot, int pv) {
    const int s = j >> 1;
    const int p0 = __builtin_amdgcn_readlane(pv, (2 * s) & 63);
    const int p1 = __builtin_amdgcn_readlane(pv, (2 * s + 1) & 63);
    if (!(j & 1)) {
      const int sh = 2 * (s & 15);
      valid_q = (valid_q & ~(3u << sh)) | ((uint32_t)(p0 >= 0) << sh) | ((uint32_t)(p1 >= 0) << (sh + 1));
    }
    const uint64_t cache = reinterpret_cast<uint64_t>((j & 1) ? v_cache : k_cache) + head_bytes;
    const uint64_t b0 = cache + (uint64_t)(p0 >= 0 ? p0 : 0) * page_bytes;  // keys 0..15 of the sub-tile
    const uint64_t b1 = cache + (uint64_t)(p1 >= 0 ? p1 : 0) * page_bytes;  // keys 16..31
    const unsigned dst = ring_lds + (unsigned)(slot * kSlot);
    lds_copy_slot(b0, b1, dst, dst + 4096, voff0, voff1, voff2, voff3);  // pages to the slot's two halves
  };

  // K read of step t: piece 2t + g of key li at position (2t + g) ^ kv_swz(li)
  const int k_off = li * 256 + 16 * (g ^ kv_swz(li));  // XOR 32t selects step t
  // V transpose reads.  In each group of 16 lanes, source lane s points at
  // dims base + 4(s%4) .. +3 of key kb + s/4; the read hands lane i the
  // 4 keys kb .. kb+3 of dim base + i.  Group 2g + half covers dims
  // 32d + 16 half .. +15 and keys kb = 16h + 8u + 4g (u: first or second
  // four of the lane's eight), matching the key order of the P operand.
  int v_off[4][2];
  {
    const int sl = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kk = 8 * u + 4 * g + (sl >> 2);  // + 16h (an immediate)
        const int c = 4 * d + 2 * half + ((sl & 3) >> 1);
        v_off[d][u] = kk * 256 + 16 * (c ^ kv_swz(kk)) + 8 * (sl & 1);
      }
  }

  // Q and the page ids have landed.  Issued as the builtin, which the
  // compiler's own wait tracking sees: it then knows no load of its own is
  // pending in the loop below and inserts no wait there that would also
  // drain the ring of copies.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // prologue: the first kRing loads
  const int n_pro = min(kRing, total);
  for (int j = 0; j < n_pro; ++j) {
    const int w = window_for(j);
    issue(j, j, pick_window(w, pw0, pw1, pw2, pw3, pwx));
  }

  float Ms = -INFINITY, Ls = 0.0f, Os[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) Os[k] = 0.0f;
  float mc = -INFINITY, lc = 0.0f;
  f32x16 oc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oc[d][v] = 0.0f;

  int sk = 0, sv = 1;  // slots of K(s) and V(s)
  for (int s = 0; s < nsub; ++s) {
    const int sub_base = tok_begin + s * kSub;
    const uint32_t vb = valid_q >> (2 * (s & 15));
    const bool ok0 = vb & 1u, ok1 = vb & 2u;
    // ---- S^T = K Q^T
    wait_ring(total - 1 - 2 * s);
    const unsigned char* Ks = ring + sk * kSlot;
    f32x16 sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (k_off ^ (32 * t)));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[t], sacc, 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // K slot read: refill it
    if (2 * s + kRing < total) {
      const int w = window_for(2 * s + kRing);
      issue(2 * s + kRing, sk, pick_window(w, pw0, pw1, pw2, pw3, pwx));
    }
    // ---- softmax statistics of the sub-tile (log2 domain)
    // score v of the lane is key kk = 8(v/4) + 4g + v%4 of the sub-tile; it
    // is visible when kk <= last_key - sub_base and its page is present
    float x[16];
    if (ok0 && ok1 && sub_base + kSub - 1 <= L) {  // wave-uniform: every row sees every key
#pragma unroll
      for (int v = 0; v < 16; ++v) x[v] = __fmul_rn(sacc[v], scale_log2);
    } else {
      const int lim = last_key - sub_base - 4 * g;  // compare 8(v/4) + v%4 against it
      const int lim_lo = ok0 ? lim : -1, lim_hi = ok1 ? lim : -1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = 8 * (v >> 2) + (v & 3) <= (v < 8 ? lim_lo : lim_hi);
        x[v] = ok ? __fmul_rn(sacc[v], scale_log2) : -INFINITY;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, x[v]);
    tmax = max_with_other_half(tmax);
    // The row's reference max moves only when a score exceeds it by more
    // than kLazy (log2 units), so p <= 2^kLazy and the accumulators are
    // rescaled rarely; the result is the same softmax, and the decision
    // depends on the row's own scores alone.
    const float mn = (mc == -INFINITY || tmax > mc + kLazy) ? tmax : mc;
    float alpha = 1.0f, lsum = 0.0f;
    bf16x8 pb[2];
    if (mn == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)0.0f;
        pb[1][e] = (__bf16)0.0f;
      }
    } else {
      alpha = mc == -INFINITY ? 0.0f : exp2_raw(mc - mn);  // exactly 1 when mn == mc
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2_raw(x[v] - mn);  // masked: exp2(-inf) = 0
        lsum = __fadd_rn(lsum, p);
        pb[v >> 3][v & 7] = (__bf16)p;
      }
    }
    lsum = sum_with_other_half(lsum);
    lc = __fadd_rn(__fmul_rn(lc, alpha), lsum);
    mc = mn;
    // ---- O^T += V^T P^T
    wait_ring(total - 2 - 2 * s);
    unsigned char* Vs = ring + sv * kSlot;
    if (!(ok0 && ok1 && sub_base + kSub <= n_tok)) {  // wave-uniform: zero V rows of masked keys
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = 4 * i + (lane >> 4);
        const bool ok = (i < 4 ? ok0 : ok1) && sub_base + key < n_tok;
        if (!ok) *reinterpret_cast<u32x4*>(Vs + 1024 * i + 16 * lane) = zero;  // row of key 4i + lane/16
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // wave-uniform; rows that keep their max multiply by exactly 1, and a
    // chunk's first visible sub-tile finds its accumulators still zero
    const bool rescale = __any(alpha != 1.0f && alpha != 0.0f);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (rescale) {
#pragma unroll
        for (int v = 0; v < 16; ++v) oc[d][v] = __fmul_rn(oc[d][v], alpha);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(Vs + v_off[d][0] + 4096 * h));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(Vs + v_off[d][1] + 4096 * h));
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[h], oc[d], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // V slot read: refill it
    if (2 * s + 1 + kRing < total) {
      const int w = window_for(2 * s + 1 + kRing);
      issue(2 * s + 1 + kRing, sv, pick_window(w, pw0, pw1, pw2, pw3, pwx));
    }
    sk = sk + 2 >= kRing ? sk + 2 - kRing : sk + 2;
    sv = sv + 2 >= kRing ? sv + 2 - kRing : sv + 2;
    // ---- end of a chunk: fold its partial into the segment result
    // (ascending), or, in a later part of a split segment, write it out
    if ((s + 1) % subs_per_chunk == 0 || s + 1 == nsub) {
      float o[64];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[16 * d + v] = oc[d][v];
      if constexpr (kParts) {
        if (first_part) {
          fold_into<64>(Ms, Ls, Os, mc, lc, o);
        } else {
          const int64_t chunk = ((int64_t)v * Hkv + kvh) * nseg_max * (seg_tokens / kChunk) + sub_base / kChunk;
          store_partial<false>(ws.chunk_o, ws.chunk_ml, chunk, lane, row_ok, mc, lc, o);
        }
      } else {
        fold_into<64>(Ms, Ls, Os, mc, lc, o);
      }
      mc = -INFINITY;
      lc = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) oc[d][v] = 0.0f;
    }
  }

  if (!first_part) return;  // its chunk partials are out
  // value k = 16d + v of lane (li, g): dim 32d + 8(v/4) + 4g + v%4 of row li
  if (nseg == 1 && !split) {
    if (!row_ok) return;
    const float inv = Ls > 0.0f ? __fdiv_rn(1.0f, Ls) : 0.0f;
    uint16_t* orow = out + (qtok * Hq + hq) * kHD;
#pragma unroll
    for (int k4 = 0; k4 < 16; ++k4) {
      const int d = k4 >> 2, v0 = 4 * (k4 & 3);
      uint32_t w0 = (uint32_t)f2bf(__fmul_rn(Os[16 * d + v0 + 0], inv)) |
                    ((uint32_t)f2bf(__fmul_rn(Os[16 * d + v0 + 1], inv)) << 16);
      uint32_t w1 = (uint32_t)f2bf(__fmul_rn(Os[16 * d + v0 + 2], inv)) |
                    ((uint32_t)f2bf(__fmul_rn(Os[16 * d + v0 + 3], inv)) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * d + 8 * (k4 & 3) + 4 * g) = make_uint2(w0, w1);
    }
    return;
  }
  // the segment result (or, for a split segment, the fold of its first
  // part's chunks) -> workspace; attn_combine_kernel folds on from there.
  // Grids of about one round of waves store it through the caches, where
  // the fold that follows finds it (the 8B-shaped pass's attention 2.8%
  // faster); grids long enough for a work list stream it past them (2.5%
  // faster at 64 requests of U[512, 32768], whose partials are many).
  const int64_t pslot = ((int64_t)v * Hkv + kvh) * nseg_max + seg;
  if (items)
    store_partial<true>(ws.part_o, ws.part_ml, pslot, lane, row_ok, Ms, Ls, Os);
  else
    store_partial<false>(ws.part_o, ws.part_ml, pslot, lane, row_ok, Ms, Ls, Os);
}

// Work list for large grids: every full segment first, then the partial last
// segments, longest first, so that the dispatcher's list scheduling leaves
// the short items for the end of the grid (LPT order).  Only the order of
// the work changes: each item's arithmetic and its workspace slot are fixed
// by (request, segment), so the results are the same bits.  One workgroup;
// partial lengths are bucketed in 128 classes.
__global__ __launch_bounds__(1024) void attn_plan_kernel(const int32_t* __restrict__ ctx,
                                                        const int32_t* __restrict__ q_off, int Rv, int q_len,
                                                        int max_blocks, int seg_tokens, int nseg_max, int blk_pos,
                                                        int n_rb, int32_t* __restrict__ items) {
  constexpr int NB = 128;
  __shared__ int n_full, full_cur, bucket_cnt[NB], bucket_start[NB], bucket_cur[NB];
  const int tid = threadIdx.x;
  if (tid == 0) {
    n_full = 0;
    full_cur = 0;
  }
  if (tid < NB) {
    bucket_cnt[tid] = 0;
    bucket_cur[tid] = 0;
  }
  __syncthreads();
  const int cap = max_blocks * 16;
  const int bw = (seg_tokens + NB - 1) / NB;
  // keys of row block v: up to the block's last query position (none for a
  // block past its request's rows)
  auto block_tokens = [&](int v) {
    const int r = v / n_rb, j0 = (v - r * n_rb) * blk_pos;
    const int jn = min(blk_pos, req_rows(q_off, r, q_len).n - j0);
    return jn <= 0 ? 0 : min(ctx[r] + j0 + jn, cap);
  };
  for (int v = tid; v < Rv; v += 1024) {
    const int nt = block_tokens(v);
    const int full = nt / seg_tokens, part = nt - full * seg_tokens;
    atomicAdd(&n_full, full);
    if (part > 0) atomicAdd(&bucket_cnt[(part - 1) / bw], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = n_full;
    for (int b = NB - 1; b >= 0; --b) {
      bucket_start[b] = acc;
      acc += bucket_cnt[b];
    }
  }
  __syncthreads();
  for (int v = tid; v < Rv; v += 1024) {
    const int nt = block_tokens(v);
    const int full = nt / seg_tokens, part = nt - full * seg_tokens;
    const int base = atomicAdd(&full_cur, full);
    for (int k = 0; k < full; ++k) items[base + k] = v * nseg_max + k;
    if (part > 0) {
      const int b = (part - 1) / bw;
      items[bucket_start[b] + atomicAdd(&bucket_cur[b], 1)] = v * nseg_max + full;
    }
  }
  const int n_items = bucket_start[0] + bucket_cnt[0];
  for (int i = n_items + tid; i < Rv * nseg_max; i += 1024) items[i] = -1;
}

// Parts per segment: halve the parts' length while the grid of segments
// holds fewer than kSplitBelow potential waves (one round of resident waves
// on a 256-CU device: a CU streams fastest with all four of its wave slots
// busy), down to one chunk per part.  From the call's shape alone.
constexpr int64_t kSplitBelow = 1024;
static int attn_parts(int64_t Rv, int Hkv, int64_t nseg_max, int seg_tokens) {
  const int cps = seg_tokens / kChunk;
  const int64_t potential = Rv * Hkv * nseg_max;
  int w = 1;
  while (cps % (2 * w) == 0 && potential * w < kSplitBelow) w *= 2;
  return w;
}

// Workspace: segment partials [Rv * Hkv * nseg_max] (4096 values + 128 for
// (m, l) each), the work list (Rv * nseg_max entries, padded to 4), then,
// when segments are split, the chunk partials [Rv * Hkv * nseg_max * chunks
// per segment] in the same format.
static size_t attn_ws_floats(int64_t Rv, int Hkv, int64_t nseg_max, int seg_tokens, int parts) {
  const int64_t slots = Rv * Hkv * nseg_max;
  const int64_t items = (Rv * nseg_max + 3) / 4 * 4;
  const int64_t cslots = parts > 1 ? slots * (seg_tokens / kChunk) : 0;
  return (size_t)(slots * (4096 + 128) + items + cslots * (4096 + 128));
}
static int32_t* attn_ws_items(void* workspace, int64_t Rv, int Hkv, int64_t nseg_max) {
  return reinterpret_cast<int32_t*>(static_cast<float*>(workspace) + Rv * Hkv * nseg_max * (4096 + 128));
}
static AttnWs attn_ws_layout(void* workspace, int64_t Rv, int Hkv, int64_t nseg_max, int seg_tokens, int parts) {
  const int64_t slots = Rv * Hkv * nseg_max;
  AttnWs ws;
  ws.part_o = static_cast<float*>(workspace);
  ws.part_ml = ws.part_o + slots * 4096;
  ws.chunk_o = ws.part_ml + slots * 128 + (Rv * nseg_max + 3) / 4 * 4;
  ws.chunk_ml = ws.chunk_o + (parts > 1 ? slots * (seg_tokens / kChunk) * 4096 : 0);
  return ws;
}

// Waves of the segment kernel resident at once on the current device (four
// per CU: its LDS ring takes a quarter of a CU's 160 KiB).
static int resident_attn_waves() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = 4 * cus;
  }
  return cached[dev];
}

// Second pass for requests with more than one segment or a split segment:
// per segment, in ascending order, its result -- from the first pass, or,
// for a split segment, as attn_chunk_fold_kernel completed it (the first
// part's fold with the later chunks folded on in ascending order) -- and
// the segment results left-folded in ascending order from the first one
// (the fold above, element by element), and the output written.  Four
// workgroups of 256 threads per (KV head, row block) (measured: 1-7% faster
// than one of 1024, same bits); thread t of workgroup z takes lane t % 64 of
// the first pass and its values 4q .. 4q+3, q = 4z + t / 64 (dims
// 32(q/4) + 8(q%4) + 4g .. +3 of row (t%64) % 32).  Up to kCombBatch segment
// partials are loaded at once.
//
// Split segments are completed before this pass, all segments of a request
// in parallel (a chain of chunk folds inside this pass was what bounded it
// at small batch).
constexpr int kCombZ = 4;  // workgroups per (KV head, row block)
constexpr int kCombThreads = 1024 / kCombZ, kCombBatch = 8, kChunkFoldBatch = 8;

// A split segment's partial: the fold of its first part's chunks from the
// first pass, then its later chunks folded on in ascending order; written to
// the segment's first chunk slot, which the first pass leaves unused (the
// first part folds its chunks in registers).  Grid (segment x KV head, row
// block, kCombZ); threads as in the second pass.
__global__ __launch_bounds__(kCombThreads) void attn_chunk_fold_kernel(const int32_t* __restrict__ ctx,
                                                                       const int32_t* __restrict__ q_off, int q_len,
                                                                       int Hq, int Hkv, int max_blocks, int seg_tokens,
                                                                       int nseg_max, AttnWs ws, int blk_pos, int n_rb,
                                                                       int parts) {
  const int sg = (int)(blockIdx.x / (unsigned)Hkv), kvh = (int)blockIdx.x - sg * Hkv, v = blockIdx.y;
  const int r = v / n_rb, j0 = (v - r * n_rb) * blk_pos;
  const int tid = threadIdx.x, q = blockIdx.z * (kCombThreads / 64) + (tid >> 6), lane = tid & 63,
            li = lane & 31;
  const ReqRows rr = req_rows(q_off, r, q_len);
  const int G = Hq / Hkv, jn = min(blk_pos, rr.n - j0), nrows = jn * G;
  if (jn <= 0 || li >= nrows) return;
  const int n_tok = min(ctx[r] + j0 + jn, max_blocks * 16);
  const int nseg = (n_tok + seg_tokens - 1) / seg_tokens;
  if (sg >= nseg) return;
  const int part_tok = seg_tokens / parts, cps = seg_tokens / kChunk, cpp = part_tok / kChunk;
  const int keys = min((sg + 1) * seg_tokens, n_tok) - sg * seg_tokens;
  if (keys <= part_tok) return;  // not split: its partial is complete
  const int nch = (keys + kChunk - 1) / kChunk;
  const int64_t slot = ((int64_t)v * Hkv + kvh) * nseg_max + sg;
  float o[4], m, l;
  {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ws.part_o + slot * 4096) + q * 64 + lane);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = w[c];
    m = ws.part_ml[slot * 128 + lane * 2 + 0];
    l = ws.part_ml[slot * 128 + lane * 2 + 1];
  }
  for (int c0 = cpp; c0 < nch; c0 += kChunkFoldBatch) {
    float co[kChunkFoldBatch][4], cm[kChunkFoldBatch], cl[kChunkFoldBatch];
#pragma unroll
    for (int e = 0; e < kChunkFoldBatch; ++e) {
      if (c0 + e < nch) {
        const int64_t cs = slot * cps + c0 + e;
        const f32x4 w = *(reinterpret_cast<const f32x4*>(ws.chunk_o + cs * 4096) + q * 64 + lane);
#pragma unroll
        for (int c = 0; c < 4; ++c) co[e][c] = w[c];
        cm[e] = ws.chunk_ml[cs * 128 + lane * 2 + 0];
        cl[e] = ws.chunk_ml[cs * 128 + lane * 2 + 1];
      }
    }
#pragma unroll
    for (int e = 0; e < kChunkFoldBatch; ++e)
      if (c0 + e < nch) fold_into<4>(m, l, o, cm[e], cl[e], co[e]);
  }
  const int64_t cs0 = slot * cps;  // chunk 0 of the segment: never written by the first pass
  *(reinterpret_cast<f32x4*>(ws.chunk_o + cs0 * 4096) + q * 64 + lane) = f32x4{o[0], o[1], o[2], o[3]};
  if (q == 0) {  // (m, l) of a row are the same in every thread of its lane
    ws.chunk_ml[cs0 * 128 + lane * 2 + 0] = m;
    ws.chunk_ml[cs0 * 128 + lane * 2 + 1] = l;
  }
}

__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(const int32_t* __restrict__ ctx,
                                                                    const int32_t* __restrict__ q_off,
                                                                    uint16_t* __restrict__ out, int q_len, int Hq,
                                                                    int Hkv, int max_blocks, int seg_tokens,
                                                                    int nseg_max, AttnWs ws, int blk_pos, int n_rb,
                                                                    int parts) {
  const int kvh = blockIdx.x, v = blockIdx.y;  // v: row block, as in the first pass
  const int r = v / n_rb, j0 = (v - r * n_rb) * blk_pos;
  const int tid = threadIdx.x, q = blockIdx.z * (kCombThreads / 64) + (tid >> 6), lane = tid & 63, g = lane >> 5,
            li = lane & 31;
  const ReqRows rr = req_rows(q_off, r, q_len);
  const int G = Hq / Hkv, jn = min(blk_pos, rr.n - j0), nrows = jn * G;
  if (jn <= 0) return;
  const int n_tok = min(ctx[r] + j0 + jn, max_blocks * 16);
  const int nseg = (n_tok + seg_tokens - 1) / seg_tokens;
  const int part_tok = seg_tokens / parts, cps = seg_tokens / kChunk;
  // keys of segment s; it was split when they exceed one part
  auto seg_keys = [&](int sg) { return min((sg + 1) * seg_tokens, n_tok) - sg * seg_tokens; };
  if ((nseg <= 1 && seg_keys(0) <= part_tok) || li >= nrows) return;  // written by the first pass
  const int jq = j0 + li / G, hq = kvh * G + li % G;
  const int64_t slot0 = ((int64_t)v * Hkv + kvh) * nseg_max;
  float M = -INFINITY, Lt = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < nseg; s0 += kCombBatch) {
    float o[kCombBatch][4], m[kCombBatch], l[kCombBatch];
#pragma unroll
    for (int b = 0; b < kCombBatch; ++b) {
      if (s0 + b < nseg) {
        // a split segment, completed by attn_chunk_fold_kernel, sits in its first chunk slot
        const bool done = seg_keys(s0 + b) > part_tok;
        const int64_t sl = done ? (slot0 + s0 + b) * cps : slot0 + s0 + b;
        const float* po = done ? ws.chunk_o : ws.part_o;
        const float* pml = done ? ws.chunk_ml : ws.part_ml;
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(po + sl * 4096) + q * 64 + lane);
#pragma unroll
        for (int c = 0; c < 4; ++c) o[b][c] = w[c];
        m[b] = pml[sl * 128 + lane * 2 + 0];
        l[b] = pml[sl * 128 + lane * 2 + 1];
      }
    }
#pragma unroll
    for (int b = 0; b < kCombBatch; ++b) {
      const int sg = s0 + b;
      if (sg >= nseg) continue;
      if (sg == 0) {
        M = m[b];
        Lt = l[b];
#pragma unroll
        for (int c = 0; c < 4; ++c) O[c] = o[b][c];
      } else {
        fold_into<4>(M, Lt, O, m[b], l[b], o[b]);
      }
    }
  }
  const float inv = Lt > 0.0f ? __fdiv_rn(1.0f, Lt) : 0.0f;
  uint16_t* orow = out + ((rr.first + jq) * Hq + hq) * kHD + 32 * (q >> 2) + 8 * (q & 3) + 4 * g;
  const uint32_t w0 = (uint32_t)f2bf(__fmul_rn(O[0], inv)) | ((uint32_t)f2bf(__fmul_rn(O[1], inv)) << 16);
  const uint32_t w1 = (uint32_t)f2bf(__fmul_rn(O[2], inv)) | ((uint32_t)f2bf(__fmul_rn(O[3], inv)) << 16);
  *reinterpret_cast<uint2*>(orow) = make_uint2(w0, w1);
}

// fp32 path: one wave per (query row, query head, request).  Same chunking:
// 256-key chunks at absolute positions, chunk partials (natural-exp domain)
// left-folded in ascending order.  Lanes own keys for the scores and
// dimensions for the weighted sum; every sum runs in a fixed order.
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, int64_t q_stride,
                                                      const float* __restrict__ k_cache,
                                                      const float* __restrict__ v_cache,
                                                      const int32_t* __restrict__ block_table,
                                                      const int32_t* __restrict__ ctx,
                                                      const int32_t* __restrict__ q_off, float* __restrict__ out,
                                                      int q_len, int Hq, int Hkv, int D, int max_blocks,
                                                      int num_blocks, float scale) {
  __shared__ float qs[128];
  __shared__ float ps[kF32Chunk];
  const int j = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x;
  const ReqRows rr = req_rows(q_off, r, q_len);
  if (j >= rr.n) return;
  const int G = Hq / Hkv, kvh = h / G;
  const int L = ctx[r];
  const int n_keys = min(L + j + 1, max_blocks * 16);
  const int32_t* bt = block_table + (int64_t)r * max_blocks;
  const int64_t qtok = rr.first + j;
  const int64_t qrow = qtok * Hq + h;
  for (int d = lane; d < D; d += 64) qs[d] = q[qtok * q_stride + (int64_t)h * D + d];
  __syncthreads();
  float M = -INFINITY, Ls = 0.0f, O0 = 0.0f, O1 = 0.0f;
  for (int cb = 0; cb < n_keys; cb += kF32Chunk) {
    const int ce = min(cb + kF32Chunk, n_keys);
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

// Query positions per 32-row block (G query heads per KV head share a block)
// and the number of blocks a request's q_len rows take.
static inline int attn_blk_pos(int Hq, int Hkv) { return 32 / (Hq / Hkv); }
static inline int attn_row_blocks(int q_len, int Hq, int Hkv) { return (int)cdiv(q_len, attn_blk_pos(Hq, Hkv)); }

// invariant: the batch-invariant call (kChunk-key chunks; small batches'
// segments split over waves, same bits); otherwise the comparison path
// (kAdaptiveChunk-key chunks, one wave per segment).
static biv_status launch_attn_bf16(const char* who, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* ctx, const int32_t* q_off, void* out,
                                   int R, int q_len,
                                   int Hq, int Hkv, int max_blocks, int num_blocks, float scale, int seg_tokens,
                                   bool invariant, void* workspace, size_t workspace_bytes, hipStream_t s) {
  const int G = Hq / Hkv;
  BIV_REQUIRE(G >= 1 && 32 % G == 0, "%s: bf16 path needs Hq/Hkv dividing 32 (got %d)", who, G);
  const int blk_pos = attn_blk_pos(Hq, Hkv), n_rb = attn_row_blocks(q_len, Hq, Hkv);
  BIV_REQUIRE((int64_t)R * n_rb <= 65535, "%s: %d requests x %d row blocks exceed the grid", who, R, n_rb);
  const int Rv = R * n_rb;  // row blocks
  BIV_REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && q_stride % 8 == 0,
              "%s: q (and its row stride) and the caches must be 16-byte aligned", who);
  // the invariant call's chunks, or the comparison path's
  const int chunk = invariant ? kChunk : kAdaptiveChunk;
  BIV_REQUIRE(seg_tokens > 0 && seg_tokens % chunk == 0, "%s: segment size %d is not a multiple of %d", who,
              seg_tokens, chunk);
  const int64_t nseg_max64 = cdiv((int64_t)max_blocks * 16, seg_tokens);
  BIV_REQUIRE(nseg_max64 <= 0x7fffffff, "%s: too many segments", who);
  const int nseg_max = (int)nseg_max64;
  // Segments split over several waves where the grid would otherwise hold
  // few waves (decided by the call's shape alone; no bits change).
  const int parts = invariant ? attn_parts(Rv, Hkv, nseg_max, seg_tokens) : 1;
  // the layout this launch uses (biv_attn_workspace_bytes, which allows for
  // splits, is never smaller)
  const size_t need = attn_ws_floats(Rv, Hkv, nseg_max, seg_tokens, parts) * sizeof(float);
  BIV_REQUIRE(workspace != nullptr && workspace_bytes >= need, "%s: workspace needs %zu bytes (got %zu)", who, need,
              workspace_bytes);
  BIV_REQUIRE(aligned16(workspace), "%s: workspace must be 16-byte aligned", who);
  const AttnWs ws = attn_ws_layout(workspace, Rv, Hkv, nseg_max, seg_tokens, parts);
  // A grid of at least four rounds of resident waves is launched in LPT
  // order from a work list (decided by the call's shape alone).
  const int64_t waves = (int64_t)Rv * nseg_max * Hkv * parts;
  int32_t* items = nullptr;
  dim3 grid((unsigned)(nseg_max * parts), Hkv, Rv);
  if (parts == 1 && waves >= 4 * (int64_t)resident_attn_waves() && waves <= 0x7fffffff) {
    items = attn_ws_items(workspace, Rv, Hkv, nseg_max);
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, s, ctx, q_off, Rv, q_len, max_blocks, seg_tokens, nseg_max,
                       blk_pos, n_rb, items);
    biv_status st = launched(who);
    if (st != BIV_OK) return st;
    grid = dim3((unsigned)waves);
  }
  // Without a list, calls whose requests may span four or more segments
  // launch the KV heads of a segment (part) together, so the eight waves
  // reading adjacent pieces of the same pages run at once (decided by the
  // call's shape alone): 5-7% faster for 16 and 32 requests of
  // U[512, 32768], while the 8B pass's contexts (at most three segments)
  // run 0.8% faster segment first.
  const bool head_fastest = items == nullptr && nseg_max >= 4 && nseg_max * parts <= 65535;
  if (head_fastest) grid = dim3((unsigned)Hkv, (unsigned)(nseg_max * parts), (unsigned)Rv);
  // segments split over waves take the kernel with the chunk-partial path;
  // the others a kernel without it (same arithmetic, leaner code)
  if (parts > 1)
    hipLaunchKernelGGL(attn_bf16_kernel<true>, grid, dim3(64), 0, s, static_cast<const uint16_t*>(q), q_stride,
                       static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table, ctx,
                       q_off, static_cast<uint16_t*>(out), q_len, Hq, Hkv, max_blocks, num_blocks, scale * kLog2e,
                       seg_tokens, nseg_max, ws, items, blk_pos, n_rb, parts, head_fastest ? 1 : 0, chunk / kSub);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<false>, grid, dim3(64), 0, s, static_cast<const uint16_t*>(q), q_stride,
                       static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table, ctx,
                       q_off, static_cast<uint16_t*>(out), q_len, Hq, Hkv, max_blocks, num_blocks, scale * kLog2e,
                       seg_tokens, nseg_max, ws, items, blk_pos, n_rb, 1, head_fastest ? 1 : 0, chunk / kSub);
  biv_status st = launched(who);
  if (st != BIV_OK || (nseg_max <= 1 && parts == 1)) return st;
  if (parts > 1) {  // complete the split segments, every segment of a request at once
    BIV_REQUIRE((int64_t)Hkv * nseg_max <= 0x7fffffff, "%s: too many segments", who);
    hipLaunchKernelGGL(attn_chunk_fold_kernel, dim3((unsigned)(Hkv * nseg_max), Rv, kCombZ), dim3(kCombThreads), 0, s,
                       ctx, q_off, q_len, Hq, Hkv, max_blocks, seg_tokens, nseg_max, ws, blk_pos, n_rb, parts);
    st = launched(who);
    if (st != BIV_OK) return st;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hkv, Rv, kCombZ), dim3(kCombThreads), 0, s, ctx, q_off, static_cast<uint16_t*>(out),
                     q_len, Hq, Hkv, max_blocks, seg_tokens, nseg_max, ws, blk_pos, n_rb, parts);
  return launched(who);
}

}  // namespace biv

extern "C" size_t biv_attn_workspace_bytes(int R, int Hkv, int max_blocks, int seg_tokens) {
  using namespace biv;
  if (R <= 0 || Hkv <= 0 || max_blocks <= 0 || seg_tokens <= 0 || seg_tokens % kAdaptiveChunk != 0) return 0;
  const int64_t nseg = cdiv((int64_t)max_blocks * 16, seg_tokens);
  // room for the split layout wherever the invariant call could split (its
  // segments are whole chunks); the comparison path never splits
  const int parts = seg_tokens % kChunk == 0 ? attn_parts(R, Hkv, nseg, seg_tokens) : 1;
  return attn_ws_floats(R, Hkv, nseg, seg_tokens, parts) * sizeof(float);
}

extern "C" size_t biv_attn_workspace_bytes_q(int R, int q_len, int Hq, int Hkv, int max_blocks, int seg_tokens) {
  using namespace biv;
  if (R <= 0 || q_len <= 0 || Hkv <= 0 || Hq < Hkv || Hq % Hkv != 0 || 32 % (Hq / Hkv) != 0) return 0;
  const int64_t rv = (int64_t)R * attn_row_blocks(q_len, Hq, Hkv);
  if (rv > 0x7fffffff) return 0;
  return biv_attn_workspace_bytes((int)rv, Hkv, max_blocks, seg_tokens);
}

extern "C" biv_status attn_decode_bi(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* ctx, const int32_t* q_off, void* out,
                                     int R, int q_len,
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
    if (32 % (Hq / Hkv) != 0)
      return fail(BIV_EUNSUPPORTED, "attn_decode_bi: bf16 path needs Hq/Hkv dividing 32 (got %d)", Hq / Hkv);
    return launch_attn_bf16("attn_decode_bi", q, q_stride, k_cache, v_cache, block_table, ctx, q_off, out, R, q_len, Hq, Hkv,
                            max_blocks, num_blocks, scale, BIV_ATTN_SEG_TOKENS, true, workspace, workspace_bytes, s);
  }
  if (D != 64 && D != 128) return fail(BIV_EUNSUPPORTED, "attn_decode_bi: fp32 path supports D in {64,128} (D=%d)", D);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(q_len, Hq, R), dim3(64), 0, s, static_cast<const float*>(q), q_stride,
                     static_cast<const float*>(k_cache), static_cast<const float*>(v_cache), block_table, ctx, q_off,
                     static_cast<float*>(out), q_len, Hq, Hkv, D, max_blocks, num_blocks, scale);
  return launched("attn_decode_bi/f32");
}

extern "C" int biv_attn_adaptive_split(int R, int Hkv, int max_blocks) {
  using namespace biv;
  if (R <= 0 || Hkv <= 0 || max_blocks <= 0) return kAdaptiveChunk;
  const int64_t cap = (int64_t)max_blocks * 16;
  const int64_t want = cdiv(1024, (int64_t)R * Hkv);  // segments per (request, head): one wave per SIMD
  int64_t split = cdiv(cdiv(cap, want), kAdaptiveChunk) * kAdaptiveChunk;
  return (int)std::max<int64_t>(kAdaptiveChunk, split);
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
  if (32 % (Hq / Hkv) != 0) return fail(BIV_EUNSUPPORTED, "attn_decode_adaptive: needs Hq/Hkv dividing 32");
  BIV_REQUIRE(split_tokens >= 0 && split_tokens % kAdaptiveChunk == 0,
              "attn_decode_adaptive: split_tokens must be a multiple of %d", kAdaptiveChunk);
  const int split = split_tokens == 0 ? biv_attn_adaptive_split(R, Hkv, max_blocks) : split_tokens;
  return launch_attn_bf16("attn_decode_adaptive", q, q_stride, k_cache, v_cache, block_table, ctx, nullptr, out, R, q_len, Hq, Hkv,
                          max_blocks, num_blocks, scale, split, false, workspace, workspace_bytes,
                          static_cast<hipStream_t>(stream));
}

// ----------------------------------------------------------------------------
// attn_decode_bi_static: attn_decode_bi with its workspace in memory the
// library holds, for callers that cannot allocate.  `scratch` is a file-scope
// device array; in host code its name only stands in for the symbol, so its
// device address on each GPU is looked up once (hipGetSymbolAddress, with
// that GPU current, at the entry point's first call there) and only that
// address is ever handed to a kernel.
namespace biv {

static __device__ __align__(256) unsigned char scratch[BIV_ATTN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {nullptr};

static biv_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BIV_EHIP, "attn_decode_bi_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BIV_EUNSUPPORTED, "attn_decode_bi_static: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(BIV_EHIP, "attn_decode_bi_static: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BIV_OK;
}

}  // namespace biv

extern "C" biv_status attn_decode_bi_static(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                            const int32_t* block_table, const int32_t* ctx, const int32_t* q_off,
                                            void* out, int R, int q_len, int Hq, int Hkv, int D, int max_blocks,
                                            int num_blocks, float scale, biv_dtype dt, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(dt), "attn_decode_bi_static: bad dtype");
  biv_status st = check_attn("attn_decode_bi_static", q, q_stride, k_cache, v_cache, block_table, ctx, out, R, q_len,
                             Hq, Hkv, D, max_blocks, num_blocks);
  if (st != BIV_OK) return st;
  if (R == 0) return BIV_OK;
  if (dt != BIV_BF16)  // the fp32 path uses no workspace
    return attn_decode_bi(q, q_stride, k_cache, v_cache, block_table, ctx, q_off, out, R, q_len, Hq, Hkv, D,
                          max_blocks, num_blocks, scale, dt, nullptr, 0, stream);
  if (D != kHD) return fail(BIV_EUNSUPPORTED, "attn_decode_bi_static: bf16 path supports D == 128 only (D=%d)", D);
  if (32 % (Hq / Hkv) != 0)
    return fail(BIV_EUNSUPPORTED, "attn_decode_bi_static: bf16 path needs Hq/Hkv dividing 32 (got %d)", Hq / Hkv);
  const size_t need = biv_attn_workspace_bytes_q(R, q_len, Hq, Hkv, max_blocks, BIV_ATTN_SEG_TOKENS);
  BIV_REQUIRE(need > 0 && need <= (size_t)BIV_ATTN_STATIC_SCRATCH_BYTES,
              "attn_decode_bi_static: this call needs %zu bytes of workspace, more than the library's %zu-byte "
              "static scratch; use attn_decode_bi with a workspace", need, (size_t)BIV_ATTN_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != BIV_OK) return st;
  return launch_attn_bf16("attn_decode_bi_static", q, q_stride, k_cache, v_cache, block_table, ctx, q_off, out, R,
                          q_len, Hq, Hkv, max_blocks, num_blocks, scale, BIV_ATTN_SEG_TOKENS, true, ws,
                          (size_t)BIV_ATTN_STATIC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}
