// gemm_bi: batch-invariant matmul, and gemm_splitk, its non-invariant
// split-K counterpart.
//
// LLM-42 post, paragraph 1: at small batch a matmul normally splits the
// reduction dimension K into pieces computed in parallel and summed
// afterwards (split-K); the batch-invariant matmul drops split-K and always
// uses one and the same data-parallel tiling.
//
// bf16 path (gfx950 MFMA), two kernels with one per-element reduction:
// every output element is reduced by the 32x32x16 bf16 MFMA over
// k = 0, 16, 32, ... in ascending order with fp32 accumulators, so its bits
// depend only on its own row of A and column of B: not on M, not on the tile
// it lands in, not on the other rows.  This reduction is the same for every
// M; the column tiling depends on the weight shape alone, and only the rows
// per tile (32 or 64 at M <= 64, else the class's full height) follow M.
//  - gemm_dma_kernel (K a multiple of 64, the decoder's case): A and B tiles
//    copied HBM -> LDS by global_load_lds_dwordx4 into a ring of 64- or
//    128-wide k stages; tile shape and wave arrangement chosen per weight width (see
//    dma_tile_for); store, residual-accumulate and SwiGLU epilogues.
//  - gemm_bf16_kernel (any K % 8 == 0): 128 x 128 tiles, K staged 64 at a time
//    through registers into double-buffered, XOR-swizzled LDS; four waves of
//    64 x 64 outputs.
//
// Workgroup -> tile mapping is XCD aware: the dispatcher deals workgroups to
// the 8 XCDs round-robin, so workgroup b is remapped to give each XCD a
// contiguous run of tiles, M-fastest, and the M tiles that share a B tile
// meet in the same XCD's L2.
#include <algorithm>

#include "biv_internal.h"

namespace biv {

constexpr int kBM = 128, kBN = 128, kBK = 64;
// Internal epilogue of the staged kernel (not a gemm_bi epilogue): Gumbel-max
// of each row over each wave's columns, for lm_head_gumbel_verify.
constexpr int kEpiGumbel = 3;
constexpr int kGemmThreads = 256;
constexpr int kTileBytes = kBM * kBK * 2;  // 16 KiB per operand tile

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` in an LDS tile.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb >> 3;
  return (b < (per << 3)) ? (b & 7) * per + (b >> 3) : b;
}

// kSplit: write fp32 partial sums of the K range [k_begin, k_end) to `partial`
// ([split][M][N]) instead of running the epilogue.
template <int OUT_DT, int EPI, bool kSplit>
__global__ __launch_bounds__(kGemmThreads) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                                 const uint16_t* __restrict__ B, void* C,
                                                                 float* __restrict__ partial, int M, int N, int K,
                                                                 int tilesM, int tilesN, int k_per_split) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2][2][kTileBytes];  // [buf][A/B]
  const int tid = threadIdx.x;
  const int logical = xcd_remap(blockIdx.x, tilesM * tilesN);
  const int m0 = (logical % tilesM) * kBM;
  const int n0 = (logical / tilesM) * kBN;
  const int k_begin = kSplit ? blockIdx.y * k_per_split : 0;
  const int k_end = kSplit ? min(K, k_begin + k_per_split) : K;

  // global -> register staging: row = tid/8 + 32 i, chunk = tid % 8
  const int lrow = tid >> 3, lch = tid & 7;
  uint4 ra[4], rb[4];
  auto load_tiles = [&](int k0) {
    const int gk = k0 + lch * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      const int gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M && gk < k_end) ? *reinterpret_cast<const uint4*>(A + (int64_t)gm * K + gk) : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < N && gk < k_end) ? *reinterpret_cast<const uint4*>(B + (int64_t)gn * K + gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<uint4*>(&smem[buf][0][swz(row, lch)]) = ra[i];
      *reinterpret_cast<uint4*>(&smem[buf][1][swz(row, lch)]) = rb[i];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, li = lane & 31;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (int)cdiv(k_end - k_begin, kBK);
  load_tiles(k_begin);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(k_begin + (kt + 1) * kBK);
    const unsigned char* As = smem[cur][0];
    const unsigned char* Bs = smem[cur][1];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = 2 * ks + g;  // lanes 0-31 take k 0..7 of the step, lanes 32-63 k 8..15
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(As + swz(64 * wm + 32 * i + li, chunk));
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(64 * wn + 32 * j + li, chunk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column li; value v is row 8(v/4) + 4g + v%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wn + 32 * j + li;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= M) continue;
        const int64_t idx = (int64_t)m * N + n;
        const float x = acc[i][j][v];
        if (kSplit) {
          partial[(int64_t)blockIdx.y * M * N + idx] = x;
        } else if (EPI == BIV_EPI_ACCUM) {
          store_from_f32(C, idx, __fadd_rn(load_as_f32(C, idx, OUT_DT), x), OUT_DT);
        } else {
          store_from_f32(C, idx, x, OUT_DT);
        }
      }
    }
}

// ----------------------------------------------------------------------------
// bf16 path with K staged straight from HBM into a ring of LDS stages.
//
// The same per-element reduction as gemm_bf16_kernel -- one 32x32x16 MFMA
// shape, k ascending in steps of 16, lanes 0-31 holding k 0..7 and lanes 32-63
// k 8..15 of each step -- so the two kernels give identical bits, and a row's
// bits never depend on M or on the tile it lands in.  K advances KB (64 or
// 128) per stage; each stage's A (BM x KB) and B (BN x KB) tiles are copied
// HBM -> LDS by global_load_lds_dwordx4 in 1 KiB windows of 8 rows x 128 B or
// 4 rows x 256 B (whole 128-byte lines: half-line rows move at roughly half
// the rate), STAGES - 1 stages in flight ahead of the one being multiplied.
// WAVES_M x WAVES_N waves own (BM/WAVES_M) x (BN/WAVES_N) outputs each.  The
// tile shape is chosen from the weight shape (N) alone, its k width from K.
constexpr int kDBK = 64;

// 16-byte chunk c of LDS row r is stored at position c ^ gemm_swz<KB>(r).
// 128-byte rows (KB = 64): any 16 consecutive rows read at one logical chunk
// land in 16 distinct 16-byte slots of the 256-byte span they share two by
// two.  256-byte rows (KB = 128): each row spans all 64 banks, and 16
// consecutive rows put one logical chunk in 16 distinct slots.  Either way a
// ds_read_b128 of 32 rows is bank-conflict free.
template <int KB>
__device__ __forceinline__ int gemm_swz(int r) {
  return KB == 64 ? ((r >> 1) & 7) : (r & 15);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int kN>
__device__ __forceinline__ void vm_wait() {
  __builtin_amdgcn_s_waitcnt((kN & 15) | (7 << 4) | (15 << 8) | (((kN >> 4) & 3) << 14));
}
template <int kPer, int kMax>
__device__ __forceinline__ void vm_wait_stages(int ahead) {  // ahead in [0, kMax]
  if constexpr (kMax == 0) {
    vm_wait<0>();
  } else {
    if (ahead >= kMax)
      vm_wait<kPer * kMax>();
    else
      vm_wait_stages<kPer, kMax - 1>(ahead);
  }
}

// One reduce-scatter step of the Gumbel epilogue over lane offset O: keep
// HALF of the rows (the upper half when bit O of the lane is set), fold in the
// partner lane's copy of them.
template <int O, int HALF>
__device__ __forceinline__ void gumbel_fold_step(float* bv, int* bi, int li) {
  const bool up = (li & O) != 0;
#pragma unroll
  for (int k = 0; k < HALF; ++k) {
    const float send_v = up ? bv[k] : bv[k + HALF];
    const int send_i = up ? bi[k] : bi[k + HALF];
    float keep_v = up ? bv[k + HALF] : bv[k];
    int keep_i = up ? bi[k + HALF] : bi[k];
    const float rv = __shfl_xor(send_v, O, 64);
    const int ri = __shfl_xor(send_i, O, 64);
    take_better(keep_v, keep_i, rv, ri);
    bv[k] = keep_v;
    bi[k] = keep_i;
  }
}

template <int BM, int BN, int STAGES, int WAVES_M, int WAVES_N, int OUT_DT, int EPI, bool kSplit, int KB>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_dma_kernel(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B, void* C,
                                                       float* __restrict__ partial, int M, int N, int K,
                                                       int tilesM, int tilesN, int k_per_split) {
  static_assert(KB == 64 || KB == 128, "k width per stage");
  constexpr int ROW = KB * 2;     // bytes of K per row per stage: 128 or 256
  constexpr int RPW = 1024 / ROW;  // rows per 1 KiB copy window: 8 or 4
  constexpr int CPR = ROW / 16;    // 16-byte chunks per row: 8 or 16
  constexpr int A_BYTES = BM * ROW;
  constexpr int STAGE = (BM + BN) * ROW;
  constexpr int WIN = (BM + BN) / RPW;  // 1 KiB windows per stage
  constexpr int NW = WAVES_M * WAVES_N;
  static_assert(WIN % NW == 0, "windows must split evenly over the waves");
  constexpr int PER_WAVE = WIN / NW;
  static_assert(PER_WAVE * (STAGES - 2) <= 63, "vmcnt range");
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 block");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * STAGE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int logical = xcd_remap(blockIdx.x, tilesM * tilesN);
  const int m0 = (logical % tilesM) * BM;
  const int n0 = (logical / tilesM) * BN;
  const int k_begin = kSplit ? blockIdx.y * k_per_split : 0;
  const int k_end = kSplit ? min(K, k_begin + k_per_split) : K;
  const int nk = (k_end - k_begin) / KB;

  // This wave's DMA windows: j = wave + NW q, A windows first, then B.  Window
  // j holds rows RPW j .. RPW j + RPW - 1 of its operand; lane -> row
  // lane / CPR of the window, LDS chunk lane % CPR holding logical chunk
  // (lane % CPR) ^ gemm_swz(RPW j + lane / CPR).
  const int r_in = lane / CPR;
  const unsigned char* gbase[PER_WAVE];
  unsigned voff[PER_WAVE];
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q) {
    const int j = wave + NW * q;
    const bool isA = j < BM / RPW;
    const int row0 = isA ? m0 + RPW * j : n0 + RPW * (j - BM / RPW);
    const int rows = isA ? M : N;
    const int first = min(row0, rows - 1);       // window base row, in range
    const int row = min(row0 + r_in, rows - 1);  // rows past the edge re-read the last row
    const int c_log = (lane % CPR) ^ gemm_swz<KB>(RPW * j + r_in);
    const uint16_t* src = isA ? A : B;
    gbase[q] = reinterpret_cast<const unsigned char*>(src + (int64_t)first * K + k_begin);
    voff[q] = (unsigned)((row - first) * K * 2 + c_log * 16);
  }
  // Window q of every wave is an A window for q < A_PER_WAVE, a B window
  // after.  The weight (B) is streamed with the non-temporal hint in the
  // tiles where that measured faster -- rows per tile <= 64 (3-9% at M = 64)
  // and the 256-column tiles (lm_head 2.5% at M = 512) -- which keeps the
  // activation rows that every column block re-reads in the L2.
  constexpr int A_PER_WAVE = (BM / RPW) / NW;
  static_assert((BM / RPW) % NW == 0, "A windows must split evenly over the waves");
  constexpr bool kStreamB = BM <= 64 || BN >= 256;
  auto issue = [&](int kt) {
    unsigned char* slot = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
      if (q < A_PER_WAVE)
        lds_dma16(gbase[q] + (int64_t)kt * ROW, voff[q], slot + (wave + NW * q) * 1024);
      else
        lds_dma16<kStreamB>(gbase[q] + (int64_t)kt * ROW, voff[q], slot + (wave + NW * q) * 1024);
    }
  };

  // fragment offsets: row li of a 32-row block, logical chunk 2 ks + g
  const int xs = gemm_swz<KB>(li);
  int off[KB / 16];
#pragma unroll
  for (int ks = 0; ks < KB / 16; ++ks) off[ks] = li * ROW + 16 * ((2 * ks + g) ^ xs);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st);
  for (int kt = 0; kt < nk; ++kt) {
    vm_wait_stages<PER_WAVE, STAGES - 2>(min(STAGES - 2, nk - 1 - kt));  // stage kt has landed
    __builtin_amdgcn_s_barrier();  // for every wave; and stage kt-1's slot is free
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
    const unsigned char* As = smem + (kt % STAGES) * STAGE;
    const unsigned char* Bs = As + A_BYTES;
    // Fragments are read ahead of the MFMAs that use them, so that LDS
    // latency overlaps matrix work (with one wave per SIMD nothing else
    // hides it).  Small wave tiles read the whole stage up front; large ones
    // read step ks + 1 while step ks multiplies.  The sched_barrier keeps the
    // compiler from sinking the reads back next to their uses.
    constexpr int KS = KB / 16;
    constexpr bool kWhole = (FM + FN) <= 3;
    constexpr int NBUF = kWhole ? KS : 2;
    bf16x8 a[NBUF][FM], b[NBUF][FN];
    auto read = [&](int ks, int buf) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[buf][i] = *reinterpret_cast<const bf16x8*>(As + (wm * WM + 32 * i) * ROW + off[ks]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[buf][j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * WN + 32 * j) * ROW + off[ks]);
    };
    if constexpr (kWhole) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) read(ks, ks);
    } else {
      read(0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int buf = kWhole ? ks : (ks & 1);
      if constexpr (!kWhole) {
        if (ks + 1 < KS) read(ks + 1, (ks + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][i], b[buf][j], acc[i][j], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: lane holds column li; value v is row 8(v/4) + 4g + v%4.
  if constexpr (EPI == kEpiGumbel) {
    // C is the noise [M, N] fp32; `partial` receives, per row m and per
    // group of WN columns (this wave's), the best (score bits, index) pair
    // of s = fl32(acc + noise) under take_better's order: the same scores as
    // storing the fp32 product and adding the noise afterwards.  Branch
    // free: rows past M read row M-1 and are not written; columns past N
    // enter as (-inf, INT_MAX), which never beats a real entry.
    static_assert(!kSplit && OUT_DT == BIV_F32, "Gumbel epilogue: fp32 scores, no split");
    const float* noise = static_cast<const float*>(C);
    uint2* part = reinterpret_cast<uint2*>(partial);
    const int groups = (N + WN - 1) / WN;
    const int ncol0 = n0 + wn * WN;
    if (ncol0 < N) {
      const int grp = ncol0 / WN;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float bv[16];
        int bi[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          bv[v] = -INFINITY;
          bi[v] = 0x7fffffff;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = min(m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3), M - 1);
          const float* nrow = noise + (int64_t)m * N;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int n = ncol0 + 32 * j + li;
            const bool ok = n < N;
            const float sc = acc[i][j][v] + nrow[ok ? n : N - 1];
            take_better(bv[v], bi[v], ok ? sc : -INFINITY, ok ? n : 0x7fffffff);
          }
        }
        // The 32 lanes of each half hold the same 16 rows.  Reduce-scatter:
        // at offset o a lane keeps half of its rows (the upper half if bit o
        // of its lane is set) and folds in its partner's copy of them, so
        // after offsets 16, 8, 4, 2 lane li holds row li >> 1 over 16 lanes,
        // and offset 1 completes it (31 exchanges instead of 80).
        gumbel_fold_step<16, 8>(bv, bi, li);
        gumbel_fold_step<8, 4>(bv, bi, li);
        gumbel_fold_step<4, 2>(bv, bi, li);
        gumbel_fold_step<2, 1>(bv, bi, li);
        {
          const float rv = __shfl_xor(bv[0], 1, 64);
          const int ri = __shfl_xor(bi[0], 1, 64);
          take_better(bv[0], bi[0], rv, ri);
        }
        const int v = li >> 1;
        const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if ((li & 1) == 0 && m < M) part[(int64_t)m * groups + grp] = make_uint2(__float_as_uint(bv[0]), (unsigned)bi[0]);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * WN + 32 * j + li;
      if constexpr (EPI == BIV_EPI_SWIGLU) {
        // fragment pair (j, j + 1) = gate and up blocks of the same 32
        // outputs: packed columns 64b .. 64b+63 -> outputs 32b .. 32b+31
        static_assert(FN % 2 == 0 && !kSplit, "SwiGLU pairs the wave's gate and up fragments");
        if (j & 1) continue;
        const int nc = n0 + wn * WN + 32 * j;  // a multiple of 64
        if (nc >= N) continue;
        const int col = (nc >> 1) + li;
        const int64_t n_out = N >> 1;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
          if (m >= M) continue;
          const float gt = acc[i][j][v], up = acc[i][j + 1][v];
          const float act = __fdiv_rn(gt, __fadd_rn(1.0f, expf(-gt)));
          store_from_f32(C, (int64_t)m * n_out + col, __fmul_rn(act, up), OUT_DT);
        }
        continue;
      }
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        if (m >= M) continue;
        const int64_t idx = (int64_t)m * N + n;
        const float x = acc[i][j][v];
        if (kSplit) {
          partial[(int64_t)blockIdx.y * M * N + idx] = x;
        } else if (EPI == BIV_EPI_ACCUM) {
          store_from_f32(C, idx, __fadd_rn(load_as_f32(C, idx, OUT_DT), x), OUT_DT);
        } else {
          store_from_f32(C, idx, x, OUT_DT);
        }
      }
    }
}

// fp32 path: 64 x 64 tiles, K staged 16 at a time, each lane owns 4 x 4
// outputs; every output is one fused multiply-add chain over k ascending.
constexpr int kFT = 64, kFK = 16;

template <int OUT_DT, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                       void* C, int M, int N, int K) {
  __shared__ float As[kFK][kFT + 4];
  __shared__ float Bs[kFK][kFT + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * kFT, n0 = blockIdx.x * kFT;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kFK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      const int row = idx >> 4, kk = idx & 15;
      const int gk = k0 + kk;
      As[kk][row] = (m0 + row < M && gk < K) ? A[(int64_t)(m0 + row) * K + gk] : 0.0f;
      Bs[kk][row] = (n0 + row < N && gk < K) ? B[(int64_t)(n0 + row) * K + gk] : 0.0f;
    }
    __syncthreads();
    const int kmax = min(kFK, K - k0);
    for (int kk = 0; kk < kmax; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __fmaf_rn(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const int64_t idx = (int64_t)m * N + n;
      if (EPI == BIV_EPI_ACCUM)
        store_from_f32(C, idx, __fadd_rn(load_as_f32(C, idx, OUT_DT), acc[i][j]), OUT_DT);
      else
        store_from_f32(C, idx, acc[i][j], OUT_DT);
    }
  }
}

// Split-K second pass: C = sum over splits (ascending) of the partials.
template <int OUT_DT, int EPI>
__global__ void splitk_reduce_kernel(const float* __restrict__ partial, void* C, int64_t MN, int splits) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += (int64_t)gridDim.x * blockDim.x) {
    float s = partial[e];
    for (int k = 1; k < splits; ++k) s = __fadd_rn(s, partial[(int64_t)k * MN + e]);
    if (EPI == BIV_EPI_ACCUM) s = __fadd_rn(load_as_f32(C, e, OUT_DT), s);
    store_from_f32(C, e, s, OUT_DT);
  }
}

// The same second pass with SwiGLU applied (the gate/up weight interleaved in
// blocks of 32 rows, as for gemm_bi's BIV_EPI_SWIGLU): output (m, j) sums
// packed columns 64(j/32) + j%32 (gate) and that + 32 (up) over the splits,
// then silu(g) * u, rounded once.
template <int OUT_DT>
__global__ void splitk_reduce_swiglu_kernel(const float* __restrict__ partial, void* C, int64_t M, int64_t N,
                                            int splits) {
  const int64_t n_out = N >> 1, MN = M * N;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < M * n_out; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / n_out, j = e - m * n_out;
    const int64_t cg = m * N + 64 * (j >> 5) + (j & 31), cu = cg + 32;
    float g = partial[cg], u = partial[cu];
    for (int k = 1; k < splits; ++k) {
      g = __fadd_rn(g, partial[(int64_t)k * MN + cg]);
      u = __fadd_rn(u, partial[(int64_t)k * MN + cu]);
    }
    const float act = __fdiv_rn(g, __fadd_rn(1.0f, expf(-g)));
    store_from_f32(C, e, __fmul_rn(act, u), OUT_DT);
  }
}

template <int OUT_DT, int EPI, bool kSplit>
static void launch_bf16(const void* A, const void* B, void* C, float* partial, int M, int N, int K, int splits,
                        int k_per_split, hipStream_t s) {
  const int tilesM = (int)cdiv(M, kBM), tilesN = (int)cdiv(N, kBN);
  hipLaunchKernelGGL((gemm_bf16_kernel<OUT_DT, EPI, kSplit>), dim3(tilesM * tilesN, splits), dim3(kGemmThreads), 0,
                     s, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), C, partial, M, N, K,
                     tilesM, tilesN, k_per_split);
}

// Tile of the staged kernel for a weight with N outputs: one column tiling
// per weight shape, the same for every M (rows per tile are cut for M <= 64,
// below).  (Each output's reduction order is the
// same under every tile -- one MFMA shape, ascending k -- so the tile only
// decides which workgroup computes which outputs.)  Chosen by measurement:
// at M = 512 on the decoder's weights, and for the 8192 <= N < 16384 class
// (no decoder weight) across M = 1 .. 512.
enum DmaTile { kTileL = 0, kTileS = 1, kTileQ = 2, kTileT = 3 };
#ifndef BIV_GEMM_L_TILE
#define BIV_GEMM_L_TILE 256, 256, 2, 2, 4  // BM, BN, stages, waves along M, waves along N
#endif
#ifndef BIV_GEMM_S_TILE
#define BIV_GEMM_S_TILE 128, 64, 3, 4, 2
#endif
#ifndef BIV_GEMM_Q_TILE
#define BIV_GEMM_Q_TILE 128, 96, 2, 4, 1  // 128-wide k stages (K % 128 == 0)
#endif
#ifndef BIV_GEMM_Q64_TILE
#define BIV_GEMM_Q64_TILE 128, 96, 4, 4, 1  // the same tile with 64-wide k stages
#endif
#ifndef BIV_GEMM_T_TILE
#define BIV_GEMM_T_TILE 128, 64, 4, 4, 2
#endif

// Columns per wave of a tile: the group width of the Gumbel epilogue's
// per-row partial results (lm_head_gumbel_verify runs the L tile).
template <int BM, int BN, int STAGES, int WAVES_M, int WAVES_N>
constexpr int wave_cols() {
  return BN / WAVES_N;
}
constexpr int kGumbelGroup = wave_cols<BIV_GEMM_L_TILE>();

static DmaTile dma_tile_for(int64_t N) {
  if (N >= 16384) return kTileL;  // 256 x 256, 8 waves of 128 x 64, 2 stages (128 KiB LDS)
  if (N >= 8192) return kTileS;   // 128 x 64, 8 waves of 32 x 32, 3 stages (72 KiB)
  if (N > 4096) return kTileQ;    // 128 x 96, 4 waves of 32 x 96, 2 stages of 128-wide k (112 KiB)
  return kTileT;                  // 128 x 64, 8 waves of 32 x 32, 4 stages (96 KiB)
}

template <int BM, int BN, int STAGES, int WAVES_M, int WAVES_N, int OUT_DT, int EPI, bool kSplit, int KB = kDBK>
static void launch_dma_t(const void* A, const void* B, void* C, float* partial, int M, int N, int K, int splits,
                         int k_per_split, hipStream_t s) {
  const int tilesM = (int)cdiv(M, BM), tilesN = (int)cdiv(N, BN);
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, STAGES, WAVES_M, WAVES_N, OUT_DT, EPI, kSplit, KB>), dim3(tilesM * tilesN, splits),
                     dim3(64 * WAVES_M * WAVES_N),
                     0, s, static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B), C, partial, M, N, K,
                     tilesM, tilesN, k_per_split);
}

// Few rows (M <= 64, decode-sized batches): the same tiling of N (tile
// width, waves along N, hence the same workgroup per output column block)
// and the same per-element reduction, with the tile's rows cut to 32 or 64.
// No copies are spent on rows past M (a 128-row tile at M = 1 copies 128
// activation rows per stage for one useful row), and the LDS this frees holds
// a deeper ring of weight stages: small-M calls stream the weight, so the
// weight bytes in flight per CU set their speed.  Rows, columns, stages,
// waves along M and along N, for the tile classes above:
#define BIV_GEMM_L32_TILE 32, 256, 4, 1, 4   // 144 KiB, three weight stages in flight
#define BIV_GEMM_L64_TILE 64, 256, 3, 2, 4   // 120 KiB
#define BIV_GEMM_N32_TILE 32, 64, 8, 1, 2    // S and T classes: 96 KiB, seven stages in flight
#define BIV_GEMM_N64_TILE 64, 64, 8, 2, 2    // 128 KiB
#define BIV_GEMM_Q64R_TILE 64, 96, 3, 2, 1   // Q class, 128-wide k: 120 KiB
#define BIV_GEMM_Q64K64_TILE 64, 96, 4, 2, 1  // Q class, 64-wide k: 80 KiB
constexpr int kSmallRows = 64;
static_assert(wave_cols<BIV_GEMM_L32_TILE>() == kGumbelGroup && wave_cols<BIV_GEMM_L64_TILE>() == kGumbelGroup,
              "the Gumbel epilogue's group width is the L tile's columns per wave at every row count");

// kSplit: the split-K comparison path on the same small tiles (k ranges of
// k_per_split, a multiple of 64).
template <int OUT_DT, int EPI, bool kSplit = false>
static void launch_dma_small(DmaTile t, const void* A, const void* B, void* C, float* partial, int M, int N, int K,
                             hipStream_t s, int splits = 1, int k_per_split = 0) {
  const bool r32 = M <= 32;
  const int kps = kSplit ? k_per_split : K;
  if constexpr (EPI == BIV_EPI_SWIGLU || EPI == kEpiGumbel) {  // these epilogues run the L tile only
    (void)t;
    if (r32) launch_dma_t<BIV_GEMM_L32_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
    else launch_dma_t<BIV_GEMM_L64_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
  } else if (t == kTileL) {
    if (r32) launch_dma_t<BIV_GEMM_L32_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
    else launch_dma_t<BIV_GEMM_L64_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
  } else if (t == kTileQ) {
    // the 64-row tiles at every M <= 64: their two waves along M issue the
    // copies twice as fast as the 32-row tile's single wave (QKV at M = 1:
    // 45.7 us with 32 rows, 38.3 us with 64)
    if (!kSplit && K % 128 == 0)
      launch_dma_t<BIV_GEMM_Q64R_TILE, OUT_DT, EPI, kSplit, 128>(A, B, C, partial, M, N, K, splits, kps, s);
    else
      launch_dma_t<BIV_GEMM_Q64K64_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
  } else {  // S and T: 64 columns, two waves along N
    if (r32) launch_dma_t<BIV_GEMM_N32_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
    else launch_dma_t<BIV_GEMM_N64_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, kps, s);
  }
}

template <int OUT_DT, int EPI, bool kSplit>
static void launch_dma(DmaTile t, const void* A, const void* B, void* C, float* partial, int M, int N, int K,
                       int splits, int k_per_split, hipStream_t s) {
  if (M <= kSmallRows) {
    launch_dma_small<OUT_DT, EPI, kSplit>(t, A, B, C, partial, M, N, K, s, splits, k_per_split);
    return;
  }
  if (t == kTileL)
    launch_dma_t<BIV_GEMM_L_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, k_per_split, s);
  else if (t == kTileS)
    launch_dma_t<BIV_GEMM_S_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, k_per_split, s);
  else if (t == kTileQ) {
    // 256-byte row copies (128-wide k stages) where K allows; split-K
    // ranges are multiples of 64
    if constexpr (!kSplit) {
      if (K % 128 == 0) {
        launch_dma_t<BIV_GEMM_Q_TILE, OUT_DT, EPI, kSplit, 128>(A, B, C, partial, M, N, K, splits, k_per_split, s);
        return;
      }
    }
    launch_dma_t<BIV_GEMM_Q64_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, k_per_split, s);
  }
  else
    launch_dma_t<BIV_GEMM_T_TILE, OUT_DT, EPI, kSplit>(A, B, C, partial, M, N, K, splits, k_per_split, s);
}

static biv_status check_gemm_args(const char* who, const void* A, const void* B, void* C, int64_t M, int64_t N,
                                  int64_t K, int out_dt, int epilogue) {
  BIV_REQUIRE(valid_dt(out_dt), "%s: bad out dtype %d", who, out_dt);
  BIV_REQUIRE(epilogue == BIV_EPI_STORE || epilogue == BIV_EPI_ACCUM || epilogue == BIV_EPI_SWIGLU,
              "%s: bad epilogue %d", who, epilogue);
  BIV_REQUIRE(M >= 0 && N >= 1 && K >= 1, "%s: bad sizes M=%lld N=%lld K=%lld", who, (long long)M, (long long)N,
              (long long)K);
  BIV_REQUIRE(M <= (1 << 30) && N <= (1 << 30) && K <= (1 << 30), "%s: size too large", who);
  if (M > 0) BIV_REQUIRE(A && B && C, "%s: NULL pointer", who);
  return BIV_OK;
}

}  // namespace biv

extern "C" biv_status gemm_bi(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                              biv_dtype in_dt, biv_dtype out_dt, int epilogue, biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(valid_dt(in_dt), "gemm_bi: bad in dtype %d", (int)in_dt);
  biv_status st = check_gemm_args("gemm_bi", A, B, C, M, N, K, out_dt, epilogue);
  if (st != BIV_OK) return st;
  if (M == 0) return BIV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (epilogue == BIV_EPI_SWIGLU) {
    BIV_REQUIRE(in_dt == BIV_BF16, "gemm_bi: the SwiGLU epilogue needs bf16 inputs");
    BIV_REQUIRE(N % 64 == 0 && K % kDBK == 0, "gemm_bi: the SwiGLU epilogue needs N %% 64 == 0 and K %% 64 == 0 "
                "(N=%lld K=%lld)", (long long)N, (long long)K);
    BIV_REQUIRE(aligned16(A) && aligned16(B), "gemm_bi: bf16 path needs 16-byte aligned A and B");
    BIV_REQUIRE((int64_t)K * 2 * 16 <= 0x7fffffff, "gemm_bi: K too large");
    // the wide tile for every N: its waves hold two 32-column fragments, a
    // gate block and the matching up block
    if (m <= kSmallRows) {
      if (out_dt == BIV_BF16) launch_dma_small<BIV_BF16, BIV_EPI_SWIGLU>(kTileL, A, B, C, nullptr, m, n, k, s);
      else launch_dma_small<BIV_F32, BIV_EPI_SWIGLU>(kTileL, A, B, C, nullptr, m, n, k, s);
    } else if (out_dt == BIV_BF16) {
      launch_dma_t<BIV_GEMM_L_TILE, BIV_BF16, BIV_EPI_SWIGLU, false>(A, B, C, nullptr, m, n, k, 1, k, s);
    } else {
      launch_dma_t<BIV_GEMM_L_TILE, BIV_F32, BIV_EPI_SWIGLU, false>(A, B, C, nullptr, m, n, k, 1, k, s);
    }
    return launched("gemm_bi/bf16-swiglu");
  }
  if (in_dt == BIV_BF16) {
    BIV_REQUIRE(K % 8 == 0, "gemm_bi: bf16 path needs K %% 8 == 0 (K=%lld)", (long long)K);
    BIV_REQUIRE(aligned16(A) && aligned16(B), "gemm_bi: bf16 path needs 16-byte aligned A and B");
    BIV_REQUIRE(cdiv(M, kBM) * cdiv(N, kBN) <= 0x7fffffff, "gemm_bi: too many tiles");
    BIV_REQUIRE((int64_t)K * 2 * 16 <= 0x7fffffff, "gemm_bi: K too large");
    if (K % kDBK == 0) {  // staged kernel (same reduction, identical bits); chosen by K alone, never by M
      const DmaTile t = dma_tile_for(N);
      if (out_dt == BIV_BF16) {
        if (epilogue == BIV_EPI_ACCUM) launch_dma<BIV_BF16, BIV_EPI_ACCUM, false>(t, A, B, C, nullptr, m, n, k, 1, k, s);
        else launch_dma<BIV_BF16, BIV_EPI_STORE, false>(t, A, B, C, nullptr, m, n, k, 1, k, s);
      } else {
        if (epilogue == BIV_EPI_ACCUM) launch_dma<BIV_F32, BIV_EPI_ACCUM, false>(t, A, B, C, nullptr, m, n, k, 1, k, s);
        else launch_dma<BIV_F32, BIV_EPI_STORE, false>(t, A, B, C, nullptr, m, n, k, 1, k, s);
      }
      return launched("gemm_bi/bf16-staged");
    }
    if (out_dt == BIV_BF16) {
      if (epilogue == BIV_EPI_ACCUM) launch_bf16<BIV_BF16, BIV_EPI_ACCUM, false>(A, B, C, nullptr, m, n, k, 1, k, s);
      else launch_bf16<BIV_BF16, BIV_EPI_STORE, false>(A, B, C, nullptr, m, n, k, 1, k, s);
    } else {
      if (epilogue == BIV_EPI_ACCUM) launch_bf16<BIV_F32, BIV_EPI_ACCUM, false>(A, B, C, nullptr, m, n, k, 1, k, s);
      else launch_bf16<BIV_F32, BIV_EPI_STORE, false>(A, B, C, nullptr, m, n, k, 1, k, s);
    }
    return launched("gemm_bi/bf16");
  }
  dim3 grid((unsigned)cdiv(N, kFT), (unsigned)cdiv(M, kFT));
  BIV_REQUIRE(cdiv(M, kFT) <= 65535, "gemm_bi: fp32 path supports M <= %d", 65535 * kFT);
  const float* a = static_cast<const float*>(A);
  const float* b = static_cast<const float*>(B);
  if (out_dt == BIV_F32) {
    if (epilogue == BIV_EPI_ACCUM) hipLaunchKernelGGL((gemm_f32_kernel<BIV_F32, BIV_EPI_ACCUM>), grid, dim3(256), 0, s, a, b, C, m, n, k);
    else hipLaunchKernelGGL((gemm_f32_kernel<BIV_F32, BIV_EPI_STORE>), grid, dim3(256), 0, s, a, b, C, m, n, k);
  } else {
    if (epilogue == BIV_EPI_ACCUM) hipLaunchKernelGGL((gemm_f32_kernel<BIV_BF16, BIV_EPI_ACCUM>), grid, dim3(256), 0, s, a, b, C, m, n, k);
    else hipLaunchKernelGGL((gemm_f32_kernel<BIV_BF16, BIV_EPI_STORE>), grid, dim3(256), 0, s, a, b, C, m, n, k);
  }
  return launched("gemm_bi/f32");
}

namespace biv {
// Tiles of the staged kernel's grid for an (M, N) output: the column tiling
// of N's weight class, and its rows per tile (32 or 64 at M <= 64).
static int64_t staged_tiles(int64_t M, int64_t N) {
  int64_t bm, bn;
  switch (dma_tile_for(N)) {
    case kTileL: bm = 256; bn = 256; break;
    case kTileQ: bm = 128; bn = 96; break;
    default: bm = 128; bn = 64; break;
  }
  if (M <= kSmallRows) bm = M <= 32 && dma_tile_for(N) != kTileQ ? 32 : 64;
  return cdiv(M, bm) * cdiv(N, bn);
}

// Split count of gemm_splitk's automatic choice: double it while the staged
// kernel's grid holds fewer workgroups than the GPU has compute units (one
// workgroup per CU is what these tiles run at), up to 8 and while every
// split keeps at least four 64-wide k stages.  1 means no split: the plain
// staged kernel, with no partial sums or second pass.
static int auto_splits(int64_t M, int64_t N, int64_t K) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                  hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  if (K % kDBK != 0) return std::max<int64_t>(1, std::min<int64_t>(cdiv(2 * cus, cdiv(M, kBM) * cdiv(N, kBN)), 8));
  const int64_t tiles = staged_tiles(M, N);
  int s = 1;
  while (s < 8 && tiles * s < cus && K / (2 * s) >= 4 * kDBK) s *= 2;
  return s;
}
static int split_len(int64_t K, int splits) { return (int)(cdiv(cdiv(K, splits), kBK) * kBK); }
}  // namespace biv

extern "C" int biv_splitk_auto_splits(int64_t M, int64_t N, int64_t K) {
  using namespace biv;
  if (M <= 0 || N <= 0 || K <= 0) return 1;
  const int sp = auto_splits(M, N, K);
  return (int)cdiv(K, split_len(K, sp));
}

extern "C" size_t biv_splitk_workspace_bytes(int64_t M, int64_t N, int splits) {
  if (M <= 0 || N <= 0 || splits < 1) return 0;
  return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

extern "C" biv_status gemm_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                  biv_dtype out_dt, int epilogue, int splits, void* workspace,
                                  size_t workspace_bytes, biv_stream stream) {
  using namespace biv;
  biv_status st = check_gemm_args("gemm_splitk", A, B, C, M, N, K, out_dt, epilogue);
  if (st != BIV_OK) return st;
  BIV_REQUIRE(epilogue != BIV_EPI_SWIGLU || (N % 64 == 0 && K % kDBK == 0),
              "gemm_splitk: the SwiGLU epilogue needs N %% 64 == 0 and K %% 64 == 0");
  BIV_REQUIRE(splits >= 0 && splits <= 64, "gemm_splitk: splits must be in [0, 64]");
  if (M == 0) return BIV_OK;
  BIV_REQUIRE(K % 8 == 0 && aligned16(A) && aligned16(B), "gemm_splitk: needs K %% 8 == 0 and aligned A, B");
  int sp = splits == 0 ? auto_splits(M, N, K) : splits;
  const int kps = split_len(K, sp);
  sp = (int)cdiv(K, kps);  // drop empty splits
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sp == 1) {  // no split: the invariant kernel itself, no partials
    const biv_status st1 = gemm_bi(A, B, C, M, N, K, BIV_BF16, out_dt, epilogue, stream);
    return st1;
  }
  BIV_REQUIRE(workspace != nullptr && workspace_bytes >= biv_splitk_workspace_bytes(M, N, sp),
              "gemm_splitk: workspace needs %zu bytes", biv_splitk_workspace_bytes(M, N, sp));
  float* part = static_cast<float*>(workspace);
  if (K % kDBK == 0)
    launch_dma<BIV_F32, BIV_EPI_STORE, true>(dma_tile_for(N), A, B, C, part, (int)M, (int)N, (int)K, sp, kps, s);
  else
    launch_bf16<BIV_F32, BIV_EPI_STORE, true>(A, B, C, part, (int)M, (int)N, (int)K, sp, kps, s);
  st = launched("gemm_splitk/partials");
  if (st != BIV_OK) return st;
  const int64_t MN = M * N;
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(MN, 256), 16384);
  if (epilogue == BIV_EPI_SWIGLU) {
    if (out_dt == BIV_BF16) hipLaunchKernelGGL((splitk_reduce_swiglu_kernel<BIV_BF16>), dim3(blocks), dim3(256), 0, s, part, C, M, N, sp);
    else hipLaunchKernelGGL((splitk_reduce_swiglu_kernel<BIV_F32>), dim3(blocks), dim3(256), 0, s, part, C, M, N, sp);
    return launched("gemm_splitk/reduce-swiglu");
  }
  if (out_dt == BIV_BF16) {
    if (epilogue == BIV_EPI_ACCUM) hipLaunchKernelGGL((splitk_reduce_kernel<BIV_BF16, BIV_EPI_ACCUM>), dim3(blocks), dim3(256), 0, s, part, C, MN, sp);
    else hipLaunchKernelGGL((splitk_reduce_kernel<BIV_BF16, BIV_EPI_STORE>), dim3(blocks), dim3(256), 0, s, part, C, MN, sp);
  } else {
    if (epilogue == BIV_EPI_ACCUM) hipLaunchKernelGGL((splitk_reduce_kernel<BIV_F32, BIV_EPI_ACCUM>), dim3(blocks), dim3(256), 0, s, part, C, MN, sp);
    else hipLaunchKernelGGL((splitk_reduce_kernel<BIV_F32, BIV_EPI_STORE>), dim3(blocks), dim3(256), 0, s, part, C, MN, sp);
  }
  return launched("gemm_splitk/reduce");
}

extern "C" size_t biv_gumbel_workspace_bytes(int M, int V) {
  using namespace biv;
  if (M <= 0 || V <= 0) return 0;
  return (size_t)M * (size_t)((V + kGumbelGroup - 1) / kGumbelGroup) * 8;
}

extern "C" biv_status lm_head_gumbel_verify(const void* h, const void* w_head, const float* noise, const int32_t* cand,
                                            int R, int K, int V, int H, int32_t* target, int32_t* accept_len,
                                            int32_t* next_token, void* workspace, size_t workspace_bytes,
                                            biv_stream stream) {
  using namespace biv;
  BIV_REQUIRE(R >= 0 && K >= 1 && V >= 1 && H >= 1, "lm_head_gumbel_verify: need R >= 0, K >= 1, V >= 1, H >= 1");
  BIV_REQUIRE((int64_t)R * K <= (1 << 30) && V <= (1 << 30), "lm_head_gumbel_verify: size too large");
  BIV_REQUIRE(H % kDBK == 0 && (int64_t)H * 2 * 16 <= 0x7fffffff,
              "lm_head_gumbel_verify: H must be a multiple of %d (H=%d)", kDBK, H);
  if (R == 0) return BIV_OK;
  BIV_REQUIRE(h && w_head && noise && cand && target && accept_len && next_token && workspace,
              "lm_head_gumbel_verify: NULL pointer");
  BIV_REQUIRE(aligned16(h) && aligned16(w_head), "lm_head_gumbel_verify: h and w_head must be 16-byte aligned");
  BIV_REQUIRE(((uintptr_t)workspace & 7) == 0, "lm_head_gumbel_verify: workspace must be 8-byte aligned");
  const int M = R * K;
  BIV_REQUIRE(workspace_bytes >= biv_gumbel_workspace_bytes(M, V),
              "lm_head_gumbel_verify: workspace %zu < %zu bytes", workspace_bytes, biv_gumbel_workspace_bytes(M, V));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M <= kSmallRows)
    launch_dma_small<BIV_F32, kEpiGumbel>(kTileL, h, w_head, const_cast<float*>(noise), static_cast<float*>(workspace),
                                          M, V, H, s);
  else
    launch_dma_t<BIV_GEMM_L_TILE, BIV_F32, kEpiGumbel, false>(h, w_head, const_cast<float*>(noise),
                                                             static_cast<float*>(workspace), M, V, H, 1, H, s);
  const biv_status st = launched("lm_head_gumbel_verify/gemm");
  if (st != BIV_OK) return st;
  return launch_gumbel_finish(static_cast<const uint2*>(workspace), (V + kGumbelGroup - 1) / kGumbelGroup, cand, R, K, target,
                              accept_len, next_token, s);
}
