/*
 * biverify.h — C ABI of the batch-invariant verifier step for MI355X (gfx950).
 *
 * The verifier step of decode-verify-rollback inference: a decoder forward
 * over W = N*K candidate tokens (K from each of N requests) built from
 * batch-invariant RMSNorm, matmul and attention, ending in Gumbel-max
 * verification of the candidates and an overwrite of the fast path's KV.
 *
 * Sources (web pages; cited by title and paragraph):
 *   [LLM42]  Telegram post on batch-invariant kernels and LLM-42
 *            (tgstat.com/ru/channel/@ashnskt/392):
 *            para 1 - batch-invariant matmul (no split-K, one data-parallel
 *            tiling), RMSNorm (fixed split over hidden), attention (fixed
 *            KV-split size); para 3 - fast path vs fixed-batch verifier,
 *            reference point = last known-correct token, overwrite of the
 *            fast path's KV at every verification; para 4 - W = N*K.
 *   [GUMBEL] Reading-club post on "Coupling without Communication and
 *            Drafter-Invariant Speculative Decoding"
 *            (tginsight.xyz/en/channel/AIexTime/post/185): Gumbel-max trick
 *            (argmax of logits + Gumbel noise, noise prepared in advance);
 *            Gumbel coupling (same noise for draft and target; verification
 *            compares the two tokens; no draft logits needed).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are device memory owned by the
 *     caller; the library never frees them.  Entry points allocate nothing
 *     (workspaces are passed in).
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL =
 *     the default stream).  Nothing synchronises.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns BIV_EINVAL (or BIV_EUNSUPPORTED for a shape the
 *     library has no kernel for) and launches nothing.  biv_last_error() then holds
 *     a message (thread-local).  A failed launch returns BIV_EHIP.  Device
 *     faults surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 *   - Layouts are row-major; "[a, b]" lists dimensions slowest first.
 *   - bf16 = IEEE binary32 truncated to its top 16 bits; every bf16 result
 *     is rounded once from fp32, to nearest even.
 *   - Batch invariance: for every entry point marked "_bi", each output row
 *     is a function of that row's inputs only (its own activations, its own
 *     request's KV); the bits do not change with M, with the number of
 *     requests, with which other rows share the call, or with a row's
 *     position in the batch.
 */
#ifndef BIVERIFY_H
#define BIVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BIV_OK = 0,
  BIV_EINVAL = 1,       /* bad argument: null pointer, size, alignment, dtype */
  BIV_EUNSUPPORTED = 2, /* valid request the library has no kernel for */
  BIV_EHIP = 3          /* the HIP runtime reported an error */
} biv_status;

typedef enum { BIV_F32 = 0, BIV_BF16 = 1 } biv_dtype;

typedef void* biv_stream; /* hipStream_t */

/* Version of this interface (increments when a signature changes). */
int biv_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* biv_last_error(void);

/* --------------------------------------------------------------------------
 * rmsnorm_bi — batch-invariant RMSNorm ([LLM42] para 1: RMSNorm with a fixed
 * split over the hidden dimension, independent of how many compute units are
 * busy), with an optional residual add in the same pass.
 *
 *   residual == NULL:  s[m, i] = x[m, i]
 *   residual != NULL:  s[m, i] = fl32(x[m, i] + residual[m, i]), rounded once
 *                      to x_dt and written back to residual[m, i]
 *   y[m, i] = s[m, i] * gamma[i] / sqrt(mean_k s[m, k]^2 + eps)
 *
 * x [M, H] and residual [M, H] (nullable) in x_dt; gamma [H] and y [M, H] in
 * y_dt (device).  The sum of squares of a row is accumulated in fp32 with
 * fused multiply-adds in an order fixed by H alone, never by M, the
 * pointers' alignment or the other rows: one 256-lane workgroup per row;
 * when H is a multiple of 1024, lane t adds the 4-element groups
 * 4t + 1024j (j ascending, the four elements in ascending order), otherwise
 * elements t, t+256, ... in ascending order; then a fixed butterfly over
 * the 64 lanes of each wave and the four wave sums added in ascending order.
 * M >= 0 (M = 0 launches nothing), 1 <= H <= 65536.  x, residual and y may
 * not overlap (BIV_EINVAL).
 *
 * The decoder forward here keeps its residual stream in fp32 and adds each
 * sublayer's output inside the matmul that produces it (gemm_bi's
 * BIV_EPI_ACCUM), so it calls rmsnorm_bi with residual == NULL; the fused
 * form serves callers whose sublayer outputs are separate tensors.
 * ------------------------------------------------------------------------ */
biv_status rmsnorm_bi(const void* x, biv_dtype x_dt, void* residual, const void* gamma, void* y, biv_dtype y_dt,
                      int64_t M, int64_t H, float eps, biv_stream stream);

/* --------------------------------------------------------------------------
 * gemm_bi — batch-invariant matmul ([LLM42] para 1: no split-K; one and the
 * same data-parallel tiling of the reduction for every batch size: each
 * output is reduced by one workgroup in one fixed order, while the rows per
 * output tile may shrink for small batches, which moves no bits).
 *
 *   acc[m, n] = sum_k A[m, k] * B[n, k]          (fp32 accumulation)
 *   epilogue BIV_EPI_STORE:  C[m, n] = acc
 *   epilogue BIV_EPI_ACCUM:  C[m, n] = C[m, n] + acc   (residual add, in place)
 *
 * A [M, K] and B [N, K] (the weight in linear-layer layout: row n holds the
 * K inputs of output n) in in_dt; C [M, N] in out_dt (device).
 *   in_dt BIV_BF16: bf16 MFMA (32x32x16), fp32 accumulators; every output is
 *     reduced over k in ascending 16-wide steps by one instruction shape,
 *     whatever M is, so a row's bits never depend on M.  Requires K % 8 == 0
 *     and 16-byte aligned A, B.
 *   in_dt BIV_F32: fp32 FMA chain over k ascending.
 * The rounding of C is once, from fp32.  M >= 0, N >= 1, K >= 1.
 * ------------------------------------------------------------------------ */
enum { BIV_EPI_STORE = 0, BIV_EPI_ACCUM = 1, BIV_EPI_SWIGLU = 2 };
/* epilogue BIV_EPI_SWIGLU (SwiGLU feed-forward, gate and up projections in one
 * product): B holds the gate and up weights interleaved in blocks of 32 rows
 * (rows 64b .. 64b+31 are gate rows 32b .. 32b+31, rows 64b+32 .. 64b+63 the
 * up rows 32b .. 32b+31); C is [M, N/2] and C[m, j] = silu(g) * u with g, u the
 * fp32 results of gate and up row j, silu(g) = g / (1 + exp(-g)), rounded once.
 * bf16 inputs only, N % 64 == 0 and K % 64 == 0. */

biv_status gemm_bi(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                   biv_dtype in_dt, biv_dtype out_dt, int epilogue, biv_stream stream);

/* --------------------------------------------------------------------------
 * attn_decode_bi — batch-invariant paged decode/verify attention ([LLM42]
 * para 1: a fixed KV-split size, no adaptation to sequence length or load;
 * para 3-4: the verifier runs K query rows per request).
 *
 * Row (r, j), j < q_len_r, is the query of the token at absolute position
 * ctx[r] + j; it attends to keys at positions 0 .. ctx[r] + j of request r:
 *   out = softmax(q . k_p * scale) . v_p,  q head h reads KV head h / (Hq/Hkv).
 *
 * Rows of a request (the K candidates of each of N requests, [LLM42] para 4;
 * requests may bring different numbers of candidates):
 *   q_off == NULL: every request has q_len rows; row (r, j) is row
 *                  r*q_len + j of q and out.
 *   q_off != NULL: device int32 [R+1], non-decreasing, q_off[0] = 0; request
 *                  r has q_len_r = q_off[r+1] - q_off[r] rows (0 <= q_len_r
 *                  <= q_len; q_len is then the largest q_len_r, which sizes
 *                  the grid and the workspace), row (r, j) is row
 *                  q_off[r] + j of q and out, and q and out hold q_off[R]
 *                  rows.  The offsets are read on the device; rows past
 *                  q_len of a request are not computed.  A row's bits are the
 *                  same as with q_off == NULL and that request alone: they do
 *                  not depend on the other requests' row counts.
 *
 * q   the rows above, Hq*D elements each, consecutive rows q_stride
 *     elements apart (>= Hq*D; a slice of a fused QKV output can be passed
 *     directly)                                    dt, device
 * k_cache, v_cache [num_blocks, Hkv, 16, D]        dt, device (pages of 16)
 * block_table [R, max_blocks] int32: physical page of each logical page;
 *             entries outside [0, num_blocks) are treated as empty pages
 *             (their keys are masked, their values read as zero).
 * ctx [R] int32: verified context length L_r >= 0 of each request.
 * out [rows, Hq, D]                                dt, device
 *
 * Keys are cut into chunks of BIV_ATTN_CHUNK_TOKENS (256) tokens, aligned at
 * absolute position 0.  Each
 * chunk gives a partial (max, sum, weighted values) for each row; partials
 * are left-folded in ascending chunk order within fixed segments of
 * BIV_ATTN_SEG_TOKENS tokens, and the segment results are left-folded in
 * ascending order.  Every split point is a fixed absolute position, so a
 * row's result depends only on its own request's data and length.
 * Positions >= ctx[r] + q_len_r read as empty (values zero, keys masked).
 * Launches: the chunk/segment pass, then (only when some request spans
 * more than one segment, or segments are split) the fold of the partials;
 * large grids add a one-workgroup launch before them that orders the
 * segments.  Where the grid of segments would hold fewer than 1024 waves
 * (decided by R, Hkv and max_blocks alone), each segment is taken by
 * several waves over consecutive chunks: the first folds its
 * chunks, the later ones store their chunk partials, and a launch between
 * the two folds those on in the same ascending order, every segment of a
 * request at once -- the same fold, so the same bits.  The fp32 path folds all chunk partials of a row in one ascending
 * left fold (one launch).
 *
 * Supported: dt BIV_BF16 with D == 128 and Hq/Hkv dividing 32 (bf16 MFMA
 * path; any q_len: the rows of a request are taken 32/(Hq/Hkv) positions at a
 * time, each such row block with its own keys 0 .. ctx[r] + its last
 * position, so q_len up to a whole prompt gives a causal prefill whose rows
 * are the same bits as decoding them one at a time); dt BIV_F32 with D in
 * {64, 128} (fp32 path, any q_len).  Hq % Hkv == 0, ctx[r] + q_len_r <=
 * max_blocks * 16, R * row blocks <= 65535.
 *
 * workspace: device memory of at least
 * biv_attn_workspace_bytes_q(R, q_len, Hq, Hkv, max_blocks, BIV_ATTN_SEG_TOKENS)
 * bytes (equal to biv_attn_workspace_bytes(R, Hkv, max_blocks, ...) when
 * q_len * Hq/Hkv <= 32),
 * 16-byte aligned (bf16 path; may be NULL for the fp32 path); it holds the
 * segment (and, for split segments, chunk) partials between the two
 * launches and, for grids of at least four rounds of resident waves, the
 * work list that launches the segments in longest-first order (same
 * results); it needs no initialisation.
 * Calls that share a workspace must be ordered (same stream).
 * ------------------------------------------------------------------------ */
#define BIV_ATTN_CHUNK_TOKENS 256
#define BIV_ATTN_SEG_TOKENS 4096

size_t biv_attn_workspace_bytes(int R, int Hkv, int max_blocks, int seg_tokens);
/* The same for any q_len: R requests of q_len rows (0 for unsupported shapes). */
size_t biv_attn_workspace_bytes_q(int R, int q_len, int Hq, int Hkv, int max_blocks, int seg_tokens);

biv_status attn_decode_bi(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* ctx, const int32_t* q_off, void* out, int R,
                          int q_len, int Hq, int Hkv, int D, int max_blocks, int num_blocks, float scale,
                          biv_dtype dt, void* workspace, size_t workspace_bytes, biv_stream stream);

/* --------------------------------------------------------------------------
 * attn_decode_bi_static — attn_decode_bi without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It allocates
 * nothing: the segment partials (and work list) go to a static array of
 * BIV_ATTN_STATIC_SCRATCH_BYTES in the library's device code, one per GPU,
 * held from the library's load until the process ends.  Arguments, results
 * and bits are those of attn_decode_bi (same kernels).
 *
 * The call needs biv_attn_workspace_bytes_q(R, q_len, Hq, Hkv, max_blocks,
 * BIV_ATTN_SEG_TOKENS) <= BIV_ATTN_STATIC_SCRATCH_BYTES (32 MiB) and returns
 * BIV_EINVAL, launching nothing, when it needs more.  That covers, e.g., the
 * verify step of 64 requests x 8 KV heads at contexts up to 12288 (26 MB) or
 * one request up to 32768 (18 MB); batches small enough for their segments to be
 * split over several waves reserve room for every chunk's partial
 * (16 per segment) and reach the limit sooner.  Every call
 * on a GPU shares that GPU's array (it keeps the last call's contents; the
 * kernels need no initialisation), so calls that overlap on one GPU -- on two
 * streams, or from two threads -- race: order them on one stream.  The
 * array's address on a GPU is looked up at the first call there, with that
 * GPU current (BIV_EHIP if the runtime cannot give it).
 * ------------------------------------------------------------------------ */
#define BIV_ATTN_STATIC_SCRATCH_BYTES (32u << 20)

biv_status attn_decode_bi_static(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* ctx, const int32_t* q_off, void* out,
                                 int R, int q_len, int Hq, int Hkv, int D, int max_blocks, int num_blocks,
                                 float scale, biv_dtype dt, biv_stream stream);

/* --------------------------------------------------------------------------
 * gumbel_verify — Gumbel-max coupled verification ([GUMBEL]: add Gumbel(0,1)
 * noise to the logits and take the argmax; the same noise couples draft and
 * target, so verification compares the draft token with the target token).
 *
 * logits, noise [R*K, V] fp32 (row r*K + j; device).  noise row (r, j) must be
 *   the noise of the token at position ctx[r] + j + 1 (prepared in advance).
 * cand [R, K] int32: the fast path's candidate for position ctx[r] + j + 1.
 * Outputs (device, always fully written):
 *   target [R, K] int32:  argmax_v fl32(logits + noise); exact ties go to the
 *                         lowest index; NaN never wins; -0 equals +0.
 *   accept_len [R] int32: first j with target != cand, K if none.
 *   next_token [R] int32: target[r, accept_len[r]], or -1 if accept_len == K.
 * Two launches (per-row argmax, per-request decision), no workspace.
 * ------------------------------------------------------------------------ */
biv_status gumbel_verify(const float* logits, const float* noise, const int32_t* cand, int R, int K,
                         int V, int32_t* target, int32_t* accept_len, int32_t* next_token,
                         biv_stream stream);

/* --------------------------------------------------------------------------
 * gumbel_topk — the k largest perturbed scores of each row (Gumbel post: the
 * Gumbel-max trick gives top-k sampling for free; the top k of l + g are k
 * draws without replacement from the softmax).
 *
 * logits, noise [rows, V] fp32; idx [rows, k] int32: the indices in
 * descending order of s = fl32(l + g), equal scores in ascending index order,
 * a NaN score counted as -inf; score [rows, k] fp32 (nullable): those scores
 * (NaN as -inf).  k = 1 gives gumbel_verify's targets.  1 <= k <= V;
 * k > 8 returns BIV_EUNSUPPORTED.
 * ------------------------------------------------------------------------ */
biv_status gumbel_topk(const float* logits, const float* noise, int rows, int V, int k, int32_t* idx,
                       float* score, biv_stream stream);

/* --------------------------------------------------------------------------
 * lm_head_gumbel_verify — the lm_head matmul and gumbel_verify in one pass,
 * without the fp32 logits in HBM (Gumbel post: argmax of logits + noise,
 * then the candidate comparison; the noise is an input prepared in advance).
 *
 * h [R*K, H] bf16: final-normed hidden rows (row r*K + j as for gumbel_verify);
 * w_head [V, H] bf16: the lm_head weight (gemm_bi's B layout); noise
 * [R*K, V] fp32; cand [R, K] int32.  Scores are s = fl32(l + g) with l the
 * fp32 result gemm_bi gives for the same h and w_head (same per-element
 * reduction), so target, accept_len and next_token are bit for bit those of
 * gemm_bi(h, w_head -> fp32 logits) followed by gumbel_verify.  H must be a
 * multiple of 64, h and w_head 16-byte aligned.
 * workspace: device memory of at least biv_gumbel_workspace_bytes(R*K, V)
 * bytes, 8-byte aligned (per-row best pairs of each 64-column group); it need
 * not be initialised, and calls that share it must not overlap.
 * ------------------------------------------------------------------------ */
size_t biv_gumbel_workspace_bytes(int M, int V);
biv_status lm_head_gumbel_verify(const void* h, const void* w_head, const float* noise, const int32_t* cand,
                                 int R, int K, int V, int H, int32_t* target, int32_t* accept_len,
                                 int32_t* next_token, void* workspace, size_t workspace_bytes,
                                 biv_stream stream);

/* --------------------------------------------------------------------------
 * kv_overwrite — write the verifier's K/V into the slots the fast path wrote
 * ([LLM42] para 3: at every verification the fast path's KV, computed at some
 * other batch size, is overwritten with the verifier's consistent values).
 *
 * k_new, v_new: T token rows of Hkv*D elements, consecutive rows src_stride
 *   elements apart (so a slice of a fused QKV output can be passed directly).
 * slot [T] int64: physical slot page*16 + offset of token t.
 * k_cache, v_cache [num_blocks, Hkv, 16, D] (device), element size by dt.
 * Bit copy; every other slot is left unchanged.  Slots outside
 * [0, num_blocks*16) are skipped.  Slots must be distinct.
 * ------------------------------------------------------------------------ */
biv_status kv_overwrite(const void* k_new, const void* v_new, int64_t src_stride, const int64_t* slot,
                        void* k_cache, void* v_cache, int T, int Hkv, int D, int num_blocks,
                        biv_dtype dt, biv_stream stream);

/* --------------------------------------------------------------------------
 * Tree verification by branches.  A draft tree (for example the top-k tokens
 * a drafter proposes from the shared Gumbel noise at each position, [GUMBEL]:
 * top-k sampling comes with the Gumbel-max trick) is verified as B root-to-
 * leaf chains per request, each chain an ordinary row block of the verifier
 * step.  With the noise keyed by (request, absolute position), chains that
 * share a prefix get the same targets on it, and every chain's bits are those
 * of one-token-at-a-time decoding (batch invariance); the output therefore
 * does not depend on the tree ([GUMBEL]: at a fixed seed the output does not
 * depend on the drafter).  Each chain writes its K/V into private pages for
 * positions L_r .. L_r+K-1; the selected chain's pages then take the place
 * of the request's.
 *
 * kv_copy_pages: whole-page bit copies inside one layer's cache, page
 *   dst_page[i] <- page src_page[i] (all Hkv heads, 16 tokens, K and V), so
 *   that each chain's private page starts with the request's context tokens
 *   of the page holding position L_r.  src_page, dst_page [n] int32 (device);
 *   pairs with a page outside [0, num_blocks) or src == dst are skipped.  The
 *   dst pages must be distinct and none may appear in src_page (copies run
 *   in parallel).  Caches [num_blocks, Hkv, 16, D], 16-byte aligned.
 *
 * tree_select: for R requests of B chains each (accept_len, next_token
 *   [R*B] int32, chain-major within a request, as gumbel_verify writes them
 *   for R*B chains), best[r] = the chain with the longest accepted prefix,
 *   the lowest chain index among equals; accept_out[r] and next_out[r] are
 *   that chain's values.  All device pointers, [R] int32 outputs.
 * ------------------------------------------------------------------------ */
biv_status kv_copy_pages(const int32_t* src_page, const int32_t* dst_page, int n, void* k_cache, void* v_cache,
                         int num_blocks, int Hkv, int D, biv_dtype dt, biv_stream stream);
biv_status tree_select(const int32_t* accept_len, const int32_t* next_token, int R, int B, int32_t* best,
                       int32_t* accept_out, int32_t* next_out, biv_stream stream);

/* --------------------------------------------------------------------------
 * Elementwise helpers of the decoder forward (no reductions; row-local).
 * ------------------------------------------------------------------------ */

/* out[t, :] = table[ids[t], :] converted to out_dt (bf16 -> fp32 is exact).
 * ids outside [0, V) give a zero row.  table [V, H] in table_dt. */
biv_status embed_rows(const int32_t* ids, const void* table, biv_dtype table_dt, void* out,
                      biv_dtype out_dt, int T, int V, int H, biv_stream stream);

/* Host-side RoPE table (rotate-half convention): for p < max_pos, i < D/2,
 * cos_sin[(p * D/2 + i) * 2 + 0] = cos(p * theta^(-2i/D)),
 * cos_sin[(p * D/2 + i) * 2 + 1] = sin(...), computed in fp64, rounded to fp32.
 * cos_sin is HOST memory of max_pos * D floats. */
biv_status biv_rope_table(float* cos_sin, int max_pos, int D, double theta);

/* In-place rotate-half RoPE on n_heads heads of D elements starting at
 * element 0 of each of T rows (row stride `stride` elements):
 * (a, b) = (x[i], x[i + D/2]) -> (a cos - b sin, b cos + a sin), fp32 math,
 * rounded once to dt.  pos [T] int32 absolute positions (< max_pos of the
 * table; others leave the row unchanged).  cos_sin: device copy of the
 * biv_rope_table output. */
biv_status rope_apply(void* x, int64_t stride, const int32_t* pos, const float* cos_sin, int T,
                      int n_heads, int D, int max_pos, biv_dtype dt, biv_stream stream);

/* rope_apply on the Q and K heads of a fused QKV output followed by
 * kv_overwrite of its (rotated) K and V heads, in one pass over the rows
 * (RoPE as above; the overwrite as in [LLM42] para 3).  qkv: T rows of at
 * least (Hq + 2*Hkv)*D elements, `stride` elements apart: Q heads at element
 * 0, K heads at Hq*D, V heads at (Hq+Hkv)*D; Q and K are rotated in place.
 * pos, cos_sin, max_pos as for rope_apply; slot, k_cache, v_cache, num_blocks
 * as for kv_overwrite.  Results are bit for bit those of
 * rope_apply(qkv, stride, pos, cos_sin, T, Hq + Hkv, D, max_pos) followed by
 * kv_overwrite(qkv + Hq*D, qkv + (Hq+Hkv)*D, stride, slot, ...).  bf16 rows
 * with D a multiple of 16, stride a multiple of 8 and 16-byte aligned
 * pointers take the fused kernel; anything else runs those two calls. */
biv_status rope_kv_overwrite(void* qkv, int64_t stride, const int32_t* pos, const float* cos_sin,
                             const int64_t* slot, void* k_cache, void* v_cache, int T, int Hq, int Hkv, int D,
                             int max_pos, int num_blocks, biv_dtype dt, biv_stream stream);

/* out[m, n] = silu(g) * u, silu(g) = g / (1 + exp(-g)), fp32 math; gu [M, 2N],
 * out [M, N], both in dt.  block == 0: g = gu[m, n], u = gu[m, N + n] (gate
 * and up halves); block > 0 (dividing N): the columns come in groups of
 * 2*block, gate block then up block, as in the BIV_EPI_SWIGLU weight layout
 * (block 32): g = gu[m, 2*block*(n/block) + n%block], u = that + block. */
biv_status swiglu(const void* gu, void* out, int64_t M, int64_t N, int64_t block, biv_dtype dt,
                  biv_stream stream);

/* --------------------------------------------------------------------------
 * Non-invariant comparison variants (same contracts as above, NOT batch
 * invariant): what a serving engine does by default at small batch ([LLM42]
 * para 1: split-K matmul; attention whose split adapts to length and load).
 * ------------------------------------------------------------------------ */

/* gemm_splitk: bf16 A/B as in gemm_bi (epilogues STORE, ACCUM and SWIGLU),
 * fp32 partial sums of `splits` slices of K (each a multiple of 64 wide)
 * computed by the staged kernel on its own tiles and summed in ascending
 * slice order by a second pass that applies the epilogue.  A split count of 1
 * is gemm_bi itself (no partials, no second pass).  splits == 0 picks the
 * count from M, N, K: doubled from 1 while the staged kernel's grid holds
 * fewer workgroups than the GPU has compute units, up to 8, keeping at least
 * four k stages per slice.  Which count is fastest depends on the shape; a
 * caller tuning for speed times the candidates (the results differ in the
 * last bits between counts and between M, which is the point of the
 * comparison).  workspace: biv_splitk_workspace_bytes() (unused at 1). */
size_t biv_splitk_workspace_bytes(int64_t M, int64_t N, int splits);
/* The split count gemm_splitk uses for splits == 0. */
int biv_splitk_auto_splits(int64_t M, int64_t N, int64_t K);
biv_status gemm_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                       biv_dtype out_dt, int epilogue, int splits, void* workspace,
                       size_t workspace_bytes, biv_stream stream);

/* attn_decode_adaptive: bf16 attention whose segment size (tokens per
 * workgroup, a multiple of 256) is chosen from the batch:
 * biv_attn_adaptive_split() returns the largest split that still gives at
 * least 512 workgroups (2 per compute unit), or the whole capacity when the
 * batch alone gives that many.  split_tokens == 0 uses that choice.
 * Workspace: biv_attn_workspace_bytes(R, Hkv, max_blocks, split). */
int biv_attn_adaptive_split(int R, int Hkv, int max_blocks);
biv_status attn_decode_adaptive(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* ctx, void* out, int R,
                                int q_len, int Hq, int Hkv, int D, int max_blocks, int num_blocks,
                                float scale, int split_tokens, void* workspace,
                                size_t workspace_bytes, biv_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* BIVERIFY_H */
