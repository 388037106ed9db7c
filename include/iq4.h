/*
 * iq4.h -- C ABI of the MI355X (gfx950) library for matrix products against IQ4
 * block-quantised weights decoded on the fly.
 *
 * Block format.  32 weights per block, stored in 18 bytes: an IEEE binary16 scale d
 * (bytes 0-1, little-endian) and 32 four-bit indices into the fixed codebook
 * {-127,-104,-83,-65,-49,-35,-22,-10,1,13,25,38,53,69,89,113}; byte 2+i holds index
 * q_i in its low nibble and q_{i+16} in its high nibble.  The decoded weight is
 * w = d * codebook[q], exact in binary32.  Page 2 of the sources (Strata pull request
 * "sm_80 (GA100) tuning", PLE-compact commit message) fixes the block at 18 bytes per
 * 32 values; the nibble order is this library's reading, shared with its CPU oracle.
 *
 * A weight matrix W has N rows and K columns (K a multiple of 32); row r is K/32
 * consecutive blocks.  This "row-block" layout is what iq4_quantize_blocks writes and
 * iq4_dequant_blocks / iq4_pack_weights read.  The product calls read the "packed"
 * layout written by iq4_pack_weights (same 18 bytes per block, rearranged so that one
 * 128-bit load feeds one matrix-core fragment; see iq4_pack_weights).
 *
 * Conventions shared by every call:
 *  - All pointers are device pointers unless stated otherwise; the caller owns every
 *    buffer.  The library never allocates device memory and never synchronises the
 *    stream inside a call: work is enqueued on `stream` (a hipStream_t; NULL means the
 *    legacy default stream) and inputs must stay valid and unmodified until the stream
 *    has passed the call.  Outputs are overwritten, never accumulated into.
 *  - Every call returns IQ4_OK (0) or a negative IQ4_E_* status.  Arguments are
 *    validated on the host before anything is enqueued; on error nothing is enqueued
 *    and iq4_last_error() describes the problem.
 *  - Activations are token-major: X[t][k] at X + t*ldx + k (ldx in elements).
 *  - Calls are safe from several host threads; the last-error text is per thread.
 */
#ifndef IQ4_H
#define IQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define IQ4_OK 0
#define IQ4_E_ARG (-1)         /* a size, count or dtype is out of range          */
#define IQ4_E_ALIGN (-2)       /* a pointer or leading dimension is misaligned    */
#define IQ4_E_UNSUPPORTED (-3) /* a shape this library does not implement         */
#define IQ4_E_HIP (-4)         /* the HIP runtime reported an error at launch     */
#define IQ4_E_WORKSPACE (-5)   /* the workspace is missing or too small           */

/* element types */
#define IQ4_F32 0
#define IQ4_F16 1

/* iq4_moe_expert_gemm flags */
#define IQ4_MOE_ATOMIC_COMBINE 1u    /* prefill: add slot rows into `out` with atomics
                                        (not bit-reproducible run to run)             */
#define IQ4_MOE_KEEP_INTERMEDIATE 2u /* also keep the gate and up products g, u (fp32)
                                        in the workspace, and always run the gather;
                                        offsets: iq4_moe_intermediate_layout          */

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * thread's next iq4_* call. */
const char* iq4_last_error(void);

/* ABI version of this header (incremented on incompatible change). */
#define IQ4_ABI_VERSION 1
int iq4_abi_version(void);

/*
 * Encode float32 weights into blocks (the quantiser of the block format).
 *   src      [n_blocks][32] float32, finite, with max|w|/127 <= 65504.
 *   blocks   [n_blocks][18] bytes (row-block layout; 2-byte aligned).
 * Per block: d = f16_rne(f32(max|w|) / 127) (IEEE binary32 division); each element
 * takes the codebook level nearest to w/d, ties to the lower index; d == 0 stores
 * index 8 everywhere.  The index decision is exact, so the bytes are unique.
 * Source: the workload definition of the format (scale absmax/127, nearest level).
 * Errors: IQ4_E_ARG if n_blocks < 0; IQ4_E_ALIGN if src is not 16-byte aligned or
 * blocks is not 2-byte aligned.
 */
int iq4_quantize_blocks(const float* src, int64_t n_blocks, void* blocks, void* stream);

/*
 * Decode blocks: out[b][i] = d_b * codebook[q_{b,i}], in block order.
 *   blocks   [n_blocks][18] bytes (row-block layout; 2-byte aligned).
 *   out      [n_blocks][32] of out_dtype: IQ4_F32 (exact) or IQ4_F16 (the exact
 *            value rounded to nearest even, subnormals kept, overflow to inf).
 * Bitwise equal to the host decode -- page 2 (pull request "sm_80 (GA100) tuning"),
 * PLE-compact commit message: the device dequant yields the host dequant's floats
 * bit for bit.
 * Errors: IQ4_E_ARG (n_blocks < 0, bad dtype), IQ4_E_ALIGN (blocks not 2-byte or out
 * not 16-byte aligned).
 */
int iq4_dequant_blocks(const void* blocks, int64_t n_blocks, int32_t out_dtype, void* out,
                       void* stream);

/*
 * Size in bytes of the packed form of an n x k matrix (= n*k/32*18), or -1 if
 * n % 16 != 0, k % 128 != 0 or either is not positive.
 */
int64_t iq4_packed_bytes(int64_t n, int64_t k);

/*
 * Rearrange an n x k matrix from the row-block layout into the packed layout read by
 * the product calls (one-time, at weight-load time).
 *   blocks   [n][k/32][18] bytes, 2-byte aligned.
 *   packed   iq4_packed_bytes(n, k) bytes, 256-byte aligned, not overlapping blocks.
 * Packed layout (16-row x 4-block tiles, tile (rt, kq) for rows 16rt..16rt+15 and
 * blocks 4kq..4kq+3, tiles ordered rt-major):
 *   nibble plane: tile at (rt*(k/128) + kq) * 1024 bytes; 64 entries of 16 bytes;
 *     entry l = 16g + j (g = 0..3, j = 0..15) holds, for blocks b = 0..3 of the tile,
 *     the indices of elements 8g..8g+7 of block (row 16rt+j, block 4kq+b) at bytes
 *     4b..4b+3: element 8g+2i in the low and 8g+2i+1 in the high nibble of byte 4b+i.
 *   scale plane (after n*k/32*16 bytes of nibbles): tile at (rt*(k/128)+kq)*128 bytes;
 *     row j's four scales (binary16) at bytes 8j..8j+7.
 * Errors: IQ4_E_UNSUPPORTED (n % 16, k % 128), IQ4_E_ALIGN.
 */
int iq4_pack_weights(const void* blocks, int64_t n, int64_t k, void* packed, void* stream);

/*
 * Workspace bytes iq4_qmv_multi and iq4_qmv_q8 need for an n x k matrix (written to
 * *bytes; 0 when the shape is covered without splitting K over workgroups).  Depends on
 * n and k only.
 */
int iq4_qmv_workspace_size(int64_t n, int64_t k, size_t* bytes);

/*
 * T-column quantised matrix-vector product (the verify window's dense product):
 *   Y[t][r] = sum_k W[r][k] * X[t][k],  t < T,  r < n,
 * fp32 activations, fp32 result.  Page 1 (Strata commit "wire multi-token kernels
 * into Verifier and MtpDrafter CUDA graphs", verify.hpp header): T tokens read the
 * dense weights once, and each token's column is the single-token result bit for bit.
 * This call guarantees that: column t of a T-column call is bitwise equal to a 1-column
 * call on X[t] (same n, k), for every T, and results are run-to-run deterministic.
 *   packed     W in the packed layout (iq4_pack_weights), 256-byte aligned.
 *   x          [T][ldx] float32, 16-byte aligned, ldx >= k, ldx % 4 == 0.
 *   y          [T][ldy] float32, ldy >= n.
 *   T          1..8.
 *   workspace  >= iq4_qmv_workspace_size(n, k) bytes, 256-byte aligned (may be NULL
 *              when that size is 0).  It must be zero-filled before its first use;
 *              each call leaves it ready for the next one (its arrival counters back
 *              at zero).  Calls that overlap in time must not share a workspace.
 * Errors: IQ4_E_ARG (T, ldx, ldy), IQ4_E_UNSUPPORTED (n % 16, k % 128),
 * IQ4_E_ALIGN, IQ4_E_WORKSPACE.
 */
int iq4_qmv_multi(const void* packed, int64_t n, int64_t k, const float* x, int64_t ldx,
                  int32_t T, float* y, int64_t ldy, void* workspace, size_t ws_bytes,
                  void* stream);

/*
 * iq4_qmv_multi for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * without the workspace, the same results (bitwise: each column equals iq4_qmv_multi's
 * and the 1-column call's), the same errors.  The split-K scratch that iq4_qmv_multi
 * takes from a workspace (needed only when k > 4096) comes instead from a device array
 * inside the library, IQ4_QMV_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.
 *   - Nothing is allocated or freed in any call.
 *   - A shape whose iq4_qmv_workspace_size exceeds IQ4_QMV_NOALLOC_SCRATCH_BYTES is
 *     rejected with IQ4_E_WORKSPACE before anything is enqueued.
 *   - `stream` must belong to the current device.  The first call on a device looks up
 *     the array's address there and clears the array with a fill kernel on `stream`
 *     (make that first call outside graph capture; later calls may be captured).
 *   - All calls on one GPU share that GPU's array: calls that overlap in time on one GPU
 *     (different streams, or graphs replayed concurrently) race and give wrong results.
 *     Calls in one stream order are safe; each leaves the array ready for the next.
 * Errors: as iq4_qmv_multi; IQ4_E_WORKSPACE for a shape above the array's size;
 * IQ4_E_HIP if the array's address cannot be found.
 */
#define IQ4_QMV_NOALLOC_SCRATCH_BYTES (4u << 20)
int iq4_qmv_multi_noalloc(const void* packed, int64_t n, int64_t k, const float* x, int64_t ldx,
                          int32_t T, float* y, int64_t ldy, void* stream);

/*
 * 8-bit block quantisation of fp32 activations (the activation side of page 1's
 * decode products: its verify.hpp keeps the window's T activation columns as q8_1
 * blocks; the pages name that format without printing it).  Per column t and block of
 * 32 consecutive k:
 *   d = f32(absmax) / 127 and r = 1 / d (IEEE binary32 divisions; r = 0 when d rounds
 *   to a zero binary16), q_i = nearest integer of f32(x_i * r), halves away from zero,
 *   clamped to [-127, 127];  stored: q (int8) and d rounded to binary16.
 * The format's sum field (needed only by zero-offset weight formats) is not produced.
 *   x   [T][ldx] float32, 16-byte aligned, ldx >= k, ldx % 4 == 0, finite values.
 *   q   [T][k] int8 (row stride k), 8-byte aligned.
 *   d   [T][k/32] binary16 (row stride k/32), 2-byte aligned.
 *   T >= 0 (0: no-op), k > 0, k % 32 == 0.
 * Bit-exact: the codes and scales are a function of x alone.
 * Errors: IQ4_E_ARG (sizes, ldx, null pointer), IQ4_E_ALIGN.
 */
int iq4_quantize_q8_1(const float* x, int64_t T, int64_t k, int64_t ldx, int8_t* q, uint16_t* d,
                      void* stream);

/*
 * T-column quantised matrix-vector product on 8-bit activations (page 1's decode
 * numerics; page 2's interleaved-matvec commit messages describe its integer block
 * dots):
 *   Y[t][r] = sum_b dw[r][b] * dx[t][b] * sum_i c[qw[r][32b+i]] * q[t][32b+i],
 * each block's dot an exact integer, scaled by the exact product of the two binary16
 * scales with one fp32 fused multiply-add, fp32 result.  Column t of a T-column call is
 * bitwise equal to a 1-column call on column t; results are deterministic.
 *   packed     W in the packed layout (iq4_pack_weights), 256-byte aligned.
 *   q, d       as iq4_quantize_q8_1 writes them for T columns of this k.
 *   y          [T][ldy] float32, ldy >= n, 4-byte aligned.   T: 1..8.
 *   workspace  as for iq4_qmv_multi (iq4_qmv_workspace_size covers both calls; the
 *              two may share one workspace on one stream).
 * Errors: IQ4_E_ARG (T, ldy, null pointer), IQ4_E_UNSUPPORTED (n % 16, k % 128),
 * IQ4_E_ALIGN, IQ4_E_WORKSPACE.
 */
int iq4_qmv_q8(const void* packed, int64_t n, int64_t k, const int8_t* q, const uint16_t* d, int32_t T,
               float* y, int64_t ldy, void* workspace, size_t ws_bytes, void* stream);

/*
 * Top-k routing from router logits: ids[t] = the top_k experts with the largest
 * logits, in descending logit order, ties to the lower expert id (page 3, DSpark
 * tp2.py: both the TP-2 layout notes and markov_local_argmax resolve ties toward the
 * smaller index); w[t][j] = softmax over the top_k selected logits (binary32 math).
 *   logits   [n_tok][n_expert] float32.   ids [n_tok][top_k] int32.
 *   w        [n_tok][top_k] float32.      1 <= top_k <= min(n_expert, 16), n_expert <= 1024.
 * Errors: IQ4_E_ARG.
 */
int iq4_route_topk(const float* logits, int64_t n_tok, int32_t n_expert, int32_t top_k,
                   int32_t* ids, float* w, void* stream);

/*
 * Token gather of routed pairs (pair p = t*top_k + j).  Bit-exact:
 *   counts[e]    number of pairs routed to expert e                  [n_expert]
 *   offsets[e]   exclusive prefix sum of counts                      [n_expert+1]
 *   pairs[i]     pair ids grouped by expert, ascending within one    [n_pairs]
 *   slot_row[p]  position of pair p in `pairs`                       [n_pairs]
 * This is the per-expert count / start / token list of page 1's expert plan block.
 * ids must lie in [0, n_expert) (not checked on the device).  n_pairs <= 2^24,
 * n_expert <= 1024.  Errors: IQ4_E_ARG.
 */
int iq4_moe_gather(const int32_t* ids, int64_t n_pairs, int32_t n_expert, int32_t* counts,
                   int32_t* offsets, int32_t* pairs, int32_t* slot_row, void* stream);

/*
 * Workspace bytes needed by iq4_moe_expert_gemm for these sizes (written to *bytes).
 */
int iq4_moe_workspace_size(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                           int64_t inter, int32_t act_dtype, size_t* bytes);

/*
 * Where a call with IQ4_MOE_KEEP_INTERMEDIATE leaves its intermediate results in the
 * workspace (byte offsets, written to layout[0 .. IQ4_MOE_LAYOUT_N - 1]), and how large
 * that workspace must be (layout[IQ4_MOE_LAYOUT_TOTAL]; it exceeds
 * iq4_moe_workspace_size by the g and u regions).  Page 1 (verify.hpp, PoolMultiFn)
 * defines the layer's per-slot rows (n_tok * k, n_embd) and the expert plan (per-expert
 * count, start and token list); they are kept here as:
 *   COUNTS, OFFSETS, PAIRS, SLOT_ROW  the gather (int32), as iq4_moe_gather writes it;
 *   G, U      g = Wg_e x_t and u = Wu_e x_t, float32 [P][inter], P = n_tok * top_k,
 *             in pair-sorted order: row i belongs to pair PAIRS[i] (p = t * top_k + j);
 *   H         h = silu(g) * u in the same order: binary16 (IQ4_F16) or float32 (IQ4_F32);
 *   ROWS      the per-slot rows w[t][j] * (Wd_e h), [P][hidden], row p = pair p
 *             (token-major: the (n_tok * top_k, hidden) layout): float32 (IQ4_F32) or
 *             binary16 (IQ4_F16: the fp32 product rounded to nearest even); not written
 *             by a call with IQ4_MOE_ATOMIC_COMBINE.
 * shared != 0: the layout of iq4_moe_expert_gemm_shared, whose pairs include the shared
 * expert as slot top_k of every token (P = n_tok * (top_k + 1)).
 * Errors: IQ4_E_ARG (sizes as for the calls).
 */
#define IQ4_MOE_LAYOUT_TOTAL 0
#define IQ4_MOE_LAYOUT_COUNTS 1
#define IQ4_MOE_LAYOUT_OFFSETS 2
#define IQ4_MOE_LAYOUT_PAIRS 3
#define IQ4_MOE_LAYOUT_SLOT_ROW 4
#define IQ4_MOE_LAYOUT_H 5
#define IQ4_MOE_LAYOUT_ROWS 6
#define IQ4_MOE_LAYOUT_G 7
#define IQ4_MOE_LAYOUT_U 8
#define IQ4_MOE_LAYOUT_N 9
int iq4_moe_intermediate_layout(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                                int64_t inter, int32_t act_dtype, int32_t shared, int64_t* layout);

/*
 * Mixture-of-experts FFN over routed tokens (SwiGLU experts, gate-weighted sum):
 *   for token t, slot j, e = ids[t][j]:  g = Wg_e x_t, u = Wu_e x_t,
 *   h = silu(g) * u,  y_tj = Wd_e h,  out[t] = sum_j w[t][j] * y_tj (added in j order).
 * Page 1 (verify.hpp, PoolMultiFn): x (n_tok, n_embd) and ids (n_tok, k) give
 * per-slot rows (n_tok*k, n_embd) that are then summed per token.
 *   x           [n_tok][ldx] activations: IQ4_F32 (decode path, meant for a few
 *               tokens, any n_tok accepted: every product in fp32 through the grouped
 *               T-column matvec, an expert's columns 4 at a time; hidden and inter
 *               <= 4096) or IQ4_F16 (prefill path:
 *               grouped GEMM on the matrix cores, weights decoded to f16, fp32
 *               accumulation, h rounded to f16 for the down product, each slot row
 *               w[t][j] * y_tj rounded to f16 and the rows summed in fp32).
 *   ids, w      [n_tok][top_k] int32 / float32 (ids in [0, n_expert), not checked);
 *               1 <= top_k <= min(n_expert, 16), n_expert <= 1024.
 *   w_gate, w_up  n_expert packed inter x hidden matrices, expert e at
 *               e * iq4_packed_bytes(inter, hidden) bytes.
 *   w_down      n_expert packed hidden x inter matrices, expert e at
 *               e * iq4_packed_bytes(hidden, inter).
 *   out         [n_tok][ldo] float32, overwritten.
 *   workspace   >= iq4_moe_workspace_size(...) bytes, 256-byte aligned.  A prefill
 *               call, or a decode call with more than 64 routed pairs, leaves the
 *               gather (counts, offsets, pairs, slot_row) at its start; a decode call
 *               with at most 64 pairs runs no gather (its matvecs find each expert's
 *               pairs from ids) and leaves that region unspecified.
 *   flags       0 (deterministic), IQ4_MOE_ATOMIC_COMBINE (prefill only), and/or
 *               IQ4_MOE_KEEP_INTERMEDIATE (the workspace must then hold
 *               iq4_moe_intermediate_layout's total; the result is unchanged).
 * Errors: IQ4_E_ARG, IQ4_E_ALIGN, IQ4_E_UNSUPPORTED (hidden or inter not multiples of
 * 256 / 128), IQ4_E_WORKSPACE.
 */
int iq4_moe_expert_gemm(const void* x, int32_t act_dtype, int64_t n_tok, int64_t ldx,
                        const int32_t* ids, const float* w, int32_t top_k, int32_t n_expert,
                        int64_t hidden, int64_t inter, const void* w_gate, const void* w_up,
                        const void* w_down, float* out, int64_t ldo, void* workspace,
                        size_t ws_bytes, uint32_t flags, void* stream);

/*
 * Workspace bytes needed by iq4_moe_expert_gemm_shared for these sizes (written to *bytes).
 */
int iq4_moe_shared_workspace_size(int64_t n_tok, int32_t top_k, int32_t n_expert, int64_t hidden,
                                  int64_t inter, int32_t act_dtype, size_t* bytes);

/*
 * iq4_moe_expert_gemm plus a shared expert that every token passes through:
 *   out[t] = (sum_j w[t][j] * y_tj) + ys_t,  ys_t = Ws_down (silu(Ws_gate x_t) * Ws_up x_t):
 * the routed rows in slot order, then the shared expert's row.  Page 3 (the DSpark
 * drafter file, its cooperative decode with the shared expert) adds the shared
 * expert's output with weight 1 after the routed sum, in the same pass.  Here it is
 * routed as one more expert (index n_expert, slot top_k of every token, gate weight 1)
 * through the same products and the same ordered combine, so each token's row is
 * bitwise the routed call's result on a bank extended by the shared expert with that
 * routing.
 *   s_gate, s_up  packed inter x hidden matrices;  s_down  packed hidden x inter
 *               (256-byte aligned, the routed experts' sizes).
 *   workspace   >= iq4_moe_shared_workspace_size(...) bytes, 256-byte aligned.  Its
 *               gather (when one runs) is that of the extended routing.
 *   Other arguments, flags and errors as iq4_moe_expert_gemm, with top_k <=
 *   min(n_expert, 15) and n_expert <= 1023 (the extended routing within the limits).
 */
int iq4_moe_expert_gemm_shared(const void* x, int32_t act_dtype, int64_t n_tok, int64_t ldx,
                               const int32_t* ids, const float* w, int32_t top_k, int32_t n_expert,
                               int64_t hidden, int64_t inter, const void* w_gate, const void* w_up,
                               const void* w_down, const void* s_gate, const void* s_up,
                               const void* s_down, float* out, int64_t ldo, void* workspace,
                               size_t ws_bytes, uint32_t flags, void* stream);

/*
 * Dense dequant-fused GEMM over a prompt in chunks of `chunk` rows:
 *   Y[m][r] = sum_k X[m][k] * W[r][k]  (X f16, W decoded to f16, fp32 accumulation),
 * one launch per chunk of `chunk` consecutive rows of X (the last chunk may be short),
 * each launch decoding the weights again -- page 2 (pull request "sm_80 (GA100)
 * tuning"), wide-dequant commit: the prompt path decodes the dense weights for every
 * chunk; here the decode is fused into the product instead of a separate pass.
 * Results do not depend on `chunk` (bitwise).
 *   packed  W (n x k) in the packed layout.   x [m][ldx] binary16, ldx % 8 == 0.
 *   y       [m][ldy] float32.                  chunk >= 1 (0 means one launch).
 * Errors: IQ4_E_ARG, IQ4_E_ALIGN, IQ4_E_UNSUPPORTED (n % 16, k % 128).
 */
int iq4_qgemm(const void* packed, int64_t n, int64_t k, const void* x, int64_t m, int64_t ldx,
              float* y, int64_t ldy, int64_t chunk, void* stream);

/* ---------------------------------------------------------------------------------
 * IQ4_XS super-blocks.  Page 2 (pull request "sm_80 (GA100) tuning") names this dense
 * weight format in its wide-dequant commit message (decoded every prompt chunk), times
 * its matvec in the MMVQ-IL harness commit message, and gives its block dot in the
 * MMVQ-IL_PF commit message: the integer sum times the float of (ls - 32).  The bytes
 * follow the format's public definition (the pages never print them):
 *   256 weights in 136 bytes: d (binary16, bytes 0-1); a 16-bit word (bytes 2-3) whose
 *   bits 2i, 2i+1 are the high two bits of sub-block i's 6-bit code ls_i; the low four
 *   bits of ls_i in bytes 4 + i/2 (low nibble for even i); bytes 8 + 16i + m (m < 16)
 *   hold the indices of elements 32i + m (low nibble) and 32i + 16 + m (high nibble);
 *   w = d * (ls_i - 32) * codebook[q], exact in binary32.
 * A matrix is stored row-major as n rows of k/256 super-blocks, as given (no repack).
 */

/* Bytes of an n x k super-block matrix (n * k/256 * 136), or -1 if n < 1, k < 1 or
 * k % 256 != 0. */
int64_t iq4_xs_bytes(int64_t n, int64_t k);

/*
 * Decode super-blocks: out[s][j] = d_s * (ls_{s, j/32} - 32) * codebook[q_{s,j}], in
 * super-block order.
 *   sb    [n_superblocks][136] bytes, 8-byte aligned.
 *   out   [n_superblocks][256] of out_dtype: IQ4_F32 (exact) or IQ4_F16 (the exact
 *         value rounded to nearest even, subnormals kept, overflow to inf); 16-byte
 *         aligned.
 * Bitwise equal to the host decode (the same rule as iq4_dequant_blocks).
 * Errors: IQ4_E_ARG (n_superblocks < 0, bad dtype, null pointer), IQ4_E_ALIGN.
 */
int iq4_xs_dequant(const void* sb, int64_t n_superblocks, int32_t out_dtype, void* out, void* stream);

/*
 * T-column matvec on super-block weights: Y[t][r] = sum_k W[r][k] * X[t][k], t < T --
 * the verify-window product of page 1 (commit "wire multi-token kernels into Verifier
 * and MtpDrafter CUDA graphs", verify.hpp: the dense weights read once for T tokens)
 * on the format above.  fp32 activations, exact decoded weights, fp32 accumulation.
 * Column t of a call equals the T = 1 call on column t bit for bit.
 *   w     n x k super-block matrix (iq4_xs_bytes(n, k) bytes), 8-byte aligned.
 *   x     [T][ldx] float32, 16-byte aligned, ldx >= k, ldx % 4 == 0.
 *   y     [T][ldy] float32 (written, never read), ldy >= n.
 *   1 <= T <= 8; n >= 1; k >= 256, k % 256 == 0, k <= 2^20.  No workspace.
 * Errors: IQ4_E_ARG (T range, null pointer, ldx/ldy), IQ4_E_ALIGN, IQ4_E_UNSUPPORTED
 * (k % 256, sizes).
 */
int iq4_xs_qmv_multi(const void* w, int64_t n, int64_t k, const float* x, int64_t ldx, int32_t T,
                     float* y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IQ4_H */
