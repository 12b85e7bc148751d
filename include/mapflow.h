/*
 * libmapflow -- MapFlow attention-map compression and fused head-mapped
 * retrieval, native on AMD Instinct MI355X (gfx950).
 *
 * MapFlow ("Accelerating Cross-Model LLM Inference via Attention Map Reuse",
 * montaan.com/papers/2610.14688; PKU-DAIR article aitest123.com/news/zaoi86)
 * lets a receiver model reuse a sender model's attention maps.  The sender's
 * causal maps are compressed by block-level Top-p into Block Sparse Row form
 * (paper page, "Practical Implementation Details" and highlight 3; article,
 * third section, first component: block statistics first, then the choice of
 * blocks).  For each reuse receiver layer a fused kernel reads only the kept
 * blocks, mixes the sender heads into each receiver head with the learned
 * linear head map W, and multiplies by the receiver's own values, producing
 * the attention output with no dense receiver map in memory (paper page,
 * "MapFlow System Design" item 3 and highlight 4; article, third component).
 *
 * Notation: N tokens, block size B, T = ceil(N/B); H_s sender heads; H_r
 * receiver heads; H_kv receiver KV heads, G = H_r / H_kv, receiver head r
 * reads KV head r / G; d head dimension.
 *
 * Conventions for every entry point
 *  - Pointers marked "device" are device memory owned by the caller; the
 *    library never allocates, frees or retains them.  Pointers marked "host"
 *    are host memory.
 *  - Every call validates its arguments on the host before any GPU work and
 *    returns a status; it never aborts or throws across the boundary.  On a
 *    non-OK status mf_last_error() holds a message (thread-local).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  Buffers must stay alive until the stream has finished.
 *    The only host synchronisation is the one documented at
 *    mf_topp_select_bsr.
 *  - Dtype codes: MF_F32 = 0, MF_F16 = 1, MF_BF16 = 2.
 *  - The library holds no global state besides the thread-local error text
 *    (a Block Manager is an object the caller creates and destroys) and is
 *    safe to call from several host threads on different streams.
 */
#ifndef MAPFLOW_H
#define MAPFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MF_ABI_VERSION 7

typedef enum {
  MF_OK = 0,
  MF_ERR_INVALID = 1,     /* bad argument (null pointer, size, dtype, p, stride) */
  MF_ERR_UNSUPPORTED = 2, /* valid arguments, combination not built */
  MF_ERR_CAPACITY = 3,    /* BSR output larger than the caller's capacity */
  MF_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} mf_status;

typedef enum { MF_F32 = 0, MF_F16 = 1, MF_BF16 = 2 } mf_dtype;

/* Returns MF_ABI_VERSION of the built library. */
int mf_abi_version(void);

/* Static text for a status code (never NULL). */
const char* mf_status_string(int status);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* mf_last_error(void);

/*
 * Block mass -- the compressor's block statistic (article, third section,
 * first component; paper page, highlight 3).
 *
 *   mass[I][J] = (1/H_s) * sum_h sum_{i in block I, i<N} sum_{j in block J, j<N} A[h][i][j]
 *
 * for the causal blocks J <= I; entries with J > I are written as 0.
 *
 *  A     device, [H_s][N][N] row-major, dtype `dtype`: the sender layer's
 *        causal attention maps (rows sum to 1; entries above the diagonal are
 *        expected to be 0 but are read and summed as given inside the
 *        diagonal blocks).  Only the causal block tiles are read.
 *  mass  device, [T][T] float32, written completely.
 *  The per-block sum is formed with fp32 partial sums of at most 8
 *  consecutive elements combined in fp64, then rounded once to fp32.
 *  Alignment: A needs only its element alignment.  Rows of N*e bytes that
 *  are not a multiple of 16 (ragged N, or A off a 16-byte boundary) are read
 *  with 16-byte loads aligned to the element size, which the HSA target's
 *  unaligned global access allows; rows shorter than 16 bytes use narrower
 *  loads.
 *  Errors: MF_ERR_INVALID for a null pointer, N < 1, B not in
 *  {16,32,64,128}, H_s not in [1,64] or an unknown dtype.
 */
int mf_block_mass(const void* A, int dtype, int H_s, int N, int B,
                  float* mass, void* stream);

/* Workspace bytes of mf_block_mass_ws: H_s * T(T+1)/2 float32 (0 for bad sizes). */
size_t mf_block_mass_ws_bytes(int H_s, int N, int B);

/*
 * The same block masses as mf_block_mass (same statistic, same masses up to
 * the order of the fp64 additions; bit-reproducible run to run), computed by
 * streaming whole map rows: one workgroup per (head, block row) reads the
 * causal part of that block row's rows as contiguous runs and leaves its
 * per-tile sums, rounded once to fp32, in `workspace`; a second kernel adds
 * the heads in a fixed order in fp64 and divides by H_s.  Faster than the
 * column-strip scan of mf_block_mass, at the price of a caller-owned device
 * workspace of at least mf_block_mass_ws_bytes(H_s, N, B) bytes (overwritten).
 *  Errors: those of mf_block_mass, plus MF_ERR_INVALID for a null or short
 *  workspace.
 */
int mf_block_mass_ws(const void* A, int dtype, int H_s, int N, int B, float* mass,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mf_topp_select_bsr needs for (N, B). */
size_t mf_topp_workspace_bytes(int N, int B);

/*
 * Block-level Top-p selection and BSR build (paper page, highlight 3 and
 * "Practical Implementation Details"; article, third section, first and
 * second components).
 *
 * For each block row I, the candidates J = 0..I are ordered by decreasing
 * mass[I][J] (equal fp32 masses: lower J first) and kept until the running
 * sum, accumulated in fp64 in that order, first reaches p * total, where
 * total is the fp64 sum of mass[I][0..I] in column order; the block that
 * reaches it is kept.  p == 1 keeps every causal block.  The kept columns of
 * each row are stored in ascending order.
 *
 *  mass      device, [T][T] float32 from mf_block_mass.
 *  A         device, the same [H_s][N][N] map (source of the kept tiles).
 *  p         Top-p threshold, 0 < p <= 1.
 *  row_ptr   device, [T+1] int32, written: row_ptr[0] = 0,
 *            row_ptr[I+1] - row_ptr[I] = blocks kept in row I, row_ptr[T] = nnzb.
 *  col_idx   device, [cap_nnzb] int32, written for k < nnzb.
 *  vals      device, [cap_nnzb][H_s][B][B] of `dtype`, written for k < nnzb:
 *            vals[k][h][i][c] = A[h][I*B+i][J*B+c] copied bit for bit, 0 where
 *            I*B+i >= N or J*B+c >= N.
 *  cap_nnzb  capacity of col_idx/vals in blocks (>= 0).
 *  nnzb_out  host, may be NULL.  If non-NULL the call synchronises `stream`
 *            after enqueueing its work, stores nnzb there, and returns
 *            MF_ERR_CAPACITY if nnzb > cap_nnzb.  If NULL the call does not
 *            synchronise; read row_ptr[T] to learn nnzb.
 *  workspace device, >= mf_topp_workspace_bytes(N, B) bytes of scratch.
 *  When nnzb > cap_nnzb the kernels leave col_idx and vals untouched; row_ptr
 *  is always valid, so the caller can reallocate and call again.
 *  Errors: MF_ERR_INVALID for null pointers, bad N/B/H_s/dtype, p NaN or
 *  outside (0, 1], cap_nnzb < 0 or a workspace that is too small;
 *  MF_ERR_UNSUPPORTED if T > 4096; MF_ERR_CAPACITY as above.
 */
int mf_topp_select_bsr(const float* mass, const void* A, int dtype, int H_s,
                       int N, int B, float p, int32_t* row_ptr,
                       int32_t* col_idx, void* vals, int64_t cap_nnzb,
                       int64_t* nnzb_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * mf_topp_select_bsr for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Computes exactly what mf_topp_select_bsr(..., nnzb_out = NULL,
 * ...) computes (same kernels, bitwise the same row_ptr, col_idx and vals),
 * with the selection's scratch taken from a fixed device array inside the
 * library instead of a caller workspace.  It allocates nothing and does not
 * synchronise: read row_ptr[T] for nnzb; when nnzb > cap_nnzb, col_idx and
 * vals are left untouched, as in mf_topp_select_bsr.
 *  Limit: T = ceil(N/B) <= 1024 block rows (the array holds kept[T][T] and
 *  count[T] int32, 4.2 MB; each GPU the library runs on holds its own copy
 *  until the process ends).  The array's device address is looked up once
 *  per device on the first call there, with that device current; the calling
 *  thread's current device must be the one `stream` runs on.
 *  Every call on one GPU uses the same array: calls that overlap in time on
 *  one GPU (different streams, or different host threads) race and must not
 *  be issued.  Nothing in the array needs clearing between calls (every entry
 *  a call reads, it has written itself first).
 *  Errors: those of mf_topp_select_bsr (no workspace or nnzb_out arguments),
 *  and MF_ERR_UNSUPPORTED when T > 1024.
 */
int mf_topp_select_bsr_noalloc(const float* mass, const void* A, int dtype, int H_s,
                               int N, int B, float p, int32_t* row_ptr,
                               int32_t* col_idx, void* vals, int64_t cap_nnzb,
                               void* stream);

/*
 * Compression without a dense map (article, third section, first component:
 * the block statistics and the kept blocks are obtained without first laying
 * out the complete dense attention matrix).
 *
 * The sender layer's causal attention is the softmax of its scores,
 *   s_h[i][j] = scale[h] * (q_h,i . k_h,j),   j <= i,
 *   A[h][i][j] = exp(s_h[i][j] - lse[h][i]),  lse[h][i] = log sum_{j<=i} exp(s_h[i][j]),
 * with Q = [H_s][N][d] and K = [H_ks][N][d] (contiguous rows of d elements,
 * dtype `dtype`); sender head h reads K head h / (H_s / H_ks).  lse is the
 * per-row statistic an attention forward keeps; mf_row_lse computes it when
 * the caller does not have it.  The three calls below give the same block
 * masses and kept tiles as mf_block_mass / mf_topp_select_bsr on that map,
 * computed from Q, K, scale and lse; A is never formed.  Scores are
 * accumulated in fp32 from the stored Q and K; exponentials are fp32.
 *
 * Common arguments: Q, K device; scale device, [H_s] float32; lse device,
 * [H_s][N] float32; d in {64, 128}; H_ks >= 1 dividing H_s.  Errors:
 * MF_ERR_INVALID for null pointers, N < 1, B not in {16,32,64,128}, H_s not
 * in [1,64], H_ks not dividing H_s, d not in {64,128} or an unknown dtype.
 */

/* lse[h][i] for every sender head and row (device, [H_s][N] float32). */
int mf_row_lse(const void* Q, const void* K, int dtype, int H_s, int H_ks, int N, int d,
               const float* scale, float* lse, void* stream);

/* Workspace bytes mf_block_mass_qk needs: per-head partial sums over 16-row
 * tiles, H_s * ceil(N/16) * T float32. */
size_t mf_block_mass_qk_workspace_bytes(int H_s, int N, int B);

/*
 *   mass[I][J] = (1/H_s) * sum_h sum_{i in I, i<N} sum_{j in J, j<=i} exp(s_h[i][j] - lse[h][i])
 * for J <= I, 0 for J > I (device, [T][T] float32, written completely).  Each
 * head's sum over a 16-row tile and a column block is an fp32 sum; the tiles
 * and heads of a block are combined in fp64 in a fixed order, so the result
 * is bit-reproducible.  workspace: device, >= mf_block_mass_qk_workspace_bytes.
 */
int mf_block_mass_qk(const void* Q, const void* K, const float* scale, const float* lse,
                     int dtype, int H_s, int H_ks, int N, int d, int B, float* mass,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mf_lse_block_mass_qk needs: H_s * B * T(T+1)/2 pairs of
 * float32 (one per row and causal column block) and H_s * T(T+1)/2 float32
 * per-head block sums, or the workspace of mf_block_mass_qk where that is
 * larger. */
size_t mf_lse_block_mass_qk_workspace_bytes(int H_s, int N, int B);

/*
 * mf_row_lse and mf_block_mass_qk in one pass over the scores: lse (device,
 * [H_s][N] float32) and mass (device, [T][T] float32, written completely) as
 * those two calls define them.  While the online maximum and sum of a row run
 * over its keys, the pass also keeps, for each causal column block J, the
 * block's sum e = sum_{j in J} exp(s - m) relative to the row's running
 * maximum m after the block; then
 *   mass[I][J] = (1/H_s) * sum_h sum_{i in I} e_h[i][J] * exp(m_h[i][J] - lse[h][i]):
 * each head's terms over a block row are added in fp32 in a fixed tree order,
 * the heads in fp64 in a fixed order (bit-reproducible).  Each (m, e) pair is
 * an fp32 pair; the result agrees with mf_block_mass_qk's direct sums to
 * fp32 rounding.  The scores are computed once instead of twice.  fp32 inputs
 * and B = 16 take the two separate passes.  workspace: device, >=
 * mf_lse_block_mass_qk_workspace_bytes.  Errors as mf_block_mass_qk.
 */
int mf_lse_block_mass_qk(const void* Q, const void* K, const float* scale, int dtype, int H_s,
                         int H_ks, int N, int d, int B, float* lse, float* mass,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-level Top-p selection and BSR build as mf_topp_select_bsr (same rule,
 * same row_ptr / col_idx / capacity / nnzb_out / workspace contract), with
 * the kept tiles recomputed instead of copied:
 *   vals[k][h][i][c] = exp(s_h[I*B+i][J*B+c] - lse[h][I*B+i]) rounded once to
 *   `dtype` (round to nearest even) for J*B+c <= I*B+i < N, and 0 elsewhere;
 *   values below 2^-126 may be stored as 0.
 */
int mf_topp_select_bsr_qk(const float* mass, const void* Q, const void* K,
                          const float* scale, const float* lse, int dtype, int H_s,
                          int H_ks, int N, int d, int B, float p, int32_t* row_ptr,
                          int32_t* col_idx, void* vals, int64_t cap_nnzb,
                          int64_t* nnzb_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes mf_retrieve_fused needs for (N, B, H_kv, d, dtype).  The
 * current kernels need none and return 0 for every configuration; the
 * argument pair stays in mf_retrieve_fused so that a kernel which does need
 * scratch can be added without changing the boundary. */
size_t mf_retrieve_workspace_bytes(int N, int B, int H_kv, int d, int dtype);

/*
 * Workspace bytes that let mf_retrieve_fused split long block rows (article,
 * third section, second component: different layers and positions keep
 * different numbers of blocks, so a few long rows can set the time of a
 * launch).  With a workspace of at least this size, a launch whose average
 * row is longer than half of one CU's share of the work cuts every row of
 * more than P = ceil(nnzb * B/16 / CUs) kept blocks into parts of at most P
 * blocks, runs the parts as separate work items (rows from the last to the
 * first) and adds each split row's fp32 partial outputs in part order in a
 * second kernel, so the output is bitwise the same on every run.  It is
 * still the sum of the same products, not bitwise the unsplit output.  Returns
 * 0 when splitting does not apply to these shapes (they take the matrix-core
 * kernel with pair stages only: fp16/bf16, d = 128, B >= 32, H_s <= 40, H_r in
 * {8,16,24,32}), for nnzb <= 0 or for invalid arguments.  The size grows
 * with nnzb: (T + nnzb/P) items x B rows x H_r x 128 fp32, plus 4*T bytes.
 */
size_t mf_retrieve_split_workspace_bytes(int64_t nnzb, int dtype, int H_s, int N, int B, int H_r,
                                         int H_kv, int d);

/*
 * Which retrieval kernel mf_retrieve_fused runs for these arguments (host
 * only, no GPU work; the three pointers are inspected for alignment only and
 * may be any address with the alignment the real buffers will have).
 *  Returns 1 for the matrix-core kernel (MF_F16/MF_BF16, d = 128, B in
 *  {16,32,64,128}, H_s <= 48, H_r in {8,16,24,32} with each group of H_r/8
 *  consecutive receiver heads inside one KV head, vals and O 16-byte aligned,
 *  ldO % 8 == 0, V 16-byte aligned with ldV % 8 == 0), 0 for the plain kernel,
 *  and -MF_ERR_INVALID when mf_retrieve_fused would reject the shapes.
 */
int mf_retrieve_kernel(int dtype, int H_s, int N, int B, int H_r, int H_kv, int d,
                       const void* vals, const void* V, int64_t ldV, const void* O,
                       int64_t ldO);

/*
 * Fused head-mapped BSR retrieval (paper page, "MapFlow System Design" item 3,
 * highlights 2 and 4; article, second section and third component).
 *
 * For every kept block k = (I, J) and receiver head r:
 *   Ahat_k[r] = sum_s W[r][s] * vals[k][s]                       (B x B, on chip)
 *   O[I*B+i][r][:] += sum_c Ahat_k[r][i][c] * V[J*B+c][r/G][:]
 * accumulated in fp32 over the row's kept blocks; O is written once, rounded
 * to `dtype` with round-to-nearest-even.  Ahat is never written to memory.
 * Rows with no kept block get O = 0.
 *
 *  row_ptr, col_idx, vals  device, the BSR state from mf_topp_select_bsr
 *            (or any BSR of the same layout: row_ptr monotone from 0, col_idx
 *            in [0, T)); `nnzb` is the number of blocks in vals.  Blocks with
 *            a column outside [0, T) and indices k outside [0, nnzb) are
 *            skipped: they contribute nothing to O.  Tile positions of key
 *            columns at or beyond N (the padding of a partial last block)
 *            contribute nothing either, whatever they hold (NaN included).
 *            Tile values that are used must be finite.
 *  W         device, [H_r][H_s] float32, row-major.
 *  V         device, rows of H_kv*d elements of `dtype` at stride ldV
 *            elements (ldV >= H_kv*d, so V may be a slice of a fused QKV
 *            tensor): V[n][g][e] at V[n*ldV + g*d + e], n < N.
 *  O         device, O[n][r][e] at O[n*ldO + r*d + e], ldO >= H_r*d.
 *  workspace device scratch of >= mf_retrieve_workspace_bytes(...) bytes
 *            (NULL when that is 0, as it is for every current kernel).  A
 *            workspace of >= mf_retrieve_split_workspace_bytes(...) bytes
 *            turns on the splitting of long block rows described there; its
 *            contents need no initialisation.
 *  Precision: MF_F32 runs in fp32 throughout.  MF_BF16: the head mix runs on
 *  bf16 matrix cores with W split into two bf16 halves (W enters exactly) and
 *  fp32 accumulation; the fp32 mixed map is split the same way into hi + lo
 *  bf16 parts, each multiplied with V as stored on bf16 matrix cores with
 *  fp32 accumulation.  MF_F16: W and the mixed map are rounded to fp16 and
 *  multiplied on fp16 matrix cores with fp32 accumulation.
 *  Errors: MF_ERR_INVALID for null pointers, N < 1, nnzb < 0, bad B, d not
 *  in {64,128}, H_s/H_r not in [1,64], H_kv < 1, H_r % H_kv != 0, ldV or ldO
 *  too small, a missing or short workspace, unknown dtype.
 */
int mf_retrieve_fused(const int32_t* row_ptr, const int32_t* col_idx,
                      const void* vals, int64_t nnzb, int dtype, int H_s,
                      int N, int B, const float* W, int H_r, const void* V,
                      int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One sender state, several receivers (the pages serve several downstream
 * models from one sender's cached maps: article, second section, and its
 * three-model experiment).  Computes, for each receiver i, exactly what
 * mf_retrieve_fused(row_ptr, col_idx, vals, nnzb, dtype, H_s, N, B, W[i],
 * H_r[i], V[i], H_kv[i], d, ldV[i], O[i], ldO[i]) computes (outputs are bitwise
 * identical), in one launch when every receiver takes the matrix-core kernel:
 * the work items of the receivers for one (block row, 16-row slice) run
 * together on one XCD, so the row's tiles leave HBM once for all receivers.
 * Otherwise it runs one launch per receiver.
 *
 *  n_recv       host, number of receivers, 1..4.
 *  W, V, O      host arrays of n_recv device pointers (layouts as in
 *               mf_retrieve_fused); the O buffers must not overlap.
 *  H_r, H_kv, ldV, ldO   host arrays of n_recv entries.
 *  The BSR state, dtype, H_s, N, B and d are shared by all receivers.
 *  Errors: MF_ERR_INVALID for n_recv outside [1, 4], a null array or
 *  pointer, two receivers with the same O, and every check of
 *  mf_retrieve_fused on any receiver (the message names the receiver).
 */
int mf_retrieve_fused_multi(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                            int64_t nnzb, int dtype, int H_s, int N, int B, int n_recv,
                            const float* const* W, const int* H_r, const void* const* V,
                            const int* H_kv, int d, const int64_t* ldV, void* const* O,
                            const int64_t* ldO, void* stream);

/*
 * Fused retrieval over a packed batch of sequences in one launch (the pages'
 * serving integration runs under chunked prefill and paged KV caches: paper
 * page, "Practical Implementation Details").  For each sequence s it computes
 * exactly what mf_retrieve_fused computes for that sequence alone, with the
 * same kernels and the same arithmetic (outputs are bitwise identical).
 *
 *  S           host, number of sequences, >= 1.
 *  R           host, number of block rows of all sequences (= cu_rows[S]);
 *              it sizes the grid.
 *  cu_seqlens  device, [S+1] int32, nondecreasing from 0: sequence s holds
 *              tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of V and O
 *              (N_s = cu_seqlens[s+1] - cu_seqlens[s] tokens).
 *  cu_rows     device, [S+1] int32, nondecreasing from 0: sequence s owns
 *              global block rows cu_rows[s] .. cu_rows[s+1]-1, with
 *              cu_rows[s+1] - cu_rows[s] = ceil(N_s / B).
 *  row_ptr     device, [R+1] int32, monotone from 0: kept blocks of global
 *              block row g are k = row_ptr[g] .. row_ptr[g+1]-1 (k < nnzb).
 *  col_idx     device, [nnzb] int32: each kept block's column block, local to
 *              its sequence (in [0, ceil(N_s/B))).
 *  block_table device, [nnzb] int32 or NULL: the pool page holding kept block
 *              k's tiles.  NULL means page k (a contiguous pool).
 *  vals        device, the tile pool [n_pages][H_s][B][B] of `dtype`
 *              (n_pages is ignored when block_table is NULL: the pool then
 *              holds nnzb pages).
 *  W, V, O     as in mf_retrieve_fused, with V and O packed by token.
 *  Rows past a sequence's end, columns outside [0, ceil(N_s/B)), pages
 *  outside [0, n_pages) and indices k outside [0, nnzb) are skipped rather
 *  than read, so malformed tables cannot make the kernels read outside the
 *  caller's buffers; the device arrays are not otherwise validated.
 *  Ownership: the caller owns every buffer; nothing is retained after the call.
 *  Errors: MF_ERR_INVALID for S < 1, R < 0, nnzb < 0, n_pages < 0 with a
 *  block table, a null pointer (col_idx and vals may be NULL only when
 *  nnzb == 0; block_table may be NULL), and the dtype, B, H_s, H_r, H_kv, d
 *  and stride checks of mf_retrieve_fused.
 */
int mf_retrieve_fused_varlen(int S, int R, const int32_t* cu_seqlens, const int32_t* cu_rows,
                             const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* block_table, const void* vals, int64_t n_pages,
                             int64_t nnzb, int dtype, int H_s, int B, const float* W, int H_r,
                             const void* V, int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                             void* stream);

/* ------------------------------------------------------------------------
 * Block Manager: the prefix-hash index of cached compressed state (paper
 * page, "Practical Implementation Details": the cache is organised by a Block
 * Manager with a prefix-hash index; article, third section, second component:
 * each index key carries the information of the whole preceding context).
 *
 * Block row I of a sender layer's causal map depends on tokens 0..(I+1)B-1
 * only, so it is cached under the chained hash of exactly that prefix:
 *   h_0 = seed,
 *   h_{c+1} = FNV-1a 64-bit over (h_c as 8 little-endian bytes, then tokens
 *             cB .. cB+B-1 as 4 little-endian bytes each)
 * (FNV-1a: offset basis 14695981039346656037, prime 1099511628211), and block
 * row I of layer l is keyed by (l, h_{I+1}).  Only full chunks of B tokens are
 * cached.  An entry holds the row's kept column blocks and, per kept block,
 * the page of a caller-owned device tile pool [n_pages][H_s][B][B] that holds
 * its tiles.  It also keeps the parent hash and the chunk's tokens: lookups
 * compare both, so a hash collision can only make a row look absent.
 *
 * Pages are handed out smallest index first.  When too few are free, rows
 * that no lookup holds are evicted, least recently used first (a lookup or an
 * insert that meets a row counts as a use).  The manager is host memory only,
 * created and destroyed by the caller; each call takes the manager's mutex,
 * so one manager may be shared by host threads.  Tiles move with
 * mf_pool_store.
 * ---------------------------------------------------------------------- */
typedef struct mf_block_manager mf_block_manager;

/* The prefix hashes h_1 .. h_n of the n = n_tokens / B full chunks.
 *  tokens  host, [n_tokens] int32;  hashes  host, [n] uint64, written.
 *  Errors: MF_ERR_INVALID for B < 1, n_tokens < 0, null pointers. */
int mf_prefix_hashes(const int32_t* tokens, int64_t n_tokens, int B, uint64_t seed,
                     uint64_t* hashes);

/* A manager for block size B, n_layers sender layers and a pool of n_pages
 * tile pages, hashing from `seed` (e.g. one per sender model).  Returns NULL
 * (with mf_last_error set) for B < 1, n_layers < 1 or n_pages outside
 * [0, 2^31-1]. */
mf_block_manager* mf_bm_create(int B, int n_layers, int64_t n_pages, uint64_t seed);

/* Frees the manager (not the pool).  NULL is accepted. */
void mf_bm_destroy(mf_block_manager* m);

/* The longest cached prefix of `tokens` for `layer`, at most max_rows block
 * rows: *n_rows rows, row_ptr[0..*n_rows] (host, from 0), col_idx and pages
 * (host, row_ptr[*n_rows] entries; cap is their capacity).  Every returned
 * row is held (never evicted) until mf_bm_release.
 * Errors: MF_ERR_INVALID for a null manager / n_rows / row_ptr, a layer
 * outside [0, n_layers), negative sizes, cap > 0 with null col_idx / pages;
 * MF_ERR_CAPACITY when the rows hold more than cap blocks (*n_rows is then
 * set and nothing is held). */
int mf_bm_lookup(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                 int max_rows, int* n_rows, int32_t* row_ptr, int32_t* col_idx, int32_t* pages,
                 int64_t cap);

/* Releases the first n_rows rows of `tokens` held by a lookup.
 * Errors: MF_ERR_INVALID when a row is not held (nothing is released then). */
int mf_bm_release(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                  int n_rows);

/* Caches block rows row0 .. row0+n_rows-1 of `tokens` for `layer`: the
 * rows' kept columns as row_ptr[n_rows+1] (host, from 0) and col_idx (host,
 * ascending per row, each <= its row).  pages_out (host, row_ptr[n_rows]
 * entries) receives the pool page assigned to each kept block, or -1 for the
 * blocks of rows already cached; the caller then copies the tiles into those
 * pages (mf_pool_store).  Needs (row0 + n_rows) * B tokens.
 * Errors: MF_ERR_INVALID for bad arguments; MF_ERR_CAPACITY when not enough
 * pages are free or evictable (nothing is inserted or evicted then). */
int mf_bm_insert(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                 int row0, int n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                 int32_t* pages_out);

/* out (host, 7 entries): free pages, cached rows, held rows, row hits, row
 * misses (chunks a lookup asked for and did not get), evictions, inserted rows. */
int mf_bm_stats(mf_block_manager* m, int64_t* out);

/* Device copy of kept tiles into pool pages: pool[pages[k]] = vals[k] for
 * k < nnzb, skipping pages outside [0, n_pages) (e.g. the -1 of rows already
 * cached).  vals [nnzb][H_s][B][B] and pool [n_pages][H_s][B][B] of `dtype`,
 * both 16-byte aligned; pages device int32 [nnzb].
 * Errors: MF_ERR_INVALID for bad dtype / B / H_s, negative sizes, null
 * pointers or misaligned buffers; MF_ERR_HIP for a failed launch. */
int mf_pool_store(const void* vals, int64_t nnzb, const int32_t* pages, void* pool,
                  int64_t n_pages, int dtype, int H_s, int B, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAPFLOW_H */
