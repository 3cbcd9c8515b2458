/*
 * diffqkv.h -- C ABI of the DiffQKV attention library for AMD MI355X (gfx950).
 *
 * DiffQKV attention (the Sigma pages: "Sigma: Differential Rescaling of
 * Query, Key and Value for Efficient Language Models", architecture summary
 * page, sections 3.2 and 3.4, and its "FlexHeadFA Kernel and Deployment
 * Infrastructure" section) lets the Query, Key and Value sides carry their
 * own head counts and head dimensions:
 *
 *   n_q query heads of dimension d_k (the query is already in the key space),
 *   n_k key heads of dimension d_k, n_v value heads of dimension d_v.
 *
 * Query head i reads key head floor(i * n_k / n_q) and value head
 * floor(i * n_v / n_q) (section 3.4 Step 3, GroupSharing; FlexHeadFA's
 * separated address rule).  Its output is
 *
 *   o_i = sum_j softmax_j(scale * q_i . K_j) * V_j,   o_i in R^{d_v}
 *
 * (section 3.4 Steps 4 and 5).  Every entry point that takes `scale` reads
 * scale = 0 as the default 1/sqrt(d_k) (Step 4's divisor) and otherwise
 * requires a positive finite value (DQKV_ERR_SHAPE).
 *
 * Memory layouts (row-major, innermost last; all device memory):
 *   q (decode)   [B][n_q][d_k]
 *   q (prefill)  [B][t_new][n_q][d_k]
 *   k_cache      [B][n_k][l_cap][d_k]    separate key cache  (section 3.2 item 3)
 *   v_cache      [B][n_v][l_cap][d_v]    separate value cache
 *   k_new        [B][t_new][n_k][d_k]    token-major rows to append
 *   v_new        [B][t_new][n_v][d_v]
 *   out (decode) [B][n_q][d_v],  lse (decode)  [B][n_q]         (fp32)
 *   out (prefill)[B][t_new][n_q][d_v], lse      [B][t_new][n_q] (fp32)
 *   ctx_len, pos [B] int32
 *
 * Element type: DQKV_F32 (IEEE float) or DQKV_BF16 (bfloat16 bit patterns) for
 * q, caches, new rows and out; arithmetic is fp32 throughout, bf16 outputs are
 * rounded to nearest even.  lse is the natural-log log-sum-exp of the scaled
 * scores, always fp32, optional (NULL to skip).
 *
 * Supported sizes: 1 <= n_k <= n_q, 1 <= n_v <= n_q, n_q a multiple of n_k
 * and of n_v; d_k, d_v in {32, 64, 128, 256}, d_k = 256 bf16 only (prefill: d_k
 * in {64, 128}, d_v in {64, 128}, bf16 only).  Every device pointer must be
 * 16-byte aligned.
 *
 * Ownership and execution: the caller owns every buffer; the library neither
 * allocates nor frees device memory nor keeps any pointer after returning.
 * Every call only enqueues work on `stream` (a hipStream_t; NULL = the null
 * stream) and never synchronises.  The return value reports host-side
 * argument checks and launch errors (DQKV_ERR_HIP); faults inside a kernel
 * surface at the caller's next synchronisation.  Calls on one stream run in
 * order; calls that share output buffers on different streams race.
 */
#ifndef DIFFQKV_H
#define DIFFQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define DQKV_F32  0
#define DQKV_BF16 1

/* Status codes. */
#define DQKV_OK               0
#define DQKV_ERR_NULL        -1 /* a required pointer is NULL                 */
#define DQKV_ERR_SHAPE       -2 /* head counts / sizes violate the rules above */
#define DQKV_ERR_UNSUPPORTED -3 /* valid, but a size or dtype not built        */
#define DQKV_ERR_WORKSPACE   -4 /* workspace too small                         */
#define DQKV_ERR_HIP         -5 /* the HIP runtime refused a launch            */
#define DQKV_ERR_ALIGN       -6 /* a device pointer is not 16-byte aligned     */

/* Human-readable name of a status code (static storage). */
const char* dqkv_status_str(int32_t status);

/*
 * Context-chunk length (rows per split) that diffqkv_decode uses when it is
 * called with chunk_tokens = 0.  (diffqkv_decode_paged plans its own: half
 * as long for batches under 8 sequences.)  Pure host computation.
 */
int32_t diffqkv_decode_chunk(int32_t n_q, int32_t n_k, int32_t n_v,
                             int32_t d_k, int32_t d_v, int32_t batch,
                             int32_t max_ctx, int32_t* chunk_tokens);

/*
 * Workspace bytes diffqkv_decode needs for these sizes and chunk length
 * (chunk_tokens = 0: the automatic choices of both diffqkv_decode and
 * diffqkv_decode_paged, whichever needs more).  The workspace holds the
 * per-chunk partial results of the split step, fp32: a reference m (within
 * 8 log2 units below the chunk's largest scaled score, so the chunk's
 * weights 2^(s - m) stay below 2^8), the sum l of those weights and the
 * weighted V sum; the combine merges them exactly for any such m.  Their
 * layout is internal.  Pure host computation.
 */
int32_t diffqkv_decode_workspace(int32_t n_q, int32_t n_k, int32_t n_v,
                                 int32_t d_k, int32_t d_v, int32_t batch,
                                 int32_t max_ctx, int32_t chunk_tokens,
                                 size_t* bytes);

/*
 * kv_append -- Step 2 of section 3.4: K_t = [K_{t-1}; k_t], V_t = [V_{t-1}; v_t]
 * into the separate K and V caches.
 *
 * Token t of sequence b (k_new[b][t], v_new[b][t]) is copied, bit for bit,
 * to cache row pos[b] + t of every head.  pos is a device array.  Rows whose
 * destination falls outside [0, l_cap) are skipped (no write).  t_new = 0 or
 * batch = 0 is a no-op.
 */
int32_t kv_append(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                  int32_t d_v, int32_t dtype, int32_t batch, int32_t t_new,
                  int32_t l_cap, const void* k_new, const void* v_new,
                  const int32_t* pos, void* k_cache, void* v_cache,
                  void* stream);

/*
 * diffqkv_decode -- one decode step: every query head of every sequence
 * attends rows 0 .. ctx_len[b]-1 of its key and value heads (the newest row
 * included, section 3.4 Steps 2-5).
 *
 * Split-KV structure (FlexHeadFA section: a split kernel over context chunks
 * followed by a combine kernel): the context is cut into chunks of
 * chunk_tokens rows (0 = automatic, otherwise a multiple of 64); the split
 * kernel writes each chunk's (max, sum, weighted V sum) into `workspace`
 * (>= diffqkv_decode_workspace bytes, 16-byte aligned, contents need not be
 * initialised) and the combine kernel merges them exactly in log-sum-exp
 * form into out and lse.
 *
 * max_ctx (host) bounds ctx_len and sizes the launch: 0 <= ctx_len[b] <=
 * max_ctx <= l_cap is required.  Values beyond are clamped to
 * min(max_ctx, l_cap) (memory-safe, result then covers only those rows; the
 * fused-append forms below then write nothing for that sequence, so the
 * cache keeps its history).  ctx_len[b] = 0 yields out = 0 and lse = -inf.
 */
int32_t diffqkv_decode(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                       int32_t d_v, int32_t dtype, int32_t batch,
                       int32_t l_cap, int32_t max_ctx, float scale,
                       const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* ctx_len,
                       void* out, float* lse, int32_t chunk_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * diffqkv_decode_append -- one decode step that first appends the step's
 * new token: k_new[b] ([B][n_k][d_k], i.e. token-major with t_new = 1) and
 * v_new[b] ([B][n_v][d_v]) are written to cache row ctx_len[b] - 1 (so
 * ctx_len counts rows after the append, Step 2 of section 3.4), and every
 * query head then attends rows 0 .. ctx_len[b] - 1 as in diffqkv_decode.
 * Same result, bit for bit, as kv_append with pos[b] = ctx_len[b] - 1
 * followed by diffqkv_decode, in two kernels instead of three: the waves of
 * the split workgroup that owns row ctx_len[b] - 1 store the new row into
 * the caches and read it back with the rest of their chunk.  Requires
 * 1 <= ctx_len[b] <= max_ctx for every b that should append (ctx_len[b] = 0:
 * nothing appended, out = 0, lse = -inf).
 */
int32_t diffqkv_decode_append(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                              int32_t d_v, int32_t dtype, int32_t batch,
                              int32_t l_cap, int32_t max_ctx, float scale,
                              const void* q, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* ctx_len, void* out, float* lse,
                              int32_t chunk_tokens, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * diffqkv_decode_append_noalloc -- diffqkv_decode_append (k_new / v_new may
 * also both be NULL: then diffqkv_decode) without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The split
 * kernel's partial results go to a static device array of the library
 * (16 MiB, one per GPU, held from the first use until the process ends);
 * the call allocates nothing and frees nothing.  Sizes whose partials need
 * more than 16 MiB (diffqkv_decode_workspace bytes) return
 * DQKV_ERR_WORKSPACE.  The array of the CURRENT device is used, so the
 * stream must belong to the current device.  Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (on different
 * streams) race and must not be issued; calls in order on one stream are
 * fine (no contents need to survive between calls).  Same result, bit for
 * bit, as diffqkv_decode_append (or diffqkv_decode) with the same
 * chunk_tokens.
 */
int32_t diffqkv_decode_append_noalloc(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                      int32_t d_v, int32_t dtype, int32_t batch,
                                      int32_t l_cap, int32_t max_ctx, float scale,
                                      const void* q, const void* k_new,
                                      const void* v_new, void* k_cache, void* v_cache,
                                      const int32_t* ctx_len, void* out, float* lse,
                                      int32_t chunk_tokens, void* stream);

/*
 * diffqkv_decode_split / diffqkv_decode_combine -- the two halves of
 * diffqkv_decode (or, with k_new / v_new non-NULL, of diffqkv_decode_append),
 * for callers that time or schedule them separately: the pages measure the
 * split and combine kernels of FlexHeadFA separately.  Arguments have the
 * meaning given above; both calls of one step must pass the same sizes,
 * chunk_tokens and workspace.  The split kernel writes every non-empty
 * chunk's (reference m, sum, weighted V sum) to the workspace; the combine reads
 * them and writes out and lse.  k_cache / v_cache are written only when
 * k_new / v_new are given (both or neither).
 */
int32_t diffqkv_decode_split(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                             int32_t d_v, int32_t dtype, int32_t batch,
                             int32_t l_cap, int32_t max_ctx, float scale,
                             const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* ctx_len, int32_t chunk_tokens,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

int32_t diffqkv_decode_combine(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                               int32_t d_v, int32_t dtype, int32_t batch,
                               int32_t l_cap, int32_t max_ctx,
                               const int32_t* ctx_len, void* out, float* lse,
                               int32_t chunk_tokens, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * diffqkv_prefill -- causal attention of t_new new query rows per sequence
 * against the cache, with bf16 matrix-core (MFMA) products.
 *
 * The t_new new rows must already be in the caches (kv_append), so
 * ctx_len[b] counts rows after the append and ctx_len[b] >= t_new.  New row
 * r of sequence b sits at position p = ctx_len[b] - t_new + r and attends
 * key rows 0 .. p (each token sees all earlier tokens and itself; a reading
 * of section 3.4 Steps 2-5 applied token by token).  Rows with p < 0 (that
 * is ctx_len[b] < t_new) get out = 0, lse = -inf; ctx_len is clamped to
 * l_cap.
 *
 * workspace (optional, 16-byte aligned, contents need not be initialised):
 * when it holds diffqkv_prefill_workspace bytes and that size is non-zero,
 * small launches split every row's keys over several workgroups and merge
 * the parts exactly in log-sum-exp form (one more kernel); with NULL or too
 * small a workspace the prefill runs unsplit.  Results agree within
 * rounding either way.
 */
int32_t diffqkv_prefill_workspace(int32_t n_q, int32_t n_k, int32_t n_v,
                                  int32_t d_k, int32_t d_v, int32_t batch,
                                  int32_t t_new, size_t* bytes);

int32_t diffqkv_prefill(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                        int32_t d_v, int32_t dtype, int32_t batch,
                        int32_t t_new, int32_t l_cap, float scale,
                        const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* ctx_len,
                        void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * diffqkv_prefill_paged -- diffqkv_prefill over a paged cache (the page
 * layout of diffqkv_decode_paged: k_pages [num_pages][n_k][page_rows][d_k],
 * v_pages [num_pages][n_v][page_rows][d_v], key row j of sequence b in page
 * block_table[b][j / page_rows], page_rows a power of two >= 64).  The row
 * capacity max_blocks * page_rows takes the place of l_cap; entries of
 * block_table outside [0, num_pages) are clamped (memory-safe, the result
 * then reads another page).  Same workspace (diffqkv_prefill_workspace) and
 * the same result, bit for bit, as diffqkv_prefill on the equivalent
 * contiguous cache.  Not described by the pages (a layout choice; vLLM's
 * paged attention is the prior art they name).
 */
int32_t diffqkv_prefill_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                              int32_t d_v, int32_t dtype, int32_t batch,
                              int32_t t_new, int32_t page_rows, int32_t num_pages,
                              int32_t max_blocks, float scale, const void* q,
                              const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* ctx_len,
                              void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * diffqkv_decode_selective -- decode with selective V fetching (architecture
 * page, section "Selective V Cache Fetching"; a NEXT-step inference
 * optimisation, not part of the Sigma model itself).
 *
 * For every sequence b and query head i the attention weights
 * alpha_j = softmax_j(scale * q_i . K_j) are computed over all rows
 * j < ctx_len[b] (the whole K cache is read), then only the V rows of the
 * top_k largest weights are read and
 *
 *   out[b][i] = sum_{j in TopK} alpha_j * V[floor(i n_v / n_q)][j]
 *
 * with alpha the full softmax: the selected weights are not renormalised, so
 * the output equals diffqkv_decode's when top_k >= ctx_len[b].  Equal
 * weights are ordered by row index, lower first (the page leaves ties open).
 * The selection is decided on the kernel's fp32 logits.
 *
 *   top_k     1 .. 1024 (the page's experiments use 100).
 *   k_new, v_new  optional fused append as in diffqkv_decode_append (both or
 *             neither): row ctx_len[b] - 1 is written from them first.
 *   lse       optional [B][n_q] fp32: log-sum-exp over ALL visible rows.
 *   sel_idx   optional [B][n_q][top_k] int32: the selected rows in ascending
 *             order, -1 past min(top_k, ctx_len[b]).
 *   workspace diffqkv_decode_selective_workspace bytes, 16-byte aligned,
 *             contents need not be initialised; it holds the fp32 logits
 *             ([B][n_q][max_ctx rounded up to 64]) and per-range candidates
 *             (ranges of 4096 rows, or of 2048 when 4096-row ranges would
 *             give fewer than 256 (sequence, head, range) selections).
 * ctx_len is clamped to [0, max_ctx]; ctx_len[b] = 0 gives out = 0,
 * lse = -inf, sel_idx = -1.  Three kernels on `stream`: logits (reads K
 * once), per-range top-k, final top-k with the V gather.
 */
int32_t diffqkv_decode_selective_workspace(int32_t n_q, int32_t n_k, int32_t n_v,
                                           int32_t d_k, int32_t d_v, int32_t batch,
                                           int32_t max_ctx, int32_t top_k,
                                           size_t* bytes);

int32_t diffqkv_decode_selective(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                                 int32_t d_v, int32_t dtype, int32_t batch,
                                 int32_t l_cap, int32_t max_ctx, float scale,
                                 int32_t top_k, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* ctx_len, void* out, float* lse,
                                 int32_t* sel_idx, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Paged cache -- a serving layout (the architecture page names vLLM's paged
 * attention as prior art that treats K and V alike; here K and V keep
 * separate page pools with their own row shapes under one page table):
 *
 *   k_pages      [num_pages][n_k][page_rows][d_k]
 *   v_pages      [num_pages][n_v][page_rows][d_v]
 *   block_table  [B][max_blocks] int32 (device): row j of sequence b is
 *                slot j % page_rows of page block_table[b][j / page_rows]
 *
 * page_rows is a power of two >= 64 (a 64-row decode tile then never spans
 * two pages, so each tile costs one table read).  The row capacity of a
 * sequence is max_blocks * page_rows.  Table entries outside
 * [0, num_pages) are never written through: kv_append_paged and the fused
 * appends of the decode and selective paths skip such rows, and their reads
 * clamp the entry into [0, num_pages) (a wrong result for a malformed
 * table, never an out-of-bounds access or a write into another page).
 *
 * kv_append_paged -- kv_append into a paged cache (pos, t_new, k_new, v_new
 *   as for kv_append; rows past the capacity are skipped).
 * diffqkv_decode_paged -- diffqkv_decode / diffqkv_decode_append over a paged
 *   cache; k_new / v_new optional (both or neither) as for
 *   diffqkv_decode_append; max_ctx <= max_blocks * page_rows; the workspace is
 *   diffqkv_decode_workspace's for the same sizes.  With the same chunking
 *   the result is bit-identical to diffqkv_decode on the gathered caches.
 */
int32_t kv_append_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                        int32_t d_v, int32_t dtype, int32_t batch, int32_t t_new,
                        int32_t page_rows, int32_t num_pages, int32_t max_blocks,
                        const void* k_new, const void* v_new, const int32_t* pos,
                        const int32_t* block_table, void* k_pages, void* v_pages,
                        void* stream);

int32_t diffqkv_decode_paged(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                             int32_t d_v, int32_t dtype, int32_t batch,
                             int32_t page_rows, int32_t num_pages,
                             int32_t max_blocks, int32_t max_ctx, float scale,
                             const void* q, const void* k_new, const void* v_new,
                             void* k_pages, void* v_pages,
                             const int32_t* block_table, const int32_t* ctx_len,
                             void* out, float* lse, int32_t chunk_tokens,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * diffqkv_decode_selective_paged -- diffqkv_decode_selective over a paged
 * cache (the layout above).  max_ctx <= max_blocks * page_rows; the same
 * workspace (diffqkv_decode_selective_workspace) and the same result, bit
 * for bit, as the contiguous call on the equivalent cache.
 */
int32_t diffqkv_decode_selective_paged(
    int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k, int32_t d_v, int32_t dtype,
    int32_t batch, int32_t page_rows, int32_t num_pages, int32_t max_blocks,
    int32_t max_ctx, float scale, int32_t top_k, const void* q, const void* k_new,
    const void* v_new, void* k_pages, void* v_pages, const int32_t* block_table,
    const int32_t* ctx_len, void* out, float* lse, int32_t* sel_idx, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * kv_group_sharing -- the compatibility expansion for frameworks whose
 * kernels need n_k = n_v (architecture page, FlexHeadFA section: the
 * kv_group_sharing wrapper, which the page warns negates the K saving).
 * Writes k_out [B][n_h][l_cap][d_k] and v_out [B][n_h][l_cap][d_v] with
 * n_h = max(n_k, n_v): output head h copies input head floor(h * n_k / n_h)
 * of K (floor(h * n_v / n_h) of V), so each head of the smaller side appears
 * n_h / n_smaller times in a row and the larger side is copied unchanged.
 * Decoding the expanded caches with (n_q, n_h, n_h, d_k, d_v) gives the same
 * result as the original layout.  A bit-exact copy of all l_cap rows; the
 * outputs must not overlap the inputs.
 */
int32_t kv_group_sharing(int32_t n_q, int32_t n_k, int32_t n_v, int32_t d_k,
                         int32_t d_v, int32_t dtype, int32_t batch, int32_t l_cap,
                         const void* k_cache, const void* v_cache, void* k_out,
                         void* v_out, void* stream);

/*
 * augq_forward -- the augmented-Q projection (architecture page, section 3.2
 * item 4: Augmented Q with SwiGLU gating), bf16 in and out, fp32
 * accumulation:
 *
 *   a = silu(h W_gate^T) * (h W_up^T)   [M][d_i], rounded to bf16 (workspace)
 *   q = a W_down^T                       [M][d_out]
 *
 * h [M][d_m] (M tokens); weights given PACKED by augq_pack from the (out,
 * in) layout: w_gate, w_up from [d_i][d_m], w_down from [d_out][d_i]
 * (d_i = 3072, d_m = 2048, d_out = n_q * d_k = 2048 for SIGMA-1.5B).  For
 * decode, q [M][d_out] is the query tensor [B][n_q][d_k] that diffqkv_decode
 * takes.  d_m and d_i multiples of 1024, d_out a multiple of 16; h, the
 * packed weights and q 16-byte aligned.  workspace: augq_workspace bytes
 * (M * d_i bf16), 16-byte aligned; it receives a, row-major [M][d_i], except
 * for M <= 16, where it is chunk-major [d_i / 8][M][8] (element (r, c) at
 * ((c / 8) M + r) 8 + c % 8: the order in which the down product's operand
 * loads read it).  Two kernels on `stream`.
 *
 * augq_pack -- one-time weight layout change for augq_forward: w [n_out][n_in]
 * (bf16, row-major) -> w_packed [n_out / 16][n_in / 32][64][8], element
 * (nb, kb, l, e) = w[16 nb + l % 16][32 kb + 8 (l / 16) + e]: the operand
 * order of the matrix-core instruction, so each 1 KiB fragment is read in one
 * contiguous wave load.  n_out a multiple of 16, n_in of 32; w_packed holds
 * n_out * n_in elements and must not overlap w.
 */
int32_t augq_pack(int32_t n_out, int32_t n_in, const void* w, void* w_packed,
                  void* stream);

int32_t augq_workspace(int32_t M, int32_t d_m, int32_t d_i, int32_t d_out,
                       size_t* bytes);

int32_t augq_forward(int32_t M, int32_t d_m, int32_t d_i, int32_t d_out,
                     const void* h, const void* w_gate, const void* w_up,
                     const void* w_down, void* q, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIFFQKV_H */
