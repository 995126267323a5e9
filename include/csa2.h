/*
 * csa2.h -- C ABI of the gfx950 (MI355X) library for CSA2 sparse attention
 * over an FP4 KV cache (E2M1 elements, one E4M3 scale per 16 channels).
 *
 * Three calls cover the three statically assigned layer modes described in
 * the course brief "DeepSeek-V4.1-Flash" (section "CSA2: most layers don't
 * keep their own cache", mode table) and in the metallab.ai article on the
 * V4.1-Flash KV cache (paragraph on the three modes):
 *
 *   Full    : csa2_quantize_kv_fp4 (write own main KV)
 *             -> csa2_index_topk(CSA2_FULL, ..., pool_size)   own indexer
 *             -> csa2_sparse_attn
 *   Reindex : csa2_index_topk(CSA2_REINDEX, pool = last Full's pool)
 *             -> csa2_sparse_attn
 *   Reuse   : csa2_sparse_attn(idx = last Full/Reindex selection)
 *
 * Variants: csa2_sparse_attn_swa joins each layer's local FP8 window to the
 * selection (csa2_quantize_swa_fp8 writes window entries);
 * csa2_index_topk_mxfp4 scores MXFP4 indexer keys (csa2_quantize_idx_mxfp4
 * writes them).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *     every buffer (inputs, outputs, workspace); the library never allocates,
 *     frees, synchronizes or copies to the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Inputs are read-only (except win_codes, when csa2_sparse_attn_swa is
 *     given new_x).  Outputs are overwritten in full, padding too.
 *   - Return value: CSA2_OK (0) or a negative status.  Only host-visible
 *     arguments are checked; device data are never read by the host.
 *     Data-dependent conditions are defined behaviour, not errors: an index
 *     < 0 or >= the row's visible count is skipped, an empty selection
 *     gives output 0 and lse = -inf.
 *   - csa2_last_error() returns a thread-local message for the last failing
 *     call of the calling thread.
 *   - Calls that share a workspace must be ordered on one stream.
 *
 * Packed variable-length batches work like cu_seqlens: every row r owns a
 * segment of the cache starting at row_kv_start[r]; entry (token position)
 * j of that row lives at cache row row_kv_start[r] + j.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CSA2_OK 0
#define CSA2_E_INVALID (-1)     /* null pointer, bad dtype, shape or alignment */
#define CSA2_E_UNSUPPORTED (-2) /* valid request this build does not implement */
#define CSA2_E_WORKSPACE (-3)   /* workspace missing or smaller than required  */
#define CSA2_E_HIP (-4)         /* a HIP launch failed; message has the reason */

/* element types */
#define CSA2_F32 0
#define CSA2_BF16 1
#define CSA2_MXFP4 2 /* indexer keys only: OCP MXFP4, see csa2_quantize_idx_mxfp4 */

/* indexer modes */
#define CSA2_FULL 0
#define CSA2_REINDEX 1
#define CSA2_FULL_SHARED 2 /* Full for rows that share one key segment (a prefill chunk) */

/* geometry of one cache entry ("FP4 cache entries, and why they're safe":
 * 512 values x 4 bits + 512/16 scales x 1 byte = 256 + 32 = 288 bytes) */
#define CSA2_HEAD_DIM 512
#define CSA2_CODE_BYTES 256
#define CSA2_SCALE_BYTES 32
#define CSA2_MAX_TOP_K 4096

/*
 * Quantize-on-write ("FP4 cache entries, and why they're safe", course
 * brief "DeepSeek-V4.1-Flash": E2M1 elements with one E4M3 scale per group
 * of 16 channels, no second-level global scale).  Per group g:
 *   amax = max|x_c|; s = E4M3(amax / 6) (fp32 division, round to nearest
 *   even, saturating at 448); code_c = E2M1(x_c / s) (fp32 division, round
 *   to nearest even, saturating at 6, sign kept); a group with s = 0 gets
 *   all-zero codes.
 *
 * x            [n_tokens, x_row_stride] elements of x_dtype (CSA2_F32 or
 *              CSA2_BF16); the first 512 of each row are quantized.  Must be
 *              16-byte aligned with x_row_stride * element size a multiple
 *              of 16.  Values must be finite.
 * dst_rows     [n_tokens] int64 cache row of each token, or NULL for rows
 *              0..n_tokens-1 (then n_tokens <= cap_rows is required).  A
 *              destination outside [0, cap_rows) is skipped; two tokens of
 *              one call with the same destination leave either one there.
 * kv_codes     [cap_rows, 256] uint8: byte i = code of channel 2i (low
 *              nibble) | code of channel 2i+1 (high nibble).
 * kv_scales    [cap_rows, 32] uint8: E4M3 scale byte of group g.
 * Errors: CSA2_E_INVALID for null buffers, n_tokens < 0, bad dtype,
 * misalignment, x_row_stride < 512, or (dst_rows NULL and n_tokens > cap_rows).
 */
int32_t csa2_quantize_kv_fp4(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                             const int64_t* dst_rows, uint8_t* kv_codes, uint8_t* kv_scales,
                             int64_t cap_rows, void* stream);

/*
 * Indexer + top-K ("The global branch: compress, index, select" and "The
 * hierarchical indexer" in the course brief; "The Paper" in the talk
 * write-up "DeepSeek V4.1 Flash: pushing the limits").
 *
 * Score of entry j for row r (fp32, fixed operation order, bit-reproducible):
 *   acc_h = fmaf chain over c = 0..63 of idx_q[r,h,c] * idx_k[j,c] from +0;
 *   score = sum over h = 0..H-1, left to right, of max(acc_h, +0).
 * Selection: the top_k entries by (score desc, position asc); out_idx[r] holds
 * their positions ascending, padded with -1.
 *
 * mode = CSA2_FULL: candidates are positions 0..row_visible[r]-1.  With
 *   pool_size > 0 (block_size must be 8) it also emits the hierarchical
 *   candidate pool: blocks of 8 positions scored by their best member, the
 *   top pool_size/8 blocks by (block score desc, block asc), their member
 *   positions ascending in out_pool[r] (padded with -1), the count in
 *   out_pool_len[r].
 * mode = CSA2_REINDEX: candidates are pool[r, i] for i < pool_len[r] (or
 *   i < pool_stride if pool_len is NULL); entries < 0 or >= row_visible[r]
 *   are skipped.  Valid entries must be unique and ascending (as
 *   CSA2_FULL emits them); ties are broken by pool order.
 * mode = CSA2_FULL_SHARED: CSA2_FULL for query rows that all read the same
 *   key segment, the one starting at row_kv_start[0] (row_kv_start[r] for
 *   r > 0 is not read), row r seeing its first row_visible[r] entries: a
 *   prefill chunk whose token r sits at position P0 + r sees
 *   row_visible[r] = P0 + r + 1.  Results are identical to CSA2_FULL over
 *   that segment.  With bf16 queries and keys, n_heads in {4, 8, 16} and no
 *   pool, the rows are first scored as one bf16 MFMA product with a proven
 *   bound on its error, every entry that the bound cannot exclude from the
 *   top_k is rescored with the exact chain above, and the selection among
 *   them is exact; a row with more than 16,384 such candidates is scanned
 *   exactly in full.  Otherwise it runs as CSA2_FULL does.
 *
 * idx_q        [n_rows, n_heads, head_dim] of q_dtype.
 * idx_k        [cache rows, head_dim] of k_dtype; row_kv_start[r] + j.
 * k_heads      indexer keys per entry: 1, one key shared by the n_heads query
 *              heads (the only layout built: the brief's per-entry byte count
 *              of the indexer cache holds one key vector per entry); any other
 *              value returns CSA2_E_UNSUPPORTED.
 * row_kv_start [n_rows] int64;  row_visible [n_rows] int32.
 * max_visible  host-side upper bound of row_visible (sizes grids and
 *              workspace); larger row_visible values are clamped to it.
 * head_dim must be 64; n_heads in 1..32; 1 <= top_k <= CSA2_MAX_TOP_K.
 * out_idx      [n_rows, top_k] int32.
 * workspace    device scratch of csa2_index_topk_workspace_size(...) bytes,
 *              256-byte aligned.
 */
int32_t csa2_index_topk(int32_t mode, int32_t n_rows,
                        const void* idx_q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                        const void* idx_k, int32_t k_dtype, int32_t k_heads,
                        const int64_t* row_kv_start, const int32_t* row_visible, int32_t max_visible,
                        const int32_t* pool, const int32_t* pool_len, int32_t pool_stride,
                        int32_t top_k, int32_t* out_idx,
                        int32_t pool_size, int32_t block_size, int32_t* out_pool, int32_t* out_pool_len,
                        void* workspace, size_t workspace_bytes, void* stream);

size_t csa2_index_topk_workspace_size(int32_t mode, int32_t n_rows, int32_t n_heads, int32_t max_visible,
                                      int32_t pool_stride, int32_t top_k, int32_t pool_size);

/*
 * MXFP4 indexer keys.  The course brief "DeepSeek-V4.1-Flash" ("FP4 cache
 * entries, and why they're safe") assumes the indexer keys are stored in
 * OCP MXFP4: blocks of 32 values share one 8-bit power-of-two scale (E8M0,
 * value 2^(b - 127)), elements are E2M1.  A 64-channel key is 32 code bytes
 * + 2 scale bytes = 34 B, against 128 B in bf16.
 *
 * csa2_quantize_idx_mxfp4 writes keys in that format, converting as the OCP
 * Microscaling specification does: per block of 32 channels,
 *   X = 2^(floor(log2 max|x|) - 2) (E8M0 code clamped to 0..254; a block of
 *   zeros gets code 0); code_c = E2M1(x_c / X) (fp32 division, nearest, ties
 *   to even, |.| > 6 clamped to 6, sign kept).
 * x            [n_tokens, x_row_stride] of x_dtype (CSA2_F32 or CSA2_BF16),
 *              16-byte aligned rows; the first 64 values of a row are used;
 *              values must be finite.
 * dst_rows     [n_tokens] int64 destination rows or NULL (rows 0..n_tokens-1,
 *              then n_tokens <= cap_rows); rows outside [0, cap_rows) are
 *              skipped; repeated destinations in one call leave either token.
 * k_codes      [cap_rows, 32] uint8 (byte i: channel 2i low nibble, 2i+1 high),
 *              16-byte aligned.
 * k_scales     [cap_rows, 2] uint8 E8M0 (block 0 = channels 0..31), 2-byte aligned.
 *
 * csa2_index_topk_mxfp4 is csa2_index_topk over such keys: each key value is
 * the exact fp32 product E2M1(code) * 2^(b - 127), and the score is the
 * same fixed-order fmaf chain, ReLU and head sum over those values; so the
 * result equals csa2_index_topk over the dequantized keys bit for bit.
 * CSA2_FULL_SHARED takes the MFMA passes (on the keys widened to bf16, which is
 * exact) and the exact rescoring, as with bf16 keys.
 * Arguments and errors as csa2_index_topk, with (idx_k, k_dtype) replaced by
 * (idx_k_codes, idx_k_scales); the workspace size is
 * csa2_index_topk_workspace_size's.
 */
int32_t csa2_quantize_idx_mxfp4(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                                const int64_t* dst_rows, uint8_t* k_codes, uint8_t* k_scales, int64_t cap_rows,
                                void* stream);

int32_t csa2_index_topk_mxfp4(int32_t mode, int32_t n_rows,
                              const void* idx_q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                              const uint8_t* idx_k_codes, const uint8_t* idx_k_scales, int32_t k_heads,
                              const int64_t* row_kv_start, const int32_t* row_visible, int32_t max_visible,
                              const int32_t* pool, const int32_t* pool_len, int32_t pool_stride,
                              int32_t top_k, int32_t* out_idx,
                              int32_t pool_size, int32_t block_size, int32_t* out_pool, int32_t* out_pool_len,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse attention over the selected entries ("The Paper" in the talk
 * write-up: K and V are the same Main KV entry, the selected entries are
 * attended with the normal attention operation; "The global branch" in the
 * course brief: one 512-dim latent per entry shared by every query head).
 * For row r, head h, over S = {idx[r,i] : 0 <= idx[r,i] < row_visible[r]}:
 *   x_j = E2M1(code) * E4M3(scale) dequantized entry j;
 *   z_j = softmax_scale * q[r,h] . x_j;  p = softmax(z) over S;
 *   out[r,h] = sum_j p_j x_j;  lse[r,h] = ln sum_j exp(z_j).
 * S empty: out = 0, lse = -inf.  Duplicate indices count as often as listed.
 *
 * q            [n_rows, n_heads, 512] of q_dtype (CSA2_F32 or CSA2_BF16);
 *              16-byte aligned.  The products run in fp16 on the matrix
 *              cores.  bf16 queries: decode launches (bf16, n_heads a
 *              multiple of 32, n_rows * n_heads / 32 <= 256, and not
 *              n_rows * n_heads / 64 >= 256; with a window, also
 *              top_k > 256 and n_rows * n_heads / 32 a multiple of 8 below
 *              256) first scale each head by
 *              the power of two that puts its largest |q| in [2^14, 2^15)
 *              (undone in the logit scale), so every finite value at least
 *              2^-28 of its head's largest is used exactly over the selected
 *              entries; other launches, and a window's entries
 *              (csa2_sparse_attn_swa), use a bf16 value exactly when
 *              2^-14 <= |q| < 65520 (the fp16
 *              normal range): smaller values lose low bits (below 2^-24 they
 *              count as 0) and larger ones overflow.  fp32 queries are split
 *              into two fp16 halves (about 22 significant bits in the fp16
 *              normal range) and must stay below 65504 in magnitude.
 * n_heads      a multiple of 16, at most 128; head_dim must be 512.
 * kv_codes/kv_scales  the cache written by csa2_quantize_kv_fp4.
 * idx          [n_rows, top_k] int32 positions (e.g. out_idx of the indexer).
 * row_visible  [n_rows] int32 or NULL (NULL: every idx >= 0 is valid).
 * out          [n_rows, n_heads, 512] of out_dtype (CSA2_F32 or CSA2_BF16).
 * lse          [n_rows, n_heads] fp32 or NULL.
 * workspace    csa2_sparse_attn_workspace_size(...) bytes (may be 0 when
 *              that function returns 0), 256-byte aligned.  Its first 4 KiB
 *              hold counters through which the workgroups of a key-split
 *              launch hand their partials to the workgroups that merge them:
 *              they must be zero when a workspace is first used (allocate it
 *              zero-filled) and every call leaves them zero again, so only
 *              other writers of that memory need to restore them.
 * Results are deterministic: the same inputs give the same bits.
 */
int32_t csa2_sparse_attn(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                         const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                         const int32_t* idx, int32_t top_k, const int32_t* row_visible,
                         float softmax_scale, void* out, int32_t out_dtype, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

size_t csa2_sparse_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t q_dtype, int32_t top_k);

/*
 * csa2_sparse_attn without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Arguments, results and errors are those of
 * csa2_sparse_attn (the same kernels run); the split partials and merge
 * counters live instead in one array of CSA2_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends.
 *   - A call whose csa2_sparse_attn_workspace_size(...) exceeds
 *     CSA2_NOALLOC_SCRATCH_BYTES (16 MiB) returns CSA2_E_WORKSPACE and
 *     launches nothing.  Nearly every shape fits; the largest workspaces
 *     (up to about 16.1 MiB) come with 129..255 row x 32-head pairs at
 *     top_k above 2048, for example 255 rows of 32 heads at top_k 4096.
 *   - Every call on a device uses that device's one array: calls that may
 *     overlap on one device (other streams, other threads) race and must be
 *     ordered by the caller.  The array keeps the last call's partials; the
 *     counters in its first 4 KiB are cleared on the device's first call
 *     (a kernel on `stream`) and every call leaves them zero.
 *   - The call allocates nothing, neither device nor host memory.  The first
 *     call on a device looks up the array's device address
 *     (hipGetSymbolAddress) and is best made once before any capture.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t csa2_sparse_attn_noalloc(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                                 const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                                 const int32_t* idx, int32_t top_k, const int32_t* row_visible, float softmax_scale,
                                 void* out, int32_t out_dtype, float* lse, void* stream);

/*
 * Local sliding-window branch.  Every CSA2 layer also runs exact sliding-
 * window attention over the 128 most recent tokens with its own window
 * cache, kept in FP8, and the selected Main KV entries are joined to that
 * window's KV for one attention ("The Paper" in the talk write-up "DeepSeek
 * V4.1 Flash: pushing the limits"; course brief "DeepSeek-V4.1-Flash",
 * sections "Two attention paths in every layer", "The global branch" and
 * "FP4 cache entries, and why they're safe").  The first layers are window
 * only (top_k = 0 below).
 *
 * Window entry: 512 bytes, one signed E4M3 (E4M3FN) byte per channel of the
 * layer's 512-channel latent, no scale; K = V = the entry, as for Main KV.
 */
#define CSA2_SWA_WINDOW 128

/*
 * Quantize-on-write of window entries: byte c = nearest E4M3 value of
 * x[t, c] (round to nearest even, |x| > 448 saturating to 448, sign bit of
 * x kept, so a negative value that rounds to zero is 0x80).
 * x            [n_tokens, x_row_stride] of x_dtype (CSA2_F32 or CSA2_BF16),
 *              16-byte aligned rows; values must be finite.
 * dst_rows     [n_tokens] int64 window-cache row per token, or NULL for rows
 *              0..n_tokens-1 (then n_tokens <= cap_rows).  A destination
 *              outside [0, cap_rows) is skipped; two tokens of one call with
 *              the same destination leave either one there.  A per-sequence
 *              ring of 128 rows (row = position mod 128) keeps a decode window.
 * win_codes    [cap_rows, 512] uint8, 16-byte aligned.
 * Errors: CSA2_E_INVALID for null buffers, n_tokens < 0, bad dtype,
 * misalignment, x_row_stride < 512, or (dst_rows NULL and n_tokens > cap_rows).
 */
int32_t csa2_quantize_swa_fp8(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t x_row_stride,
                              const int64_t* dst_rows, uint8_t* win_codes, int64_t cap_rows, void* stream);

/*
 * csa2_sparse_attn with the row's window joined into the same softmax.
 * For row r, head h, the attended set is S (as csa2_sparse_attn defines it,
 * empty when top_k = 0) plus the window entries W_r = rows
 * row_win_start[r] .. row_win_start[r] + n_r - 1 of win_codes, with
 * n_r = row_win_len[r] clamped to [0, 128]:
 *   w_i = E4M3(win_codes[i, c]) per channel;  z over S and W_r as in
 *   csa2_sparse_attn;  p = softmax over S and W_r together;
 *   out[r,h] = sum p x over S + sum p w over W_r;  lse over both.
 * Entries are not de-duplicated between S and W_r (they come from
 * different caches).  Nothing to attend: out = 0, lse = -inf.
 * Window entries of a row may be stored in any order (a ring buffer's valid
 * prefix works as it is): the result does not depend on their order.
 *
 * Arguments as for csa2_sparse_attn, plus:
 * top_k        0..CSA2_MAX_TOP_K; with 0, kv_codes, kv_scales, row_kv_start,
 *              idx and row_visible are not read and may be NULL.
 * win_codes    window entries written by csa2_quantize_swa_fp8, 16-byte aligned;
 *              read only, unless new_x is given.
 * row_win_start [n_rows] int64;  row_win_len [n_rows] int32.
 * new_x        optional (NULL: none): [n_rows, new_x_stride] of new_x_dtype
 *              (CSA2_F32 or CSA2_BF16), 16-byte aligned rows.  Row r's token
 *              new_x[r] is written, as csa2_quantize_swa_fp8 writes it, to
 *              window row new_rows[r] (skipped if negative; a non-negative
 *              value must be a row of win_codes) by this call, and
 *              row r attends over it if that row lies in its window: the
 *              decode step's newest token, without a separate write call.
 *              Precondition: no new row of the call lies in another row's
 *              window (true for one ring per sequence; a prefill chunk, whose
 *              windows overlap, writes first with csa2_quantize_swa_fp8).
 * workspace    csa2_sparse_attn_swa_workspace_size(...) bytes, 256-byte aligned,
 *              first 4 KiB zero as for csa2_sparse_attn.
 * Results are deterministic.
 */
int32_t csa2_sparse_attn_swa(int32_t n_rows, const void* q, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                             const uint8_t* kv_codes, const uint8_t* kv_scales, const int64_t* row_kv_start,
                             const int32_t* idx, int32_t top_k, const int32_t* row_visible,
                             uint8_t* win_codes, const int64_t* row_win_start, const int32_t* row_win_len,
                             const void* new_x, int32_t new_x_dtype, int64_t new_x_stride, const int64_t* new_rows,
                             float softmax_scale, void* out, int32_t out_dtype, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

size_t csa2_sparse_attn_swa_workspace_size(int32_t n_rows, int32_t n_heads, int32_t q_dtype, int32_t top_k);

/*
 * Visible entries of layers whose cache entries fold m consecutive tokens
 * ("The global branch: compress, index, select" in the course brief: the
 * encoder layers compress m = 2 tokens into one entry, the decoder's keep
 * m = 1).  Entry e covers tokens m*e .. m*e + m - 1, and a query at token
 * position t sees only entries whose whole block lies at or before t:
 *   row_visible[r] = (token_pos[r] + 1) / tokens_per_entry   (0 if token_pos[r] < 0),
 * computed on the device, ready for the row_visible argument of the calls above.
 * token_pos    [n_rows] int64 (device).   row_visible  [n_rows] int32 (device), written.
 * Errors: CSA2_E_INVALID for null buffers, n_rows < 0 or tokens_per_entry < 1.
 */
int32_t csa2_visible_entries(const int64_t* token_pos, int32_t tokens_per_entry, int32_t n_rows,
                             int32_t* row_visible, void* stream);

/* Thread-local description of the last non-zero status of this thread. */
const char* csa2_last_error(void);

/*
 * Measurement hook.  When `start_event`/`stop_event` (hipEvent_t as void*)
 * are non-NULL, later calls record them on the launch stream immediately
 * before and after every launch of kernel `kernel_id`; NULL pointers stop
 * the recording.  Process-wide; not thread-safe.  Returns CSA2_E_INVALID
 * for an unknown id.
 */
#define CSA2_KERNEL_QUANT 1
#define CSA2_KERNEL_INDEX_SCAN 2
#define CSA2_KERNEL_REINDEX_SCORE 3
#define CSA2_KERNEL_ATTN 4
#define CSA2_KERNEL_ATTN_COMBINE 5
#define CSA2_KERNEL_QUANT_FP8 6
#define CSA2_KERNEL_SWA_ATTN 7
#define CSA2_KERNEL_QUANT_MXFP4 8
int32_t csa2_profile_kernel_events(int32_t kernel_id, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
