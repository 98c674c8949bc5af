/*
 * csa2.h -- C ABI of the CSA2 sparse-attention hot path on MI355X (gfx950).
 *
 * The method (arXiv 2609.19969, "DeepSeek-V4.1-Flash: Pushing the Limits of
 * KV Cache Compression"), as described by the jaehun.me review of that paper
 * (sections "2) CSA2" and "3) FP4 main KV + SWA Bounded Replay", and the
 * worked example of the three modes) and by the ainewsway.com article on it:
 *   - every CSA2 layer has a static mode.  Full: scores all compressed
 *     main-KV entries with an indexer and keeps the Top-K (K = 512); the
 *     decoder's first Full layer also builds a candidate pool of 2,048
 *     blocks x 8 positions.  Reindex: rescores only the pool with its own
 *     indexer query and keeps 512.  Reuse: takes the latest Full layer's
 *     main KV and indices as they are.  Every mode has its own query and its
 *     own sliding-window (SWA) KV.
 *   - main KV is stored as FP4 E2M1 with one E4M3 scale per 16 channels; the
 *     window KV (n_win = 128 tokens) is FP8 E4M3.
 *
 * Layer modes map onto calls: Full = csa2_index_full + attention; Reindex =
 * csa2_reindex (with the Full layer's pool and key cache) + attention; Reuse =
 * attention with the same topk_idx / kv pointers and no indexer call.
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers owned by the caller; `stream` is
 *     a hipStream_t (NULL = the null stream).  The library never allocates,
 *     frees or synchronises: it checks its scalar arguments on the host,
 *     enqueues kernels on `stream` and returns.  Device-side contents are
 *     trusted (see the preconditions of each call).
 *   - Workspace `ws` (>= the size the matching *_workspace_bytes returns,
 *     256-byte aligned) is scratch owned by the caller; its contents need no
 *     initialisation and are meaningless after the call.  Calls that overlap
 *     on different streams need different workspaces.
 *   - Entry indices are int32 and local to their sequence; row offsets are
 *     int64.  Index outputs are written in ascending order, padded with -1,
 *     and fully overwritten.  Outputs must not alias inputs.
 *   - Selection order: higher score first, ties to the lower index (lower
 *     block id for the pool).  With integer-valued indexer inputs whose dot
 *     products stay below 2^24 the fp32 scores are exact and the selection
 *     is exactly the one of the definition.
 *   - Return value: a csa2_status.  No C++ exception crosses this boundary.
 */
#ifndef CSA2_H
#define CSA2_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_NULL = 1,        /* a required pointer is NULL                      */
    CSA2_ERR_SHAPE = 2,       /* a size is negative or inconsistent              */
    CSA2_ERR_UNSUPPORTED = 3, /* valid, but outside what the kernels implement   */
    CSA2_ERR_WORKSPACE = 4,   /* ws_bytes below the *_workspace_bytes figure     */
    CSA2_ERR_HIP = 5          /* a launch failed; see csa2_last_hip_error()      */
} csa2_status;

/* Name of a status code (static string). */
const char* csa2_status_str(int status);
/* hipError_t of the last CSA2_ERR_HIP returned on this host thread. */
int csa2_last_hip_error(void);

/* Limits of this implementation. */
#define CSA2_MAX_TOPK 2048          /* topk and pool_blocks                     */
#define CSA2_MAX_POOL_CAND 16384    /* pool_blocks * block_size (2,048 x 8)    */

/* ------------------------------------------------------------------------
 * Full-mode indexer: scoring + Top-K (+ candidate pool).
 *
 * Defines (jaehun.me review, section "2) CSA2" and the worked example; the
 * pages give no score formula, the plain head sum is used):
 *   s(q, t) = sum_{h < Hi} sum_{d < Di} qI[q,h,d] * kI[row0(q) + t, h mod Hk, d]
 * for every visible entry t < q_nvis[q], row0(q) = seq_row_off[q_seq[q]].
 * topk_idx[q] = the min(topk, q_nvis[q]) entries of highest score.
 * With pool_blocks > 0 (decoder's first Full layer, 2,048 blocks x 8
 * positions): block b covers entries [b*block_size, (b+1)*block_size) ∩
 * [0, q_nvis); it scores the maximum of its entries' scores;
 * pool_block_idx[q] = the min(pool_blocks, #blocks) best blocks.
 *
 *   qI             [Q, Hi, Di] fp32
 *   kI             [rows, Hk, Di] fp32, Hk == Hi or Hk == 1 (one key row
 *                  shared by all indexer heads); Hk*Di must be 256, 512 or
 *                  1024 (Hk == Hi) or Di must be (Hk == 1)
 *   seq_row_off    [S] int64: first kI row of each sequence
 *   q_seq          [Q] int32: sequence of each query.  May be NULL: then all
 *                  queries belong to sequence 0 (a chunk of prefill queries
 *                  of one prompt) and the call is scheduled as a
 *                  query-tile x key-tile contraction instead of one key
 *                  stream per query.
 *   q_nvis         [Q] int32: visible entries of each query (causality; for
 *                  an encoder chunk with m tokens per entry the caller passes
 *                  floor((p+1)/m)).  0 <= q_nvis[q] <= max_nvis; a larger
 *                  value is read as max_nvis (never past the rows scored).
 *   max_nvis       host bound on q_nvis (sizes the grid and the workspace)
 *   topk           0..CSA2_MAX_TOPK; topk_idx [Q, topk] int32 (may be NULL iff 0)
 *   pool_blocks    0..CSA2_MAX_TOPK; block_size in {1,2,4,8};
 *                  pool_block_idx [Q, pool_blocks] int32 (NULL iff pool_blocks 0)
 * Workspace: csa2_index_full_workspace_bytes for q_seq != NULL;
 * csa2_index_prefill_workspace_bytes (which also holds bf16 copies of the
 * chunk's query rows and the sequence's key rows) for q_seq == NULL, or
 * csa2_index_prefill_workspace_bytes_ex when that form also builds a pool.
 * The prefill form's pool is the encoder-side form of the hierarchical
 * indexer (the jaehun.me review's "next steps" suggest extending the
 * decoder-only candidate pool to the encoder): each query of the chunk gets
 * the same block pool a decode query with its q_nvis would.  Too small a
 * workspace: CSA2_ERR_WORKSPACE.
 * Accuracy of the prefill form: its scores come from bf16 matrix products of
 * a two-part split of every input value, x = hi + lo (hi = bf16(x),
 * lo = bf16(x - hi)); hi*hi + hi*lo + lo*hi is accumulated in fp32 and the
 * lo*lo product is dropped.  Integer-valued inputs (|x| <= 256 splits with
 * lo = 0) give the exact scores of the decode form and the selection of the
 * definition.  Other fp32 inputs: each score is within about
 * 2^-14 * sum_i |q_i k_i| of the exact one (the dropped lo*lo term and the
 * split's residual, each at most 2^-18 of a product, plus fp32 accumulation),
 * so an entry can trade places with another only when their exact scores
 * are that close.
 * Preconditions (device data): rows read stay inside kI.
 * ---------------------------------------------------------------------- */
size_t csa2_index_full_workspace_bytes(int32_t Q, int32_t max_nvis, int32_t topk,
                                       int32_t pool_blocks, int32_t block_size);
size_t csa2_index_prefill_workspace_bytes(int32_t Q, int32_t max_nvis, int32_t topk,
                                          int32_t Hk, int32_t Di);
size_t csa2_index_prefill_workspace_bytes_ex(int32_t Q, int32_t max_nvis, int32_t topk,
                                             int32_t pool_blocks, int32_t block_size,
                                             int32_t Hk, int32_t Di);
int csa2_index_full(const float* qI, const float* kI, const int64_t* seq_row_off,
                    const int32_t* q_seq, const int32_t* q_nvis, int32_t Q, int32_t Hi,
                    int32_t Hk, int32_t Di, int32_t max_nvis, int32_t topk, int32_t* topk_idx,
                    int32_t pool_blocks, int32_t block_size, int32_t* pool_block_idx, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Reindex mode (jaehun.me review, section "2) CSA2"; paper 2.3.2): rescore
 * only the candidate pool with this layer's own indexer query against the
 * shared key cache and keep the Top-K.  Candidates of query q:
 *   { b*block_size + j : b = pool_block_idx[q, i] >= 0, j < block_size,
 *     b*block_size + j < q_nvis[q] }
 * at most pool_blocks * block_size <= CSA2_MAX_POOL_CAND (2,048 x 8).
 * Score as in csa2_index_full; ties go to the lower ENTRY index.
 *   pool_block_idx [Q, pool_blocks] int32, -1 = empty slot.
 * Preconditions (device data): the valid block ids of a row are distinct.
 * ---------------------------------------------------------------------- */
size_t csa2_reindex_workspace_bytes(int32_t Q, int32_t pool_blocks, int32_t block_size);
int csa2_reindex(const float* qI, const float* kI, const int64_t* seq_row_off,
                 const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_block_idx,
                 int32_t pool_blocks, int32_t block_size, int32_t Q, int32_t Hi, int32_t Hk,
                 int32_t Di, int32_t topk, int32_t* topk_idx, void* ws, size_t ws_bytes,
                 void* stream);

/* ------------------------------------------------------------------------
 * Allocation-free Reindex, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): csa2_reindex with its workspace replaced by a static device
 * array of CSA2_NOALLOC_MAX_CAND candidate score keys (8 MiB) that each GPU the
 * library runs on holds until the process ends.  Same arguments, results and
 * errors as csa2_reindex, without ws / ws_bytes; the array of the CURRENT
 * device (hipGetDevice) is used, so `stream` must belong to that device.
 * Q * pool_blocks * block_size above CSA2_NOALLOC_MAX_CAND (for example 128
 * queries of 2,048 x 8 candidates) gives CSA2_ERR_UNSUPPORTED before anything
 * is enqueued.  The call allocates nothing (no hipMalloc, no hipFree).  All
 * calls on one GPU share its array, and every call overwrites what it uses
 * before reading it: calls that overlap on one GPU (different streams or
 * host threads without ordering) race and must not be issued.
 * ---------------------------------------------------------------------- */
#define CSA2_NOALLOC_MAX_CAND 2097152
int csa2_reindex_noalloc(const float* qI, const float* kI, const int64_t* seq_row_off,
                         const int32_t* q_seq, const int32_t* q_nvis,
                         const int32_t* pool_block_idx, int32_t pool_blocks, int32_t block_size,
                         int32_t Q, int32_t Hi, int32_t Hk, int32_t Di, int32_t topk,
                         int32_t* topk_idx, void* stream);

/* ------------------------------------------------------------------------
 * Compact indexer-key cache: the same Full-mode and Reindex calls over keys
 * stored as one E4M3FN byte per value (a quarter of the fp32 cache's bytes).
 * The pages (jaehun.me review, TL;DR and section "2) CSA2": the global KV
 * cache, indexer keys included, takes 890 bytes per token; indexer K is a
 * projection of main KV) give no storage format for indexer keys.  Reading
 * used: plain OCP E4M3FN values with no scale, decoded exactly to fp32 before
 * the dot product; a scale common to all keys can be folded into qI.  With
 * integer-valued keys of magnitude <= 16 (exact in E4M3) and integer queries
 * whose dot products stay below 2^24 the selection is exactly the one of the
 * fp32 cache holding the same values.
 *   kI  [rows, Hk, Di] u8 (E4M3FN; S.1111.111 = NaN must not occur), 16-byte
 *       aligned; every other argument, the workspace sizes
 *       (csa2_index_full_workspace_bytes, csa2_index_prefill_workspace_bytes,
 *       csa2_reindex_workspace_bytes), the shapes supported and the errors
 *       are those of csa2_index_full and csa2_reindex.
 * ---------------------------------------------------------------------- */
int csa2_index_full_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                         const int32_t* q_seq, const int32_t* q_nvis, int32_t Q, int32_t Hi,
                         int32_t Hk, int32_t Di, int32_t max_nvis, int32_t topk,
                         int32_t* topk_idx, int32_t pool_blocks, int32_t block_size,
                         int32_t* pool_block_idx, void* ws, size_t ws_bytes, void* stream);
int csa2_reindex_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                      const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_block_idx,
                      int32_t pool_blocks, int32_t block_size, int32_t Q, int32_t Hi, int32_t Hk,
                      int32_t Di, int32_t topk, int32_t* topk_idx, void* ws, size_t ws_bytes,
                      void* stream);

/* ------------------------------------------------------------------------
 * General form of the Full-mode indexer: the key cache's format and the
 * candidate pool's block score are parameters.  The pages (jaehun.me review,
 * section "2) CSA2") give the pool as 2,048 blocks x 8 positions and no block
 * score; the reading used everywhere else is the block's maximum entry score
 * (CSA2_BLOCK_MAX), which also equals taking the blocks of the top entries in
 * rank order until pool_blocks distinct blocks are held.  CSA2_BLOCK_SUM, a
 * variant, scores a block by the sum of its visible entries' scores (exact
 * for integer-valued inputs while the sums stay below 2^24 in magnitude;
 * otherwise fp32 sums).
 *   kI          key_format CSA2_KEYS_F32: const float* [rows, Hk, Di];
 *               CSA2_KEYS_E4M3: const uint8_t* [rows, Hk, Di] (E4M3FN)
 *   block_rule  CSA2_BLOCK_MAX or CSA2_BLOCK_SUM (used when pool_blocks > 0)
 * Every other argument, the workspace sizes and the errors are those of
 * csa2_index_full; an unknown key_format or block_rule gives
 * CSA2_ERR_UNSUPPORTED.  csa2_index_full = (CSA2_KEYS_F32, CSA2_BLOCK_MAX),
 * csa2_index_full_e4m3 = (CSA2_KEYS_E4M3, CSA2_BLOCK_MAX).
 * ---------------------------------------------------------------------- */
#define CSA2_KEYS_F32 0
#define CSA2_KEYS_E4M3 1
#define CSA2_BLOCK_MAX 0
#define CSA2_BLOCK_SUM 1
int csa2_index_full_ex(const float* qI, const void* kI, int32_t key_format,
                       const int64_t* seq_row_off, const int32_t* q_seq, const int32_t* q_nvis,
                       int32_t Q, int32_t Hi, int32_t Hk, int32_t Di, int32_t max_nvis,
                       int32_t topk, int32_t* topk_idx, int32_t pool_blocks, int32_t block_size,
                       int32_t* pool_block_idx, int32_t block_rule, void* ws, size_t ws_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * Sparse attention, decode (one query token per sequence; any layer mode).
 * (jaehun.me review, sections "2) CSA2" and "3) FP4 main KV"; ainewsway.com
 * article: window and global sparse retrieval form one attention.)
 * For sequence b and head h, one softmax over the union of
 *   - main-KV entries t = topk_idx[b, i] >= 0: key = value = dequantised row
 *     seq_row_off[b] + t, v[c] = E2M1(code[c]) * E4M3(scale[c/16]) (channel
 *     c = low nibble of byte c/2 for even c, high nibble for odd c);
 *   - window tokens w < min(swa_len[b], W): key E4M3(swa_k[b,w,:]),
 *     value E4M3(swa_v[b,w,:]);
 * with logits softmax_scale * q.k:  out[b,h] = sum_j p_j v_j,
 * lse[b,h] = log sum_j exp(logit_j).  No key at all: out = 0, lse = -inf.
 *   q        [B, H, D] fp32          kv_codes [rows, D/2] u8
 *   kv_scales [rows, D/16] u8        topk_idx [B, topk] int32 (-1 skipped)
 *   swa_k/swa_v [B, W, D] u8 (E4M3FN)  swa_len [B] int32
 *   out [B, H, D] fp32; lse [B, H] fp32 or NULL
 * Supported: D == 512, H a multiple of 16, B <= 65535,
 * 0 <= topk <= CSA2_MAX_TOPK, 0 <= W <= 1024.
 * Preconditions (device data): every valid index addresses a row of kv and
 * is below 2^23 (the gathers address a sequence's rows with 32-bit byte
 * offsets; a padding slot is read out of range and returns 0).
 * ---------------------------------------------------------------------- */
size_t csa2_decode_workspace_bytes(int32_t B, int32_t H, int32_t D, int32_t topk, int32_t W);
int csa2_sparse_attn_decode(const float* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                            const int64_t* seq_row_off, const int32_t* topk_idx, int32_t topk,
                            const uint8_t* swa_k, const uint8_t* swa_v, const int32_t* swa_len,
                            int32_t W, int32_t B, int32_t H, int32_t D, float softmax_scale,
                            float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Sparse attention, decode, for a layer group in one call: L layers (a Full
 * or Reindex layer and its Reuse layers) that share topk_idx and the main KV
 * and differ in their query and window (jaehun.me review, section "2) CSA2"
 * and its worked example: Reuse layers attend with their own query and SWA
 * KV over the latest Full layer's KV and indices).  Layer l equals
 * csa2_sparse_attn_decode with q[l], swa_k[l], swa_v[l], out[l], lse[l] and
 * the shared arguments; one launch covers all L x B query-layers, so small
 * batches need fewer key-range splits (and often no merge step).
 *   q, swa_k, swa_v, out   HOST arrays of L device pointers (each as in
 *                          csa2_sparse_attn_decode); swa_k/swa_v may be NULL
 *                          when W == 0
 *   lse                    NULL, or a HOST array of L device pointers (entries
 *                          may be NULL)
 *   1 <= L <= 8 and L x B <= 65535 (else CSA2_ERR_UNSUPPORTED); workspace:
 *   csa2_decode_layers_workspace_bytes.  Other arguments, shapes and errors
 *   as csa2_sparse_attn_decode; the per-layer call is this one with L = 1.
 * ---------------------------------------------------------------------- */
size_t csa2_decode_layers_workspace_bytes(int32_t L, int32_t B, int32_t H, int32_t D,
                                          int32_t topk, int32_t W);
int csa2_sparse_attn_decode_layers(int32_t L, const float* const* q, const uint8_t* kv_codes,
                                   const uint8_t* kv_scales, const int64_t* seq_row_off,
                                   const int32_t* topk_idx, int32_t topk,
                                   const uint8_t* const* swa_k, const uint8_t* const* swa_v,
                                   const int32_t* swa_len, int32_t W, int32_t B, int32_t H,
                                   int32_t D, float softmax_scale, float* const* out,
                                   float* const* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Sparse attention over a prefill chunk of ONE sequence: query i sits at
 * position p = p0 + i and equals a decode query with index row topk_idx[i]
 * and the window of the W tokens ending at p (those at positions >= 0).
 * (jaehun.me review: encoder CSA2 layers, m = 2; window n_win = 128.)
 *   q [Qn, H, D] fp32; kv_codes/kv_scales: this sequence's rows
 *   topk_idx [Qn, topk] int32 (-1 skipped)
 *   swa_k/swa_v [Qn + W - 1, D] u8: row r holds position p0 - W + 1 + r;
 *   rows of negative position may be read but never contribute (their bytes
 *   need not be valid E4M3).
 *   out [Qn, H, D]; lse [Qn, H] or NULL.   Supported shapes as for decode
 *   (Qn <= 65535).
 * ---------------------------------------------------------------------- */
size_t csa2_prefill_workspace_bytes(int32_t Qn, int32_t H, int32_t D, int32_t topk, int32_t W);
int csa2_sparse_attn_prefill_chunk(const float* q, int64_t p0, const uint8_t* kv_codes,
                                   const uint8_t* kv_scales, const int32_t* topk_idx,
                                   int32_t topk, const uint8_t* swa_k, const uint8_t* swa_v,
                                   int32_t W, int32_t Qn, int32_t H, int32_t D,
                                   float softmax_scale, float* out, float* lse, void* ws,
                                   size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FP4 main-KV writer: quantises fp32 rows into the main-KV format the
 * attention calls read (jaehun.me review, section "3) FP4 main KV"; the
 * ainewsway.com article: E2M1 values with one scale per 16 channels).  The
 * pages fix the format, not the rounding; this writer's rule: a group's
 * scale is the smallest positive finite E4M3 value s with 6 s >= its
 * largest magnitude (448 and saturation at 6 beyond 6 x 448; scale byte 0
 * and all-zero codes for an all-zero group); each value takes the E2M1
 * magnitude nearest to |x| / s, ties to the even code, the sign of x and no
 * negative zero.
 *   x      [rows, D] fp32, 16-byte aligned, finite
 *   codes  [rows, D/2] u8: channel c in the low nibble of byte c/2 when c is
 *          even, the high nibble when odd; 2-byte aligned
 *   scales [rows, D/16] u8 (E4M3FN)
 * D must be a multiple of 16 (else CSA2_ERR_UNSUPPORTED).  No workspace.
 * ---------------------------------------------------------------------- */
int csa2_kv_quantize_fp4(const float* x, int64_t rows, int32_t D, uint8_t* codes,
                         uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * FP8 window ring append (jaehun.me review, section "3) FP4 main KV + SWA
 * Bounded Replay": the last 128 tokens are kept in FP8 beside the sparse main
 * KV; ainewsway.com article: a 128-token sliding window).  Reading of the
 * ring: sequence b keeps W slots; its token at position pos[b] goes to slot
 * pos[b] mod W, so after position p the ring holds tokens max(0, p-W+1) .. p
 * and csa2_sparse_attn_decode reads it as the window with
 * swa_len = min(W, p + 1) (the attention does not depend on the order of the
 * window's tokens).  A window-only layer is csa2_sparse_attn_decode with
 * topk = 0.  Encoding: E4M3FN, round to nearest even, the sign of zero kept,
 * magnitudes beyond 448 saturated to 448 (never NaN for finite input).
 *   k_new, v_new [B, D] fp32, 16-byte aligned, finite
 *   pos          [B] int64, device; a negative position appends nothing
 *   swa_k, swa_v [B, W, D] u8 (E4M3FN), 8-byte aligned; only slot
 *                pos[b] mod W of each sequence is written
 * D must be a multiple of 8 (else CSA2_ERR_UNSUPPORTED).  No workspace.
 * ---------------------------------------------------------------------- */
int csa2_swa_append(const float* k_new, const float* v_new, const int64_t* pos, int32_t B,
                    int32_t D, int32_t W, uint8_t* swa_k, uint8_t* swa_v, void* stream);

/* ------------------------------------------------------------------------
 * Optional per-kernel timing (for measurement tools).  While enabled, every
 * kernel the library launches is bracketed by hipEvents recorded on the
 * launch stream; csa2_profile_read synchronises on the last event and
 * returns, per kernel name, the launch count and summed milliseconds.
 * Not thread-safe; disabled by default.
 * ---------------------------------------------------------------------- */
int csa2_profile_enable(int enable);
int csa2_profile_read(int slot, const char** name, int* launches, double* total_ms);
int csa2_profile_reset(void);

/* Test hook: decodes every byte value with the device codecs the attention
 * kernels use.  fp4_hw/fp4_ref [512]: entry 2b / 2b+1 = low / high nibble of
 * byte b through the gfx950 FP4 conversion / through the E2M1 definition;
 * fp8_hw/fp8_ref [256]: byte b through the gfx950 FP8 conversion / the
 * E4M3FN definition.  Device pointers. */
int csa2_debug_decode_tables(float* fp4_hw, float* fp4_ref, float* fp8_hw, float* fp8_ref,
                             void* stream);

/* Test hook: the attention kernels' own dequantisation to fp16, read back as
 * fp32.  main_out [256 * 16 * 8]: entry (s * 16 + c) * 8 + p = E2M1 code c at
 * nibble position p of a code dword, times E4M3 scale byte s (every E2M1 x
 * E4M3 product is exact in fp16).  win_out [256 * 8]: entry b * 8 + p =
 * E4M3 byte b at byte position p of an 8-byte window chunk.  The other
 * positions hold other values, so a wrong byte or nibble selection shows.
 * Device pointers; CSA2_ERR_NULL on a null pointer. */
int csa2_debug_dequant_tables(float* main_out, float* win_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
