/*
 * csa2.h -- C ABI of the CSA2 decode hot path on MI355X (gfx950).
 *
 * Four compute calls follow the pages' statement of one CSA2 decode layer
 * ("DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
 * sections "CSA2: share cache, refresh selection only when needed" (mode
 * table), "Hierarchical Sparse Indexer" (Figure 5), "FP4 main KV: trade
 * precision for bytes"; "Inside DeepSeek V4.1 Flash: CED, CSA2 and the
 * 890-Byte KV Cache", sections "CSA2: reuse memory and reuse selection
 * independently", "Hierarchical indexing bounds later searches, not every
 * search", "Reconstructing the 890-byte cache budget"):
 *
 *   csa2_quantize_kv    -- FP4 main-KV cache write (E2M1 + E4M3 per 16 ch)
 *   csa2_index_full     -- Full mode: score every visible entry, top-k, and
 *                          the block-max candidate pool (<= 2,048 blocks of 8)
 *   csa2_index_reindex  -- Reindex mode: score only the pool, top-k
 *   csa2_sparse_attn    -- gather + dequantize the selected entries and run
 *                          one softmax over them and the 128-row FP8 window.
 *                          Reuse mode is this call with a previous layer's
 *                          top-k buffer passed in unchanged.
 *
 * Conventions (all calls):
 *  - Every pointer argument except `stream` is a DEVICE pointer (HBM) owned
 *    by the caller; the library never allocates, frees or synchronizes.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the null stream).  Inputs are read-only; outputs are fully written.
 *  - Return value: CSA2_OK, or a negative status detected on the host before
 *    any launch (argument and size checks), or CSA2_ERR_LAUNCH if the launch
 *    itself failed.  On an error return nothing has been enqueued.
 *  - Fixed dimensions: main KV 512 channels, indexer key 128 channels,
 *    64 entries per page, pool blocks of 8 entries, window of 128 rows.
 *  - Formats: bf16 = IEEE bfloat16 bits; FP8 = OCP E4M3 (E4M3FN, max 448,
 *    codes 0x7F/0xFF are NaN); FP4 = OCP E2M1 nibbles.
 *  - Preconditions not checked on the device: inputs finite, no FP8 NaN
 *    codes, indexer weights w finite with |w| = 0 or 2^-100 <= |w| <= 2^90,
 *    top-k indices distinct.  Page ids outside [0, n_pages) and positions
 *    outside [0, n_entries[b]) are treated as not visible (never read).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_D 512                 /* main-KV channels */
#define CSA2_DI 128                /* indexer-key channels */
#define CSA2_PAGE 64               /* entries per page */
#define CSA2_ENTRY_CODE_BYTES 256  /* 512 E2M1 nibbles */
#define CSA2_ENTRY_SCALE_BYTES 32  /* one E4M3 scale per 16 channels */
#define CSA2_ENTRY_BYTES 288       /* 256 + 32 */
#define CSA2_PAGE_BYTES 18432      /* 64 x 288: 64 x 256 B codes, then 64 x 32 B scales */
#define CSA2_KIDX_PAGE_BYTES 8192  /* 64 x 128 B FP8 indexer keys */
#define CSA2_MX_KIDX_PAGE_BYTES 4352  /* 64 x (64 B E2M1 codes) + 64 x 4 E8M0 scales */
#define CSA2_BLOCK 8               /* positions per pool block */
#define CSA2_SWA 128               /* sliding-window rows per query token */
#define CSA2_MAX_TOPK 2048
#define CSA2_MAX_POOL_BLOCKS 2048
#define CSA2_MAX_ENTRIES 262144    /* per sequence: 1M tokens at 4:1 */
#define CSA2_MAX_INDEX_HEADS 64    /* indexer heads HI */
#define CSA2_MAX_T 256             /* query tokens per sequence (decode: 1..4; prefill chunks up to 256) */
#define CSA2_MAX_WRITE_ROWS 1024   /* rows of the cache write fused into csa2_index_full_write */
/* Output marks of the indexer calls (every output slot of the (b, t) row): */
#define CSA2_ROW_BAD_SCALE (-2)    /* an MXFP4 key of the row has a scale code outside 119..133 */
#define CSA2_ROW_UNRANKED (-3)     /* test aid csa2_test_select_path(2) only: the fast path declined */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20) /* fixed per-GPU scratch of csa2_index_full_noalloc */

enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_INVALID_ARG = -1, /* null pointer, negative or zero size, k > limit */
  CSA2_ERR_UNSUPPORTED = -2, /* a size outside what the kernels are built for */
  CSA2_ERR_WORKSPACE = -3,   /* ws NULL or ws_bytes below csa2_workspace_bytes */
  CSA2_ERR_LAUNCH = -4,      /* the HIP launch reported an error */
  CSA2_ERR_SCRATCH = -5      /* a no-allocation call needs more than its fixed scratch */
};

enum csa2_op {
  CSA2_OP_INDEX_FULL = 1,
  CSA2_OP_INDEX_REINDEX = 2,
  CSA2_OP_SPARSE_ATTN = 3
};

typedef void *csa2_stream_t; /* hipStream_t */

/*
 * FP4 main-KV cache write.  Knowledge note, "FP4 main KV": E2M1 elements,
 * one E4M3 scale per 16 channels, no second-level scale, applied after RoPE;
 * "Inside DeepSeek V4.1 Flash", "Reconstructing the 890-byte cache budget":
 * 288 B per 512-channel entry.
 *   kv_bf16   [rows][512] bf16, post-RoPE rows to store.
 *   dst_slot  [rows] int64: physical page * 64 + offset of each row; rows
 *             whose slot is outside [0, n_pages * 64) are skipped.
 *   kv_pool   [n_pages][18432] bytes.  Page layout: entry e's 256 code bytes
 *             at e * 256 (channel 2i in the low nibble of byte i, nibble =
 *             sign << 3 | magnitude code), then entry e's 32 scale bytes at
 *             16384 + e * 32.
 * Per 16-channel group: scale = E4M3 nearest to amax / 6 (ties to even,
 * saturating at 448); element = E2M1 nearest to |x| / scale (ties to even,
 * saturating at 6), sign copied from x; a zero scale gives zero magnitudes.
 */
int csa2_quantize_kv(const uint16_t *kv_bf16, int64_t rows, const int64_t *dst_slot,
                     uint8_t *kv_pool, int64_t n_pages, csa2_stream_t stream);

/*
 * Non-overlapping sequence compressor, the producer of the main-KV entries.
 * "Inside DeepSeek V4.1 Flash", deep dive "Causal Encoder-Decoder" (symbol
 * table, equation 1): C (main KV) and Z (compression weights) are projected
 * per source position and one entry stands for m positions; CSA2 groups
 * non-overlapping positions and has no absolute positional term.  The pages
 * give no formula; this call computes, per channel c of entry g,
 *   entry[g][c] = sum_i w_i C[g m + i][c],  w_i = softmax_i(Z[g m + i][c]),
 * i < m (a softmax over the group's positions), in binary32 with the weights
 * exp(Z - max Z) from the hardware base-2 exponential, rounded to bf16
 * (nearest, ties to even).  Error: within 2^-8 |entry| (the bf16 rounding)
 * plus 2^-18 sum_i w_i |C_i| of the exact value.
 *   c_bf16, z_bf16 [rows][512] finite bf16 (16-byte aligned), the source
 *                  positions.
 *   m              1, 2, 4 or 8 (the pages: 2 in the encoder, 1 in the
 *                  decoder; 4 for 4:1 compression).
 *   out_bf16       [rows / m][512] bf16 (16-byte aligned): the entries of the
 *                  complete groups; a trailing partial group forms none.
 * Feed out_bf16 to csa2_quantize_kv to write the entries into the FP4 pool.
 * Returns CSA2_ERR_INVALID_ARG for rows < 0, m <= 0, a null or misaligned
 * pointer (when an entry is formed), CSA2_ERR_UNSUPPORTED for other m,
 * CSA2_ERR_LAUNCH if the launch fails.
 */
int csa2_compress(const uint16_t *c_bf16, const uint16_t *z_bf16, int64_t rows, int32_t m,
                  uint16_t *out_bf16, csa2_stream_t stream);

/*
 * Fused RoPE + cache writes.  Knowledge note, "FP4 main KV": the main KV is
 * quantized after RoPE; the indexer keys are FP8 (E4M3).  The pages do not
 * give the rotary channels or the angles; this call takes them as follows.
 * The last 64 channels of each main-KV row (448..511) and of each indexer
 * key (64..127) are rotary: channels (2i, 2i + 1) of that slice, i < 32,
 * turn by the angle of pair i at the row's position, given by the caller as
 * rope_cs[pos][i] = (cos, sin).  With x, y the pair's bf16 values:
 *   x' = fl(fl(x cos) - fl(y sin)),  y' = fl(fl(x sin) + fl(y cos))
 * (each product and sum one binary32 operation, no fused multiply-add),
 * then x', y' rounded to bf16, nearest with ties to even.  The rotated main
 * KV is written exactly as csa2_quantize_kv writes it; the rotated indexer
 * key as E4M3 codes, nearest with ties to even, saturating at +-448, sign
 * copied (so -0 and negative values that round to 0 give 0x80).
 *   kv_bf16   [rows][512] bf16 (16-byte aligned), pre-RoPE main-KV rows.
 *   kidx_bf16 [rows][128] bf16 (8-byte aligned), pre-RoPE indexer keys.
 *   pos       [rows] int64 positions; rope_cs [max_pos][32][2] float
 *             (16-byte aligned).
 *   dst_slot  [rows] int64 physical page * 64 + offset, shared by both pools.
 *   kv_pool   [n_pages][18432] bytes, the layout of csa2_quantize_kv.
 *   kidx_pool [n_pages][64][128] bytes, the E4M3 key pool of csa2_index_full.
 * Rows whose slot lies outside [0, n_pages * 64) or whose position lies
 * outside [0, max_pos) are skipped (neither pool is written).  Inputs are
 * only read.  Returns CSA2_ERR_INVALID_ARG for negative sizes, a null or
 * misaligned pointer (rows > 0), CSA2_ERR_UNSUPPORTED beyond 2^40 bytes of
 * pool or table, CSA2_ERR_LAUNCH if the launch fails.
 */
int csa2_rope_write_caches(const uint16_t *kv_bf16, const uint16_t *kidx_bf16, int64_t rows,
                           const int64_t *pos, const float *rope_cs, int64_t max_pos,
                           const int64_t *dst_slot, uint8_t *kv_pool, uint8_t *kidx_pool,
                           int64_t n_pages, csa2_stream_t stream);

/*
 * Full mode of the hierarchical indexer.  Knowledge note, "Hierarchical
 * Sparse Indexer" (Figure 5): the Full layer scores all visible positions,
 * ranks blocks of 8 positions by their maximum score and keeps up to 2,048
 * blocks as the candidate pool; it also keeps its own top-k.
 *   q_idx      [B][T][HI][128] FP8 indexer queries.
 *   w          [B][T][HI] float head weights.
 *   kidx_pool  [n_pages][64][128] FP8 indexer keys (shared by later layers).
 *   page_table [B][max_pages] int32 physical page of each logical page.
 *   n_entries  [B] int32 visible entries per sequence (device).
 *   max_n_entries  host upper bound of n_entries (sizes the grid).
 * Score of entry j for token t (exact per-head dot rounded once to fp32,
 * ReLU, weighted, then a balanced binary tree of binary32 adds over 64 head
 * slots in ascending head order, slots HI..63 holding +0):
 *   r_h = max(fl(sum_c q[h][c] k_j[c]), +0),  t_h = fl(w_h r_h) (h < HI),
 *   s(j) = (((t_0 + t_1) + (t_2 + t_3)) + ... + (t_62 + t_63)) + 0.
 * Outputs, per (b, t):
 *   out_topk   [B][T][topk]: the topk best entries by (score desc, index asc),
 *              written in ascending index order, -1 padded when n < topk.
 *   out_pool   [B][T][pool_blocks]: the pool_blocks best blocks (block b =
 *              entries [8b, 8b+8) clipped to n) by (max score desc, block
 *              asc), ascending, -1 padded; out_pool_n [B][T] their count.
 * Requires topk <= pool_blocks (then the top-k lies inside the pool),
 * 4 <= HI <= 64 with HI % 4 == 0, 1 <= T <= 256, B * T <= 65535,
 * max_n_entries <= 262144.  Every token of a sequence sees all n_entries[b]
 * entries (csa2_index_full_causal gives each token its own count).
 */
int csa2_index_full(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                    int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                    const int32_t *n_entries, int32_t max_n_entries, int32_t B, int32_t T,
                    int32_t HI, int32_t topk, int32_t pool_blocks, int32_t *out_topk,
                    int32_t *out_pool, int32_t *out_pool_n, void *ws, size_t ws_bytes,
                    csa2_stream_t stream);

/*
 * csa2_index_full together with the step's FP4 cache write (csa2_quantize_kv
 * of `rows` rows into kv_pool, kv_pages pages), in the same launches: the
 * Full selection's workgroups write the rows before their selections.
 * The indexer reads nothing the write changes, and a reader of the new
 * entries (csa2_sparse_attn) launched after this call on the same stream sees
 * them, so the results equal the two calls in sequence; the step saves one
 * kernel launch (the selection's workgroups share the rows).  Arguments as csa2_index_full and csa2_quantize_kv (rows
 * whose slot lies outside the pool are skipped); csa2_index_full_mxfp4_write
 * takes the indexer keys in the MXFP4 layout of csa2_index_full_mxfp4.
 * Returns CSA2_ERR_INVALID_ARG for rows < 0, kv_pages < 0, or (rows > 0) a
 * null or misaligned row or pool pointer; CSA2_ERR_UNSUPPORTED for rows >
 * CSA2_MAX_WRITE_ROWS; otherwise as csa2_index_full.
 */
int csa2_index_full_write(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                          int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                          const int32_t *n_entries, int32_t max_n_entries, int32_t B, int32_t T,
                          int32_t HI, int32_t topk, int32_t pool_blocks, int32_t *out_topk,
                          int32_t *out_pool, int32_t *out_pool_n, const uint16_t *kv_bf16,
                          int64_t rows, const int64_t *dst_slot, uint8_t *kv_pool,
                          int64_t kv_pages, void *ws, size_t ws_bytes, csa2_stream_t stream);
int csa2_index_full_mxfp4_write(const uint8_t *q_idx, const float *w, const uint8_t *kidx_mx,
                                int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                                const int32_t *n_entries, int32_t max_n_entries, int32_t B,
                                int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                                int32_t *out_topk, int32_t *out_pool, int32_t *out_pool_n,
                                const uint16_t *kv_bf16, int64_t rows, const int64_t *dst_slot,
                                uint8_t *kv_pool, int64_t kv_pages, void *ws, size_t ws_bytes,
                                csa2_stream_t stream);

/*
 * Multi-token (prefill chunk) variants with causal visibility.  "Inside
 * DeepSeek V4.1 Flash", "CED: build decoder memory without running the whole
 * decoder", and the knowledge note's "CSA2: share cache, refresh selection
 * only when needed": during prefill many query tokens of a sequence run the
 * same Full / Reindex layers, each seeing only the compressed entries that
 * are complete before it.  Arguments, outputs and errors as
 * csa2_index_full / csa2_index_reindex, plus
 *   n_visible [B][T] int32 (device): token t of sequence b sees its first
 *             min(n_entries[b], n_visible[b][t]) entries (negative: none);
 *             with 4:1 compression, a token at position p sees
 *             floor((p + 1) / 4) entries.
 * Each token's top-k and pool are those of csa2_index_full over its visible
 * entries only (a pool block is clipped to them).  csa2_index_reindex_causal
 * takes the pool csa2_index_full_causal wrote for the same tokens.
 * Returns CSA2_ERR_INVALID_ARG when n_visible is NULL.
 */
int csa2_index_full_causal(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                           int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                           const int32_t *n_entries, const int32_t *n_visible, int32_t max_n_entries,
                           int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                           int32_t *out_topk, int32_t *out_pool, int32_t *out_pool_n, void *ws,
                           size_t ws_bytes, csa2_stream_t stream);
int csa2_index_reindex_causal(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                              int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                              const int32_t *n_entries, const int32_t *n_visible, int32_t B, int32_t T,
                              int32_t HI, const int32_t *pool, const int32_t *pool_n, int32_t pool_blocks,
                              int32_t topk, int32_t *out_topk, void *ws, size_t ws_bytes,
                              csa2_stream_t stream);

/*
 * csa2_index_full for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, outputs, errors and kernels, without the workspace
 * argument.  The workspace lives in a library-owned device array of
 * CSA2_NOALLOC_SCRATCH_BYTES, one copy per GPU, looked up on the first call
 * on that GPU (the caller's current device) and held until the process ends.
 * The call allocates nothing and calls no allocating routine.  Every call on
 * one GPU uses that GPU's one array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialized by the caller;
 * calls in sequence on one stream are safe.  Nothing in the array needs to
 * start at zero: each call writes every part it later reads.
 * Returns CSA2_ERR_SCRATCH (before anything is enqueued) when
 * csa2_workspace_bytes(CSA2_OP_INDEX_FULL, B, T, HI, max_n_entries, topk)
 * exceeds CSA2_NOALLOC_SCRATCH_BYTES (e.g. B * T = 4 at 262,144 entries fits),
 * CSA2_ERR_LAUNCH if the array's address cannot be found; otherwise as
 * csa2_index_full.
 */
int csa2_index_full_noalloc(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                            int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                            const int32_t *n_entries, int32_t max_n_entries, int32_t B, int32_t T,
                            int32_t HI, int32_t topk, int32_t pool_blocks, int32_t *out_topk,
                            int32_t *out_pool, int32_t *out_pool_n, csa2_stream_t stream);

/*
 * Reindex mode.  Knowledge note, "Hierarchical Sparse Indexer": later
 * Reindex layers score only the pool with their own indexer query and pick
 * their own top-k inside it; the pool is query-specific.
 *   pool [B][T][pool_blocks], pool_n [B][T]: as written by csa2_index_full.
 * Same score, ranking and output format as csa2_index_full's out_topk,
 * restricted to the positions of the first pool_n[b][t] pool blocks.
 * Returns CSA2_ERR_UNSUPPORTED when n_pages * 64 exceeds INT32_MAX.
 */
int csa2_index_reindex(const uint8_t *q_idx, const float *w, const uint8_t *kidx_pool,
                       int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                       const int32_t *n_entries, int32_t B, int32_t T, int32_t HI,
                       const int32_t *pool, const int32_t *pool_n, int32_t pool_blocks,
                       int32_t topk, int32_t *out_topk, void *ws, size_t ws_bytes,
                       csa2_stream_t stream);

/*
 * Full and Reindex modes over indexer keys in the pages' own format: E2M1
 * elements with one E8M0 scale per 32 channels, 68 B per 128-channel entry
 * (knowledge note, "FP4 main KV"; "Inside DeepSeek V4.1 Flash",
 * "Reconstructing the 890-byte cache budget").  Arguments, outputs, errors
 * and the score are those of csa2_index_full / csa2_index_reindex, except the
 * key pool:
 *   kidx_mx [n_pages][4352] bytes.  Page layout: entry e's 64 code bytes at
 *           e * 64 (channel 2i in the low nibble of byte i, nibble = sign << 3
 *           | magnitude code), then entry e's 4 scale bytes at 4096 + e * 4
 *           (byte g scales channels 32g .. 32g + 31; code s means 2^(s - 127)).
 * Scale codes 119 <= s <= 133 (2^-8 .. 2^6) are supported: every key value
 * is then a multiple of 2^-9 of magnitude <= 384 and the scores are exact as
 * above.  A (b, t) row whose scanned entries (Full: the token's visible
 * entries; Reindex: the entries of its pool blocks) hold another scale code
 * is reported instead of ranked: every out_topk slot of the row holds
 * CSA2_ROW_BAD_SCALE, and in Full mode every out_pool slot and out_pool_n
 * as well.  Other rows are unaffected.
 */
int csa2_index_full_mxfp4(const uint8_t *q_idx, const float *w, const uint8_t *kidx_mx,
                          int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                          const int32_t *n_entries, int32_t max_n_entries, int32_t B, int32_t T,
                          int32_t HI, int32_t topk, int32_t pool_blocks, int32_t *out_topk,
                          int32_t *out_pool, int32_t *out_pool_n, void *ws, size_t ws_bytes,
                          csa2_stream_t stream);
int csa2_index_reindex_mxfp4(const uint8_t *q_idx, const float *w, const uint8_t *kidx_mx,
                             int64_t n_pages, const int32_t *page_table, int32_t max_pages,
                             const int32_t *n_entries, int32_t B, int32_t T, int32_t HI,
                             const int32_t *pool, const int32_t *pool_n, int32_t pool_blocks,
                             int32_t topk, int32_t *out_topk, void *ws, size_t ws_bytes,
                             csa2_stream_t stream);

/*
 * Sparse attention over the selected FP4 entries merged with the FP8 window.
 * "Inside DeepSeek V4.1 Flash", "CSA2: reuse memory and reuse selection
 * independently": the main query attends to the selected global entries
 * together with the local window; knowledge note, "FP4 main KV": entries are
 * dequantized before attention, the window stays FP8.  Reuse mode passes the
 * latest Full/Reindex top-k buffer as topk_idx.
 *   q        [B][T][H][512] bf16 main queries.
 *   topk_idx [B][T][topk] int32 entry positions, -1 = empty slot.
 *   swa      [B][127 + T][512] FP8 window rows; token t uses rows t..t+127.
 *   out      [B][T][H][512] float; out_lse [B][T][H] float (natural log) or NULL.
 * For each (b, t, h) one softmax over J = {valid selected entries} U {window
 * rows}: logits sm_scale * q . x_j, out = sum_j p_j x_j (each 512-channel
 * row serves as key and value).  H must be 16, 32 or 64; 1 <= T <= 256
 * (a prefill chunk's tokens each with their own index set and window rows).
 */
int csa2_sparse_attn(const uint16_t *q, float sm_scale, const uint8_t *kv_pool, int64_t n_pages,
                     const int32_t *page_table, int32_t max_pages, const int32_t *n_entries,
                     const int32_t *topk_idx, int32_t topk, const uint8_t *swa, int32_t B,
                     int32_t T, int32_t H, float *out, float *out_lse, void *ws, size_t ws_bytes,
                     csa2_stream_t stream);

/* Kernels the library launches, for csa2_time_kernel. */
enum csa2_kernel {
  CSA2_K_QUANTIZE = 1,        /* cache write */
  CSA2_K_SCORE_FULL = 2,      /* Full-mode score scan */
  CSA2_K_SELECT_FULL = 3,     /* Full-mode pool + top-k selection */
  CSA2_K_SCORE_REINDEX = 4,   /* Reindex-mode score scan over the pool */
  CSA2_K_SELECT_REINDEX = 5,  /* Reindex-mode top-k selection */
  CSA2_K_ATTN_SPLIT = 6,      /* attention over row splits */
  CSA2_K_ATTN_COMBINE = 7,    /* merge of the splits */
  CSA2_K_ROPE_WRITE = 8,      /* fused RoPE + cache writes */
  CSA2_K_COMPRESS = 9,        /* sequence compressor */
  CSA2_K_COUNT = 10
};

/*
 * Measurement aid (not part of the method): from now on, record
 * `start_event` immediately before and `stop_event` immediately after each
 * launch of `kernel` on its launch stream (both are hipEvent_t created by
 * the caller; NULL, NULL turns recording off).  Lets a benchmark time one
 * kernel of a multi-kernel call with events on the right stream.  Process-
 * wide setting; not thread-safe.  Returns CSA2_OK or CSA2_ERR_INVALID_ARG.
 */
int csa2_time_kernel(int kernel, void *start_event, void *stop_event);

/*
 * Test aid (not part of the method): the path of the indexer selections.
 * The scan leaves, per row, list and workgroup, the keys at or above a local
 * threshold; the selection ranks their union when it can prove that union
 * holds the exact top-k (or pool), and the whole list otherwise.
 *   mode 0 (default): that choice; 1: always the whole lists; 2: the union
 *   only: a row it cannot rank exactly gets CSA2_ROW_UNRANKED in every
 *   output slot (and out_pool_n) instead.
 * Modes 0 and 1 give identical results; 1 and 2 let a test reach each path.
 * Process-wide setting, not thread-safe.  Returns CSA2_OK, or
 * CSA2_ERR_INVALID_ARG for another mode.
 */
int csa2_test_select_path(int mode);

/* Workspace bytes a call needs (op = enum csa2_op; `heads` = HI for the
 * indexer calls, H for attention; `max_n_entries` unused for attention). */
size_t csa2_workspace_bytes(int op, int32_t B, int32_t T, int32_t heads, int32_t max_n_entries,
                            int32_t topk);

/* Static description of a status code. */
const char *csa2_status_str(int status);

/* ABI version of this header (major * 100 + minor). */
int csa2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
