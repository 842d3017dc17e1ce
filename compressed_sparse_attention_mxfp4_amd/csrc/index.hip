// C ABI of the hierarchical sparse indexer (knowledge note
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
// "Hierarchical Sparse Indexer"; "Inside DeepSeek V4.1 Flash", section
// "Hierarchical indexing bounds later searches, not every search"): argument
// checks, the workspace layout, and the launches of the score scan
// (score.hip) and the selection (select.hip).
//
// Workspace, each part 256-byte aligned:
//   Full:    scores [B][T][s_stride(max_n)] f32, block maxima
//            [B][T][bm_stride(max_n)] f32, segment headers [B][T][2][S],
//            segment candidates [B][T][2][seg_off_at(P, S)] (segment i at
//            seg_off_at(P, i)), segment counts [B][T] int32
//   Reindex: scores [B][T][pool_blocks * 8] f32, then the same segments
// where S is the most segments a row can have: the static plan's
// workgroups per row, or for the balanced plan up to 8 times the even share.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "index_common.h"

// ---------------------------------------------------------------- C ABI
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_index_common(const void* q_idx, const void* w, const void* kidx, int64_t n_pages,
                       const void* page_table, int32_t max_pages, const void* n_entries,
                       int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks) {
  if (!q_idx || !w || !kidx || !page_table || !n_entries) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || HI <= 0 || n_pages <= 0 || max_pages <= 0) return CSA2_ERR_INVALID_ARG;
  if (topk <= 0 || topk > CSA2_MAX_TOPK || pool_blocks <= 0 || pool_blocks > CSA2_MAX_POOL_BLOCKS)
    return CSA2_ERR_INVALID_ARG;
  if (HI > CSA2_MAX_INDEX_HEADS || (HI % 4) != 0) return CSA2_ERR_UNSUPPORTED;
  if (T > CSA2_MAX_T) return CSA2_ERR_UNSUPPORTED;
  if (topk > pool_blocks) return CSA2_ERR_UNSUPPORTED;
  if (B > 65535 / T) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}
}  // namespace

namespace {
struct IndexLayout {
  size_t s_off, bm_off, hdr_off, cand_off, segn_off, total;
  int max_segs, seg_k, segs_guess;
  int64_t region;
};

// Full mode: rows of the scan are (sequence, group of up to 4 tokens);
// Reindex: (b, t).
IndexLayout index_layout(bool full, int32_t B, int32_t T, int32_t max_n, int32_t pool_blocks) {
  IndexLayout L{};
  int rows, chunks, t_slots;
  if (full) {
    rows = B * ((T + csa2::kGroupT - 1) / csa2::kGroupT);
    chunks = (max_n + csa2::kChunk - 1) / csa2::kChunk;
    t_slots = T >= csa2::kGroupT ? csa2::kGroupT : (T == 3 ? 4 : T);
  } else {
    rows = B * T;
    chunks = (pool_blocks * csa2::kBlock + csa2::kChunk - 1) / csa2::kChunk;
    t_slots = 1;
  }
  int per = 0, W = 0;
  csa2_score_grid(rows, chunks, t_slots, &per, &W);
  L.seg_k = pool_blocks;  // >= topk
  if (full && csa2_scan_balanced(rows, chunks)) {
    // a row may take up to 8 times its even share of the workgroups
    const int need = std::max(1, (chunks + csa2::kMaxWgChunks - 1) / csa2::kMaxWgChunks);
    const int even = (csa2::kScanTarget + rows - 1) / rows;
    L.max_segs = std::min(csa2::kMaxSegs, std::max(std::max(W, need), 8 * even));
    L.segs_guess = std::max(1, csa2::kScanTarget / rows);
  } else {
    L.max_segs = W;
    L.segs_guess = W;
  }
  L.region = csa2::seg_off_at(L.seg_k, L.max_segs);
  const size_t bt = (size_t)B * T;
  L.s_off = 0;
  const size_t s_bytes = full ? bt * csa2::s_stride(max_n) * 4 : bt * pool_blocks * csa2::kBlock * 4;
  L.bm_off = align256(s_bytes);
  const size_t bm_bytes = full ? bt * csa2::bm_stride(max_n) * 4 : 0;
  L.hdr_off = L.bm_off + align256(bm_bytes);
  L.cand_off = L.hdr_off + align256(bt * 2 * L.max_segs * sizeof(csa2::SegHeader));
  L.segn_off = L.cand_off + align256(bt * 2 * (size_t)L.region * sizeof(csa2::Cand));
  L.total = L.segn_off + align256(bt * sizeof(int32_t));
  return L;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}
}  // namespace

extern "C" size_t csa2_index_ws_bytes(int op, int32_t B, int32_t T, int32_t max_n,
                                      int32_t pool_blocks) {
  if (B <= 0 || T <= 0 || pool_blocks <= 0) return 0;
  if (op == CSA2_OP_INDEX_FULL) return max_n > 0 ? index_layout(true, B, T, max_n, pool_blocks).total : 0;
  return index_layout(false, B, T, 0, pool_blocks).total;
}

namespace {
int index_full_impl(bool mx, const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool, int64_t n_pages,
                    const int32_t* page_table, int32_t max_pages, const int32_t* n_entries,
                    const int32_t* n_vis, int32_t max_n_entries, int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                    int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, void* ws, size_t ws_bytes,
                    csa2_stream_t stream, const uint16_t* wr_rows = nullptr, int64_t wr_n = 0,
                    const int64_t* wr_slots = nullptr, uint8_t* wr_pool = nullptr,
                    int64_t wr_pages = 0) {
  int st = check_index_common(q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, B, T,
                              HI, topk, pool_blocks);
  if (st) return st;
  if (!out_topk || !out_pool || !out_pool_n) return CSA2_ERR_INVALID_ARG;
  if (max_n_entries <= 0) return CSA2_ERR_INVALID_ARG;
  if (max_n_entries > CSA2_MAX_ENTRIES) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_index_ws_bytes(CSA2_OP_INDEX_FULL, B, T, max_n_entries, pool_blocks);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  csa2::ScoreArgs sa{};
  sa.q_idx = q_idx;
  sa.w = w;
  sa.kidx = kidx_pool;
  sa.n_pages = n_pages;
  sa.page_table = page_table;
  sa.max_pages = max_pages;
  sa.n_entries = n_entries;
  sa.max_n = max_n_entries;
  sa.T = T;
  sa.HI = HI;
  sa.n_vis = n_vis;
  sa.n_groups = (T + csa2::kGroupT - 1) / csa2::kGroupT;
  const IndexLayout lay = index_layout(true, B, T, max_n_entries, pool_blocks);
  sa.pool_blocks = pool_blocks;
  sa.topk = topk;
  sa.out_s = ws_at<float>(ws, lay.s_off);
  sa.out_bm = ws_at<float>(ws, lay.bm_off);
  sa.seg_hdr = ws_at<csa2::SegHeader>(ws, lay.hdr_off);
  sa.seg_cand = ws_at<csa2::Cand>(ws, lay.cand_off);
  sa.seg_n = ws_at<int32_t>(ws, lay.segn_off);
  sa.max_segs = lay.max_segs;
  sa.seg_k = lay.seg_k;
  sa.seg_region = lay.region;
  sa.rows = B * sa.n_groups;
  sa.chunks_per_row = (max_n_entries + csa2::kChunk - 1) / csa2::kChunk;
  const int t_slots = T >= csa2::kGroupT ? csa2::kGroupT : (T == 3 ? 4 : T);
  st = csa2_launch_scan(false, mx, sa, t_slots, (hipStream_t)stream);
  if (st) return st;
  csa2::SelectArgs se{};
  se.s = sa.out_s;
  se.bm = sa.out_bm;
  se.n_entries = n_entries;
  se.n_vis = n_vis;
  se.max_n = max_n_entries;
  se.max_pages = max_pages;
  se.T = T;
  se.topk = topk;
  se.pool_blocks = pool_blocks;
  se.out_topk = out_topk;
  se.out_pool = out_pool;
  se.out_pool_n = out_pool_n;
  se.seg_hdr = sa.seg_hdr;
  se.seg_cand = sa.seg_cand;
  se.seg_n = sa.seg_n;
  se.max_segs = sa.max_segs;
  se.seg_k = sa.seg_k;
  se.seg_region = sa.seg_region;
  se.segs_guess = lay.segs_guess;
  se.wr_rows = wr_rows;
  se.wr_slots = wr_slots;
  se.wr_pool = wr_pool;
  se.wr_n = wr_n;
  se.wr_pages = wr_pages;
  return csa2_launch_select(true, se, B * T, (hipStream_t)stream);
}

int index_reindex_impl(bool mx, const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                       int64_t n_pages, const int32_t* page_table, int32_t max_pages, const int32_t* n_entries,
                       const int32_t* n_vis, int32_t B, int32_t T, int32_t HI, const int32_t* pool, const int32_t* pool_n,
                       int32_t pool_blocks, int32_t topk, int32_t* out_topk, void* ws, size_t ws_bytes,
                       csa2_stream_t stream) {
  int st = check_index_common(q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, B, T,
                              HI, topk, pool_blocks);
  if (st) return st;
  if (!pool || !pool_n || !out_topk) return CSA2_ERR_INVALID_ARG;
  // the scan keeps physical entry indices (page * 64 + entry) in 32 bits
  if (n_pages > (int64_t)INT32_MAX / csa2::kPage) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_index_ws_bytes(CSA2_OP_INDEX_REINDEX, B, T, 0, pool_blocks);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  const int max_n = (int)std::min<int64_t>((int64_t)max_pages * csa2::kPage, CSA2_MAX_ENTRIES);
  csa2::ScoreArgs sa{};
  sa.q_idx = q_idx;
  sa.w = w;
  sa.kidx = kidx_pool;
  sa.n_pages = n_pages;
  sa.page_table = page_table;
  sa.max_pages = max_pages;
  sa.n_entries = n_entries;
  sa.max_n = max_n;
  sa.T = T;
  sa.HI = HI;
  sa.n_vis = n_vis;
  sa.n_groups = 1;
  sa.pool = pool;
  sa.pool_n = pool_n;
  sa.pool_blocks = pool_blocks;
  const IndexLayout lay = index_layout(false, B, T, 0, pool_blocks);
  sa.topk = topk;
  sa.out_s = ws_at<float>(ws, lay.s_off);
  sa.seg_hdr = ws_at<csa2::SegHeader>(ws, lay.hdr_off);
  sa.seg_cand = ws_at<csa2::Cand>(ws, lay.cand_off);
  sa.seg_n = ws_at<int32_t>(ws, lay.segn_off);
  sa.max_segs = lay.max_segs;
  sa.seg_k = lay.seg_k;
  sa.seg_region = lay.region;
  sa.rows = B * T;
  sa.chunks_per_row = (pool_blocks * csa2::kBlock + csa2::kChunk - 1) / csa2::kChunk;
  st = csa2_launch_scan(true, mx, sa, 1, (hipStream_t)stream);
  if (st) return st;
  csa2::SelectArgs se{};
  se.s = sa.out_s;
  se.n_entries = n_entries;
  se.n_vis = n_vis;
  se.max_n = max_n;
  se.max_pages = max_pages;
  se.T = T;
  se.topk = topk;
  se.pool_blocks = pool_blocks;
  se.pool_in = pool;
  se.pool_n_in = pool_n;
  se.out_topk = out_topk;
  se.seg_hdr = sa.seg_hdr;
  se.seg_cand = sa.seg_cand;
  se.seg_n = sa.seg_n;
  se.max_segs = sa.max_segs;
  se.seg_k = sa.seg_k;
  se.seg_region = sa.seg_region;
  se.segs_guess = lay.segs_guess;
  return csa2_launch_select(false, se, B * T, (hipStream_t)stream);
}
}  // namespace

extern "C" int csa2_index_full(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                               int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                               const int32_t* n_entries, int32_t max_n_entries, int32_t B,
                               int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                               int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, void* ws,
                               size_t ws_bytes, csa2_stream_t stream) {
  return index_full_impl(false, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, nullptr,
                         max_n_entries, B,
                         T, HI, topk, pool_blocks, out_topk, out_pool, out_pool_n, ws, ws_bytes, stream);
}

extern "C" int csa2_index_full_mxfp4(const uint8_t* q_idx, const float* w, const uint8_t* kidx_mx,
                                     int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                     const int32_t* n_entries, int32_t max_n_entries, int32_t B,
                                     int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                                     int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, void* ws,
                                     size_t ws_bytes, csa2_stream_t stream) {
  return index_full_impl(true, q_idx, w, kidx_mx, n_pages, page_table, max_pages, n_entries, nullptr,
                         max_n_entries, B,
                         T, HI, topk, pool_blocks, out_topk, out_pool, out_pool_n, ws, ws_bytes, stream);
}

extern "C" int csa2_index_reindex(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                                  int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                  const int32_t* n_entries, int32_t B, int32_t T, int32_t HI,
                                  const int32_t* pool, const int32_t* pool_n, int32_t pool_blocks,
                                  int32_t topk, int32_t* out_topk, void* ws, size_t ws_bytes,
                                  csa2_stream_t stream) {
  return index_reindex_impl(false, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, nullptr, B, T,
                            HI, pool,
                            pool_n, pool_blocks, topk, out_topk, ws, ws_bytes, stream);
}

extern "C" int csa2_index_reindex_mxfp4(const uint8_t* q_idx, const float* w, const uint8_t* kidx_mx,
                                        int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                        const int32_t* n_entries, int32_t B, int32_t T, int32_t HI,
                                        const int32_t* pool, const int32_t* pool_n, int32_t pool_blocks,
                                        int32_t topk, int32_t* out_topk, void* ws, size_t ws_bytes,
                                        csa2_stream_t stream) {
  return index_reindex_impl(true, q_idx, w, kidx_mx, n_pages, page_table, max_pages, n_entries, nullptr, B, T,
                            HI, pool,
                            pool_n, pool_blocks, topk, out_topk, ws, ws_bytes, stream);
}

extern "C" int csa2_index_full_causal(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                                      int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                      const int32_t* n_entries, const int32_t* n_visible, int32_t max_n_entries,
                                      int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                                      int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, void* ws,
                                      size_t ws_bytes, csa2_stream_t stream) {
  if (!n_visible) return CSA2_ERR_INVALID_ARG;
  return index_full_impl(false, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, n_visible,
                         max_n_entries, B, T, HI, topk, pool_blocks, out_topk, out_pool, out_pool_n, ws, ws_bytes,
                         stream);
}

extern "C" int csa2_index_reindex_causal(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                                         int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                         const int32_t* n_entries, const int32_t* n_visible, int32_t B, int32_t T,
                                         int32_t HI, const int32_t* pool, const int32_t* pool_n,
                                         int32_t pool_blocks, int32_t topk, int32_t* out_topk, void* ws,
                                         size_t ws_bytes, csa2_stream_t stream) {
  if (!n_visible) return CSA2_ERR_INVALID_ARG;
  return index_reindex_impl(false, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, n_visible, B, T,
                            HI, pool, pool_n, pool_blocks, topk, out_topk, ws, ws_bytes, stream);
}

static int index_full_write_impl(bool mx, const uint8_t* q_idx, const float* w,
                                 const uint8_t* kidx_pool, int64_t n_pages,
                                 const int32_t* page_table, int32_t max_pages,
                                 const int32_t* n_entries, int32_t max_n_entries, int32_t B,
                                 int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                                 int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n,
                                 const uint16_t* kv_bf16, int64_t rows, const int64_t* dst_slot,
                                 uint8_t* kv_pool, int64_t kv_pages, void* ws, size_t ws_bytes,
                                 csa2_stream_t stream) {
  if (rows < 0 || kv_pages < 0) return CSA2_ERR_INVALID_ARG;
  if (rows > CSA2_MAX_WRITE_ROWS) return CSA2_ERR_UNSUPPORTED;
  if (rows > 0 && (!kv_bf16 || !dst_slot || !kv_pool || ((uintptr_t)kv_bf16 & 15) ||
                   ((uintptr_t)kv_pool & 7)))
    return CSA2_ERR_INVALID_ARG;
  if (kv_pages > ((int64_t)1 << 40) / csa2::kPageBytes) return CSA2_ERR_UNSUPPORTED;
  return index_full_impl(mx, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, nullptr,
                         max_n_entries, B, T, HI, topk, pool_blocks, out_topk, out_pool, out_pool_n,
                         ws, ws_bytes, stream, kv_bf16, rows, dst_slot, kv_pool, kv_pages);
}

#define CSA2_INDEX_FULL_WRITE_PARAMS                                                            \
  const uint8_t *q_idx, const float *w, const uint8_t *kidx, int64_t n_pages,                   \
      const int32_t *page_table, int32_t max_pages, const int32_t *n_entries,                   \
      int32_t max_n_entries, int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks, \
      int32_t *out_topk, int32_t *out_pool, int32_t *out_pool_n, const uint16_t *kv_bf16,       \
      int64_t rows, const int64_t *dst_slot, uint8_t *kv_pool, int64_t kv_pages, void *ws,       \
      size_t ws_bytes, csa2_stream_t stream
#define CSA2_INDEX_FULL_WRITE_ARGS                                                              \
  q_idx, w, kidx, n_pages, page_table, max_pages, n_entries, max_n_entries, B, T, HI, topk,     \
      pool_blocks, out_topk, out_pool, out_pool_n, kv_bf16, rows, dst_slot, kv_pool, kv_pages,  \
      ws, ws_bytes, stream

extern "C" int csa2_index_full_write(CSA2_INDEX_FULL_WRITE_PARAMS) {
  return index_full_write_impl(false, CSA2_INDEX_FULL_WRITE_ARGS);
}

extern "C" int csa2_index_full_mxfp4_write(CSA2_INDEX_FULL_WRITE_PARAMS) {
  return index_full_write_impl(true, CSA2_INDEX_FULL_WRITE_ARGS);
}

// ---------------------------------------------------------------- no allocation
// csa2_index_full with its workspace in a fixed library-owned device array,
// for callers that cannot allocate.  In host code `scratch` names a host-side
// stand-in, not the device copy: its device address is looked up once per
// GPU (with that GPU current) and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// Device address of the current GPU's copy of `scratch`.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return CSA2_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CSA2_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}
}  // namespace

extern "C" int csa2_index_full_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                                       int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                       const int32_t* n_entries, int32_t max_n_entries, int32_t B,
                                       int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                                       int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n,
                                       csa2_stream_t stream) {
  int st = check_index_common(q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, B, T, HI,
                              topk, pool_blocks);
  if (st) return st;
  if (!out_topk || !out_pool || !out_pool_n || max_n_entries <= 0) return CSA2_ERR_INVALID_ARG;
  if (max_n_entries > CSA2_MAX_ENTRIES) return CSA2_ERR_UNSUPPORTED;
  if (csa2_index_ws_bytes(CSA2_OP_INDEX_FULL, B, T, max_n_entries, pool_blocks) > CSA2_NOALLOC_SCRATCH_BYTES)
    return CSA2_ERR_SCRATCH;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st) return st;
  return index_full_impl(false, q_idx, w, kidx_pool, n_pages, page_table, max_pages, n_entries, nullptr,
                         max_n_entries, B,
                         T, HI, topk, pool_blocks, out_topk, out_pool, out_pool_n, ws,
                         CSA2_NOALLOC_SCRATCH_BYTES, stream);
}
