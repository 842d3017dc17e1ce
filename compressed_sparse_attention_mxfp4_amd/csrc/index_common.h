// Shared definitions of the hierarchical sparse indexer's kernels (score
// scan, selection) and of the C ABI that launches them.
#pragma once
#include "common.h"

namespace csa2 {

constexpr int kScoreThreads = 512;           // 8 waves
constexpr int kWaves = kScoreThreads / 64;
constexpr int kChunk = 64;                   // entries scored together per wave: one page
constexpr int kSub = kChunk / 16;            // 16-entry MFMA sub-tiles per chunk
constexpr int kRT = 4;                       // row tiles of 16 heads (HI <= 64)
constexpr int kMaxWaveChunks = 1024;         // chunks one wave may take in one launch
// A workgroup's chunks of one row: at most 1016 * 64 = 65,024 entries per
// token, so its 16-bit histogram counters cannot overflow.
constexpr int kMaxWgChunks = 1016;
// Coarse histogram of a workgroup's score keys: their top 10 bits.
constexpr int kHistBins = 1024;
// Fine histogram of the keys inside one coarse bin: the next 12 bits.
constexpr int kFineBins = 4096;
// Full mode: a workgroup scores the keys for a group of at most 4 query
// tokens of one sequence (each token's query limbs and histograms in LDS)
constexpr int kGroupT = 4;
// MXFP4 indexer keys: per page 64 entries x 64 code bytes (channel 2i in the
// low nibble of byte i), then 64 x 4 E8M0 scale bytes (byte g: channels
// 32g .. 32g + 31)
constexpr int kMxCodes = 64;
constexpr int kMxScaleOff = kPage * kMxCodes;        // 4,096
constexpr int kMxPageBytes = kMxScaleOff + kPage * 4;  // 4,352
constexpr int kMxScaleMin = 119, kMxScaleMax = 133;  // supported E8M0 codes (2^-8 .. 2^6)
constexpr int kBufferFlags = 0x00020000;     // raw buffer descriptor word 3 (32-bit data, no swizzle)
// The scan aims at this many workgroups in all (one per compute unit:
// each takes most of a unit's LDS), hence at most this many per row.
constexpr int kScanTarget = 256;
constexpr int kMaxSegs = kScanTarget;

// Row stride of the block-maxima buffer: ceil(max_n / 8) rounded up to a
// multiple of 4 so every row starts 16-byte aligned.
__host__ __device__ __forceinline__ int bm_stride(int max_n) {
  return ((max_n + kBlock - 1) / kBlock + 3) & ~3;
}
// Row stride of the Full-mode score buffer: max_n rounded up to a multiple
// of 8, so each 8-entry block is 32-byte aligned.
__host__ __device__ __forceinline__ int s_stride(int max_n) { return (max_n + 7) & ~7; }

// ---- candidate segments
// Every scan workgroup ends by writing, for each (b, t) row it scored and
// each of the row's lists (0: entry scores; 1: block maxima, Full mode
// only), a segment: the keys of its part of the list at or above a local
// threshold chosen so that the part's share of the list's top K lies among
// them with a wide margin, in list order, with their list positions.  A
// segment's header holds its count, the threshold key (every valid key of
// the part below it was dropped) and flags.  The selection takes the top K
// of the row's concatenated segments and checks that no dropped key could
// have ranked in it.
enum SegFlags : uint32_t {
  kSegDropped = 1u,    // some valid key of the part was below the threshold
  kSegOverflow = 2u,   // more keys reached the threshold than the segment holds
  kSegBadScale = 4u,   // an MXFP4 key of the part has a scale code outside 119..133
};
// Header of a segment, 8 bytes (read with one load, both words used):
// count in bits 0..23 and SegFlags in bits 24..31, then the threshold key.
struct SegHeader {
  uint32_t count_flags;
  uint32_t thr;
};
struct Cand {
  uint32_t key;
  int32_t pos;
};

struct ScoreArgs {
  const uint8_t* q_idx;
  const float* w;
  const uint8_t* kidx;
  int64_t n_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* n_entries;
  int max_n;
  int T;
  int HI;
  const int32_t* n_vis;   // [B][T] per-token visible entries (causal counts), or null
  int n_groups;           // full: token groups per sequence, ceil(T / 4)
  const int32_t* pool;    // pool mode
  const int32_t* pool_n;  // pool mode
  int pool_blocks;
  int topk;
  float* out_s;           // full: [B][T][s_stride(max_n)]; pool: [B][T][pool_blocks*8]
  float* out_bm;          // full: [B][T][bm_stride(max_n)]
  int rows;               // full: B * n_groups; pool: B*T
  int chunks_per_row;     // full: ceil(max_n/64); pool: ceil(pool_blocks/8)
  // static plan: every row gets wg_per_row workgroups of chunks_per_wg chunks
  int chunks_per_wg;
  int wg_per_row;
  // balanced plan (Full mode): kScanTarget workgroups shared out in
  // proportion to the rows' visible chunks times tokens (scan_plan_balanced)
  int balanced;
  SegHeader* seg_hdr;     // [B*T][2][max_segs]
  Cand* seg_cand;         // [B*T][2][seg_region]: segment i at seg_off_at(seg_k, i)
  int32_t* seg_n;         // [B*T]: segments of the row (written by segment 0)
  int max_segs;
  int seg_k;              // the larger K of the two lists (capacities)
  int64_t seg_region;
};

struct SelectArgs {
  const float* s;        // full: [B][T][s_stride(max_n)]; reindex: [B][T][pool_blocks*8] (pool order)
  const float* bm;       // full: [B][T][bm_stride(max_n)]
  const int32_t* n_entries;
  const int32_t* n_vis;      // [B][T] per-token visible entries, or null
  int max_n;
  int max_pages;
  int T;
  int topk;
  int pool_blocks;
  const int32_t* pool_in;    // reindex: [B][T][pool_blocks]
  const int32_t* pool_n_in;  // reindex: [B][T]
  int32_t* out_topk;         // [B][T][topk]
  int32_t* out_pool;         // full: [B][T][pool_blocks]
  int32_t* out_pool_n;       // full: [B][T]
  const SegHeader* seg_hdr;  // the scan's segments (ScoreArgs)
  const Cand* seg_cand;
  const int32_t* seg_n;
  int max_segs;
  int seg_k;
  int64_t seg_region;
  int segs_guess;            // the usual segment count (the candidates' early loads assume it)
  int mode;                  // test aid: 0 normal, 1 skip the segments, 2 segments only
  // full, optional: the step's cache write, spread over the workgroups
  const uint16_t* wr_rows;   // [wr_n][512] bf16
  const int64_t* wr_slots;   // [wr_n]
  uint8_t* wr_pool;          // [wr_pages][18432]
  int64_t wr_n, wr_pages;
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trip).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane((int)wave_incl_scan((uint32_t)v), 63);
}

// Segment capacities.  Segment i of a row exists only when the row has more
// than i segments, so its part's expected share of the top K is at most
// 1.5 K / (i + 1); capacities come in bands of i + 1 in [2^b, 2^(b+1)):
// twice the band's largest share plus a margin, at most K + 64.  Segment i
// of a (row, list) starts at seg_off_at(K, i) of the list's region.
__host__ __device__ __forceinline__ int seg_band(int i) {
  int b = 0;
  while ((2 << b) <= i + 1) ++b;
  return b;
}
__host__ __device__ __forceinline__ int band_cap(int K, int b) {
  const int c = (((3 * K) >> b) + 128 + 15) & ~15;
  return c < K + 64 ? c : K + 64;
}
__host__ __device__ __forceinline__ int seg_cap_at(int K, int i) { return band_cap(K, seg_band(i)); }
__host__ __device__ __forceinline__ int64_t seg_off_at(int K, int i) {
  const int b = seg_band(i);
  int64_t off = 0;
  for (int bb = 0; bb < b; ++bb) off += (int64_t)(1 << bb) * band_cap(K, bb);
  return off + (int64_t)(i + 1 - (1 << b)) * band_cap(K, b);
}

// Test aid: 0 normal; 1 the selections ignore the segments (full lists);
// 2 they use the segments only (a row whose segments cannot give the exact
// result gets -3 in every output slot and count).
int& select_mode();

}  // namespace csa2

// Static plan of the scan (workgroups per row etc.).
int csa2_score_grid(int rows, int chunks_per_row, int T_slots, int* chunks_per_wg, int* wg_per_row);
// Whether a Full-mode scan of `rows` rows of up to chunks_per_row chunks
// takes the balanced plan (its kScanTarget workgroups cover any lengths).
bool csa2_scan_balanced(int rows, int chunks_per_row);
// Launches the scan over E4M3 (mx = false) or MXFP4 indexer keys; Full mode
// (pool = false) or Reindex mode over the pool.  Fills in the grid fields.
int csa2_launch_scan(bool pool, bool mx, csa2::ScoreArgs& sa, int T_slots, hipStream_t stream);
// Launches the selection (Full: pool and top-k; Reindex: top-k) over B*T rows.
int csa2_launch_select(bool full, const csa2::SelectArgs& se, int rows, hipStream_t stream);
