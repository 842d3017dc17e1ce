// Hierarchical sparse indexer: Full scan, block-max pool, Reindex over the
// pool (knowledge note "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression", section "Hierarchical Sparse Indexer", Figure 5; "Inside
// DeepSeek V4.1 Flash", section "Hierarchical indexing bounds later searches,
// not every search").
//
// Score of entry j for one query token (per indexer head h):
//   d_h = exact sum_c q[h][c] k_j[c], rounded once to binary32
//   t_h = fl(w_h * max(d_h, +0)) for h < HI, +0 for HI <= h < 64
//   s_j = balanced binary tree of binary32 adds over t_0 .. t_63 in
//         ascending order, ((t_0 + t_1) + (t_2 + t_3)) + ..., then + 0.
//
// Exactness on MFMA.  Every E4M3 value is M * 2^-9 with M an integer,
// |M| <= 229,376 < 2^18.
//  - Fast path (f16 MFMA): keys are converted to f16 (exact for every code);
//    the query, when every |q| < 32, is split as M = ql + 2^7 qm with ql in
//    [0, 127] and qm in [-128, 127], both exact in f16.  S_l = ql . k and
//    S_m = qm . k come from v_mfma_f32_16x16x32_f16; when the entry's
//    sum_c k_c^2 < 500 (so sum_c |k_c| < 253), every partial sum of either
//    is a multiple of 2^-9 below 2^15, exact in binary32 in any order, and
//    fl(2^9 q.k) = fl(S_l + 2^7 S_m) is one fused multiply-add.
//  - General path (int8 MFMA), for chunks with an entry over that bound or
//    rows whose query has some |q| >= 32: three limbs per side,
//    M = lo + 2^7 mid + 2^14 top (lo, mid in [0, 127], top signed), every
//    limb-pair dot an exact int32 from v_mfma_i32_16x16x64_i8, five weighted
//    partial sums combined exactly in binary64 (at most 43 significant
//    bits) and rounded once.
// The FP8 MFMA is not used: it aligns each group of 8 products to the group
// maximum and keeps about 13 bits, so it does not return the exactly
// rounded dot.
//
// MFMA lane layout (16x16 tiles): lane l holds row (l & 15) of A and column
// (l & 15) of B, K elements 8*(l >> 4) .. +7 of a 32-deep f16 slice (16*(l >>
// 4) .. +15 of a 64-deep int8 slice); the 4 outputs of lane l are rows
// 4*(l >> 4) + i, column l & 15.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "fp4.h"

// Every multiply and add of the score is its own binary32 operation: no
// multiply-add contraction anywhere in this file.
#pragma clang fp contract(off)

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
// Level-1 histogram of the selections: score keys by their top 10 bits.
constexpr int kHistBins = 1024;
// Full mode: a workgroup scores the keys for a group of at most 4 query
// tokens of one sequence (each token's query limbs and histograms in LDS)
constexpr int kGroupT = 4;
// MXFP4 indexer keys: per page 64 entries x 64 code bytes (channel 2i in the
// low nibble of byte i), then 64 x 4 E8M0 scale bytes (byte g: channels
// 32g .. 32g + 31)
constexpr int kMxCodes = 64;
constexpr int kMxScaleOff = kPage * kMxCodes;        // 4,096
constexpr int kMxPageBytes = kMxScaleOff + kPage * 4;  // 4,352
constexpr int kBufferFlags = 0x00020000;     // raw buffer descriptor word 3 (32-bit data, no swizzle)

// General split of the 4 FP8 codes of one dword: M = value * 2^9 (exact
// integer in binary32, |M| < 2^18) = lo + 2^7 mid + 2^14 top with lo, mid
// in [0, 127] and top signed; byte i of each plane is code i's limb.
__device__ __forceinline__ void limbs3_word(uint32_t x, uint32_t& lo, uint32_t& mid, uint32_t& top) {
  const v2f a01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 512.0f, false);
  const v2f a23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 512.0f, true);
  const uint32_t M[4] = {(uint32_t)(int)a01[0], (uint32_t)(int)a01[1], (uint32_t)(int)a23[0],
                         (uint32_t)(int)a23[1]};
  lo = mid = top = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= (M[i] & 127u) << (8 * i);
    mid |= ((M[i] >> 7) & 127u) << (8 * i);
    top |= ((M[i] >> 14) & 255u) << (8 * i);  // low byte of the arithmetic shift
  }
}

// 16 FP8 codes -> general lo, mid and top limb planes.
__device__ __forceinline__ void limbs3(v4u codes, v4i& lo, v4i& mid, v4i& top) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t l, m, t;
    limbs3_word(codes[d], l, m, t);
    lo[d] = (int)l;
    mid[d] = (int)m;
    top[d] = (int)t;
  }
}

// E8M0 scale code -> its binary32 value times 2^e (codes 119 .. 133 and
// small e keep it a normal number)
__device__ __forceinline__ float e8m0_times_pow2(uint32_t s, int e) { return __uint_as_float((s + e) << 23); }

// General limbs of one MXFP4 half (s2 = 0: channels [16g, 16g+16), 1:
// [64+16g, 64+16g+16)), in the layout limbs3 gives FP8 codes: M = value * 2^9
// is an exact integer (|M| <= 384 * 2^9 < 2^18) under the supported scales.
__device__ __forceinline__ void limbs3_mx(const v4u (&mx)[2], int s2, int g, v4i& lo, v4i& mid, v4i& top) {
  const uint32_t s = (mx[1][0] >> (8 * (2 * s2 + (g >> 1)))) & 0xFFu;
  const float sc = e8m0_times_pow2(s, 9);  // scale * 2^9
  uint32_t M[16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t wd = mx[0][2 * s2 + i];
    const v2f m0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 0);
    const v2f m1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 1);
    const v2f m2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 2);
    const v2f m3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, sc, 3);
    const float v[8] = {m0[0], m0[1], m1[0], m1[1], m2[0], m2[1], m3[0], m3[1]};
#pragma unroll
    for (int e = 0; e < 8; ++e) M[8 * i + e] = (uint32_t)(int)v[e];
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t l = 0u, m = 0u, t = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = M[4 * d + i];
      l |= (x & 127u) << (8 * i);
      m |= ((x >> 7) & 127u) << (8 * i);
      t |= ((x >> 14) & 255u) << (8 * i);
    }
    lo[d] = (int)l;
    mid[d] = (int)m;
    top[d] = (int)t;
  }
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Eight f16 ones (an MFMA operand whose rows all sum the other operand).
__device__ __forceinline__ v8h ones8() {
  const v8h o = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                 (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  return o;
}

__device__ __forceinline__ v4i mfma8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Maximum over each aligned group of 8 lanes, in every lane of the group
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror).
__device__ __forceinline__ uint32_t group8_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
  return m;
}

// Row stride of the block-maxima buffer: ceil(max_n / 8) rounded up to a
// multiple of 4 so every row starts 16-byte aligned.
__host__ __device__ __forceinline__ int bm_stride(int max_n) {
  return ((max_n + kBlock - 1) / kBlock + 3) & ~3;
}
// Row stride of the Full-mode score buffer: max_n rounded up to a multiple
// of 8, so each 8-entry block is 32-byte aligned.
__host__ __device__ __forceinline__ int s_stride(int max_n) { return (max_n + 7) & ~7; }

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
  float* out_s;           // full: [B][T][s_stride(max_n)]; pool: [B][T][pool_blocks*8]
  float* out_bm;          // full: [B][T][bm_stride(max_n)]
  int rows;               // full: B * n_groups; pool: B*T
  int chunks_per_row;     // full: ceil(max_n/64); pool: ceil(pool_blocks/8)
  int chunks_per_wg;      // chunks of one row per workgroup
  int wg_per_row;         // workgroups per row
  uint32_t* hist;         // [B][T][2][kHistBins]: counts of the visible entries' and the
                          // blocks' score keys by their top 10 bits (cleared by the scan)
  int clear_hist;         // 0 only under the test aid that keeps the histograms
};

// Adds 1 to bin `bin` of a histogram of 16-bit counters packed two per word.
__device__ __forceinline__ void hist_add16(uint32_t* h, uint32_t bin) {
  atomicAdd(&h[bin >> 1], 1u << ((bin & 1u) << 4));
}

// Keys of one chunk for one wave: lane (g, col) holds entry 16*st + col of
// the chunk, channels [16g, 16g+16) and [64+16g, 64+16g+16).
struct ChunkKeys {
  v4u k[kSub][2];
};

// Row context of a wave: sequence b, token t, visible entries n, pool row.
struct RowCtx {
  int b = 0, t = 0, n = 0, n_pos = 0;
  const int32_t* pool_row = nullptr;
};

// Full mode: row = b * n_groups + token group, t_full the wave's token
// (live: the token exists; the dead fourth slot of a group of three sees
// nothing).  Token t of sequence b sees its first min(n_entries[b],
// n_vis[b][t]) entries.
template <bool POOL>
__device__ __forceinline__ void row_ctx(const ScoreArgs& a, int row, int t_full, bool live, RowCtx& r) {
  if (POOL) {
    r.b = row / a.T;
    r.t = row % a.T;
  } else {
    r.b = row / a.n_groups;
    r.t = t_full;
  }
  int n = a.n_entries[r.b];
  n = min(n, a.max_n);
  n = max(0, min(n, a.max_pages * kPage));
  if (a.n_vis != nullptr) n = max(0, min(n, a.n_vis[(int64_t)r.b * a.T + r.t]));
  if (!live) n = 0;
  r.n = n;
  if (POOL) {
    r.pool_row = a.pool + (int64_t)row * a.pool_blocks;
    const int pn = max(0, min(a.pool_n[row], a.pool_blocks));
    r.n_pos = pn * kBlock;
  } else {
    r.n_pos = n;
  }
}

// Position p of the row's list -> entry index j, or -1 when not visible.
template <bool POOL>
__device__ __forceinline__ int entry_of(const ScoreArgs& a, const RowCtx& r, int p) {
  if (p >= r.n_pos) return -1;
  int j = p;
  if (POOL) {
    const int blk = r.pool_row[p >> 3];
    j = (blk >= 0 && blk < (r.n + kBlock - 1) / kBlock) ? blk * kBlock + (p & 7) : r.n;
  }
  if (j >= r.n) return -1;
  return phys_page(a.page_table, a.max_pages, a.n_pages, r.b, j >> 6) >= 0 ? j : -1;
}

// Physical page of a Full-mode chunk (logical page `chunk`), or -1 when
// none of its entries is visible or the page is not usable.
__device__ __forceinline__ int64_t chunk_page(const ScoreArgs& a, const RowCtx& r, int chunk) {
  return chunk * kChunk < r.n ? phys_page(a.page_table, a.max_pages, a.n_pages, r.b, chunk) : -1;
}

// Loads the keys of sub-tile st (entries 16 st .. 16 st + 15) of a chunk:
// lane (g, col) gets entry 16 st + col, channels [16g, 16g+16) and
// [64+16g, 64+16g+16); entries that are not visible read as zero.  Full
// mode: `pg` is the chunk's page (chunk_page), read through a buffer
// descriptor whose record count ends at the sub-tile's last visible entry,
// so the loads need no predicate (the hardware returns zero past the count).
// MXFP4 keys (MX): k[0] holds the 16 + 16 channels' code bytes (dwords 0, 1:
// channels [16g, 16g+16); dwords 2, 3: [64+16g, 64+16g+16)), k[1][0] the
// entry's 4 scale bytes.
template <bool POOL, bool MX>
__device__ __forceinline__ void load_sub(const ScoreArgs& a, const RowCtx& r, int chunk, int64_t pg, int st,
                                         int g, int col, v4u (&k)[2]) {
  if (MX) {
    v2u c0 = {0u, 0u}, c1 = {0u, 0u};
    uint32_t sw = 0u;
    if (!POOL) {
      const int nv = pg >= 0 ? min(r.n - chunk * kChunk, kChunk) : 0;
      const uint8_t* page = a.kidx + (pg >= 0 ? pg * kMxPageBytes : 0);
      const int nst = __builtin_amdgcn_readfirstlane(min(max(nv - 16 * st, 0), 16));
      const __amdgpu_buffer_rsrc_t rc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(page + st * 16 * kMxCodes), 0, nst * kMxCodes, kBufferFlags);
      const __amdgpu_buffer_rsrc_t rsc =
          __builtin_amdgcn_make_buffer_rsrc((void*)(page + kMxScaleOff + st * 16 * 4), 0, nst * 4, kBufferFlags);
      const uint32_t lofs = (uint32_t)(col * kMxCodes + 8 * g);
      c0 = __builtin_amdgcn_raw_buffer_load_b64(rc, lofs, 0, 0);
      c1 = __builtin_amdgcn_raw_buffer_load_b64(rc, lofs + 32, 0, 0);
      sw = __builtin_amdgcn_raw_buffer_load_b32(rsc, (uint32_t)(col * 4), 0, 0);
    } else {
      const int j = entry_of<POOL>(a, r, chunk * kChunk + st * 16 + col);
      if (j >= 0) {
        const int64_t p = phys_page(a.page_table, a.max_pages, a.n_pages, r.b, j >> 6);
        const uint8_t* page = a.kidx + p * kMxPageBytes;
        c0 = *reinterpret_cast<const v2u*>(page + (j & 63) * kMxCodes + 8 * g);
        c1 = *reinterpret_cast<const v2u*>(page + (j & 63) * kMxCodes + 32 + 8 * g);
        sw = *reinterpret_cast<const uint32_t*>(page + kMxScaleOff + (j & 63) * 4);
      }
    }
    k[0] = v4u{c0[0], c0[1], c1[0], c1[1]};
    k[1] = v4u{sw, 0u, 0u, 0u};
    return;
  }
  if (!POOL) {
    const int nv = pg >= 0 ? min(r.n - chunk * kChunk, kChunk) : 0;
    const uint8_t* base = a.kidx + (pg >= 0 ? pg * (kPage * kDI) : 0) + st * 16 * kDI;
    // readfirstlane: the clamp would otherwise become a vector med3 and the
    // descriptor a per-lane value, loaded through a waterfall loop
    const int nst = __builtin_amdgcn_readfirstlane(min(max(nv - 16 * st, 0), 16));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nst * kDI, kBufferFlags);
    const uint32_t lofs = (uint32_t)(col * kDI + 16 * g);
    k[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, lofs, 0, 0);
    k[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lofs + 64, 0, 0);
    return;
  }
  const int j = entry_of<POOL>(a, r, chunk * kChunk + st * 16 + col);
  v4u k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0};
  if (j >= 0) {
    const int64_t p = phys_page(a.page_table, a.max_pages, a.n_pages, r.b, j >> 6);
    const v4u* src = reinterpret_cast<const v4u*>(a.kidx + p * (kPage * kDI) + (j & 63) * kDI + 16 * g);
    k0 = __builtin_nontemporal_load(src);
    k1 = __builtin_nontemporal_load(src + 4);
  }
  k[0] = k0;
  k[1] = k1;
}

// Loads all sub-tiles of a chunk; returns whether the page is usable (Full
// mode; true in pool mode).
template <bool POOL, bool MX>
__device__ __forceinline__ bool load_chunk(const ScoreArgs& a, const RowCtx& r, int chunk, int g, int col,
                                           ChunkKeys& ck) {
  const int64_t pg = POOL ? 0 : chunk_page(a, r, chunk);
#pragma unroll
  for (int st = 0; st < kSub; ++st) load_sub<POOL, MX>(a, r, chunk, pg, st, g, col, ck.k[st]);
  return POOL || pg >= 0;
}

// Writes the chunk's scores (lane e: entry e of the chunk; NaN, i.e. key 0,
// for positions that are not visible) and, in Full mode, the maxima of its
// blocks of 8.  Counts the visible entries' keys in hist_s and the blocks'
// in hist_bm (LDS, 16-bit counters).
template <bool POOL>
__device__ __forceinline__ void emit_chunk(const ScoreArgs& a, const RowCtx& rc, int chunk, float s,
                                           bool page_ok, uint32_t* hist_s, uint32_t* hist_bm) {
  const int lane = lane_id();
  const int p = chunk * kChunk + lane;
  const bool valid = POOL ? entry_of<POOL>(a, rc, p) >= 0 : (page_ok && p < rc.n);
  float* out_s_row = a.out_s + ((int64_t)rc.b * a.T + rc.t) *
                                   (POOL ? (int64_t)a.pool_blocks * kBlock : (int64_t)s_stride(a.max_n));
  // order-preserving key of the score; 0 (stored as NaN) when not visible
  const uint32_t key = valid ? score_key(s) : 0u;
  if (p < rc.n_pos) out_s_row[p] = key_score(key);
  if (valid) hist_add16(hist_s, key >> 22);
  if (!POOL) {
    const uint32_t m = group8_max(key);
    if ((lane & 7) == 0 && p < rc.n_pos) {
      a.out_bm[((int64_t)rc.b * a.T + rc.t) * bm_stride(a.max_n) + (p >> 3)] = key_score(m);
      if (m != 0u) hist_add16(hist_bm, m >> 22);
    }
  }
}

// Head of MFMA row r = 4 g + i of row tile rt: 16 g + 4 rt + i.  Lane
// (g, col) then holds, for entry col of a sub-tile, the 16 consecutive heads
// 16 g .. 16 g + 15 of the pairwise head sum (element i of tile rt).
__device__ __forceinline__ int tile_head(int rt, int row) { return 16 * (row >> 2) + 4 * rt + (row & 3); }

// Pairwise sum of the 64 head terms of entry col (lane (g, col) holds
// p[rt][i] = term of head 16 g + 4 rt + i): levels 1..4 inside the lane,
// 5 and 6 across the lanes l, l ^ 16, l ^ 32, then + 0 (no -0).  Every
// lane (g, col) returns the sum of entry col.
__device__ __forceinline__ float head_sum(const v4f (&p)[kRT]) {
  float q4[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) q4[rt] = (p[rt][0] + p[rt][1]) + (p[rt][2] + p[rt][3]);
  const float s16 = (q4[0] + q4[1]) + (q4[2] + q4[3]);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s16), __float_as_uint(s16), false, false);
  const float s32 = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s32), __float_as_uint(s32), false, false);
  return (__uint_as_float(r[0]) + __uint_as_float(r[1])) + 0.0f;
}

// The same from the in-lane sums q4[rt] = (p[rt][0] + p[rt][1]) +
// (p[rt][2] + p[rt][3]) (levels 1 and 2).
__device__ __forceinline__ float head_sum4(const float (&q4)[kRT]) {
  const float s16 = (q4[0] + q4[1]) + (q4[2] + q4[3]);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s16), __float_as_uint(s16), false, false);
  const float s32 = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s32), __float_as_uint(s32), false, false);
  return (__uint_as_float(r[0]) + __uint_as_float(r[1])) + 0.0f;
}

// Lane e = 16 g + col keeps the sum of entry e: sub-tile g's sum (every
// lane (g', col) holds the sum of entry 16 st + col of sub-tile st).
__device__ __forceinline__ float keep_subtile(float mine, float sum, int st, int lane) {
  return (lane >> 4) == st ? sum : mine;
}

// Query of one token in the general split: for row tile rt and half s2,
// the lo, mid and top planes of channels [64 s2 + 16 g, 64 s2 + 16 g + 16)
// of head tile_head(rt, col), as lane (g, col) feeds them to the int8 MFMA.
struct GenQuery {
  v4i lo[kRT][2], mid[kRT][2], top[kRT][2];
};

__device__ __forceinline__ void general_query(const ScoreArgs& a, int64_t qrow0, GenQuery& gq) {
  const int lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int h = tile_head(rt, col);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      v4u qc = {0, 0, 0, 0};
      if (h < a.HI) qc = reinterpret_cast<const v4u*>(a.q_idx + (qrow0 + h) * kDI + 16 * g)[4 * s2];
      limbs3(qc, gq.lo[rt][s2], gq.mid[rt][s2], gq.top[rt][s2]);
    }
  }
}

// General exact path for one chunk: three limb planes on both sides, five
// partial sums per dot combined exactly in binary64 and rounded once.
// Reads the chunk's codes again; returns this lane's entry score before
// validity masking.  wreg[rt][i] holds w * 2^-9 of head tile_head(rt, 4 g + i).
template <bool POOL, bool MX>
__device__ __forceinline__ float general_chunk(const ScoreArgs& a, const RowCtx& rc, int chunk, const GenQuery& gq,
                                               const v4f (&wreg)[kRT], bool& page_ok) {
  const int lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  ChunkKeys raw;
  page_ok = load_chunk<POOL, MX>(a, rc, chunk, g, col, raw);
  float s_mine = 0.0f;
#pragma unroll
  for (int st = 0; st < kSub; ++st) {
    v4i kl[2], km[2], kt[2];
    if (MX) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) limbs3_mx(raw.k[st], s2, g, kl[s2], km[s2], kt[s2]);
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) limbs3(raw.k[st][s2], kl[s2], km[s2], kt[s2]);
    }
    v4f p[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const v4i z = {0, 0, 0, 0};
      v4i acc[5] = {z, z, z, z, z};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const v4i ql = gq.lo[rt][s2], qm = gq.mid[rt][s2], qt = gq.top[rt][s2];
        acc[0] = mfma8(ql, kl[s2], acc[0]);
        acc[1] = mfma8(ql, km[s2], acc[1]);
        acc[1] = mfma8(qm, kl[s2], acc[1]);
        acc[2] = mfma8(ql, kt[s2], acc[2]);
        acc[2] = mfma8(qm, km[s2], acc[2]);
        acc[2] = mfma8(qt, kl[s2], acc[2]);
        acc[3] = mfma8(qm, kt[s2], acc[3]);
        acc[3] = mfma8(qt, km[s2], acc[3]);
        acc[4] = mfma8(qt, kt[s2], acc[4]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // every term and the sum are integers below 2^53: exact, one rounding
        const double D = (double)acc[0][i] + (double)acc[1][i] * 128.0 + (double)acc[2][i] * 16384.0 +
                         (double)acc[3][i] * 2097152.0 + (double)acc[4][i] * 268435456.0;
        const float f = (float)D * 0x1p-9f;  // fl(2^9 d): the weights hold w * 2^-9
        p[rt][i] = wreg[rt][i] * (f > 0.0f ? f : 0.0f);
      }
    }
    s_mine = keep_subtile(s_mine, head_sum(p), st, lane);
  }
  return s_mine;
}

// Scan.  POOL = false: Full mode, rows = sequences, the waves split
// T tokens x chunk slices.  POOL = true: Reindex mode, rows = (b, t),
// positions are the entries of the row's pool blocks.  Each workgroup takes
// a range of 64-entry chunks inside one row; each wave loads its next
// chunk's keys while it scores the current one.
//
// The workgroup first splits its tokens' queries into f16 limbs once, in
// LDS, while every wave's first keys are in flight; each wave then copies
// its token's limbs into registers.  Per chunk a wave takes its 4 sub-tiles
// of 16 entries in turn: convert the keys to f16, run the MFMAs of the 4 row
// tiles and the sub-tile's Gram matrix, form fl(w_h * relu(d_h)) and the
// pairwise head sum in registers.  Chunks with an entry over the fast
// path's bound, and rows whose query has some |q| >= 32, are only marked
// here and scored after the main loop by the general path.
template <bool POOL, bool MX>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  struct __attribute__((aligned(16))) Lds {
    // per token: the f16 limbs ql, qm of the query, in the order the waves
    // hold them: [row tile][slice][limb][lane]
    v8h qlimb[kGroupT][kRT][4][2][64];
    float wsh[kGroupT][kRT * 16];                 // w * 2^-9 per head, 0 past HI
    uint32_t qbad[kGroupT];                       // nonzero: some |q| >= 32
    uint32_t defer[kWaves][kMaxWaveChunks / 32];  // chunks left to the general path
    // per token: level-1 histograms of entry scores and block maxima,
    // 16-bit counters packed two per word
    uint32_t hist[kGroupT][2][kHistBins / 2];
  };
  __shared__ Lds sm;

  for (int i = threadIdx.x; i < kWaves * kMaxWaveChunks / 32; i += blockDim.x) (&sm.defer[0][0])[i] = 0u;
  for (int i = threadIdx.x; i < kGroupT * kHistBins; i += blockDim.x) (&sm.hist[0][0][0])[i] = 0u;
  if (threadIdx.x < kGroupT) sm.qbad[threadIdx.x] = 0u;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4;   // K slice group of the MFMA operands; head group of the outputs
  const int col = lane & 15;
  const int HI = a.HI;
  const int row = blockIdx.x / a.wg_per_row;
  // Full mode: tokens t0 .. t0 + Tg - 1 of the sequence, in Ts token slots
  // (a group of three keeps a dead fourth slot, so that the slots divide the
  // 8 waves); each wave takes one slot and a slice of the chunk range
  const int t0 = POOL ? 0 : (row % a.n_groups) * kGroupT;
  const int Tg = POOL ? 1 : min(kGroupT, a.T - t0);
  const int Ts = Tg == 3 ? 4 : Tg;
  const int slot = POOL ? 0 : wave % Ts;
  const int t_full = POOL ? 0 : t0 + min(slot, Tg - 1);
  const int slice = POOL ? wave : wave / Ts;
  const int n_slices = POOL ? kWaves : kWaves / Ts;
  const int c0 = (blockIdx.x % a.wg_per_row) * a.chunks_per_wg;
  const int c1 = min(a.chunks_per_row, c0 + a.chunks_per_wg);
  const bool have_row = row < a.rows;
  int chunk = c0 + slice;
  const bool active = have_row && chunk < c1 && slot < Tg;
  uint32_t* hist_s = sm.hist[slot][0];
  uint32_t* hist_bm = sm.hist[slot][1];
  RowCtx rc;
  if (have_row) row_ctx<POOL>(a, row, t_full, slot < Tg, rc);
  const int64_t qrow0 = ((int64_t)rc.b * a.T + rc.t) * HI;
  const int n_tok = POOL ? 1 : Ts;

  // ---- every load that needs nothing loaded first is issued here, ahead of
  // the keys (the wait counter retires loads in issue order): the raw query
  // words of this thread's limb items, the head weights, and (Full mode)
  // the page-table words of this wave's first 64 chunks, read before the
  // row's length is known and checked against it afterwards.  The loads are
  // unconditional (clamped indices; words that are not needed are masked
  // by opaque masks at their use), so that no branch separates them and the
  // compiler keeps no load of them inside one.
  // Limb item (token, row tile rt, slice s, lane L): head tile_head(rt, L &
  // 15), channels 16 gL + 8 s + e (s < 2) or 64 + 16 gL + 8 (s - 2) + e
  // (e < 8, gL = L >> 4), the keys' order in the slices.
  constexpr int kLimbIters = kGroupT * kRT * 4 * 64 / kScoreThreads;
  const int n_items = n_tok * kRT * 4 * 64;  // 1024 n_tok, a power of two
  uint32_t qraw[kLimbIters][2], qkeep[kLimbIters];
#pragma unroll
  for (int j = 0; j < kLimbIters; ++j) {
    const int it = (int)threadIdx.x + j * kScoreThreads;
    const int iw = it & (n_items - 1);
    const int L = iw & 63, sl = (iw >> 6) & 3, rt = (iw >> 8) & 3, tk = iw >> 10;
    const int t = POOL ? rc.t : t0 + min(tk, Tg - 1);
    const int h = tile_head(rt, L & 15), gL = L >> 4;
    const int ch = sl < 2 ? 16 * gL + 8 * sl : 64 + 16 * gL + 8 * (sl - 2);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        a.q_idx + (((int64_t)rc.b * a.T + t) * HI + min(h, HI - 1)) * kDI + ch);
    qraw[j][0] = src[0];
    qraw[j][1] = src[1];
    qkeep[j] = (it < n_items && h < HI && (POOL || tk < Tg)) ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(qkeep[j]));
  }
  uint32_t wraw, wkeep;
  {
    const int i = min((int)threadIdx.x, n_tok * 64 - 1);
    const int tk = i >> 6, h = i & 63;
    const int t = POOL ? rc.t : t0 + min(tk, Tg - 1);
    wraw = __float_as_uint(a.w[((int64_t)rc.b * a.T + t) * HI + min(h, HI - 1)]);
    wkeep = ((int)threadIdx.x < n_tok * 64 && h < HI && (POOL || tk < Tg)) ? 0xFFFFFFFFu : 0u;
    asm volatile("" : "+v"(wkeep));
  }
  int page_word = -1;
  if (!POOL) {
    const int ck = c0 + slice + lane * n_slices;
    page_word = a.page_table[(int64_t)rc.b * a.max_pages + max(0, min(ck, a.max_pages - 1))];
  }
  // clear this workgroup's share of its row's global level-1 histograms: the
  // row's workgroups add into them only at their ends.  Device-scope atomics,
  // so that the clear and the other workgroups' adds are ordered at the same
  // point whichever caches they pass.  A workgroup that starts only after
  // another of its row has already added would drop those counts; the
  // selection checks its counts against the list and then counts the list's
  // keys itself, so such a histogram costs time, not correctness.
  if (row < a.rows && a.clear_hist) {
    const int words = Tg * 2 * kHistBins;
    uint32_t* gh = a.hist + (POOL ? (int64_t)row : (int64_t)rc.b * a.T + t0) * 2 * kHistBins;
    const int k = blockIdx.x % a.wg_per_row;
    const int per = (words + a.wg_per_row - 1) / a.wg_per_row;
    const int w1 = min(words, (k + 1) * per);
    for (int i = k * per + (int)threadIdx.x; i < w1; i += blockDim.x) atomicAnd(&gh[i], 0u);
  }
  lds_barrier();

  // Full mode: the physical pages of this wave's chunks, lane k holding the
  // page of its chunk number k0 + k (refilled every 64 chunks), so the loop
  // reads them with readlane and issues no memory load of its own for them
  // (a vector load there would wait for the key prefetch as well)
  int wave_pages = -1;
  auto fill_pages = [&](int k0) {
    const int ck = c0 + slice + (k0 + lane) * n_slices;
    wave_pages = (!POOL && ck < c1) ? (int)chunk_page(a, rc, ck) : -1;
  };
  auto page_of = [&](int k) -> int64_t {
    return POOL ? 0 : (int64_t)__builtin_amdgcn_readlane(wave_pages, k & 63);
  };
  // every early load has arrived here (they went out together): waiting
  // for them before the key loads leaves nothing to wait for in the limb work
#pragma unroll
  for (int j = 0; j < kLimbIters; ++j) asm volatile("" ::"v"(qraw[j][0]), "v"(qraw[j][1]));
  asm volatile("" ::"v"(wraw), "v"(page_word));
  ChunkKeys cur;
  bool cur_ok = false;
  if (active) {
    if (!POOL) {
      // chunk_page on the early page-table word
      const int ck = c0 + slice + lane * n_slices;
      wave_pages = (ck < c1 && ck * kChunk < rc.n && ck < a.max_pages && page_word >= 0 && page_word < a.n_pages)
                       ? page_word : -1;
    }
    const int64_t pg0 = page_of(0);
#pragma unroll
    for (int st = 0; st < kSub; ++st) load_sub<POOL, MX>(a, rc, chunk, pg0, st, g, col, cur.k[st]);
    cur_ok = POOL || pg0 >= 0;
  }

  // ---- the workgroup's queries in f16 limbs: ql = Mq mod 2^7 and qm =
  // floor(Mq / 2^7) of M = q * 2^9 (exact small integers), from the raw words
  if (have_row) {
#pragma unroll
    for (int j = 0; j < kLimbIters; ++j) {
      const int it = (int)threadIdx.x + j * kScoreThreads;
      if (it >= n_items) break;
      const int L = it & 63, sl = (it >> 6) & 3, rt = (it >> 8) & 3, tk = it >> 10;
      v8h ql, qm;
      bool bad = false;
#pragma unroll
      for (int wd = 0; wd < 2; ++wd)
#pragma unroll
        for (int wsel = 0; wsel < 2; ++wsel) {
          const uint32_t c = qraw[j][wd] & qkeep[j];
          const v2f m2 = wsel ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 512.0f, true)
                              : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 512.0f, false);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int e = 4 * wd + 2 * wsel + jj;
            const float hi = floorf(m2[jj] * 0x1p-7f);
            const float lo = m2[jj] - hi * 128.0f;  // exact: both are small integers
            ql[e] = (_Float16)lo;
            qm[e] = (_Float16)hi;
            bad = bad || !(fabsf(m2[jj]) < 16384.0f);
          }
        }
      sm.qlimb[tk][rt][sl][0][L] = ql;
      sm.qlimb[tk][rt][sl][1][L] = qm;
      if (bad) atomicOr(&sm.qbad[tk], 1u);
    }
    if ((int)threadIdx.x < n_tok * 64) {
      const int tk = (int)threadIdx.x >> 6, h = (int)threadIdx.x & 63;
      sm.wsh[tk][h] = __uint_as_float(wraw & wkeep) * 0x1p-9f;  // 0 past HI
    }
  }
  lds_barrier();

  if (active) {
  // this wave's token: limbs (A operands, row col of row tile rt is head
  // tile_head(rt, col)), weights of its output heads, fast-path condition
  v8h ql[kRT][4], qm[kRT][4];
  v4f wreg[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      ql[rt][sl] = sm.qlimb[slot][rt][sl][0][lane];
      qm[rt][sl] = sm.qlimb[slot][rt][sl][1][lane];
    }
    wreg[rt] = *reinterpret_cast<const v4f*>(&sm.wsh[slot][16 * g + 4 * rt]);
  }
  const bool fast_q = sm.qbad[slot] == 0u;
  uint32_t* my_defer = sm.defer[wave];
  int k_seq = 0;  // index of the current chunk among this wave's chunks

  for (; chunk < c1; chunk += n_slices, ++k_seq) {
    const int next = chunk + n_slices;
    if (!fast_q) {
      my_defer[k_seq >> 5] |= 1u << (k_seq & 31);
      continue;
    }
    const bool page_ok = cur_ok;
    if (!POOL && ((k_seq + 1) & 63) == 0) fill_pages(k_seq + 1);
    // past the range the prefetch reads nothing (Full mode: page -1, a
    // zero record count) but is still issued: a conditional load would make
    // the compiler merge old and new keys and wait for the loads at the loop
    // edge
    const int64_t next_pg = POOL ? 0 : (next < c1 ? page_of(k_seq + 1) : -1);
    cur_ok = POOL || next_pg >= 0;
    float gmax = 0.0f;
    float s_mine = 0.0f;
#pragma unroll
    for (int st = 0; st < kSub; ++st) {
      // ---- the sub-tile's keys as f16 (exact for every E4M3 code), in the
      // channel order of the query slices
      __builtin_amdgcn_sched_barrier(0);
      v8h kf[4];
      if (MX) {
        // MXFP4: E2M1 codes times the group's power-of-two scale, exact in
        // f16 for the supported scales (multiples of 2^-9 up to 384); code
        // dword i of half hf holds the 8 channels of slice 2 hf + i
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float sc = e8m0_times_pow2((cur.k[st][1][0] >> (8 * (2 * hf + (g >> 1)))) & 0xFFu, 0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t wd = cur.k[st][0][2 * hf + i];
            const h2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 0);
            const h2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 1);
            const h2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 2);
            const h2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, sc, 3);
            kf[2 * hf + i] = v8h{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
          }
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const h2_t lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[st][hf][d], 1.0f, false);
            const h2_t hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[st][hf][d], 1.0f, true);
            const int slice = 2 * hf + (d >> 1), e = 4 * (d & 1);
            kf[slice][e + 0] = lo2[0];
            kf[slice][e + 1] = lo2[1];
            kf[slice][e + 2] = hi2[0];
            kf[slice][e + 3] = hi2[1];
          }
      }
      // the same sub-tile of the next chunk streams into the freed registers
      // (after the conversions have read them)
      __builtin_amdgcn_sched_barrier(0);
      load_sub<POOL, MX>(a, rc, next, next_pg, st, g, col, cur.k[st]);
      __builtin_amdgcn_sched_barrier(0);
      // the 8 MFMAs of each row tile, then the sub-tile's Gram matrix
      v4f sl4[kRT], sm4[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
        v4f cl = z, cm = z;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[rt][sl], kf[sl], cl, 0, 0, 0);
          cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(qm[rt][sl], kf[sl], cm, 0, 0, 0);
        }
        sl4[rt] = cl;
        sm4[rt] = cm;
      }
      // K K^T over the 128 channels: its diagonal holds sum_c k_c^2 of each
      // entry, and no other element exceeds the largest diagonal one
      // (Cauchy-Schwarz), so the maximum over all outputs is the largest
      // sum of squares of the sub-tile
      v4f gram = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) gram = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[sl], kf[sl], gram, 0, 0, 0);
      float q4[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        const v4f wv = wreg[rt];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // fl(2^9 d) = fl(S_l + 2^7 S_m): both sums exact, one rounding
          const float r = __builtin_fmaf(128.0f, sm4[rt][i], sl4[rt][i]);
          p[i] = wv[i] * (r > 0.0f ? r : 0.0f);
        }
        q4[rt] = (p[0] + p[1]) + (p[2] + p[3]);
      }
      gmax = fmaxf(gmax, fmaxf(fmaxf(gram[0], gram[1]), fmaxf(gram[2], gram[3])));
      s_mine = keep_subtile(s_mine, head_sum4(q4), st, lane);
    }
    // every entry of the chunk has sum_c k_c^2 < 500, hence (Cauchy-Schwarz
    // over 128 channels) sum_c |k_c| < sqrt(128 * 500) < 253: the fast path
    // is exact, since every partial sum of ql * k or qm * k (|ql|, |qm| <=
    // 128) is then a multiple of 2^-9 below 2^15
    const bool exact_ok = gmax < 500.0f;
    if (__ballot(!exact_ok) != 0) {
      // rare: scored after the main loop by the general path
      my_defer[k_seq >> 5] |= 1u << (k_seq & 31);
      continue;
    }
    emit_chunk<POOL>(a, rc, chunk, s_mine, page_ok, hist_s, hist_bm);
  }

  // ---- deferred chunks: general exact path
  wave_lds_order();
  bool any_deferred = false;
  for (int k = 0; k < (k_seq + 31) / 32; ++k) any_deferred = any_deferred || my_defer[k] != 0u;
  if (any_deferred) {
    GenQuery gq;
    general_query(a, qrow0, gq);
    for (int k = 0; k < k_seq; ++k) {
      if (!((my_defer[k >> 5] >> (k & 31)) & 1u)) continue;
      const int ck = c0 + slice + k * n_slices;
      bool ok;
      const float s = general_chunk<POOL, MX>(a, rc, ck, gq, wreg, ok);
      emit_chunk<POOL>(a, rc, ck, s, ok, hist_s, hist_bm);
    }
  }
  }  // this wave's chunks

  // ---- the workgroup's histograms into the row's (global, 32-bit) ones
  __syncthreads();
  if (row < a.rows) {
    for (int i = threadIdx.x; i < Tg * kHistBins; i += blockDim.x) {
      const uint32_t v = (&sm.hist[0][0][0])[i];
      if (v == 0u) continue;
      const int t = i / kHistBins, h = (i / (kHistBins / 2)) & 1, wd = i % (kHistBins / 2);
      const int64_t grow = POOL ? (int64_t)row : (int64_t)rc.b * a.T + t0 + t;  // (b, t)
      uint32_t* gh = a.hist + (grow * 2 + h) * kHistBins + 2 * wd;
      if (v & 0xFFFFu) atomicAdd(gh, v & 0xFFFFu);
      if (v >> 16) atomicAdd(gh + 1, v >> 16);
    }
  }
}

// ---------------------------------------------------------------- selection
//
// One workgroup per (b, t) row.  Keys are order-preserving uint32 images of
// the scores (key 0 = empty); thread t owns list positions t + 1024 r, so
// every load instruction of a wave covers 64 consecutive positions and the
// position order of a wave's keys for one r is the order of its lanes (ballot
// masks give ranks).
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;     // 2,048: 32 per lane of one wave
constexpr int kMaxKPT = 32;

struct SelShared {
  uint32_t stage[kMaxKPT * kSelThreads];  // the block maxima, in transit to their threads
  uint32_t bins[kBins];                   // one radix level's histogram
  int wave_tot[kSelWaves];
  int wave_tot2[kSelWaves];
  int misc[8];
  int pool_blk[CSA2_MAX_POOL_BLOCKS];
};

// Dword of SelShared::stage holding list position p: thread t = p / 32
// reads its 32 positions as 8 16-byte pieces q = (p / 4) % 8, placed at
// piece q ^ ((t / 2) % 8) of its row, so that both the coalesced writes and
// the per-thread reads of 16 lanes cover all 64 banks.
__device__ __forceinline__ int stage_addr(int p) {
  const int t = p >> 5, q = (p >> 2) & 7;
  return (t << 5) + ((q ^ ((t >> 1) & 7)) << 2) + (p & 3);
}

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

// Exclusive prefix sum over the workgroup in thread order; returns the
// thread's offset and writes the total to *total.
__device__ int block_excl_scan(int v, SelShared& sh, int* total) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) sh.wave_tot[wave] = x;
  lds_barrier();
  // lanes 0..15 hold the wave totals: one read, then a scan in registers
  const int wt = (int)wave_incl_scan(lane < kSelWaves ? (uint32_t)sh.wave_tot[lane] : 0u);
  const int before = wave > 0 ? __builtin_amdgcn_readlane(wt, wave - 1) : 0;
  *total = __builtin_amdgcn_readlane(wt, kSelWaves - 1);
  lds_barrier();
  return before + x - v;
}

// Sum over the workgroup (every thread returns it).
__device__ int block_sum(int v, SelShared& sh) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int x = wave_sum(v);
  if (lane == 0) sh.wave_tot2[wave] = x;
  lds_barrier();
  // wave_tot2 is written again only after later barriers
  return wave_sum(lane < kSelWaves ? sh.wave_tot2[lane] : 0);
}

// One wave, histogram h of 2,048 bins (lane l owns bins [2048 - 32(l+1),
// 2048 - 32l), lane 0 has the highest digits).  For the rank x >= 1 (counted
// from the top) returns the bin holding it (-1 if the histogram holds fewer
// than x keys) and writes the count above that bin.  The lane whose range
// holds the rank is found by a scan of the lane totals; its 32 bins are then
// scanned across lanes 0..31.
__device__ __forceinline__ int wave_crossing(const uint32_t* h, uint32_t x, uint32_t* above_bin, int lane) {
  const v4u* hv = reinterpret_cast<const v4u*>(h + kBins - 32 * (lane + 1));
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const v4u v = hv[q];
    sum += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint64_t who = __ballot(incl - sum < x && x <= incl);
  if (who == 0) {
    *above_bin = 0;
    return -1;
  }
  const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(who));
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), src);
  // lane j < 32 takes the j-th highest bin of lane src
  const int top_bin = kBins - 32 * src - 1;
  const uint32_t c = lane < 32 ? h[top_bin - lane] : 0u;
  const uint32_t ci = wave_incl_scan(c);
  const uint64_t hit = __ballot(lane < 32 && above + ci >= x);
  const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  *above_bin = above + (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), j);
  return top_bin - j;
}

// Top-K selection among the keys of a list (thread t holds positions
// KPT t + r), order (key desc, position asc); key 0 marks an empty slot.
// Two steps, so that the first overlaps the loads of the keys:
//
// topk_level1: the number of valid keys of the list (from each thread's
//    count) and, with more than K, the first radix digit of the K-th largest
//    key from `l1v`, the histogram the scan accumulated of the list's keys by
//    their top 10 bits (thread t holds bin t).  The histogram may count more
//    keys than the list holds, but only keys below the K-th: bins above the
//    crossing then hold the same counts as the list's own keys, and the
//    crossing bin is the same.
// topk_finish: the next two digits (11 + 11 bits) from histograms of the
//    list's keys that match the prefix so far, which gives the K-th largest
//    key tau; then every key above tau, and the first keys (in position
//    order) equal to tau up to K, are emitted: emit(rank, pos) with rank =
//    place in ascending position order.  A thread's rank base is a prefix
//    over the threads' counts, since its positions are contiguous.  Returns
//    the number selected.
//    The histogram is only a hint: such a selection (every key above tau and
//    the first keys equal to tau) holds every key that ranks above one of its
//    own, so it is the top K exactly when it holds K keys.  The count is
//    checked before anything is emitted; when the histogram disagrees with
//    the list (a workgroup of the scan cleared its share after another had
//    flushed into it), the first digit is counted from the list's own keys
//    and the selection is redone.
struct TopkState {
  uint32_t prefix, msk;
  int rem;
  bool l1_ok;
};

// One wave finds the bin holding rank `rem` of sh.bins; all threads return it.
__device__ __forceinline__ int bins_cross(SelShared& sh, int rem, int* above) {
  const int lane = lane_id();
  if (threadIdx.x < 64) {
    uint32_t ab;
    const int d = wave_crossing(sh.bins, (uint32_t)rem, &ab, lane);
    if (lane == 0) {
      sh.misc[0] = d;
      sh.misc[1] = (int)ab;
    }
  }
  lds_barrier();
  *above = sh.misc[1];
  return sh.misc[0];
}

__device__ TopkState topk_level1(uint32_t l1v, int K, SelShared& sh) {
  static_assert(kBins == 2 * kSelThreads, "two bins per thread");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tid = (int)threadIdx.x;
  TopkState st{0u, 0u, K, true};
  // the level-1 digits occupy bins [0, 1024)
  sh.bins[tid] = l1v;
  sh.bins[tid + kSelThreads] = 0u;
  const int wv = wave_sum((int)l1v);
  if (lane == 0) sh.wave_tot[wave] = wv;
  lds_barrier();
  // the crossing is looked for whenever the histogram holds K keys; whether
  // the list holds more than K is decided from its own keys
  const int n_hist = wave_sum(lane < kSelWaves ? sh.wave_tot[lane] : 0);
  st.l1_ok = n_hist >= K;
  if (st.l1_ok) {
    int ab;
    const int d = bins_cross(sh, K, &ab);
    if (d < 0) {
      st.l1_ok = false;
    } else {
      st.prefix = (uint32_t)d << 22;
      st.msk = 1023u << 22;
      st.rem = K - ab;
    }
  }
  // sh.bins and sh.wave_tot are reused next: every thread has read them
  lds_barrier();
  return st;
}

template <int KPT, typename Emit>
__device__ int topk_finish(const uint32_t (&key)[KPT], int K, TopkState st, SelShared& sh, Emit emit) {
  static_assert(KPT <= kMaxKPT, "keys per thread");
  const int tid = (int)threadIdx.x;
  uint32_t* bins = sh.bins;
  // valid keys of the list
  int nv = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) nv += key[r] != 0u ? 1 : 0;
  const int n_valid = block_sum(nv, sh);
  const int expect = min(K, n_valid);
#pragma clang loop unroll(disable)
  for (int attempt = 0;; ++attempt) {
    // the digit shifts pass through an empty asm in every attempt, so that
    // the compiler does not hoist the keys' digits out of the loop (that
    // would hold several copies of the keys in registers)
    int sh0 = 0;
    asm volatile("" : "+s"(sh0));
    uint32_t tau = 0;  // with tau = 0 every valid key is selected
    int need_eq = 0;
    if (n_valid > K) {
      uint32_t prefix = st.prefix, msk = st.msk;
      int rem = st.rem;
      // histogram of digit (key >> shift) & dmask over the keys matching the prefix
      auto build = [&](int shift, uint32_t dmask) {
        bins[tid] = 0u;
        bins[tid + kSelThreads] = 0u;
        lds_barrier();
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          const uint32_t k = key[r];
          if (k != 0u && (k & msk) == prefix) atomicAdd(&bins[(k >> shift) & dmask], 1u);
        }
        lds_barrier();
      };
      int d, ab;
      if (!st.l1_ok) {
        // the first digit from the list's own keys
        build(22 + sh0, 1023u);
        d = bins_cross(sh, rem, &ab);
        prefix = (uint32_t)d << 22;
        msk = 1023u << 22;
        rem -= ab;
      }
#pragma unroll
      for (int shift = 11; shift >= 0; shift -= 11) {
        build(shift + sh0, 2047u);
        d = bins_cross(sh, rem, &ab);
        prefix |= (uint32_t)d << shift;
        msk |= 2047u << shift;
        rem -= ab;
      }
      tau = prefix;
      need_eq = rem;
    }

    // ---- 3. count, check, emit in position order
    uint32_t gt_m = 0, eq_m = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      gt_m |= (key[r] > tau ? 1u : 0u) << r;
      eq_m |= (key[r] != 0u && key[r] == tau ? 1u : 0u) << r;
    }
    const int ngt = __builtin_popcount(gt_m), neq = __builtin_popcount(eq_m);
    int tot;
    // both totals are at most 32,768: the 16-bit halves never carry
    const int pre = block_excl_scan(ngt | (neq << 16), sh, &tot);
    const int gt_tot = tot & 0xFFFF, eq_tot = (int)((uint32_t)tot >> 16);
    const int got = gt_tot + min(eq_tot, max(need_eq, 0));
    if (got != expect && attempt == 0) {
      // the histogram disagreed with the list (workgroup-uniform decision)
      st.l1_ok = false;
      st.prefix = 0u;
      st.msk = 0u;
      st.rem = K;
      continue;
    }
    const int gt_before = pre & 0xFFFF, eq_before = (int)((uint32_t)pre >> 16);
    // this thread's keys equal to tau that are taken: the first ones in
    // position order, up to need_eq over the whole list
    uint32_t sel = gt_m, m = eq_m;
    for (int take = min(max(need_eq - eq_before, 0), neq); take > 0; --take) {
      sel |= m & (~m + 1u);
      m &= m - 1u;
    }
    // ranks stay below K whatever the counts (only a wrong count could
    // exceed it, and the recount above leaves none)
    int rank = gt_before + min(eq_before, max(need_eq, 0));
    while (sel != 0u && rank < K) {
      emit(rank++, KPT * tid + __builtin_ctz(sel));
      sel &= sel - 1u;
    }
    return min(got, K);
  }
}

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
  const uint32_t* hist;      // [B][T][2][1024]: level-1 counts of entry scores, block maxima
  // full, optional: the step's cache write, done by workgroup 0 before its selection
  const uint16_t* wr_rows;   // [wr_n][512] bf16
  const int64_t* wr_slots;   // [wr_n]
  uint8_t* wr_pool;          // [wr_pages][18432]
  int64_t wr_n, wr_pages;
};

// One workgroup per (b, t).  FULL: select the pool from block maxima, then
// the top-k inside the pool (the top-k lies inside the pool whenever
// topk <= pool_blocks).  REINDEX: top-k over the pool-order scores.
template <bool FULL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int row = blockIdx.x;  // b * T + t
  const int tid = (int)threadIdx.x;
  if (FULL && row == 0 && a.wr_n > 0) {
    // FP4 cache write of wr_n rows, 32 threads (16-channel groups) per row: whole rows per
    // wave, so the four lanes of each scale dword are active together.  Nothing the indexer
    // reads is written; the attention that reads these entries runs after this kernel.
    for (int64_t t = tid; t < a.wr_n * 32; t += kSelThreads) {
      const int64_t r = t >> 5;
      const int g = (int)(t & 31);
      const v4u* src = reinterpret_cast<const v4u*>(a.wr_rows + r * kD + g * 16);
      const v4u x0 = src[0], x1 = src[1];
      const uint32_t h[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const int64_t s = a.wr_slots[r];
      store_fp4_group(fp4_group(h), g, s >= 0 && s < a.wr_pages * kPage, s, a.wr_pool);
    }
  }
  const int b = row / a.T;
  int n = min(a.n_entries[b], min(a.max_n, a.max_pages * kPage));
  if (a.n_vis != nullptr) n = min(n, a.n_vis[row]);
  n = max(n, 0);
  const int nb = (n + kBlock - 1) / kBlock;
  const int P = a.pool_blocks;
  // level-1 histograms the scan accumulated (thread t: bin t), loaded early
  const uint32_t l1_s = a.hist[((int64_t)row * 2 + 0) * kHistBins + tid];
  const uint32_t l1_bm = FULL ? a.hist[((int64_t)row * 2 + 1) * kHistBins + tid] : 0u;
  int pool_n;
  if (FULL) {
    // ---- the pool: thread t holds the maxima of blocks 32 t .. 32 t + 31,
    // loaded coalesced (piece q of thread t: blocks 4096 q + 4 t .. + 3) and
    // passed through LDS
    constexpr int KPT = 32;  // 32,768 blocks = 262,144 entries
    static_assert(KPT <= kMaxKPT, "stage size");
    const float* bm = a.bm + (int64_t)row * bm_stride(a.max_n);
    // the whole row is read (reads past it return zero; no branch per load),
    // so the loads need not wait for n; blocks >= nb are masked below
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)bm, 0, bm_stride(a.max_n) * 4, kBufferFlags);
    v4u raw[KPT / 4];
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q)
      raw[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(4 * kSelThreads * q + 4 * tid) * 4u, 0, 0);
    for (int i = tid; i < P; i += kSelThreads) sh.pool_blk[i] = -1;
    // the first digit comes from the histogram while the loads are in flight
    const TopkState st = topk_level1(l1_bm, P, sh);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q)
      *reinterpret_cast<v4u*>(&sh.stage[stage_addr(4 * kSelThreads * q + 4 * tid)]) = raw[q];
    lds_barrier();
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) raw[q] = *reinterpret_cast<const v4u*>(&sh.stage[stage_addr(KPT * tid + 4 * q)]);
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      key[r] = KPT * tid + r < nb ? score_key(__uint_as_float(raw[r / 4][r % 4])) : 0u;
    pool_n = topk_finish<KPT>(key, P, st, sh, [&](int rank, int pos) { sh.pool_blk[rank] = pos; });
    lds_barrier();
    for (int i = tid; i < P; i += kSelThreads) a.out_pool[(int64_t)row * P + i] = sh.pool_blk[i];
    if (tid == 0) a.out_pool_n[row] = pool_n;
  } else {
    pool_n = max(0, min(a.pool_n_in[row], P));
    for (int i = tid; i < P; i += kSelThreads) sh.pool_blk[i] = i < pool_n ? a.pool_in[(int64_t)row * P + i] : -1;
    lds_barrier();
  }
  // ---- top-k over the pool's positions (list position p = 8 * slot + e):
  // thread t gathers slots 2t and 2t + 1 (16 contiguous positions) with
  // 16-byte loads straight into its keys
  constexpr int KPT2 = 16;  // 16,384 positions
  const float* srow = FULL ? a.s + (int64_t)row * s_stride(a.max_n) : a.s + (int64_t)row * P * kBlock;
  const uint32_t row_bytes = FULL ? (uint32_t)s_stride(a.max_n) * 4u : (uint32_t)P * kBlock * 4u;
  const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, row_bytes, kBufferFlags);
  uint32_t key2[KPT2];
  TopkState st2;
  {
    v4u g[2][2];
    int blk[2];
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int slot = 2 * tid + hs;
      blk[hs] = slot < pool_n ? sh.pool_blk[slot] : -1;
      const bool ok = blk[hs] >= 0 && blk[hs] < nb;
      // an offset past the row reads zeros (masked below)
      const uint32_t off = ok ? (uint32_t)(FULL ? blk[hs] : slot) * kBlock * 4u : row_bytes;
      g[hs][0] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off, 0, 0);
      g[hs][1] = __builtin_amdgcn_raw_buffer_load_b128(rs2, off + 16u, 0, 0);
    }
    // the first digit while the gathers are in flight
    st2 = topk_level1(l1_s, a.topk, sh);
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const bool ok = blk[hs] >= 0 && blk[hs] < nb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = e < 4 ? g[hs][0][e] : g[hs][1][e - 4];
        key2[8 * hs + e] = (ok && blk[hs] * kBlock + e < n) ? score_key(__uint_as_float(bits)) : 0u;
      }
    }
  }
  int32_t* out = a.out_topk + (int64_t)row * a.topk;
  // Full mode: the level-1 counts are those of every entry of the row; the
  // top-k lies inside the pool, so entries outside it all rank below the
  // k-th and the pool's own counts agree above the crossing bin
  const int got = topk_finish<KPT2>(key2, a.topk, st2, sh, [&](int rank, int p) {
    out[rank] = sh.pool_blk[p >> 3] * kBlock + (p & 7);
  });
  for (int i = got + tid; i < a.topk; i += kSelThreads) out[i] = -1;
}

}  // namespace csa2

// ---------------------------------------------------------------- C ABI
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of the scan: each takes a range of chunks inside one row, about
// one workgroup per compute unit in total (the scan uses ~138 KB of LDS).
// With T tokens sharing a workgroup, every wave covers chunks_per_wg * T / 8
// chunks of the range.
int score_grid(int rows, int chunks_per_row, int T, int* chunks_per_wg, int* wg_per_row) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      n_cu = 256;
  }
  const int slices = csa2::kWaves / T;
  const int want = std::max(1, n_cu / rows);
  int per = (chunks_per_row + want - 1) / want;
  per = ((per + slices - 1) / slices) * slices;  // whole rounds of the waves
  // each wave tracks at most kMaxWaveChunks chunks; the workgroup's 16-bit
  // histogram counters hold at most kMaxWgChunks chunks of one token
  per = std::min(per, std::min(csa2::kMaxWaveChunks * slices, csa2::kMaxWgChunks));
  *chunks_per_wg = per;
  *wg_per_row = (chunks_per_row + per - 1) / per;
  return rows * *wg_per_row;
}

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

// Workspace: scores, block maxima (Full mode), level-1 histograms.
size_t hist_bytes(int32_t B, int32_t T) { return align256((size_t)B * T * 2 * csa2::kHistBins * 4); }

extern "C" size_t csa2_index_ws_bytes(int op, int32_t B, int32_t T, int32_t max_n,
                                      int32_t pool_blocks) {
  if (op == CSA2_OP_INDEX_FULL) {
    const size_t nb = (size_t)csa2::bm_stride(max_n);
    return align256((size_t)B * T * csa2::s_stride(max_n) * 4) + align256((size_t)B * T * nb * 4) +
           hist_bytes(B, T);
  }
  return align256((size_t)B * T * pool_blocks * 8 * 4) + hist_bytes(B, T);
}

// Launches the scan (which also clears the level-1 histograms); `mx`: the
// indexer keys are in the MXFP4 page layout.
int launch_scan(bool pool, bool mx, const csa2::ScoreArgs& sa, int T_grid, hipStream_t stream) {
  csa2::ScoreArgs args = sa;
  args.clear_hist = csa2::keep_histograms() ? 0 : 1;
  const int gx = score_grid(args.rows, args.chunks_per_row, T_grid, &args.chunks_per_wg, &args.wg_per_row);
  const dim3 grid(gx), block(csa2::kScoreThreads);
  if (pool && mx)
    CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, (csa2::score_kernel<true, true>), grid, block, stream, args);
  else if (pool)
    CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, (csa2::score_kernel<true, false>), grid, block, stream, args);
  else if (mx)
    CSA2_LAUNCH(CSA2_K_SCORE_FULL, (csa2::score_kernel<false, true>), grid, block, stream, args);
  else
    CSA2_LAUNCH(CSA2_K_SCORE_FULL, (csa2::score_kernel<false, false>), grid, block, stream, args);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
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
  sa.out_s = reinterpret_cast<float*>(ws);
  sa.out_bm = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                       align256((size_t)B * T * csa2::s_stride(max_n_entries) * 4));
  sa.hist = reinterpret_cast<uint32_t*>(
      reinterpret_cast<char*>(ws) + align256((size_t)B * T * csa2::s_stride(max_n_entries) * 4) +
      align256((size_t)B * T * csa2::bm_stride(max_n_entries) * 4));
  sa.rows = B * sa.n_groups;
  sa.chunks_per_row = (max_n_entries + csa2::kChunk - 1) / csa2::kChunk;
  const int t_slots = T >= csa2::kGroupT ? csa2::kGroupT : (T == 3 ? 4 : T);
  st = launch_scan(false, mx, sa, t_slots, (hipStream_t)stream);
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
  se.hist = sa.hist;
  se.wr_rows = wr_rows;
  se.wr_slots = wr_slots;
  se.wr_pool = wr_pool;
  se.wr_n = wr_n;
  se.wr_pages = wr_pages;
  CSA2_LAUNCH(CSA2_K_SELECT_FULL, csa2::select_kernel<true>, dim3(B * T), dim3(csa2::kSelThreads),
              (hipStream_t)stream, se);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
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
  sa.out_s = reinterpret_cast<float*>(ws);
  sa.hist = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) +
                                        align256((size_t)B * T * pool_blocks * 8 * 4));
  sa.rows = B * T;
  sa.chunks_per_row = (pool_blocks * csa2::kBlock + csa2::kChunk - 1) / csa2::kChunk;
  st = launch_scan(true, mx, sa, 1, (hipStream_t)stream);
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
  se.hist = sa.hist;
  se.out_topk = out_topk;
  CSA2_LAUNCH(CSA2_K_SELECT_REINDEX, csa2::select_kernel<false>, dim3(B * T),
              dim3(csa2::kSelThreads), (hipStream_t)stream, se);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
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
