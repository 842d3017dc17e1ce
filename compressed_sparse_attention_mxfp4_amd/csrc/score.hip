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

#include "index_common.h"
#include "fp4.h"

// Every multiply and add of the score is its own binary32 operation: no
// multiply-add contraction anywhere in this file.
#pragma clang fp contract(off)

namespace csa2 {

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
  int n_raw = 0, nv_raw = 0, pn_raw = 0;  // the loaded counts, before row_ctx_finish
  bool live = false;
  const int32_t* pool_row = nullptr;
  // pool mode: the workgroup's pool slots slot0 .. slot0 + nslots - 1
  // resolved to physical entries (LDS, see pool_slot_word)
  const int* pslot = nullptr;
  int slot0 = 0, nslots = 0;
};

// Pool mode: the word of pool slot `slot`: (physical entry index of the
// block's first entry) | (visible entries of the block - 1), or -1 when the
// block is not visible or its page is not usable.  The physical index is a
// multiple of 8 (blocks of 8 never cross a 64-entry page).
__device__ __forceinline__ int pool_slot_word(const ScoreArgs& a, const RowCtx& r, int slot) {
  const int nb = (r.n + kBlock - 1) / kBlock;
  const int pn = r.n_pos / kBlock;
  // both loads are unconditional (clamped indices, masked after)
  const int blk = r.pool_row[max(0, min(slot, a.pool_blocks - 1))];
  const int lp = max(0, min(blk >> 3, a.max_pages - 1));
  const int pg = a.page_table[(int64_t)r.b * a.max_pages + lp];
  const bool ok = slot < pn && blk >= 0 && blk < nb && pg >= 0 && pg < a.n_pages;
  return ok ? (pg * kPage + (blk & 7) * kBlock) | (min(kBlock, r.n - blk * kBlock) - 1) : -1;
}

// Pool mode: physical entry of list position p (-1: not visible).
__device__ __forceinline__ int pool_entry(const RowCtx& r, int p) {
  const int li = (p >> 3) - r.slot0;
  const int w = r.pslot[max(0, min(li, r.nslots - 1))];
  const bool ok = p < r.n_pos && li >= 0 && li < r.nslots && w >= 0 && (p & 7) <= (w & 7);
  return ok ? (w & ~7) + (p & 7) : -1;
}

// Full mode: row = b * n_groups + token group, t_full the wave's token
// (live: the token exists; the dead fourth slot of a group of three sees
// nothing).  Token t of sequence b sees its first min(n_entries[b],
// n_vis[b][t]) entries.
// row_ctx_load only issues the count loads; row_ctx_finish, after the
// workgroup's other early loads have gone out, turns them into the counts
// (a load used at once would hold every later load back by a round trip).
template <bool POOL>
__device__ __forceinline__ void row_ctx_load(const ScoreArgs& a, int row, int t_full, bool live, RowCtx& r) {
  if (POOL) {
    r.b = row / a.T;
    r.t = row % a.T;
  } else {
    r.b = row / a.n_groups;
    r.t = t_full;
  }
  r.live = live;
  // vector loads (indices in VGPRs): a scalar load would share its wait
  // counter with the kernel arguments' loads, so the next argument read
  // would wait for it
  int bi = r.b, vi = r.b * a.T + r.t, pi = row;
  asm volatile("" : "+v"(bi), "+v"(vi), "+v"(pi));
  r.n_raw = a.n_entries[bi];
  r.nv_raw = a.n_vis != nullptr ? a.n_vis[vi] : 0x7FFFFFFF;
  if (POOL) {
    r.pool_row = a.pool + (int64_t)row * a.pool_blocks;
    r.pn_raw = a.pool_n[pi];
  }
}

template <bool POOL>
__device__ __forceinline__ void row_ctx_finish(const ScoreArgs& a, RowCtx& r) {
  int n = r.n_raw;
  n = min(n, a.max_n);
  n = max(0, min(n, a.max_pages * kPage));
  n = max(0, min(n, r.nv_raw));
  if (!r.live) n = 0;
  r.n = n;
  if (POOL) {
    const int pn = max(0, min(r.pn_raw, a.pool_blocks));
    r.n_pos = pn * kBlock;
  } else {
    r.n_pos = n;
  }
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
// entry's 4 scale bytes, k[1][1] nonzero when the entry is visible.
template <bool POOL, bool MX>
__device__ __forceinline__ void load_sub(const ScoreArgs& a, const RowCtx& r, int chunk, int64_t pg, int st,
                                         int g, int col, v4u (&k)[2]) {
  if (MX) {
    v2u c0 = {0u, 0u}, c1 = {0u, 0u};
    uint32_t sw = 0u, vis = 0u;
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
      vis = col < nst ? 1u : 0u;
    } else {
      // every load is issued (entry 0 stands in for positions that are not
      // visible, masked after)
      const int e = pool_entry(r, chunk * kChunk + st * 16 + col);
      const int ee = max(e, 0);
      const uint8_t* page = a.kidx + (int64_t)(ee >> 6) * kMxPageBytes;
      c0 = *reinterpret_cast<const v2u*>(page + (ee & 63) * kMxCodes + 8 * g);
      c1 = *reinterpret_cast<const v2u*>(page + (ee & 63) * kMxCodes + 32 + 8 * g);
      sw = *reinterpret_cast<const uint32_t*>(page + kMxScaleOff + (ee & 63) * 4);
      const uint32_t m = e >= 0 ? 0xFFFFFFFFu : 0u;
      c0 = v2u{c0[0] & m, c0[1] & m};
      c1 = v2u{c1[0] & m, c1[1] & m};
      sw &= m;
      vis = m & 1u;
    }
    k[0] = v4u{c0[0], c0[1], c1[0], c1[1]};
    k[1] = v4u{sw, vis, 0u, 0u};
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
  // every load is issued (entry 0 stands in for positions that are not
  // visible, masked after)
  const int e = pool_entry(r, chunk * kChunk + st * 16 + col);
  const v4u* src = reinterpret_cast<const v4u*>(a.kidx + (int64_t)max(e, 0) * kDI + 16 * g);
  const v4u k0 = __builtin_nontemporal_load(src);
  const v4u k1 = __builtin_nontemporal_load(src + 4);
  const uint32_t m = e >= 0 ? 0xFFFFFFFFu : 0u;
  k[0] = v4u{k0[0] & m, k0[1] & m, k0[2] & m, k0[3] & m};
  k[1] = v4u{k1[0] & m, k1[1] & m, k1[2] & m, k1[3] & m};
}

// Nonzero when a visible MXFP4 entry's scale word (k[1] of load_sub) holds
// a code outside kMxScaleMin .. kMxScaleMax.
__device__ __forceinline__ uint32_t mx_scale_bad(const v4u& k1) {
  uint32_t bad = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) bad |= (((k1[0] >> (8 * i)) & 0xFFu) - (uint32_t)kMxScaleMin) > (uint32_t)(kMxScaleMax - kMxScaleMin) ? 1u : 0u;
  return k1[1] != 0u ? bad : 0u;
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
  const bool valid = POOL ? pool_entry(rc, p) >= 0 : (page_ok && p < rc.n);
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

// Levels 5 and 6 of the head sum for a chunk's four sub-tiles at once.
// Lane (g, col) holds s16[st], the sum of heads 16 g .. 16 g + 15 of entry
// 16 st + col.  Swapping odd rows of one register with even rows of another
// (lane groups g, g ^ 1) pairs the quarters as Q0 + Q1 and Q2 + Q3 of two
// sub-tiles per register; swapping the upper half of one register with the
// lower half of the other (g, g ^ 2) adds those pairs, and sub-tile st's
// total lands in lane group g = st: lane e holds the sum of entry e.  Then
// + 0 (no -0).  The tree is the one head_sum4 follows.
__device__ __forceinline__ float chunk_head_sum(const float (&s16)[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s16[0]), __float_as_uint(s16[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s16[2]), __float_as_uint(s16[3]), false, false);
  const float A = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float B = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  return (__uint_as_float(c[0]) + __uint_as_float(c[1])) + 0.0f;
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
                                               const v4f (&wreg)[kRT], bool& page_ok, uint32_t& mxbad) {
  const int lane = lane_id();
  const int g = lane >> 4, col = lane & 15;
  ChunkKeys raw;
  page_ok = load_chunk<POOL, MX>(a, rc, chunk, g, col, raw);
  float s_mine = 0.0f;
#pragma unroll
  for (int st = 0; st < kSub; ++st) {
    v4i kl[2], km[2], kt[2];
    if (MX) {
      mxbad |= mx_scale_bad(raw.k[st][1]);
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

// ---------------------------------------------------------------- segments
// The plan of one segment: one token's part of one list.
struct SegPlan {
  int64_t bt;        // (b, t) row
  int list;          // 0: entry scores, 1: block maxima
  int p0, p1;        // the part's list positions [p0, p1)
  int n_valid;       // valid keys of the part
  int m;             // keys to keep at least
  int coarse;        // the coarse bin holding the m-th key (-1: keep every valid key)
  int rem;           // the m-th key's rank inside that bin
  uint32_t thr;      // keys >= thr are kept
};

// Coarse histogram (1,024 bins of 16-bit counters, two per word), one wave:
// the bin holding rank x >= 1 counted from the top, or -1 when the
// histogram holds fewer than x keys; *above: keys in higher bins; *total:
// every key.  Lane l sums bins 1008 - 16 l .. 1023 - 16 l (lane 0 the
// highest); the crossing lane's 16 bins are then scanned across lanes.
__device__ int coarse_crossing(const uint32_t* h, uint32_t x, uint32_t* above, uint32_t* total) {
  const int lane = lane_id();
  const v4u* hv = reinterpret_cast<const v4u*>(h + kHistBins / 2 - 8 * (lane + 1));
  const v4u w0 = hv[0], w1 = hv[1];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) sum += (w0[i] & 0xFFFFu) + (w0[i] >> 16) + (w1[i] & 0xFFFFu) + (w1[i] >> 16);
  const uint32_t incl = wave_incl_scan(sum);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint64_t who = __ballot(incl - sum < x && x <= incl);
  if (who == 0) {
    *above = 0;
    return -1;
  }
  const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(who));
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), src);
  const int top = kHistBins - 16 * src - 1;
  const int bin = top - lane;
  const uint32_t c = lane < 16 ? (h[bin >> 1] >> (16 * (bin & 1))) & 0xFFFFu : 0u;
  const uint32_t ci = wave_incl_scan(c);
  const uint64_t hit = __ballot(lane < 16 && base + ci >= x);
  const int k = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  *above = base + (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), k);
  return top - k;
}

// Fine histogram (4,096 bins of 32-bit counters), one wave: the bin holding
// rank x >= 1 from the top (the histogram holds at least x keys).  Lane l
// sums bins 4032 - 64 l .. 4095 - 64 l.
__device__ int fine_crossing(const uint32_t* h, uint32_t x) {
  const int lane = lane_id();
  const v4u* hv = reinterpret_cast<const v4u*>(h + kFineBins - 64 * (lane + 1));
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const v4u v = hv[i];
    sum += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint64_t who = __ballot(incl - sum < x && x <= incl);
  const int src = who ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(who)) : 63;
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), src);
  const int top = kFineBins - 64 * src - 1;
  const uint32_t c = h[top - lane];
  const uint32_t ci = wave_incl_scan(c);
  const uint64_t hit = __ballot(base + ci >= x);
  const int k = hit ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit)) : 63;
  return top - k;
}

// Exclusive prefix sum over one group of four waves (waves 4 gr .. 4 gr + 3)
// in thread order; every thread also gets its group's total.  Both groups
// call it together (its two barriers are the workgroup's).  Uses
// scan_tot[kWaves] (free again on return).
__device__ int group_excl_scan256(int v, int* scan_tot, int* total) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g0 = wave & ~3, wg = wave & 3;
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) scan_tot[wave] = x;
  lds_barrier();
  const int wt = (int)wave_incl_scan(lane < 4 ? (uint32_t)scan_tot[g0 + lane] : 0u);
  const int before = wg > 0 ? __builtin_amdgcn_readlane(wt, wg - 1) : 0;
  *total = __builtin_amdgcn_readlane(wt, 3);
  lds_barrier();
  return before + x - v;
}

// Writes this workgroup's segments (see index_common.h): for each token slot
// and list, the keys of the workgroup's part at or above a threshold key,
// in list order, with their positions.  The threshold is the lower edge of
// the fine bin (22 key bits) holding the part's m-th largest key, where m is
// one and a half times the part's expected share of the list's top K plus
// 16 (all keys when that is the whole part).  Keys and block maxima are
// read back from the workspace, where this workgroup has just written them.
// The (token, list) pairs go two at a time, one to each half of the
// workgroup (waves 0-3 and 4-7), in rounds of 16 consecutive positions per
// thread (4,096 per half and round; a part of one round is read once); both
// halves run the same steps and barriers, with the work masked off where a
// half has nothing to do, so the two pairs' dependent steps overlap.
template <bool POOL>
__device__ void write_segments(const ScoreArgs& a, const RowCtx& rc, int slot, int Ts, int Tg, int seg, int nseg,
                               int c0, int c1,
                               uint32_t (&hist)[kGroupT][2][kHistBins / 2],
                               uint32_t (&fine)[2 * kGroupT][kFineBins], const uint32_t* mxbad, SegPlan* plan,
                               int* scan_tot) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tid = threadIdx.x;
  const int n_pairs = POOL ? 1 : 2 * Tg;
  const int cap = seg_cap_at(a.seg_k, seg);
  const int64_t list_stride_s = POOL ? (int64_t)a.pool_blocks * kBlock : (int64_t)s_stride(a.max_n);

  // ---- 1. the plan of pair (token slot ts, list L), by wave ts + Ts L, which
  // holds token ts's row context: the part, its count, the coarse crossing
  const int L = POOL ? 0 : wave / Ts;
  if (POOL ? wave == 0 : (L < 2 && slot < Tg)) {
    const int ts = POOL ? 0 : slot;
    SegPlan pl;
    pl.bt = (int64_t)rc.b * a.T + rc.t;
    pl.list = L;
    const int nb = (rc.n + kBlock - 1) / kBlock;
    const int len = L == 0 ? rc.n_pos : nb;
    const int unit = L == 0 ? kChunk : kChunk / kBlock;
    pl.p0 = min(c0 * unit, len);
    pl.p1 = min(c1 * unit, len);
    const int K = L == 0 ? a.topk : a.pool_blocks;
    uint32_t total = 0, above = 0;
    pl.coarse = -1;
    pl.rem = 0;
    pl.thr = 1u;  // every valid key
    (void)coarse_crossing(hist[ts][L], 0xFFFFFFFFu, &above, &total);
    pl.n_valid = (int)total;
    // m: 1.5 x the part's share of K (its valid keys over the list's
    // length), + 16, and at most the segment's capacity less its margin
    // (which is still >= K)
    const int64_t n_row = max(len, 1);
    const int64_t share = ((int64_t)3 * K * total + 2 * n_row - 1) / (2 * n_row);
    pl.m = (int)min((int64_t)total, min(share + 16, (int64_t)(cap - 64)));
    if (pl.m < pl.n_valid) {
      pl.coarse = coarse_crossing(hist[ts][L], (uint32_t)pl.m, &above, &total);
      pl.rem = pl.m - (int)above;
    }
    if (lane == 0) plan[POOL ? 0 : 2 * ts + L] = pl;
  }
  lds_barrier();

  // ---- 2. the pairs, two at a time
  constexpr int kGT = kScoreThreads / 2;  // threads of a half
  constexpr int kPer = 16;                // positions per thread and round
  const int grp = wave >> 2;
  const int gt = tid & (kGT - 1);
  uint32_t* gfine = fine[grp];
  for (int r = 0; r < (n_pairs + 1) / 2; ++r) {
    const int p = 2 * r + grp;
    const bool mine = p < n_pairs;
    const bool two = 2 * r + 1 < n_pairs;
    const SegPlan pl0 = plan[2 * r];
    const SegPlan pl1 = plan[two ? 2 * r + 1 : 2 * r];
    SegPlan pl = grp ? pl1 : pl0;
    // rounds, and whether a fine pass runs: the same in both halves
    const int len = max(pl0.p1 - pl0.p0, two ? pl1.p1 - pl1.p0 : 0);
    const int n_rr = (len + kPer * kGT - 1) / (kPer * kGT);
    const bool fine_any = pl0.coarse >= 0 || (two && pl1.coarse >= 0);
    const bool fine_mine = mine && pl.coarse >= 0;
    const float* src = pl.list == 0 ? a.out_s + pl.bt * list_stride_s : a.out_bm + pl.bt * bm_stride(a.max_n);
    // keys of positions q0 .. q0 + 15 (0 past the part, and in a half with
    // no pair); rows start 16-byte aligned and p0 is a multiple of 8
    auto load16 = [&](int q0, uint32_t (&k)[kPer]) __attribute__((always_inline)) {
      if (mine && q0 + kPer <= pl.p1) {
        const v4u* v = reinterpret_cast<const v4u*>(src + q0);
        v4u x[kPer / 4];
#pragma unroll
        for (int i = 0; i < kPer / 4; ++i) x[i] = v[i];
#pragma unroll
        for (int i = 0; i < kPer / 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) k[4 * i + e] = score_key(__uint_as_float(x[i][e]));
      } else {
#pragma unroll
        for (int e = 0; e < kPer; ++e) k[e] = (mine && q0 + e < pl.p1) ? score_key(src[q0 + e]) : 0u;
      }
    };
    const bool one = n_rr == 1;
    uint32_t keys[kPer];
    if (fine_any) {
      // ---- fine histogram (next 12 bits) of the keys in the crossing
      // coarse bin, and its crossing: the threshold
      if (fine_mine) {
#pragma unroll
        for (int i = 0; i < kFineBins / kGT; ++i) gfine[gt + i * kGT] = 0u;
      }
      lds_barrier();
      for (int rr = 0; rr < n_rr; ++rr) {
        load16(pl.p0 + rr * kPer * kGT + kPer * gt, keys);
        if (fine_mine) {
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            if (keys[e] != 0u && (int)(keys[e] >> 22) == pl.coarse)
              atomicAdd(&gfine[(keys[e] >> 10) & (kFineBins - 1)], 1u);
        }
      }
      lds_barrier();
      if (fine_mine && (wave & 3) == 0) {
        const int c2 = fine_crossing(gfine, (uint32_t)pl.rem);
        if (lane == 0) plan[p].thr = ((uint32_t)pl.coarse << 22) | ((uint32_t)c2 << 10);
      }
      lds_barrier();
      if (mine) pl.thr = plan[p].thr;
    } else if (one) {
      load16(pl.p0 + kPer * gt, keys);
    }

    // ---- 3. compaction: kept keys in list order
    SegHeader* hdr = a.seg_hdr + (pl.bt * 2 + pl.list) * a.max_segs + seg;
    Cand* cand = a.seg_cand + (pl.bt * 2 + pl.list) * a.seg_region + seg_off_at(a.seg_k, seg);
    int written = 0;
    for (int rr = 0; rr < n_rr; ++rr) {
      const int q0 = pl.p0 + rr * kPer * kGT + kPer * gt;
      if (!one) load16(q0, keys);
      uint32_t keep = 0u;
#pragma unroll
      for (int e = 0; e < kPer; ++e) keep |= (keys[e] != 0u && keys[e] >= pl.thr ? 1u : 0u) << e;
      const int cnt = __builtin_popcount(keep);
      int tot;
      const int before = group_excl_scan256(cnt, scan_tot, &tot);
      int o = written + before;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if ((keep >> e) & 1u) {
          if (o < cap) cand[o] = Cand{keys[e], q0 + e};
          ++o;
        }
      }
      written += tot;
    }
    if (mine && gt == 0) {
      uint32_t flags = 0u;
      if (written < pl.n_valid) flags |= kSegDropped;
      if (written > cap) flags |= kSegOverflow;
      if (mxbad[POOL ? 0 : p >> 1] != 0u) flags |= kSegBadScale;
      *hdr = SegHeader{(uint32_t)min(written, cap) | (flags << 24), pl.thr};
      if (seg == 0 && pl.list == 0) a.seg_n[pl.bt] = nseg;
    }
  }
}

// Balanced plan of a Full-mode scan: the kScanTarget workgroups are shared
// out over the rows (sequence, token group) in proportion to their work,
// visible chunks (the group's largest visible count) times tokens.  Every
// row first gets the workgroups its length needs under the per-workgroup
// chunk cap, then a share of the rest; its chunks are split into whole
// rounds of its waves.  Row r's workgroups follow those of rows < r.  Every
// wave computes the whole plan from the rows' counts (at most kScanTarget
// rows; lane L holds rows j * 64 + L, so groups of 64 rows past the last one
// cost nothing), with no barrier, and takes its workgroup's part; workgroups
// past the plan's total get row = rows (none).
constexpr int kPlanRows = kScanTarget / 64;

struct PlanRows {
  int ch[kPlanRows], minw[kPlanRows], work[kPlanRows];
};

// The loaded counts of lane L's rows j * 64 + L (clamped indices, every load
// unconditional): n_entries and, with per-token counts, the group's tokens'.
struct PlanRaw {
  int n[kPlanRows];
  int v[kPlanRows][kGroupT];
};

struct PlanPart {
  int row, seg, nseg, c0, c1;
};

// floor(x / d) for 0 <= x < 2^24, 1 <= d < 2^24 and a quotient below 2^20:
// the single-precision estimate is off by at most one either way.
__device__ __forceinline__ int plan_div(int x, int d) {
  int q = (int)((float)x * __builtin_amdgcn_rcpf((float)d));
  const int r = x - q * d;
  q += (r >= d) ? 1 : 0;
  q -= (r < 0) ? 1 : 0;
  return q;
}

// The waves' rounds (slices) of a row of tg tokens: 8 / tg slots, a group of
// three taking four slots.
__device__ __forceinline__ int plan_slices(int tg) { return tg == 1 ? kWaves : tg == 2 ? kWaves / 2 : kWaves / 4; }

// Row r's token group: sequence b, first token t0, tokens tg.
__device__ __forceinline__ void plan_group(const ScoreArgs& a, int r, int& b, int& t0, int& tg) {
  if (a.n_groups == 1) {
    b = r;
    t0 = 0;
  } else {
    b = plan_div(r, a.n_groups);
    t0 = (r - b * a.n_groups) * kGroupT;
  }
  tg = min(kGroupT, a.T - t0);
}

__device__ __forceinline__ PlanRaw plan_row_loads(const ScoreArgs& a) {
  PlanRaw pr;
#pragma unroll
  for (int j = 0; j < kPlanRows; ++j) {
    const int r = min(j * 64 + lane_id(), a.rows - 1);
    int b, t0, tg;
    plan_group(a, r, b, t0, tg);
    pr.n[j] = a.n_entries[b];
#pragma unroll
    for (int k = 0; k < kGroupT; ++k)
      pr.v[j][k] = a.n_vis != nullptr ? a.n_vis[(int64_t)b * a.T + min(t0 + k, a.T - 1)] : 0x7FFFFFFF;
  }
  return pr;
}

// Lane L's rows j * 64 + L: visible chunks, workgroups their length needs
// (the per-workgroup cap is kMaxWgChunks for every token count), work.
__device__ __forceinline__ PlanRows plan_row_counts(const ScoreArgs& a, const PlanRaw& raw) {
  PlanRows pr;
#pragma unroll
  for (int j = 0; j < kPlanRows; ++j) {
    const int r = j * 64 + lane_id();
    pr.ch[j] = 0;
    pr.minw[j] = 0;
    pr.work[j] = 0;
    if (r < a.rows) {
      int b, t0, tg;
      plan_group(a, r, b, t0, tg);
      int n = min(min(raw.n[j], a.max_n), a.max_pages * kPage);
      int nm = 0;
#pragma unroll
      for (int k = 0; k < kGroupT; ++k)
        if (k < tg) nm = max(nm, min(n, raw.v[j][k]));
      n = max(nm, 0);
      const int ch = (n + kChunk - 1) / kChunk;
      pr.ch[j] = ch;
      pr.minw[j] = max(1, (ch + kMaxWgChunks - 1) / kMaxWgChunks);
      pr.work[j] = ch * tg;
    }
  }
  return pr;
}

__device__ __forceinline__ PlanPart scan_plan_balanced(const ScoreArgs& a, const PlanRows& pr) {
  const int lane = lane_id();
  int sm_ = 0, sw_ = 0;
#pragma unroll
  for (int j = 0; j < kPlanRows; ++j) {
    sm_ += pr.minw[j];
    sw_ += pr.work[j];
  }
  const int minw_tot = wave_sum(sm_), work_tot = wave_sum(sw_);
  const int budget = max(0, kScanTarget - minw_tot);
  const int wg = (int)blockIdx.x;
  int base = 0;  // workgroups of the groups of rows before j
  int hit = 0, hseg = 0, hnseg = 1, hc0 = 0, hc1 = 0;
#pragma unroll
  for (int j = 0; j < kPlanRows; ++j) {
    if (j * 64 >= a.rows) break;  // uniform
    const int r = j * 64 + lane;
    int w = 0, per = 1;
    if (r < a.rows) {
      int b, t0, tg;
      plan_group(a, r, b, t0, tg);
      const int slices = plan_slices(tg);
      // budget <= 256 and work <= 4 * 4096: the product fits 24 bits
      w = pr.minw[j] + (work_tot > 0 ? plan_div(budget * pr.work[j], work_tot) : 0);
      w = min(w, a.max_segs);
      const int ch = pr.ch[j];
      if (ch > 0) {
        per = plan_div(ch + w - 1, w);
        per = (per + slices - 1) & ~(slices - 1);  // slices is a power of two
        w = plan_div(ch + per - 1, per);
      } else {
        w = 1;
      }
    }
    const int incl = (int)wave_incl_scan((uint32_t)w);
    const int first = base + incl - w;
    if (w > 0 && wg >= first && wg < first + w) {
      hit = 1;
      hseg = wg - first;
      hnseg = w | (j << 16);
      hc0 = hseg * per;
      hc1 = min(pr.ch[j], hc0 + per);
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  const uint64_t m = __ballot(hit);
  PlanPart p{a.rows, 0, 1, 0, 0};
  if (m != 0) {
    const int src = (int)__builtin_ctzll(m);
    const int hn = __builtin_amdgcn_readlane(hnseg, src);
    p.row = (hn >> 16) * 64 + src;
    p.nseg = hn & 0xFFFF;
    p.seg = __builtin_amdgcn_readlane(hseg, src);
    p.c0 = __builtin_amdgcn_readlane(hc0, src);
    p.c1 = __builtin_amdgcn_readlane(hc1, src);
  }
  return p;
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
    union {
      // per token: the f16 limbs ql, qm of the query, in the order the
      // waves hold them: [row tile][slice][limb][lane] (read into registers
      // before the main loop)
      v8h qlimb[kGroupT][kRT][4][2][64];
      // after the main loop: per (token, list) the fine histogram of the
      // keys in the crossing coarse bin
      uint32_t fine[2 * kGroupT][kFineBins];
    };
    float wsh[kGroupT][kRT * 16];                 // w * 2^-9 per head, 0 past HI
    uint32_t qbad[kGroupT];                       // nonzero: some |q| >= 32
    uint32_t mxbad[kGroupT];                      // nonzero: an MXFP4 scale code out of range
    uint32_t defer[kWaves][kMaxWaveChunks / 32];  // chunks left to the general path
    // per token: coarse histograms (top 10 key bits) of the entry scores and
    // block maxima, 16-bit counters packed two per word
    uint32_t hist[kGroupT][2][kHistBins / 2];
    SegPlan plan[2 * kGroupT];                    // per (token, list): the segment's plan
    int pslot[CSA2_MAX_POOL_BLOCKS];              // pool mode: the workgroup's slots (pool_slot_word)
    int scan_tot[kWaves];                         // block-wide prefix sums
  };
  __shared__ Lds sm;

  for (int i = threadIdx.x; i < kWaves * kMaxWaveChunks / 32; i += blockDim.x) (&sm.defer[0][0])[i] = 0u;
  for (int i = threadIdx.x; i < kGroupT * kHistBins; i += blockDim.x) (&sm.hist[0][0][0])[i] = 0u;
  if (threadIdx.x < kGroupT) {
    sm.qbad[threadIdx.x] = 0u;
    sm.mxbad[threadIdx.x] = 0u;
  }

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4;   // K slice group of the MFMA operands; head group of the outputs
  const int col = lane & 15;
  const int HI = a.HI;
  // ---- this workgroup's row, segment of the row and chunk range: the
  // static plan first; with the balanced plan its result replaces it, and
  // the early loads below are issued again only when they differ (equal
  // rows of the greatest length give the same plan)
  int row = blockIdx.x / a.wg_per_row;
  int seg = blockIdx.x % a.wg_per_row;
  int nseg = a.wg_per_row;
  int c0 = seg * a.chunks_per_wg;
  int c1 = min(a.chunks_per_row, c0 + a.chunks_per_wg);
  // Full mode: tokens t0 .. t0 + Tg - 1 of the sequence, in Ts token slots
  // (a group of three keeps a dead fourth slot, so that the slots divide the
  // 8 waves); each wave takes one slot and a slice of the chunk range
  int t0, Tg, Ts, slot, t_full, slice, n_slices, n_tok;
  RowCtx rc;
  auto set_row = [&]() {
    const int rr = min(row, a.rows - 1);  // (a guess past the rows reads row rows - 1, unused)
    t0 = POOL ? 0 : (rr % a.n_groups) * kGroupT;
    Tg = POOL ? 1 : min(kGroupT, a.T - t0);
    Ts = Tg == 3 ? 4 : Tg;
    slot = POOL ? 0 : wave % Ts;
    t_full = POOL ? 0 : t0 + min(slot, Tg - 1);
    slice = POOL ? wave : wave / Ts;
    n_slices = POOL ? kWaves : kWaves / Ts;
    n_tok = POOL ? 1 : Ts;
    rc = RowCtx{};
    row_ctx_load<POOL>(a, rr, t_full, slot < Tg, rc);
  };
  set_row();

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
  uint32_t qraw[kLimbIters][2], qkeep[kLimbIters];
  uint32_t wraw, wkeep;
  int page_word = -1;
  auto issue_early = [&]() {
    const int n_items = n_tok * kRT * 4 * 64;  // 1024 n_tok, a power of two
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
    {
      const int i = min((int)threadIdx.x, n_tok * 64 - 1);
      const int tk = i >> 6, h = i & 63;
      const int t = POOL ? rc.t : t0 + min(tk, Tg - 1);
      wraw = __float_as_uint(a.w[((int64_t)rc.b * a.T + t) * HI + min(h, HI - 1)]);
      wkeep = ((int)threadIdx.x < n_tok * 64 && h < HI && (POOL || tk < Tg)) ? 0xFFFFFFFFu : 0u;
      asm volatile("" : "+v"(wkeep));
    }
    if (!POOL) {
      const int ck = c0 + slice + lane * n_slices;
      page_word = a.page_table[(int64_t)rc.b * a.max_pages + max(0, min(ck, a.max_pages - 1))];
    }
  };
  int wave_pages = -1;
  ChunkKeys cur;
  bool cur_ok = false;
  // Full mode: the physical pages of this wave's chunks, lane k holding the
  // page of its chunk number k0 + k (refilled every 64 chunks), so the loop
  // reads them with readlane and issues no memory load of its own for them
  // (a vector load there would wait for the key prefetch as well)
  auto fill_pages = [&](int k0) {
    const int ck = c0 + slice + (k0 + lane) * n_slices;
    wave_pages = (!POOL && ck < c1) ? (int)chunk_page(a, rc, ck) : -1;
  };
  auto page_of = [&](int k) -> int64_t {
    return POOL ? 0 : (int64_t)__builtin_amdgcn_readlane(wave_pages, k & 63);
  };
  // the balanced plan: its row counts go out first, then the early loads for
  // the static plan's part; when the balanced plan gives another part, the
  // early loads go out again for it
  if (!POOL && a.balanced) {
    const PlanRaw praw = plan_row_loads(a);
    issue_early();
    row_ctx_finish<POOL>(a, rc);
    const PlanPart pp = scan_plan_balanced(a, plan_row_counts(a, praw));
    if (pp.row >= a.rows) return;  // past the plan (the same for the whole workgroup)
    seg = pp.seg;
    nseg = pp.nseg;
    if (pp.row != row || pp.c0 != c0 || pp.c1 != c1) {
      row = pp.row;
      c0 = pp.c0;
      c1 = pp.c1;
      set_row();
      issue_early();
      row_ctx_finish<POOL>(a, rc);
    }
  } else {
    issue_early();
    row_ctx_finish<POOL>(a, rc);
  }
  const bool have_row = row < a.rows;
  int chunk = c0 + slice;
  const bool active = have_row && chunk < c1 && slot < Tg;
  uint32_t* hist_s = sm.hist[slot][0];
  uint32_t* hist_bm = sm.hist[slot][1];
  const int64_t qrow0 = ((int64_t)rc.b * a.T + rc.t) * HI;
  const int n_items = n_tok * kRT * 4 * 64;
  if (POOL && have_row) {
    // the workgroup's pool slots, resolved once to physical entries (the
    // pool word and page-table word of a slot are the only dependent loads)
    const int nsl = (c1 - c0) * kBlock;
    for (int i = (int)threadIdx.x; i < nsl; i += kScoreThreads) sm.pslot[i] = pool_slot_word(a, rc, c0 * kBlock + i);
    rc.pslot = sm.pslot;
    rc.slot0 = c0 * kBlock;
    rc.nslots = nsl;
  }
  lds_barrier();

  // every early load has arrived here (they went out together): waiting
  // for them before the key loads leaves nothing to wait for in the limb work
#pragma unroll
  for (int j = 0; j < kLimbIters; ++j) asm volatile("" ::"v"(qraw[j][0]), "v"(qraw[j][1]));
  asm volatile("" ::"v"(wraw), "v"(page_word));
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
  uint32_t mxbad = 0u;

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
    // ---- a sub-tile's keys as f16 (exact for every E4M3 code), in the
    // channel order of the query slices
    auto convert = [&](int st, v8h (&kf)[4]) __attribute__((always_inline)) {
      if (MX) {
        mxbad |= mx_scale_bad(cur.k[st][1]);
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
    };
    // fl(2^9 d) = fl(S_l + 2^7 S_m) (both sums exact, one rounding), then
    // fl(w_h * max(d_h, +0)) and the row tile's pairwise sum
    auto weigh = [&](const v4f& cl, const v4f& cm, const v4f& wv) __attribute__((always_inline)) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = __builtin_fmaf(128.0f, cm[i], cl[i]);
        p[i] = wv[i] * (r > 0.0f ? r : 0.0f);
      }
      return (p[0] + p[1]) + (p[2] + p[3]);
    };
    const v4f z4 = {0.0f, 0.0f, 0.0f, 0.0f};
    v8h kf[4];
    __builtin_amdgcn_sched_barrier(0);
    convert(0, kf);
    // the same sub-tile of the next chunk streams into the freed registers
    // (after the conversions have read them)
    __builtin_amdgcn_sched_barrier(0);
    load_sub<POOL, MX>(a, rc, next, next_pg, 0, g, col, cur.k[0]);
    __builtin_amdgcn_sched_barrier(0);
    // software pipeline over (sub-tile, row tile) steps: each step's 8 MFMAs
    // go out between the VALU work that weighs the previous step's sums, so
    // the wave's VALU work fills the matrix unit's busy cycles
    v4f pl = z4, pm = z4, gram_prev = z4;
    float q4[kRT];
    // Full mode: per sub-tile this lane's quarter of the head sum, summed
    // across the lane groups once per chunk; Reindex mode sums each
    // sub-tile on its own (no registers to spare for the four quarters)
    float s16[kSub];
    static_assert(kSub == 4, "one sub-tile per lane group");
#pragma unroll
    for (int st = 0; st < kSub; ++st) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        v4f cl = z4, cm = z4;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql[rt][sl], kf[sl], cl, 0, 0, 0);
          cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(qm[rt][sl], kf[sl], cm, 0, 0, 0);
        }
        if (st > 0 || rt > 0) {
          const int prt = rt == 0 ? kRT - 1 : rt - 1;
          q4[prt] = weigh(pl, pm, wreg[prt]);
          if (rt == 0) {
            if (POOL)
              s_mine = keep_subtile(s_mine, head_sum4(q4), st - 1, lane);
            else
              s16[st - 1] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
            gmax = fmaxf(gmax, fmaxf(fmaxf(gram_prev[0], gram_prev[1]), fmaxf(gram_prev[2], gram_prev[3])));
          }
        }
        // order: one MFMA (mask 0x008), two VALU (mask 0x002), eight times
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pl = cl;
        pm = cm;
      }
      // K K^T over the 128 channels: its diagonal holds sum_c k_c^2 of each
      // entry, and no other element exceeds the largest diagonal one
      // (Cauchy-Schwarz), so the maximum over all outputs is the largest
      // sum of squares of the sub-tile
      v4f gram = z4;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) gram = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[sl], kf[sl], gram, 0, 0, 0);
      gram_prev = gram;
      if (st + 1 < kSub) {
        v8h kn[4];
        convert(st + 1, kn);  // beside the Gram MFMAs, four VALU after each
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_sub<POOL, MX>(a, rc, next, next_pg, st + 1, g, col, cur.k[st + 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = kn[i];
      }
    }
    q4[kRT - 1] = weigh(pl, pm, wreg[kRT - 1]);
    if (POOL) {
      s_mine = keep_subtile(s_mine, head_sum4(q4), kSub - 1, lane);
    } else {
      s16[kSub - 1] = (q4[0] + q4[1]) + (q4[2] + q4[3]);
      s_mine = chunk_head_sum(s16);
    }
    gmax = fmaxf(gmax, fmaxf(fmaxf(gram_prev[0], gram_prev[1]), fmaxf(gram_prev[2], gram_prev[3])));
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
      const float s = general_chunk<POOL, MX>(a, rc, ck, gq, wreg, ok, mxbad);
      emit_chunk<POOL>(a, rc, ck, s, ok, hist_s, hist_bm);
    }
  }
  if (MX && __ballot(mxbad != 0u) != 0u && lane == 0) atomicOr(&sm.mxbad[slot], 1u);
  }  // this wave's chunks

  // ---- the candidate segments of this workgroup's part of each list
  __syncthreads();  // every wave's scores, block maxima and coarse counts are in place
  if (have_row) write_segments<POOL>(a, rc, slot, Ts, Tg, seg, nseg, c0, c1, sm.hist, sm.fine, sm.mxbad, sm.plan, sm.scan_tot);
}

}  // namespace csa2

// Workgroups of the scan: each takes a range of chunks inside one row,
// kScanTarget workgroups in all when the rows allow it.  With T_slots
// tokens sharing a workgroup, every wave covers chunks_per_wg * T_slots / 8
// chunks of the range.
int csa2_score_grid(int rows, int chunks_per_row, int T_slots, int* chunks_per_wg, int* wg_per_row) {
  const int slices = csa2::kWaves / T_slots;
  const int want = std::max(1, csa2::kScanTarget / rows);
  int per = (chunks_per_row + want - 1) / want;
  per = ((per + slices - 1) / slices) * slices;  // whole rounds of the waves
  // each wave tracks at most kMaxWaveChunks chunks; the workgroup's 16-bit
  // histogram counters hold at most kMaxWgChunks chunks of one token
  const int cap = std::min(csa2::kMaxWaveChunks * slices, csa2::kMaxWgChunks);
  per = std::min(per, cap);
  int wpr = (chunks_per_row + per - 1) / per;
  // more workgroups than one per compute unit: make the rounds whole, so
  // that a short last round does not run on a few units while the rest idle
  // (a 256-token prefill chunk at 1M context: 5 x 64 = 320 workgroups of
  // 1,016 chunks become 512 of 512)
  const int64_t total = (int64_t)rows * wpr;
  if (total > csa2::kScanTarget) {
    const int64_t rounds = (total + csa2::kScanTarget - 1) / csa2::kScanTarget;
    const int want2 = (int)((rounds * csa2::kScanTarget + rows - 1) / rows);
    int per2 = (chunks_per_row + want2 - 1) / want2;
    per2 = ((per2 + slices - 1) / slices) * slices;
    per = std::min(std::max(per2, slices), cap);
    wpr = (chunks_per_row + per - 1) / per;
  }
  *chunks_per_wg = per;
  *wg_per_row = wpr;
  return rows * wpr;
}

bool csa2_scan_balanced(int rows, int chunks_per_row) {
  const int need = (chunks_per_row + csa2::kMaxWgChunks - 1) / csa2::kMaxWgChunks;  // per row, at most
  return rows <= csa2::kScanTarget && (int64_t)rows * std::max(need, 1) <= csa2::kScanTarget;
}

int csa2_launch_scan(bool pool, bool mx, csa2::ScoreArgs& sa, int T_slots, hipStream_t stream) {
  int gx = csa2_score_grid(sa.rows, sa.chunks_per_row, T_slots, &sa.chunks_per_wg, &sa.wg_per_row);
  sa.balanced = (!pool && csa2_scan_balanced(sa.rows, sa.chunks_per_row)) ? 1 : 0;
  if (sa.balanced) gx = csa2::kScanTarget;
  else if (sa.wg_per_row > sa.max_segs) return CSA2_ERR_LAUNCH;
  if (sa.max_segs > csa2::kMaxSegs) return CSA2_ERR_LAUNCH;
  const dim3 grid(gx), block(csa2::kScoreThreads);
  if (pool && mx)
    CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, (csa2::score_kernel<true, true>), grid, block, stream, sa);
  else if (pool)
    CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, (csa2::score_kernel<true, false>), grid, block, stream, sa);
  else if (mx)
    CSA2_LAUNCH(CSA2_K_SCORE_FULL, (csa2::score_kernel<false, true>), grid, block, stream, sa);
  else
    CSA2_LAUNCH(CSA2_K_SCORE_FULL, (csa2::score_kernel<false, false>), grid, block, stream, sa);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
