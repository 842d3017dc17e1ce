// Hierarchical sparse indexer: Full scan, block-max pool, Reindex over the
// pool (knowledge note "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression", section "Hierarchical Sparse Indexer", Figure 5; "Inside
// DeepSeek V4.1 Flash", section "Hierarchical indexing bounds later searches,
// not every search").
//
// Score of entry j for one query token (per indexer head h):
//   d_h = exact sum_c q[h][c] k_j[c], rounded once to binary32
//   s_j = binary32 fold over ascending h of fl(w_h * max(d_h, +0)).
//
// Exactness on MFMA.  Every E4M3 value is M * 2^-9 with M an integer,
// |M| <= 229,376 < 2^18.  M is split into sign-magnitude 7-bit limbs
// (lo, mid, top), each in [-127, 127], so q.k * 2^18 = sum over limb pairs
// of 2^(7(a+b)) * (Q_a . K_b), and every Q_a . K_b is an exact int32 from
// the int8 MFMA.  For the common case (all |q|, |k| < 32, i.e. no top limb,
// and sum_c |Mq| < 2^17) the recombined integer fits int32 and is rounded
// to binary32 by one conversion; otherwise the five weighted partial sums
// are combined exactly in binary64 (at most 43 significant bits) and
// rounded once.  The FP8 MFMA is not used: it aligns each group of 8
// products to the group maximum and keeps about 13 bits, so it does not
// return the exactly rounded dot.
//
// Layout of v_mfma_i32_16x16x64_i8 used below: lane l holds row (l & 15) of
// A and column (l & 15) of B, bytes 16*(l >> 4) .. +15 of the 64-deep slice;
// the 4 outputs of lane l are rows 4*(l >> 4) + i, column l & 15.
#include <algorithm>

#include "common.h"

namespace csa2 {

constexpr int kScoreThreads = 512;        // 8 waves
constexpr int kWaves = kScoreThreads / 64;
constexpr int kChunk = 32;                // entries scored together per wave (half a page)
constexpr int kSub = kChunk / 16;         // 16-entry MFMA sub-tiles per chunk
constexpr int kMaxRT = 4;                 // row tiles of 16 heads (HI <= 64)
constexpr int kPassHeads = 64;            // heads folded per pass
constexpr int kPassRT = kPassHeads / 16;  // row tiles per pass
constexpr int kFoldStride = kPassHeads + 4;  // floats per entry row of the fold buffer
constexpr int kMaxWaveChunks = 1024;      // chunks one wave may take in one launch
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data, no swizzle)

// Lookup table: for every E4M3 code, its sign-magnitude 7-bit limbs of
// M = value * 2^9 packed as int8 bytes [lo, mid, top, 0]; 64 copies so the
// 64 lanes of a wave read distinct banks (address = code * 256 + lane * 4).
__device__ __forceinline__ uint32_t limb_entry(uint32_t code) {
  uint32_t e = (code >> 3) & 15u, m = code & 7u;
  uint32_t M = (e == 0) ? m : ((8u + m) << (e - 1));
  if (e == 15 && m == 7) M = 0;  // NaN codes are a precondition violation; keep them inert
  uint32_t lo = M & 127u, mid = (M >> 7) & 127u, top = M >> 14;
  if (code & 0x80u) {
    lo = (0u - lo) & 0xFFu;
    mid = (0u - mid) & 0xFFu;
    top = (0u - top) & 0xFFu;
  }
  return lo | (mid << 8) | (top << 16);
}

__device__ void build_lut(uint32_t* lut) {
  for (int i = threadIdx.x; i < 256 * 64; i += blockDim.x) lut[i] = limb_entry((uint32_t)(i >> 6));
}

__device__ __forceinline__ uint32_t lut_read(const uint8_t* lut_bytes, uint32_t lane4, uint32_t x, int k) {
  const uint32_t addr = __builtin_amdgcn_perm(x, lane4, 0x0C0C0000u | ((4u + k) << 8));
  return *reinterpret_cast<const uint32_t*>(lut_bytes + addr);
}

// 16 FP8 codes -> lo and mid limb planes; `any` collects the top limbs
// (nonzero iff some |value| >= 32).
__device__ __forceinline__ void limbs2(const uint8_t* lut_bytes, uint32_t lane4, v4u codes, v4i& lo,
                                      v4i& mid, uint32_t& any) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = codes[d];
    const uint32_t L0 = lut_read(lut_bytes, lane4, x, 0), L1 = lut_read(lut_bytes, lane4, x, 1);
    const uint32_t L2 = lut_read(lut_bytes, lane4, x, 2), L3 = lut_read(lut_bytes, lane4, x, 3);
    const uint32_t t01 = __builtin_amdgcn_perm(L1, L0, 0x05010400u);  // [lo0 lo1 mid0 mid1]
    const uint32_t t23 = __builtin_amdgcn_perm(L3, L2, 0x05010400u);
    lo[d] = (int)__builtin_amdgcn_perm(t23, t01, 0x05040100u);
    mid[d] = (int)__builtin_amdgcn_perm(t23, t01, 0x07060302u);
    any |= L0 | L1 | L2 | L3;
  }
}

// 16 FP8 codes -> all three limb planes (general path).
__device__ __forceinline__ void limbs3(const uint8_t* lut_bytes, uint32_t lane4, v4u codes, v4i& lo,
                                      v4i& mid, v4i& top) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = codes[d];
    const uint32_t L0 = lut_read(lut_bytes, lane4, x, 0), L1 = lut_read(lut_bytes, lane4, x, 1);
    const uint32_t L2 = lut_read(lut_bytes, lane4, x, 2), L3 = lut_read(lut_bytes, lane4, x, 3);
    const uint32_t t01 = __builtin_amdgcn_perm(L1, L0, 0x05010400u);
    const uint32_t t23 = __builtin_amdgcn_perm(L3, L2, 0x05010400u);
    lo[d] = (int)__builtin_amdgcn_perm(t23, t01, 0x05040100u);
    mid[d] = (int)__builtin_amdgcn_perm(t23, t01, 0x07060302u);
    const uint32_t u01 = __builtin_amdgcn_perm(L1, L0, 0x0C0C0602u);
    const uint32_t u23 = __builtin_amdgcn_perm(L3, L2, 0x0C0C0602u);
    top[d] = (int)__builtin_amdgcn_perm(u23, u01, 0x05040100u);
  }
}

__device__ __forceinline__ v4i mfma8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t abs8_sum(v4i v, uint32_t w) {
  uint32_t acc = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int b = (int)(int8_t)(((uint32_t)v[d] >> (8 * k)) & 0xFFu);
      acc += (uint32_t)(b < 0 ? -b : b) * w;
    }
  return acc;
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
  const int32_t* pool;    // pool mode
  const int32_t* pool_n;  // pool mode
  int pool_blocks;
  float* out_s;           // full: [B][T][max_n]; pool: [B][T][pool_blocks*8]
  float* out_bm;          // full: [B][T][ceil(max_n/8)]
  int rows;               // full: B; pool: B*T
  int chunks_per_row;     // full: ceil(max_n/64); pool: ceil(pool_blocks/8)
  int chunks_per_wg;
};

// Keys of one chunk for one wave: lane (g, col) holds entry 16*st + col of
// the chunk, channels [16g, 16g+16) and [64+16g, 64+16g+16).
struct ChunkKeys {
  v4u k[kSub][2];
};

// Row context of a wave: sequence b, token t, visible entries n, pool row.
struct RowCtx {
  int row = -1;
  int b = 0, t = 0, n = 0, n_pos = 0;
  const int32_t* pool_row = nullptr;
};

template <bool POOL>
__device__ __forceinline__ void row_ctx(const ScoreArgs& a, int row, int t_full, RowCtx& r) {
  r.row = row;
  if (POOL) {
    r.b = row / a.T;
    r.t = row % a.T;
  } else {
    r.b = row;
    r.t = t_full;
  }
  int n = a.n_entries[r.b];
  n = min(n, a.max_n);
  n = max(0, min(n, a.max_pages * kPage));
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

template <bool POOL>
__device__ __forceinline__ void load_chunk(const ScoreArgs& a, const RowCtx& r, int chunk, int g,
                                           int col, ChunkKeys& ck) {
  if (!POOL) {
    // a Full-mode chunk lies inside one 64-entry page: one scalar page lookup
    const int j0 = chunk * kChunk;
    const int64_t pg = j0 < r.n ? phys_page(a.page_table, a.max_pages, a.n_pages, r.b, j0 / kPage) : -1;
    // one buffer descriptor for the page (scalar registers) and a single
    // 32-bit lane offset; the sub-tile and half offsets go in the scalar
    // offset operand
    const v4u z = {0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < kSub; ++st) ck.k[st][0] = ck.k[st][1] = z;
    if (pg >= 0) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(a.kidx + pg * (kPage * kDI) + (j0 % kPage) * kDI), 0, kChunk * kDI, kBufferFlags);
      const uint32_t lofs = (uint32_t)(col * kDI + 16 * g);
      const int nv = r.n - j0;  // visible entries from the chunk start
#pragma unroll
      for (int st = 0; st < kSub; ++st) {
        if (st * 16 + col < nv) {
          ck.k[st][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, lofs, st * 16 * kDI, 0);
          ck.k[st][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lofs, st * 16 * kDI + 64, 0);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int st = 0; st < kSub; ++st) {
    const int j = entry_of<POOL>(a, r, chunk * kChunk + st * 16 + col);
    v4u k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0};
    if (j >= 0) {
      const int64_t pg = phys_page(a.page_table, a.max_pages, a.n_pages, r.b, j >> 6);
      const v4u* src = reinterpret_cast<const v4u*>(a.kidx + pg * (kPage * kDI) + (j & 63) * kDI + 16 * g);
      k0 = __builtin_nontemporal_load(src);
      k1 = __builtin_nontemporal_load(src + 4);
    }
    ck.k[st][0] = k0;
    ck.k[st][1] = k1;
  }
}

// Writes the chunk's scores (NaN, i.e. key 0, for positions that are not
// visible) and, in Full mode, the maxima of its blocks of 8.
template <bool POOL>
__device__ __forceinline__ void emit_chunk(const ScoreArgs& a, const RowCtx& rc, int chunk, float s) {
  const int lane = lane_id();
  const int p = chunk * kChunk + lane;
  bool valid;
  if (POOL) {
    valid = lane < kChunk && entry_of<POOL>(a, rc, p) >= 0;
  } else {
    const bool page_ok = chunk * kChunk < rc.n &&
                         phys_page(a.page_table, a.max_pages, a.n_pages, rc.b, chunk * kChunk / kPage) >= 0;
    valid = lane < kChunk && page_ok && p < rc.n;
  }
  float* out_s_row = a.out_s + ((int64_t)rc.b * a.T + rc.t) *
                                   (POOL ? (int64_t)a.pool_blocks * kBlock : (int64_t)s_stride(a.max_n));
  if (lane < kChunk && p < rc.n_pos) out_s_row[p] = valid ? s : u2f(0xFFFFFFFFu);
  if (!POOL) {
    float m = valid ? s : -__builtin_inff();
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    if (lane < kChunk && (lane & 7) == 0 && p < rc.n_pos) {
      a.out_bm[((int64_t)rc.b * a.T + rc.t) * bm_stride(a.max_n) + (p >> 3)] =
          (m == -__builtin_inff()) ? u2f(0xFFFFFFFFu) : m;
    }
  }
}

// General exact path for one chunk (some |value| >= 32, or a query whose
// limb sums could leave int32): three limb planes on both sides, five
// partial sums per dot combined exactly in binary64 and rounded once.
// Reads the chunk's codes again; returns this lane's entry score before
// validity masking.
template <bool POOL>
__device__ __forceinline__ float general_chunk(const ScoreArgs& a, const RowCtx& rc, int chunk, int64_t qrow0,
                                            const uint8_t* lut_bytes, float* my_fold, const float* my_w) {
  const int lane = lane_id();
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int g = lane >> 4, col = lane & 15;
  const int HI = a.HI;
  const int NRT = (HI + 15) >> 4;
  const int n_pass = (HI + kPassHeads - 1) / kPassHeads;
  ChunkKeys raw;
  load_chunk<POOL>(a, rc, chunk, g, col, raw);
  // an offset the optimizer cannot see through: keeps the query decode
  // below from being hoisted out of the chunk loop, where its 96 limb
  // registers would stay live across the common path
  int qoff = 16 * g;
  asm volatile("" : "+v"(qoff));
  float s = 0.0f;
  for (int hh = 0; hh < n_pass; ++hh) {
    for (int st = 0; st < kSub; ++st) {
      for (int rl = 0; rl < kPassRT; ++rl) {
        const int rt = kPassRT * hh + rl;
        if (rt >= NRT) break;
        const int h = rt * 16 + col;
        const v4i z = {0, 0, 0, 0};
        v4i acc[5] = {z, z, z, z, z};
        for (int s2 = 0; s2 < 2; ++s2) {
          v4u qc = {0, 0, 0, 0};
          if (h < HI) qc = reinterpret_cast<const v4u*>(a.q_idx + (qrow0 + h) * kDI + qoff)[4 * s2];
          v4i ql, qm, qt, kl, km, kt;
          limbs3(lut_bytes, lane4, qc, ql, qm, qt);
          limbs3(lut_bytes, lane4, raw.k[st][s2], kl, km, kt);
          acc[0] = mfma8(ql, kl, acc[0]);
          acc[1] = mfma8(ql, km, acc[1]);
          acc[1] = mfma8(qm, kl, acc[1]);
          acc[2] = mfma8(ql, kt, acc[2]);
          acc[2] = mfma8(qm, km, acc[2]);
          acc[2] = mfma8(qt, kl, acc[2]);
          acc[3] = mfma8(qm, kt, acc[3]);
          acc[3] = mfma8(qt, km, acc[3]);
          acc[4] = mfma8(qt, kt, acc[4]);
        }
        const v4f wv = *reinterpret_cast<const v4f*>(&my_w[rt * 16 + 4 * g]);
        v4f pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // every term and the sum are integers below 2^53: exact, one rounding
          const double D = (double)acc[0][i] + (double)acc[1][i] * 128.0 + (double)acc[2][i] * 16384.0 +
                           (double)acc[3][i] * 2097152.0 + (double)acc[4][i] * 268435456.0;
          const float f = (float)D;
          pv[i] = wv[i] * (f > 0.0f ? f : 0.0f);
        }
        *reinterpret_cast<v4f*>(&my_fold[(st * 16 + col) * kFoldStride + rl * 16 + 4 * g]) = pv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (lane < kChunk) {
      const float* frow = &my_fold[lane * kFoldStride];
      const int nh = min(kPassHeads, HI - kPassHeads * hh);
      for (int h = 0; h < nh; h += 4) {
        const v4f v = *reinterpret_cast<const v4f*>(frow + h);
        s = s + v[0];
        s = s + v[1];
        s = s + v[2];
        s = s + v[3];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
  return s;
}

// Persistent scan.  POOL = false: Full mode, rows = sequences, the 8 waves
// split T tokens x chunk slices.  POOL = true: Reindex mode, rows = (b, t),
// positions are the entries of the row's pool blocks.  Each workgroup takes a
// contiguous range of (row, 32-entry chunk) items; each wave loads its next
// chunk's keys while it scores the current one.
//
// Per chunk a wave decodes the 32 keys into limb planes once, runs the MFMAs
// of its 2 sub-tiles x 4 row tiles, writes fl(w_h * relu(d_h)) to its LDS
// fold buffer (entry-major), and lets lane e < 32 fold entry e's heads in
// ascending order.  Chunks holding a code with a top limb (or rows whose
// query could overflow int32) are only marked here and scored after the main
// loop by the general path, so the main loop keeps the common path's
// registers (no spills: a spill reload would wait for the prefetch).
template <bool POOL>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  // The lookup table sits at LDS offset 0, so a lookup address is the
  // perm result itself (code * 256 + lane * 4) with no base to add.
  struct __attribute__((aligned(16))) Lds {
    uint32_t lut[256 * 64];
    float fold[kWaves][kChunk * kFoldStride];
    float wsh[kWaves][kMaxRT * 16];  // w * 2^-18 per head
    uint32_t defer[kWaves][kMaxWaveChunks / 32];  // chunks left to the general path
  };
  __shared__ Lds sm;
  uint32_t* lut = sm.lut;

  build_lut(lut);
  for (int i = threadIdx.x; i < kWaves * kMaxWaveChunks / 32; i += blockDim.x) (&sm.defer[0][0])[i] = 0u;
  __syncthreads();
  const uint8_t* lut_bytes = reinterpret_cast<const uint8_t*>(lut);

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int g = lane >> 4;   // 16-byte K slice within a 64-deep step
  const int col = lane & 15;
  const int t_full = POOL ? 0 : wave % a.T;
  const int slice = POOL ? wave : wave / a.T;
  const int n_slices = POOL ? kWaves : kWaves / a.T;
  const int HI = a.HI;
  const int NRT = (HI + 15) >> 4;
  const int n_pass = (HI + kPassHeads - 1) / kPassHeads;

  const int total = a.rows * a.chunks_per_row;
  const int it0 = blockIdx.x * a.chunks_per_wg;
  const int it1 = min(total, it0 + a.chunks_per_wg);

  float* my_fold = sm.fold[wave];
  // this lane's fold-buffer slot for sub-tile 0, row tile 0 (the other
  // tiles sit at constant offsets from it)
  float* fold_w = my_fold + col * kFoldStride + 4 * g;
  float* my_w = sm.wsh[wave];
  uint32_t* my_defer = sm.defer[wave];
  int k_seq = 0;  // index of the current chunk among this wave's chunks

  int it = it0 + slice;
  ChunkKeys cur;
  if (it < it1) {
    RowCtx r0;
    row_ctx<POOL>(a, it / a.chunks_per_row, t_full, r0);
    load_chunk<POOL>(a, r0, it % a.chunks_per_row, g, col, cur);
  }
  while (it < it1) {
    // ---- a new row: query limbs (A operands) and head weights of token t
    RowCtx rc;
    const int row = it / a.chunks_per_row;
    row_ctx<POOL>(a, row, t_full, rc);
    const int64_t qrow0 = ((int64_t)rc.b * a.T + rc.t) * HI;
    v4i qlo[kMaxRT][2], qmid[kMaxRT][2];
    uint32_t q_any = 0, q_abs = 0;
#pragma unroll
    for (int rt = 0; rt < kMaxRT; ++rt) {
      const int h = rt * 16 + col;
      v4u c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
      if (rt < NRT && h < HI) {
        const v4u* src = reinterpret_cast<const v4u*>(a.q_idx + (qrow0 + h) * kDI + 16 * g);
        c0 = src[0];
        c1 = src[4];
      }
      limbs2(lut_bytes, lane4, c0, qlo[rt][0], qmid[rt][0], q_any);
      limbs2(lut_bytes, lane4, c1, qlo[rt][1], qmid[rt][1], q_any);
      uint32_t sabs = abs8_sum(qlo[rt][0], 1) + abs8_sum(qlo[rt][1], 1) + abs8_sum(qmid[rt][0], 128) +
                      abs8_sum(qmid[rt][1], 128);
      sabs += __shfl_xor(sabs, 16);
      sabs += __shfl_xor(sabs, 32);
      q_abs = max(q_abs, sabs);
    }
    for (int o = 1; o < 64; o <<= 1) q_abs = max(q_abs, (uint32_t)__shfl_xor((int)q_abs, o));
    // the fast path needs no top limb in q and sum_c |Mq| < 2^17, so that with
    // |Mk| < 2^14 every partial and the total stay below 2^31
    const bool fast_q = (__ballot((q_any & 0x00FF0000u) != 0) == 0) && (q_abs < (1u << 17));
    // w * 2^-18 is exact for |w| >= 2^-100 (and w = 0)
    my_w[lane] = lane < HI ? a.w[qrow0 + lane] * 0x1p-18f : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();

    const int row_end = min(it1, (row + 1) * a.chunks_per_row);
    for (; it < row_end; it += n_slices) {
      const int chunk = it % a.chunks_per_row;
      // ---- fast or general: a key code has a top limb iff |value| >= 32,
      // i.e. its exponent field is >= 12 (bits 6 and 5 of the byte both set)
      uint32_t hot = 0;
#pragma unroll
      for (int st = 0; st < kSub; ++st)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
          for (int d = 0; d < 4; ++d) hot |= cur.k[st][hs][d] & (cur.k[st][hs][d] << 1);
      const bool fast = fast_q && (__ballot((hot & 0x40404040u) != 0) == 0);
      const int itn = it + n_slices;
      // sequential head fold of one half: lane e folds entry e of this chunk
      float s = 0.0f;
      auto fold_half = [&](int hh) {
        // the fold reads what other lanes of this wave wrote
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __builtin_amdgcn_wave_barrier();
        if (lane < kChunk) {
          const float* frow = &my_fold[lane * kFoldStride];
          const int nh = min(kPassHeads, HI - kPassHeads * hh);
          for (int h = 0; h < nh; h += 4) {
            const v4f v = *reinterpret_cast<const v4f*>(frow + h);
            s = s + v[0];
            s = s + v[1];
            s = s + v[2];
            s = s + v[3];
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        __builtin_amdgcn_wave_barrier();
      };
      if (fast) {
        // ---- decode the chunk's keys into lo / mid limb planes
        v4i klo[kSub][2], kmid[kSub][2];
        uint32_t unused = 0;
#pragma unroll
        for (int st = 0; st < kSub; ++st) {
          // one sub-tile at a time: issuing all 128 lookups at once would
          // hold 128 address / result registers
          __builtin_amdgcn_sched_barrier(0);
          limbs2(lut_bytes, lane4, cur.k[st][0], klo[st][0], kmid[st][0], unused);
          limbs2(lut_bytes, lane4, cur.k[st][1], klo[st][1], kmid[st][1], unused);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the next chunk of this wave (possibly in the next row) streams into
        // the now free key registers while this one is scored
        if (itn < it1) {
          RowCtx rn;
          row_ctx<POOL>(a, itn / a.chunks_per_row, t_full, rn);
          load_chunk<POOL>(a, rn, itn % a.chunks_per_row, g, col, cur);
        }
#pragma unroll
        for (int hh = 0; hh < kMaxRT / kPassRT; ++hh) {
          if (hh >= n_pass) break;
#pragma unroll
          for (int st = 0; st < kSub; ++st) {
#pragma unroll
            for (int rl = 0; rl < kPassRT; ++rl) {
              const int rt = kPassRT * hh + rl;
              if (rt >= NRT) break;
              // keep the tiles in sequence: interleaving them needs more
              // registers than two waves per SIMD have
              __builtin_amdgcn_sched_barrier(0);
              const v4i z = {0, 0, 0, 0};
              v4i a0 = mfma8(qlo[rt][0], klo[st][0], z);
              a0 = mfma8(qlo[rt][1], klo[st][1], a0);
              v4i a1 = mfma8(qlo[rt][0], kmid[st][0], z);
              a1 = mfma8(qmid[rt][0], klo[st][0], a1);
              a1 = mfma8(qlo[rt][1], kmid[st][1], a1);
              a1 = mfma8(qmid[rt][1], klo[st][1], a1);
              v4i a2 = mfma8(qmid[rt][0], kmid[st][0], z);
              a2 = mfma8(qmid[rt][1], kmid[st][1], a2);
              const v4f wv = *reinterpret_cast<const v4f*>(&my_w[rt * 16 + 4 * g]);
              v4f pv;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                // every weighted term is bounded by sum |Mq||Mk| < 2^31: exact in int32
                const uint32_t t = (uint32_t)a1[i] + ((uint32_t)a2[i] << 7);
                const int32_t D = (int32_t)((uint32_t)a0[i] + (t << 7));
                const float r = (float)max(D, 0);
                pv[i] = wv[i] * r;
              }
              *reinterpret_cast<v4f*>(fold_w + (st * 16 * kFoldStride + rl * 16)) = pv;
            }
          }
          fold_half(hh);
        }
      } else {
        // rare: scored after the main loop, out of this loop's registers
        my_defer[k_seq >> 5] |= 1u << (k_seq & 31);
        if (itn < it1) {
          RowCtx rn;
          row_ctx<POOL>(a, itn / a.chunks_per_row, t_full, rn);
          load_chunk<POOL>(a, rn, itn % a.chunks_per_row, g, col, cur);
        }
      }

      if (fast) emit_chunk<POOL>(a, rc, chunk, s);
      ++k_seq;
    }
  }

  // ---- deferred chunks: general exact path
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int k = 0; k < k_seq; ++k) {
    if (!((my_defer[k >> 5] >> (k & 31)) & 1u)) continue;
    const int itk = it0 + slice + k * n_slices;
    RowCtx rk;
    row_ctx<POOL>(a, itk / a.chunks_per_row, t_full, rk);
    const int64_t qrow_k = ((int64_t)rk.b * a.T + rk.t) * HI;
    my_w[lane] = lane < HI ? a.w[qrow_k + lane] * 0x1p-18f : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const int chunk = itk % a.chunks_per_row;
    const float s = general_chunk<POOL>(a, rk, chunk, qrow_k, lut_bytes, my_fold, my_w);
    emit_chunk<POOL>(a, rk, chunk, s);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------- selection
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;     // 2,048: 32 per lane of one wave
constexpr int kHistCopies = 4;

constexpr int kCandCap = 4096;            // candidates kept for the single-wave exact stage

struct SelShared {
  uint32_t hist[kHistCopies][kBins];
  uint32_t cand_key[kCandCap];
  int cand_pos[kCandCap];
  int wave_tot[kSelWaves];
  uint32_t wave_min[kSelWaves], wave_max[kSelWaves];
  int misc[8];
  int pool_blk[CSA2_MAX_POOL_BLOCKS];
};

// Exclusive prefix sum over the workgroup in thread order; returns the
// thread's offset and writes the total to *total.
__device__ int block_excl_scan(int v, SelShared& sh, int* total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  // lanes 0..15 hold the wave totals: one read, then an in-register scan
  int wt = lane < kSelWaves ? sh.wave_tot[lane] : 0;
#pragma unroll
  for (int o = 1; o < kSelWaves; o <<= 1) {
    const int y = __shfl_up(wt, o);
    if (lane >= o) wt += y;
  }
  const int before = wave > 0 ? __shfl(wt, wave - 1) : 0;
  *total = __shfl(wt, kSelWaves - 1);
  __syncthreads();
  return before + x - v;
}

// Zero the 4-copy histogram (all threads), no barrier.
__device__ __forceinline__ void hist_zero(SelShared& sh) {
  for (int i = threadIdx.x; i < kHistCopies * kBins / 4; i += kSelThreads)
    reinterpret_cast<v4u*>(&sh.hist[0][0])[i] = v4u{0u, 0u, 0u, 0u};
}

// One wave: merge the 4 copies of the 32 bins lane l owns (bins
// [2048 - 32(l+1), 2048 - 32l), lane 0 has the highest digits) into copy 0
// and return their total.
__device__ __forceinline__ uint32_t wave_merge_bins(SelShared& sh, int lane) {
  uint32_t sum = 0;
  v4u* h0 = reinterpret_cast<v4u*>(&sh.hist[0][kBins - 32 * (lane + 1)]);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    v4u v = h0[q];
#pragma unroll
    for (int cp = 1; cp < kHistCopies; ++cp)
      v += reinterpret_cast<const v4u*>(&sh.hist[cp][kBins - 32 * (lane + 1)])[q];
    h0[q] = v;
    sum += v[0] + v[1] + v[2] + v[3];
  }
  return sum;
}

// Top-K selection among keys held KPT per thread (thread i owns list
// positions [i*KPT, i*KPT + KPT)), order (key desc, position asc); key 0
// marks an empty slot.  Calls emit(rank, pos) for every selected position,
// in ascending position order, and returns the number selected.
//
// 1. Block min/max and valid count; digits are the 11 bits below the
//    leading bits all keys share.
// 2. A histogram of every 8th key brackets the digit range [d_lo, d_hi]
//    that holds the K-th largest key.
// 3. One pass counts the keys above the bracket and compacts the keys inside
//    it (in position order) into LDS.  If the bracket does not hold the K-th
//    key, or holds too many keys, a block-wide radix select runs instead.
// 4. One wave finds the exact threshold among the candidates.
// 5. Every key above the threshold is taken, and the first keys (in
//    position order) equal to it up to K.
template <int KPT, typename Emit>
__device__ int block_topk(const uint32_t (&key)[KPT], int K, SelShared& sh, Emit emit) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int valid = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const uint32_t k = key[r];
    valid += k != 0;
    if (k != 0) {
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    sh.wave_min[wave] = kmin;
    sh.wave_max[wave] = kmax;
  }
  int n_valid;
  (void)block_excl_scan(valid, sh, &n_valid);  // its barriers also publish wave_min/max
  {
    uint32_t m0 = lane < kSelWaves ? sh.wave_min[lane] : 0xFFFFFFFFu;
    uint32_t m1 = lane < kSelWaves ? sh.wave_max[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      m0 = min(m0, (uint32_t)__shfl_xor((int)m0, o));
      m1 = max(m1, (uint32_t)__shfl_xor((int)m1, o));
    }
    kmin = (uint32_t)__shfl((int)m0, 0);
    kmax = (uint32_t)__shfl((int)m1, 0);
  }
  uint32_t tau = 1;             // select all valid keys (every real key is >= 1)
  int need_eq = 0x7FFFFFFF;
  if (n_valid > K) {
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0) {
      tau = kmin;
      need_eq = K;
    } else {
      const int top = 31 - __builtin_clz(diff);  // highest bit where keys differ
      const int shift1 = max(top + 1 - kDigitBits, 0);
      // ---- 2. sample histogram
      constexpr int kStride = KPT >= 16 ? 8 : 4;
      hist_zero(sh);
      __syncthreads();
#pragma unroll
      for (int r = 0; r < KPT; r += kStride) {
        const uint32_t k = key[r];
        if (k != 0) atomicAdd(&sh.hist[lane & 3][(k >> shift1) & (kBins - 1)], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        const uint32_t sum = wave_merge_bins(sh, lane);
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const float n_s = (float)__shfl((int)incl, 63);
        const float ts = (float)K * n_s / (float)n_valid;          // expected sample rank
        const float m = 3.0f * sqrtf(ts) + 8.0f;                   // margin, in samples
        const float hi_cut = ts - m, lo_cut = ts + m;
        // C(d) = samples with digit >= d; walk bins from high to low digits
        uint32_t above = incl - sum;
        int d_hi = -1, d_lo = -1;
        const v4u* h0 = reinterpret_cast<const v4u*>(&sh.hist[0][kBins - 32 * (lane + 1)]);
        for (int q = 7; q >= 0; --q) {
          const v4u v = h0[q];
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const int bin = kBins - 32 * (lane + 1) + 4 * q + e;
            const float c_prev = (float)above;   // samples with digit > bin
            above += v[e];
            const float c_here = (float)above;   // samples with digit >= bin
            if (c_here >= hi_cut && c_prev < hi_cut) d_hi = bin;
            if (c_here >= lo_cut && c_prev < lo_cut) d_lo = bin;
          }
        }
        // the crossing bins are unique across lanes; unset means "not reached"
        int dh = d_hi, dl = d_lo;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          dh = max(dh, __shfl_xor(dh, o));
          dl = max(dl, __shfl_xor(dl, o));
        }
        if (lane == 0) {
          sh.misc[0] = dh < 0 ? kBins - 1 : dh;  // hi_cut <= 0: everything above the top bin
          sh.misc[1] = dl < 0 ? 0 : dl;          // lo_cut beyond all samples: down to digit 0
        }
      }
      __syncthreads();
      const uint32_t d_hi = (uint32_t)sh.misc[0];
      const uint32_t d_lo = min((uint32_t)sh.misc[1], d_hi);
      // ---- 3. exact counts around the bracket
      int n_above = 0, n_cand = 0;
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const uint32_t k = key[r];
        const uint32_t d = (k >> shift1) & (kBins - 1);
        n_above += k != 0 && d > d_hi;
        n_cand += k != 0 && d <= d_hi && d >= d_lo;
      }
      int tot;
      const int packed_off = block_excl_scan(n_above | (n_cand << 16), sh, &tot);
      // both counts are at most 32,768, so the 16-bit halves never carry;
      // the high half can reach bit 31, hence the unsigned decode
      const int A = tot & 0xFFFF, C = (int)((uint32_t)tot >> 16);
      const bool fast = A < K && K <= A + C && C <= kCandCap;
      if (fast) {
        int o = (int)((uint32_t)packed_off >> 16);
        const int base = threadIdx.x * KPT;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
          const uint32_t k = key[r];
          const uint32_t d = (k >> shift1) & (kBins - 1);
          if (k != 0 && d <= d_hi && d >= d_lo) {
            sh.cand_key[o] = k;
            sh.cand_pos[o] = base + r;
            ++o;
          }
        }
        __syncthreads();
        // ---- 4. one wave: rank R = K - A among the C candidates
        if (threadIdx.x < 64) {
          uint32_t prefix = 0, msk = 0;
          int rem = K - A;
          for (int sh8 = 24; sh8 >= 0; sh8 -= 8) {
            // 256-bin histogram in copy 0, built by this wave only
            for (int i = lane; i < 256; i += 64) sh.hist[0][i] = 0;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            __builtin_amdgcn_wave_barrier();
            for (int i = lane; i < C; i += 64) {
              const uint32_t k = sh.cand_key[i];
              if ((k & msk) == prefix) atomicAdd(&sh.hist[0][(k >> sh8) & 255u], 1u);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            __builtin_amdgcn_wave_barrier();
            // lane l owns bins 255-4l .. 252-4l
            uint32_t cc[4], sum = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              cc[e] = sh.hist[0][255 - 4 * lane - e];
              sum += cc[e];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int o2 = 1; o2 < 64; o2 <<= 1) {
              const uint32_t y = __shfl_up(incl, o2);
              if (lane >= o2) incl += y;
            }
            uint32_t above = incl - sum;
            int dsel = -1, asel = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if ((uint32_t)rem > above && (uint32_t)rem <= above + cc[e]) {
                dsel = 255 - 4 * lane - e;
                asel = (int)above;
              }
              above += cc[e];
            }
            int dd = dsel, aa = asel;
#pragma unroll
            for (int o2 = 1; o2 < 64; o2 <<= 1) {
              const int od = __shfl_xor(dd, o2), oa = __shfl_xor(aa, o2);
              if (od > dd) {
                dd = od;
                aa = oa;
              }
            }
            prefix |= (uint32_t)dd << sh8;
            msk |= 255u << sh8;
            rem -= aa;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            __builtin_amdgcn_wave_barrier();
          }
          if (lane == 0) {
            sh.misc[2] = (int)prefix;
            sh.misc[3] = rem;
          }
        }
        __syncthreads();
        tau = (uint32_t)sh.misc[2];
        need_eq = sh.misc[3];
      } else {
        // ---- fallback: block-wide radix select over all keys
        uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
        uint32_t prefix = kmin & mask;
        int rem = K;
        int shift = top + 1;
        while (shift > 0) {
          const int width = min(kDigitBits, shift);
          shift -= width;
          const uint32_t dmask = (1u << width) - 1u;
          hist_zero(sh);
          __syncthreads();
#pragma unroll
          for (int r = 0; r < KPT; ++r) {
            const uint32_t k = key[r];
            if (k != 0 && (k & mask) == prefix) atomicAdd(&sh.hist[lane & 3][(k >> shift) & dmask], 1u);
          }
          __syncthreads();
          if (threadIdx.x < 64) {
            const uint32_t sum = wave_merge_bins(sh, lane);
            uint32_t incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const uint32_t y = __shfl_up(incl, o);
              if (lane >= o) incl += y;
            }
            uint32_t above = incl - sum;
            if (above < (uint32_t)rem && (uint32_t)rem <= incl) {
              const v4u* h0 = reinterpret_cast<const v4u*>(&sh.hist[0][kBins - 32 * (lane + 1)]);
              for (int q = 7; q >= 0; --q) {
                const v4u v = h0[q];
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                  if ((uint32_t)rem > above && (uint32_t)rem <= above + v[e]) {
                    sh.misc[0] = kBins - 32 * (lane + 1) + 4 * q + e;
                    sh.misc[1] = (int)above;
                  }
                  above += v[e];
                }
              }
            }
          }
          __syncthreads();
          const uint32_t d = (uint32_t)sh.misc[0];
          rem -= sh.misc[1];
          prefix |= d << shift;
          mask |= dmask << shift;
          __syncthreads();
        }
        tau = prefix;
        need_eq = rem;
      }
    }
  }
  // ---- 5. emit in position order: keys above tau, then the first need_eq equal to it
  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    gt += key[r] != 0 && key[r] > tau;
    eq += key[r] != 0 && key[r] == tau;
  }
  int tot2;
  const int off2 = block_excl_scan(gt | (eq << 16), sh, &tot2);
  const int gt_before = off2 & 0xFFFF, eq_before = (int)((uint32_t)off2 >> 16);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  int off = gt_before + min(eq_before, need_eq);
  const int sel_tot = (tot2 & 0xFFFF) + min((int)((uint32_t)tot2 >> 16), need_eq);
  int taken_eq = 0;
  const int base = threadIdx.x * KPT;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const uint32_t k = key[r];
    bool sel = false;
    if (k != 0 && k > tau) sel = true;
    else if (k != 0 && k == tau && taken_eq < take_eq) {
      sel = true;
      ++taken_eq;
    }
    if (sel) emit(off++, base + r);
  }
  return sel_tot;
}

struct SelectArgs {
  const float* s;        // full: [B][T][max_n]; reindex: [B][T][pool_blocks*8] (pool order)
  const float* bm;       // full: [B][T][ceil(max_n/8)]
  const int32_t* n_entries;
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
};

// One workgroup per (b, t).  FULL: select the pool from block maxima, then
// the top-k inside the pool (the top-k lies inside the pool whenever
// topk <= pool_blocks).  REINDEX: top-k over the pool-order scores.
template <bool FULL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int row = blockIdx.x;  // b * T + t
  const int b = row / a.T;
  int n = min(a.n_entries[b], min(a.max_n, a.max_pages * kPage));
  n = max(n, 0);
  const int P = a.pool_blocks;
  int pool_n;
  if (FULL) {
    const int nb = (n + kBlock - 1) / kBlock;
    const float* bm = a.bm + (int64_t)row * bm_stride(a.max_n);
    constexpr int KPT = 32;  // 32,768 blocks = 262,144 entries
    uint32_t key[KPT];
#pragma unroll
    for (int r4 = 0; r4 < KPT; r4 += 4) {
      const int blk = threadIdx.x * KPT + r4;
      v4f v = {0.f, 0.f, 0.f, 0.f};
      if (blk + 3 < nb) v = *reinterpret_cast<const v4f*>(bm + blk);
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = blk + e < nb ? bm[blk + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) key[r4 + e] = blk + e < nb ? score_key(v[e]) : 0u;
    }
    for (int i = threadIdx.x; i < P; i += kSelThreads) sh.pool_blk[i] = -1;
    __syncthreads();
    pool_n = block_topk<KPT>(key, P, sh, [&](int rank, int pos) { sh.pool_blk[rank] = pos; });
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += kSelThreads)
      a.out_pool[(int64_t)row * P + i] = sh.pool_blk[i];
    if (threadIdx.x == 0) a.out_pool_n[row] = pool_n;
  } else {
    pool_n = max(0, min(a.pool_n_in[row], P));
    for (int i = threadIdx.x; i < P; i += kSelThreads)
      sh.pool_blk[i] = i < pool_n ? a.pool_in[(int64_t)row * P + i] : -1;
    __syncthreads();
  }
  // ---- top-k over the pool's positions (list position p = 8 * slot + i)
  constexpr int KPT2 = 16;  // 2 pool slots per thread, 16,384 positions
  uint32_t key2[KPT2];
  const float* srow = FULL ? a.s + (int64_t)row * s_stride(a.max_n) : a.s + (int64_t)row * P * kBlock;
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const int slot = threadIdx.x * 2 + hs;
    const int blk = slot < pool_n ? sh.pool_blk[slot] : -1;
    const bool ok = blk >= 0 && blk < (n + kBlock - 1) / kBlock;
    // the 8 scores of this slot: block blk's entries (Full) or the slot's
    // pool-order scores (Reindex); both 32-byte aligned
    v4f v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      const v4f* src = reinterpret_cast<const v4f*>(srow + (FULL ? blk * kBlock : slot * kBlock));
      v0 = src[0];
      v1 = src[1];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = ok && blk * kBlock + e < n;
      key2[hs * 8 + e] = in ? score_key(e < 4 ? v0[e] : v1[e - 4]) : 0u;
    }
  }
  int32_t* out = a.out_topk + (int64_t)row * a.topk;
  const int got = block_topk<KPT2>(key2, a.topk, sh, [&](int rank, int p) {
    out[rank] = sh.pool_blk[p >> 3] * kBlock + (p & 7);
  });
  for (int i = got + threadIdx.x; i < a.topk; i += kSelThreads) out[i] = -1;
}

}  // namespace csa2

// ---------------------------------------------------------------- C ABI
namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// One resident workgroup per compute unit (the scan uses ~132 KB of LDS);
// each takes a contiguous range of 32-entry chunks.  With T tokens sharing a
// workgroup, every wave covers chunks_per_wg * T / 8 chunks.
int persistent_grid(int total_chunks, int T, int* chunks_per_wg) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      n_cu = 256;
  }
  const int slices = csa2::kWaves / T;
  int per = (total_chunks + n_cu - 1) / n_cu;
  per = ((per + slices - 1) / slices) * slices;  // whole rounds of the waves
  // each wave tracks at most kMaxWaveChunks chunks; beyond that, more workgroups
  per = std::min(per, csa2::kMaxWaveChunks * slices);
  *chunks_per_wg = per;
  return (total_chunks + per - 1) / per;
}

int check_index_common(const void* q_idx, const void* w, const void* kidx, int64_t n_pages,
                       const void* page_table, int32_t max_pages, const void* n_entries,
                       int32_t B, int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks) {
  if (!q_idx || !w || !kidx || !page_table || !n_entries) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || HI <= 0 || n_pages <= 0 || max_pages <= 0) return CSA2_ERR_INVALID_ARG;
  if (topk <= 0 || topk > CSA2_MAX_TOPK || pool_blocks <= 0 || pool_blocks > CSA2_MAX_POOL_BLOCKS)
    return CSA2_ERR_INVALID_ARG;
  if (HI > CSA2_MAX_INDEX_HEADS || (HI % 4) != 0) return CSA2_ERR_UNSUPPORTED;
  if (!(T == 1 || T == 2 || T == 4)) return CSA2_ERR_UNSUPPORTED;
  if (topk > pool_blocks) return CSA2_ERR_UNSUPPORTED;
  if (B > 65535 / T) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}
}  // namespace

extern "C" size_t csa2_index_ws_bytes(int op, int32_t B, int32_t T, int32_t max_n,
                                      int32_t pool_blocks) {
  if (op == CSA2_OP_INDEX_FULL) {
    const size_t nb = (size_t)csa2::bm_stride(max_n);
    return align256((size_t)B * T * csa2::s_stride(max_n) * 4) + align256((size_t)B * T * nb * 4);
  }
  return align256((size_t)B * T * pool_blocks * 8 * 4);
}

extern "C" int csa2_index_full(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                               int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                               const int32_t* n_entries, int32_t max_n_entries, int32_t B,
                               int32_t T, int32_t HI, int32_t topk, int32_t pool_blocks,
                               int32_t* out_topk, int32_t* out_pool, int32_t* out_pool_n, void* ws,
                               size_t ws_bytes, csa2_stream_t stream) {
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
  sa.out_s = reinterpret_cast<float*>(ws);
  sa.out_bm = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                       align256((size_t)B * T * csa2::s_stride(max_n_entries) * 4));
  sa.rows = B;
  sa.chunks_per_row = (max_n_entries + csa2::kChunk - 1) / csa2::kChunk;
  const int gx = persistent_grid(sa.rows * sa.chunks_per_row, T, &sa.chunks_per_wg);
  CSA2_LAUNCH(CSA2_K_SCORE_FULL, csa2::score_kernel<false>, dim3(gx), dim3(csa2::kScoreThreads),
              (hipStream_t)stream, sa);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  csa2::SelectArgs se{};
  se.s = sa.out_s;
  se.bm = sa.out_bm;
  se.n_entries = n_entries;
  se.max_n = max_n_entries;
  se.max_pages = max_pages;
  se.T = T;
  se.topk = topk;
  se.pool_blocks = pool_blocks;
  se.out_topk = out_topk;
  se.out_pool = out_pool;
  se.out_pool_n = out_pool_n;
  CSA2_LAUNCH(CSA2_K_SELECT_FULL, csa2::select_kernel<true>, dim3(B * T), dim3(csa2::kSelThreads),
              (hipStream_t)stream, se);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}

extern "C" int csa2_index_reindex(const uint8_t* q_idx, const float* w, const uint8_t* kidx_pool,
                                  int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                  const int32_t* n_entries, int32_t B, int32_t T, int32_t HI,
                                  const int32_t* pool, const int32_t* pool_n, int32_t pool_blocks,
                                  int32_t topk, int32_t* out_topk, void* ws, size_t ws_bytes,
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
  sa.pool = pool;
  sa.pool_n = pool_n;
  sa.pool_blocks = pool_blocks;
  sa.out_s = reinterpret_cast<float*>(ws);
  sa.rows = B * T;
  sa.chunks_per_row = (pool_blocks * csa2::kBlock + csa2::kChunk - 1) / csa2::kChunk;
  const int gx = persistent_grid(sa.rows * sa.chunks_per_row, 1, &sa.chunks_per_wg);
  CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, csa2::score_kernel<true>, dim3(gx), dim3(csa2::kScoreThreads),
              (hipStream_t)stream, sa);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  csa2::SelectArgs se{};
  se.s = sa.out_s;
  se.n_entries = n_entries;
  se.max_n = max_n;
  se.max_pages = max_pages;
  se.T = T;
  se.topk = topk;
  se.pool_blocks = pool_blocks;
  se.pool_in = pool;
  se.pool_n_in = pool_n;
  se.out_topk = out_topk;
  CSA2_LAUNCH(CSA2_K_SELECT_REINDEX, csa2::select_kernel<false>, dim3(B * T),
              dim3(csa2::kSelThreads), (hipStream_t)stream, se);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
