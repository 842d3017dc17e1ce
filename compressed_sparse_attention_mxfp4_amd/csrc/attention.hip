// Sparse attention over the selected FP4 main-KV entries merged with the
// FP8 sliding window ("Inside DeepSeek V4.1 Flash", section "CSA2: reuse
// memory and reuse selection independently": the main query attends to the
// selected global entries together with the local window; knowledge note
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
// "FP4 main KV": entries are dequantized before attention, the window stays
// FP8).  Each 512-channel row is both key and value; one softmax runs over
// the union of the rows.
//
// Two kernels share the row handling.  Each splits the row list [top-k
// slots | 128 window rows] of a (b, t) so that the grid has about one
// workgroup per compute unit (the splits' partial results merged by a
// combine kernel; with one split the output is written directly), resolves a
// split's rows once (index -> page -> cache slot) into LDS, and keeps the row
// loads of the next 32-row sub-chunks in flight while one is processed.  The
// head-tile kernel takes as many splits as fit one round of workgroups and
// shares the 32-row sub-chunks out evenly (a second, partly filled round
// would leave its workgroups sharing compute units, and the slowest of them
// sets the kernel's time).
//  - 64 heads, B*T >= 8 (attn_heads_kernel, below): one workgroup per (b, t, split)
//    serves every head, so each row is gathered and dequantized once into a
//    shared LDS tile of fp16 rows.
//  - otherwise (attn_split_kernel): one workgroup per (b, t, 16-head
//    tile, split); its 4 waves own 128 channels each.  Per sub-chunk a wave
//    converts its channel slice to fp16 (hardware FP4 / E4M3 conversion,
//    exact) straight into the Q.K operand and into a swizzled row-major LDS
//    tile; the four partial logits are summed in fixed order through LDS,
//    every wave runs the same online softmax and accumulates P.V for its
//    channels, reading V transposed from the tile.
#include "common.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kSub = 32;               // rows per sub-chunk
constexpr int kRowHalves = 128;        // a wave's 128-channel slice of one row (256 B, 16 chunks of 16 B)
constexpr int kMaxRows = CSA2_MAX_TOPK + CSA2_SWA;  // rows of one (b, t): 2,176
// Workgroups the split count aims at (about one per compute unit).
constexpr int kTargetWorkgroups = 256;

// LDS tile of 32 rows x 128 fp16 channels, row-major, with 16-byte chunk k of
// row r stored at chunk k ^ bitrev4(r & 15).  This one layout serves three
// access patterns without bank conflicts: the dequant stores (16 B), the
// Q.K operand loads (16 B, one row per lane) and the transposing P.V operand
// loads (8 B, 4 rows x 4 channels per 16 lanes).
__device__ __forceinline__ int swz(int row) { return (int)(__builtin_bitreverse32((uint32_t)row & 15u) >> 28); }
__device__ __forceinline__ int tile_off(int row, int chunk) {  // in halves
  return row * kRowHalves + 8 * (chunk ^ swz(row));
}

typedef _Float16 half_t;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// Reductions over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48): each
// permlane swap of a register with itself leaves the two values of a lane
// pair in the two results, in the same order on both lanes.
__device__ __forceinline__ float rows4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ v4f mfma16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

struct AttnArgs {
  const uint16_t* q;
  float sm_scale_log2;   // sm_scale * log2(e)
  const uint8_t* kv_pool;
  int64_t n_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* n_entries;
  const int32_t* topk_idx;
  int topk;
  const uint8_t* swa;
  int T;
  int H;
  int BT;
  int n_splits;
  int split_rows;  // rows per split, a multiple of 32 (the head-tile kernel: the most of any split)
  int split_base;  // head-tile kernel: split i has split_base + (i < split_extra) sub-chunks
  int split_extra;
  float* part_o;   // n_splits > 1: [B*T][H/16][n_splits][16][512]
  float* part_ml;  // n_splits > 1: [B*T][H/16][n_splits][32]  (m[16] in log2 units, l[16])
  float* out;      // n_splits == 1: [B*T][H][512]
  float* out_lse;  // n_splits == 1: [B*T][H] or null
};

// Hoisted LDS addresses: byte offsets in the workgroup's LDS, passed through
// an empty asm so that the compiler keeps them in registers instead of
// recomputing the swizzle in every sub-chunk.
typedef __attribute__((address_space(3))) half_t lds_half_t;
typedef __attribute__((address_space(3))) v8h lds_v8h_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;
__device__ __forceinline__ uint32_t lds_addr(const half_t* p) {
  uint32_t x = (uint32_t)(uintptr_t)(const lds_half_t*)p;
  asm volatile("" : "+v"(x));
  return x;
}
// Row loads through global-address-space pointers, so that they count on
// the vector-memory wait counter only (a flat load would also count on the
// LDS counter and make every LDS wait of the loop wait for the row loads).
__device__ __forceinline__ void lds_st16(uint32_t addr, v8h v) { *(lds_v8h_t*)(uintptr_t)addr = v; }
__device__ __forceinline__ v8h lds_ld16(uint32_t addr) { return *(const lds_v8h_t*)(uintptr_t)addr; }
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 4 halves that lane 4j + i / 4 points at, for j = 0..3
__device__ __forceinline__ v4h lds_ld_tr(uint32_t addr) {
  return __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(uintptr_t)addr));
}

// A row of the list: cache slot (physical page * 64 + offset) of a selected
// entry, or one of these codes.
constexpr int kRowAbsent = -1;   // empty top-k slot, or past the split's end
constexpr int kRowWindow = -2;   // a window row (its place in the list gives which)

// Kinds of row content a split can hold (decided per split, the same for
// every wave): only FP4 entries (rows < topk), only window rows, or both.
enum SubMode { kMixed = 0, kFp4Only = 1, kWindowOnly = 2 };

// The row loads of one sub-chunk for one lane (g, col): rows col and
// 16 + col, the wave's channels 128 w + 32 g .. + 31.  FP4 row: 16 code
// bytes + the 16 scale bytes 16 (w / 2) .. + 15 of the entry (the lane's two
// groups among them), or in a split of FP4 rows only just the 4 scale bytes
// holding the lane's two (hi[rt][0]); window row: 32 E4M3 bytes; absent rows
// read the pool's first bytes (discarded).
struct SubLoads {
  v4u lo[2], hi[2];
  int s[2];  // the rows' slots (or kRowAbsent / kRowWindow)
};

// The values of a batch of loads, all in flight together, are taken here
// (an empty asm that reads them): the loads cannot move into a later
// branch, and the wait for the first of them is a wait for them all.
template <int N>
__device__ __forceinline__ void resolve_fence(const int (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" ::"v"(v[k]));
}

// Cache slot of list row `row` of a (b, t) (rows past row1 are absent):
// j is its top-k index and pg the page-table word of j's page (both unused
// for a window row).
__device__ __forceinline__ int row_slot(const AttnArgs& a, int row, int row1, int n, int j, int pg) {
  if (row >= row1) return kRowAbsent;
  if (row >= a.topk) return kRowWindow;
  return (j >= 0 && j < n && pg >= 0 && pg < a.n_pages) ? (int)((int64_t)pg * kPage + (j & 63)) : kRowAbsent;
}

// The split's relative rows r0 + threadIdx.x + k * step < n_rel, one at a
// time (the kernels resolve their first rows with all loads in flight; with
// the launcher's row count per thread nothing is left here).
__device__ __forceinline__ void resolve_rest(const AttnArgs& a, const int32_t* idx_row, int b, int n, int row0,
                                          int row1, int r0, int step, int n_rel, int* rslot) {
  for (int r = r0 + (int)threadIdx.x; r < n_rel; r += step) {
    const int row = row0 + r;
    const int j = idx_row[max(0, min(row, a.topk - 1))];
    const int pg = a.page_table[(int64_t)b * a.max_pages + max(0, min(j >> 6, a.max_pages - 1))];
    rslot[r] = row_slot(a, row, row1, n, j, pg);
  }
}

typedef const __attribute__((address_space(1))) v4u gbl_v4u_t;
typedef const __attribute__((address_space(1))) uint32_t gbl_u32_t;
__device__ __forceinline__ v4u gld16(const uint8_t* p) { return *(gbl_v4u_t*)p; }
__device__ __forceinline__ uint32_t gld4(const uint8_t* p) { return *(gbl_u32_t*)p; }

// The slot of the split's relative row rel (absent from n_rel on): the LDS
// read is unconditional (index clamped), so that the reads of several rows
// can go out together.
__device__ __forceinline__ int row_at(const int* rslot, int rel, int n_rel) {
  const int v = rslot[min(rel, n_rel - 1)];
  return rel < n_rel ? v : kRowAbsent;
}

// The two 16-byte load addresses of a lane's piece of list row abs_row with
// slot s: FP4 entry -> its codes at byte c_off and its scale bytes at s_off;
// window row -> its bytes w_off and w_off + 16; absent -> the pool's first
// bytes (read and discarded).  Chosen by selects, with no branch.
struct RowPtrs {
  const uint8_t* p0;
  const uint8_t* p1;
};
__device__ __forceinline__ RowPtrs row_ptrs(const AttnArgs& a, int s, const uint8_t* win_row0, int abs_row, int c_off,
                                            int s_off, int w_off) {
  const uintptr_t pool = (uintptr_t)a.kv_pool;
  const uintptr_t page = pool + (uintptr_t)(uint32_t)(s >> 6) * kPageBytes;  // (used only for s >= 0)
  const uintptr_t f0 = page + (uint32_t)((s & 63) * kEntryCodes + c_off);
  const uintptr_t f1 = page + (uint32_t)(kPage * kEntryCodes + (s & 63) * kEntryScales + s_off);
  const uintptr_t w0 = (uintptr_t)win_row0 + (uintptr_t)(int64_t)((abs_row - a.topk) * kD + w_off);
  const bool fp4 = s >= 0, win = s == kRowWindow;
  uintptr_t q0 = win ? w0 : pool, q1 = win ? w0 + 16 : pool;
  q0 = fp4 ? f0 : q0;
  q1 = fp4 ? f1 : q1;
  return RowPtrs{(const uint8_t*)q0, (const uint8_t*)q1};
}

// The slots of a lane (g, col)'s rows col and 16 + col of the sub-chunk
// starting at relative row rel0 (read ahead of the loads they address).
struct SubSlots {
  int s[2];
};
__device__ __forceinline__ SubSlots read_sub(const int* rslot, int rel0, int n_rel, int col) {
  return SubSlots{{row_at(rslot, rel0 + col, n_rel), row_at(rslot, rel0 + 16 + col, n_rel)}};
}

// abs0: the sub-chunk's first row in the whole list (window row w = list
// row - topk).  The loads are always issued, also for sub-chunks past the
// split's end (their rows read as absent), so that every path through the
// loop has the same loads in flight and each wait counts exactly the later
// sub-chunks'.
// SC4: the split holds FP4 rows only (4-byte scale loads).
template <bool SC4>
__device__ __forceinline__ void issue_sub(const AttnArgs& a, const SubSlots& ss, int abs0, int wave, int g, int col,
                                          const uint8_t* win_row0, SubLoads& L) {
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int s = ss.s[rt];
    L.s[rt] = s;
    // the lane's groups 8 w + 2 g, + 1: scale bytes 8 (w & 1) + 2 g, + 1 of
    // the 16 at the scale offset, in the word 2 (w & 1) + g / 2
    const RowPtrs rp = row_ptrs(a, s, win_row0, abs0 + 16 * rt + col, 64 * wave + 16 * g,
                                16 * (wave >> 1) + (SC4 ? 4 * (2 * (wave & 1) + (g >> 1)) : 0), 128 * wave + 32 * g);
    // 16-byte loads at 16-byte aligned addresses inside the row they belong to
    L.lo[rt] = gld16(rp.p0);
    if (SC4) L.hi[rt] = v4u{gld4(rp.p1), 0u, 0u, 0u};
    else L.hi[rt] = gld16(rp.p1);
  }
}

// KP: rows of the list each thread resolves (KP * 256 >= the split's rows)
// MAXS > 0: every split has at most MAXS sub-chunks, and the sub-chunk loop
// is unrolled whole (no loop-carried load buffers, whose copies into the
// loop's registers would wait for the loads).  MAXS = 0: the sub-chunks go
// through a ring of NB load buffers.
// GR (with MAXS > 0): groups of 4 waves in the workgroup; group gi takes
// the split's sub-chunks gi, gi + GR, ... with its own online softmax, and
// the groups' results are merged at the end.  Two groups put two waves on
// each SIMD, so that one's waits (LDS round trips, the softmax's dependent
// steps) hide behind the other's work.  A group's j-th sub-chunk uses load
// buffer j % NB.
template <int NB, int KP, int MAXS, int GR>
__global__ __launch_bounds__(kAttnThreads * GR, GR == 1 ? 2 : 1) void attn_split_kernel(AttnArgs a) {
  static_assert(GR == 1 || MAXS > 0, "groups only with the unrolled loop");
  constexpr int kThreads = kAttnThreads * GR;
  __shared__ __attribute__((aligned(16))) half_t kr[GR][4][kSub * kRowHalves];
  __shared__ __attribute__((aligned(16))) v4f ssum[GR][2][4][2][64];  // double-buffered by sub-chunk
  __shared__ __attribute__((aligned(16))) float alph[GR][4][16];       // per wave: rescale factor per head
  __shared__ __attribute__((aligned(16))) float qmax[4][16];           // per wave: max |q| per head
  __shared__ __attribute__((aligned(16))) float gml[2][16];            // group 1's final m, l per head
  __shared__ __attribute__((aligned(16))) float gfac[4][2][16];        // group 0 wave: merge factors per head
  __shared__ __attribute__((aligned(16))) int rslot[kMaxRows + kSub];
  // STRAIGHT: each row's two load bases (FP4 entry: its codes and its scale
  // bytes; window row: its bytes and 16 bytes on; absent: the pool's first
  // bytes), so that a lane's load addresses cost one add each
  constexpr bool STRAIGHT = MAXS > 0;
  constexpr int JG = STRAIGHT ? (MAXS + GR - 1) / GR : 1;  // sub-chunks of a group, at most
  constexpr int kRB = STRAIGHT ? JG * GR * kSub : 1;
  __shared__ __attribute__((aligned(16))) uint64_t rbase[kRB][2];

  // XCD-aware order: workgroup id % 8 picks the XCD (and its L2).  The NHT
  // head tiles of one (split, b, t) unit take ids 8 apart, so they share an
  // XCD and its L2 copy of the unit's rows.
  const int NHT = a.H >> 4;
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int rest = id >> 3;
  const int ht = rest % NHT;
  const int unit = (rest / NHT) * 8 + xcd;  // split + n_splits * (b*T + t)
  if (unit >= a.n_splits * a.BT) return;
  const int split = unit % a.n_splits;
  const int bt = unit / a.n_splits;
  const int b = bt / a.T, t = bt % a.T;
  const int lane = lane_id();
  const int wave = (threadIdx.x >> 6) & 3;               // in its group
  const int grp = GR == 1 ? 0 : (int)(threadIdx.x >> 8);  // wave group
  const int g = lane >> 4, col = lane & 15;
  int n = a.n_entries[b];
  n = min(n, a.max_pages * kPage);

  const int n_rows = a.topk + kSwa;
  // the split's sub-chunks: split_base each, one more for the first
  // split_extra splits
  const int row0 = kSub * (split * a.split_base + min(split, a.split_extra));
  const int row1 = min(n_rows, row0 + kSub * (a.split_base + (split < a.split_extra ? 1 : 0)));
  const int n_sub = (row1 - row0 + kSub - 1) / kSub;
  const int32_t* idx_row = a.topk_idx + (int64_t)bt * a.topk;
  const uint8_t* win_row0 = a.swa + ((int64_t)b * (kSwa - 1 + a.T) + t) * kD;

  // the query slice's raw words go out first (used after the row resolve)
  v4u qraw[4];
  {
    const uint16_t* qrow = a.q + (((int64_t)bt * a.H) + ht * 16 + col) * kD + 128 * wave + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const v4u*>(qrow + 8 * s);
  }

  // ---- resolve the split's rows once (index, page lookup): FP4 entry slot,
  // window row, or absent (also past the split's end, up to whole sub-chunks)
  // (all index loads in flight together, then all page-table loads)
  {
    constexpr int kPer = KP;
    const int n_rel = n_sub * kSub;
    int jj[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int row = row0 + (int)threadIdx.x + k * kThreads;
      jj[k] = idx_row[max(0, min(row, a.topk - 1))];
    }
    // (unconditional, clamped; each batch of loads is taken whole before the
    // next goes out: left to itself the compiler sinks them into the
    // per-row branch below, one row's two round trips after another's)
    resolve_fence(jj);
    int pp[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int lp = max(0, min(jj[k] >> 6, a.max_pages - 1));
      pp[k] = a.page_table[(int64_t)b * a.max_pages + lp];
    }
    resolve_fence(pp);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int r = (int)threadIdx.x + k * kThreads;
      const int sl = row_slot(a, row0 + r, row1, n, jj[k], pp[k]);
      if (r < n_rel) rslot[r] = sl;
      if (STRAIGHT && r < kRB) {
        // (rows past the split's end: absent)
        const RowPtrs rp = row_ptrs(a, r < n_rel ? sl : kRowAbsent, win_row0, row0 + r, 0, 0, 0);
        *reinterpret_cast<v4u*>(&rbase[r][0]) = __builtin_bit_cast(v4u, RowPtrs{rp.p0, rp.p1});
      }
    }
    resolve_rest(a, idx_row, b, n, row0, row1, kPer * kThreads, kThreads, n_rel, rslot);
  }

  // ---- Q slice as the B operand of S^T = K.Q^T: lane (g, col) holds head
  // ht*16+col, channels 128*wave + 32*g + 8*s .. +8 as K slice s (the keys
  // use the same order of the channels, so the dot product is unchanged).
  // Each head's query is scaled by a power of two that puts its largest |q|
  // in [2^14, 2^15), so that the fp16 operand never overflows; the logits
  // take the inverse power back (exact).
  // ---- the sub-chunks' rows go through NB load buffers: the loads of NB
  // sub-chunks are in flight while the first of them is processed (the wait
  // counter retires loads in issue order, so each sub-chunk waits only for
  // its own rows)
  const int n_rel = n_sub * kSub;
  SubLoads buf[NB];
  v8h qb[4];
  float lg_scale;  // per head `col`
  {
    uint32_t mx = 0u;  // largest |q| bit pattern (bf16 in the high half)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max((qraw[s][e] << 16) & 0x7FFF0000u, qraw[s][e] & 0x7FFF0000u));
    const float m4 = rows4_max(__uint_as_float(mx));
    if (grp == 0 && lane < 16) qmax[wave][lane] = m4;
    __syncthreads();  // also publishes rslot
  }
  // the query in fp16 (after the first row loads are out)
  auto q_convert = [&]() __attribute__((always_inline)) {
    const float m = fmaxf(fmaxf(qmax[0][col], qmax[1][col]), fmaxf(qmax[2][col], qmax[3][col]));
    // exponent of the largest |q| (a normal or subnormal bf16): the scale is
    // 2^(14 - e), kept a binary32 power of two (at most 2^127)
    const int e = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 : 14;
    const int sh = min(127, 14 - e);
    const float up = __builtin_ldexpf(1.0f, sh);
    lg_scale = a.sm_scale_log2 * __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4u pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const h2_t h = {(_Float16)(u2f(qraw[s][e2] << 16) * up), (_Float16)(u2f(qraw[s][e2] & 0xFFFF0000u) * up)};
        pk[e2] = __builtin_bit_cast(uint32_t, h);
      }
      // the packed words pass through an empty asm so that the compiler
      // keeps them packed instead of re-packing the halves before every MFMA
      asm volatile("" : "+v"(pk));
      qb[s] = __builtin_bit_cast(v8h, pk);
    }
  };

  // lane (g, col) dequantizes rows col and 16 + col of each 32-row
  // sub-chunk, the wave's channels 32g .. 32g + 31 (16-byte chunks 4g ..
  // 4g + 3 of the wave's tile), straight into the A operand of S^T = K.Q^T,
  // and stores them into the tile for the transposed P.V reads
  half_t* my_kr = kr[grp][wave];
  uint32_t st_addr[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int s = 0; s < 4; ++s) st_addr[rt][s] = lds_addr(&my_kr[tile_off(16 * rt + col, 4 * g + s)]);
  // P.V operand: the V column (channel 16c + col over P's K slice, rows
  // {4g..4g+3, 16+4g..16+4g+3}) comes from the row-major tile through the
  // transposing load, so lane (g, col) points at row 4g + col / 4 (+16),
  // channels 16c + 4 (col % 4) .. +3
  uint32_t pv_addr[8];
  {
    const int tr_row = 4 * g + (col >> 2);
    const int tq = col & 3;
#pragma unroll
    for (int c = 0; c < 8; ++c) pv_addr[c] = lds_addr(&my_kr[tile_off(tr_row, 2 * c + (tq >> 1)) + 4 * (tq & 1)]);
  }
  constexpr int kRowBytes16 = 16 * kRowHalves * 2;  // 16 rows of the tile, in bytes

  float m_run = -__builtin_inff();  // running reference (log2 units) of head `col`
  float l_run = 0.0f;               // running sum of head `col`
  v4f o_acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o_acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  // One sub-chunk from its loaded bytes.
  auto process = [&](int sc, const SubLoads& L, auto mode_tag) {
    constexpr int kMode = decltype(mode_tag)::value;
    const int sub0 = sc * kSub;  // in the split's rows
    // ---- dequantize rows col, 16 + col (32 channels each) into the Q.K
    // operand.  Hardware conversions with unit scale are exact for every
    // FP4 and E4M3 code (element 0 = low nibble / low byte); the E4M3 block
    // scale is applied by one packed fp16 multiply per channel pair, exact
    // since the product has at most 6 significant bits and lies in fp16 range.
    v8h kA[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int s = L.s[rt];
      const v4u lo = L.lo[rt], hi = L.hi[rt];
      auto fp4_row = [&](bool present) {
        // absent row: zero scales, zero row (FP4 codes are all finite).  The
        // mask is opaque so that the select does not pull the loads into a
        // branch.
        uint32_t pm = present ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(pm));
        // groups 8 wave + 2 g and + 1: bytes 8 (wave & 1) + 2 g, + 1 of hi
        // (word 2 (wave & 1) + g / 2, picked by selects: g varies by lane;
        // in a split of FP4 rows only that word alone was loaded)
        const uint32_t wlo = (wave & 1) ? hi[2] : hi[0];
        const uint32_t whi = (wave & 1) ? hi[3] : hi[1];
        const uint32_t wsel = kMode == kFp4Only ? hi[0] : ((g >> 1) ? whi : wlo);
        const uint32_t sw = (wsel >> (16 * (g & 1))) & 0xFFFFu;
        const uint32_t s0 = (sw & 0xFFu) * 0x101u & pm, s1 = (sw >> 8) * 0x101u & pm;
        const h2_t sc0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, false);
        const h2_t sc1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, false);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const h2_t sc = d < 2 ? sc0 : sc1;
          const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo[d], 1.0f, 0) * sc;
          const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo[d], 1.0f, 1) * sc;
          const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo[d], 1.0f, 2) * sc;
          const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo[d], 1.0f, 3) * sc;
          kA[rt][d] = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        }
      };
      auto fp8_row = [&](bool w) {
        // window row: 32 E4M3 codes; absent row: zeros (its bytes may hold
        // NaN codes, and its V must be 0 to meet p = 0)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t c0 = w ? (d < 2 ? lo[2 * d] : hi[2 * d - 4]) : 0u;
          const uint32_t c1 = w ? (d < 2 ? lo[2 * d + 1] : hi[2 * d - 3]) : 0u;
          const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
          const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
          const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
          const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
          kA[rt][d] = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        }
      };
      if (kMode == kFp4Only) {
        fp4_row(s >= 0);
      } else if (kMode == kWindowOnly) {
        fp8_row(s == kRowWindow);
      } else {
        if (s >= 0) fp4_row(true);
        else fp8_row(s == kRowWindow);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) lds_st16(st_addr[rt][d], kA[rt][d]);
    }

    // ---- partial logits S^T (32 rows x 16 heads) over this wave's 128 channels
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      v4f sacc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 4; ++d) sacc = mfma16(kA[rt][d], qb[d], sacc);
      ssum[grp][(sc / GR) & 1][wave][rt][lane] = sacc;
    }
    // one barrier per sub-chunk: the next sub-chunk writes the other buffer,
    // and this buffer is rewritten only after the next sub-chunk's barrier;
    // it also orders this wave's tile stores before its transposed reads
    lds_barrier();
    // rows 4g..4g+3 and 16+4g..16+4g+3 present (slot or window) or not
    const v4i p0 = *reinterpret_cast<const v4i*>(&rslot[sub0 + 4 * g]);
    const v4i p1 = *reinterpret_cast<const v4i*>(&rslot[sub0 + 16 + 4 * g]);
    v4f part[4][2];
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) part[w4][rt] = ssum[grp][(sc / GR) & 1][w4][rt][lane];
    // fixed order: ((w0 + w1) + w2) + w3
    v4f st[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) st[rt] = ((part[0][rt] + part[1][rt]) + part[2][rt]) + part[3][rt];

    // ---- online softmax for head `col` over rows 4g+i (+16)
    float lg[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // fma with a zero addend is the rounded product; -inf masks the row
      lg[i] = __builtin_fmaf(st[0][i], lg_scale, p0[i] != kRowAbsent ? 0.0f : -__builtin_inff());
      lg[4 + i] = __builtin_fmaf(st[1][i], lg_scale, p1[i] != kRowAbsent ? 0.0f : -__builtin_inff());
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, lg[k]);
    mx = rows4_max(mx);
    // Lazy reference: the running reference m_run moves only when a logit
    // exceeds it by more than 8 (log2 units), so weights p stay <= 2^8 (exact
    // range for the fp16 P operand and far from fp32 overflow) and the
    // accumulator rescale is skipped while no head's reference moves.  The
    // result is the same softmax: sums and outputs share the reference.
    const bool grow = mx > m_run + 8.0f;  // m_run = -inf: any valid row grows it
    const float m_new = grow ? mx : m_run;
    // v_exp_f32 directly: its arguments are <= 8 or -inf (exp2(-inf) = 0),
    // and results below the smallest normal (weights under 2^-126 of the
    // reference) flush to 0.  While no row of head `col` has been valid,
    // m_new is -inf; subtracting 0 instead keeps p = 0 and alpha = 0 (it
    // scales only zeros then) rather than forming -inf - -inf.
    const float m_sub = (m_new == -__builtin_inff()) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
    // the sums take the weights as the P.V product sees them (rounded to
    // fp16), so that numerator and denominator use the same weights: the
    // output is then a weighted mean of the rows whatever the rounding
    float psum = 0.0f;
    v8h pa;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pa[k] = (_Float16)__builtin_amdgcn_exp2f(lg[k] - m_sub);
      psum += (float)pa[k];
    }
    psum = rows4_sum(psum);
    l_run = l_run * alpha + psum;
    // rescale output rows (heads 4g+i) by their alpha, only when some head
    // with a nonzero accumulator moved its reference (wave-uniform test;
    // every wave of the workgroup takes the same decision)
    // lane (g, col) has head col's factor; output rows are heads 4g..4g+3
    if (__ballot(grow && m_run != -__builtin_inff()) != 0) {
      if (lane < 16) alph[grp][wave][lane] = alpha;
      wave_lds_order();
      const v4f al = *reinterpret_cast<const v4f*>(&alph[grp][wave][4 * g]);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o_acc[c][i] *= al[i];
    }
    m_run = m_new;

    // ---- O (16 heads x 128 channels) += P (16 x 32 rows) . V (32 rows x 128);
    // every transposed read is issued before the first product
    v8h vb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const v4h v0 = lds_ld_tr(pv_addr[c]);
      const v4h v1 = lds_ld_tr(pv_addr[c] + kRowBytes16);
      vb[c] = v8h{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
    // (kept apart: the scheduler would otherwise pair each read with its
    // product and wait out every read's latency in turn)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) o_acc[c] = mfma16(pa, vb[c], o_acc[c]);
    // the next sub-chunk's tile stores come after these reads
    wave_lds_order();
  };

  // The loop over the sub-chunks for one kind of split (the same for every
  // wave): only FP4 entries (rows < topk), only window rows, or both.
  // Ring: each round unrolls NB sub-chunks, so buffer j always holds
  // sub-chunk NB r + j and no load result is copied inside the loop.  A
  // sub-chunk's buffer is refilled with the loads of the sub-chunk NB later
  // (absent rows past the split's end), whose slots are read from LDS before
  // the processing.
  auto ring = [&](auto mode_tag) __attribute__((always_inline)) {
    constexpr bool SC4 = decltype(mode_tag)::value == kFp4Only;
    // lane offsets from a row's load bases: FP4 rows the codes 64 w + 16 g
    // .. + 15 and the word of scale bytes 16 (w / 2) + 8 (w & 1) + 2 g (its
    // two groups); window rows the bytes 128 w + 32 g .. + 31
    const int o0 = SC4 ? 64 * wave + 16 * g : 128 * wave + 32 * g;
    const int o1 = SC4 ? 16 * (wave >> 1) + 4 * (2 * (wave & 1) + (g >> 1)) : 128 * wave + 32 * g;
    constexpr bool BASES = STRAIGHT && decltype(mode_tag)::value != kMixed;
    // the loads of sub-chunk sc into L from its rows' slots (and with BASES
    // their load bases), read from LDS beforehand
    auto issue_from = [&](int sc, const SubSlots& ss, const v4u (&rb)[2], SubLoads& L)
                          __attribute__((always_inline)) {
      if constexpr (BASES) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const RowPtrs base = __builtin_bit_cast(RowPtrs, rb[rt]);
          L.s[rt] = ss.s[rt];
          L.lo[rt] = gld16(base.p0 + o0);
          if (SC4) L.hi[rt] = v4u{gld4(base.p1 + o1), 0u, 0u, 0u};
          else L.hi[rt] = gld16(base.p1 + o1);
        }
      } else {
        issue_sub<SC4>(a, ss, row0 + sc * kSub, wave, g, col, win_row0, L);
      }
    };
    auto read_bases = [&](int sc, v4u (&rb)[2]) __attribute__((always_inline)) {
      if constexpr (BASES) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) rb[rt] = *reinterpret_cast<const v4u*>(&rbase[sc * kSub + 16 * rt + col][0]);
      }
    };
    // the group's first NB sub-chunks' row loads (everything they need read
    // from LDS together first), then the query's conversion
    {
      v4u rb[NB][2];
      SubSlots ss[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        ss[i] = read_sub(rslot, (GR * i + grp) * kSub, n_rel, col);
        read_bases(GR * i + grp, rb[i]);
      }
      // (in sub-chunk order: the wait counter retires loads in issue order,
      // so each sub-chunk then waits only for its own rows)
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        issue_from(GR * i + grp, ss[i], rb[i], buf[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    q_convert();
    if constexpr (STRAIGHT) {
      // every group runs the same number of rounds (one barrier each); a
      // group without a sub-chunk in the last round takes its barrier alone
      const int n_rounds = (n_sub + GR - 1) / GR;
#pragma unroll
      for (int j = 0; j < JG; ++j) {
        if (j < n_rounds) {
          const int sc = GR * j + grp;
          if (sc < n_sub) {
            if (j + NB < JG) {
              // the group's sub-chunk NB later refills this buffer after
              // the processing
              const int nx = GR * (j + NB) + grp;
              v4u rb[2];
              const SubSlots ns = read_sub(rslot, nx * kSub, n_rel, col);
              read_bases(nx, rb);
              process(sc, buf[j % NB], mode_tag);
              issue_from(nx, ns, rb, buf[j % NB]);
            } else {
              process(sc, buf[j % NB], mode_tag);
            }
          } else {
            lds_barrier();  // (the one its sub-chunk would have taken)
          }
        }
      }
    } else {
      for (int sc0 = 0; sc0 < n_sub; sc0 += NB) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int sc = sc0 + j;
          if (sc < n_sub) {
            const int nx = sc + NB;
            const SubSlots ns = read_sub(rslot, nx * kSub, n_rel, col);
            process(sc, buf[j], mode_tag);
            issue_sub<SC4>(a, ns, row0 + nx * kSub, wave, g, col, win_row0, buf[j]);
          }
        }
      }
    }
  };
  if (row1 <= a.topk) ring(std::integral_constant<int, kFp4Only>{});
  else if (row0 >= a.topk) ring(std::integral_constant<int, kWindowOnly>{});
  else ring(std::integral_constant<int, kMixed>{});

  if constexpr (GR == 2) {
    // ---- the groups' results merged: group 1 leaves its output
    // accumulators in LDS (wave w in its own tile, which only it used) and
    // its running (m, l) per head; group 0 rescales both to the larger
    // reference (a group with no row yet has m = -inf and contributes 0)
    if (grp == 1) {
      float* ob = reinterpret_cast<float*>(my_kr);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[(4 * c + i) * 64 + lane] = o_acc[c][i];
      if (wave == 0 && lane < 16) {
        gml[0][lane] = m_run;
        gml[1][lane] = l_run;
      }
    }
    lds_barrier();
    if (grp == 1) return;
    const float m1 = gml[0][col], l1 = gml[1][col];
    const float m = fmaxf(m_run, m1);
    const float f0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float f1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
    l_run = l_run * f0 + l1 * f1;
    m_run = m;
    // lane (g, col) has head col's factors; its output rows are heads 4g..4g+3
    if (lane < 16) {
      gfac[wave][0][lane] = f0;
      gfac[wave][1][lane] = f1;
    }
    wave_lds_order();
    const v4f a0 = *reinterpret_cast<const v4f*>(&gfac[wave][0][4 * g]);
    const v4f a1 = *reinterpret_cast<const v4f*>(&gfac[wave][1][4 * g]);
    const float* ob1 = reinterpret_cast<const float*>(kr[1][wave]);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) o_acc[c][i] = o_acc[c][i] * a0[i] + ob1[(4 * c + i) * 64 + lane] * a1[i];
  }

  if (a.n_splits == 1) {
    // ---- the whole list was this split's: normalize and write the output
    // (heads 4g+i of lane (g, col) need their sums: lanes 0..15 hold l, m)
    if (lane < 16) alph[grp][wave][lane] = 1.0f / l_run;
    wave_lds_order();
    const v4f inv = *reinterpret_cast<const v4f*>(&alph[grp][wave][4 * g]);
    float* orow = a.out + ((int64_t)bt * a.H + ht * 16) * kD;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[(4 * g + i) * kD + 128 * wave + c * 16 + col] = o_acc[c][i] * inv[i];
    if (a.out_lse && wave == 0 && lane < 16)
      a.out_lse[(int64_t)bt * a.H + ht * 16 + lane] = (m_run + log2f(l_run)) * 0.69314718055994530942f;
    return;
  }
  // ---- write this split's partials
  const int64_t pidx = ((int64_t)bt * NHT + ht) * a.n_splits + split;
  float* po = a.part_o + pidx * 16 * kD;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(4 * g + i) * kD + 128 * wave + c * 16 + col] = o_acc[c][i];
  if (wave == 0 && lane < 16) {
    a.part_ml[pidx * 32 + lane] = m_run;
    a.part_ml[pidx * 32 + 16 + lane] = l_run;
  }
}

// ---------------------------------------------------------------- 64 heads
// One workgroup per (b, t, split) serves all 64 heads, so that every row is
// gathered and dequantized once, into a shared LDS tile of 32 rows x 512
// channels (double-buffered).  Wave w = (head tile ht = w % 4, channel half
// kh = w / 4) computes the logits S^T of all 32 rows for its 16 heads over
// its 256 channels (that part of the query in registers).  Then the kh = 0
// wave adds the other half's partial logits (fixed order), runs the heads'
// online softmax and shares the fp16 weights P and the rescale factors
// through LDS, while the four kh = 1 waves dequantize the next sub-chunk's
// rows into the other tile buffer.  Wave w then owns output channels 64 w ..
// 64 w + 63 of all 64 heads and accumulates P.V from the tile, reading V
// transposed.  Two barriers per sub-chunk: after the logits, and after the
// weights and the next tile.
constexpr int kHThreads = 512;
constexpr int kTileRowHalves = kD;        // a tile row: 512 fp16 channels (64 chunks of 16 B)
constexpr int kPStride = 40;              // P row (one head): 32 rows of fp16, padded to 80 B

// Chunk k (8 channels) of tile row r sits at chunk k ^ bitrev4(r % 16) of
// the row, which keeps all three access patterns free of bank conflicts: the
// dequant stores and the Q.K operand loads (16 lanes: one chunk of 16 rows)
// and the transposed P.V loads (16 lanes: 2 chunks of 4 rows).
__device__ __forceinline__ int htile_off(int row, int chunk) {  // in halves
  return row * kTileRowHalves + 8 * (chunk ^ swz(row));
}

// The row loads of one sub-chunk for lane L of kh = 1 wave w (v = w % 4):
// row 16 (v % 2) + L % 16, channel pieces 32 c .. + 31 for c = 4 (v / 2) +
// L / 16 and c + 8.  FP4 piece: 16 code bytes + the 16 scale bytes 16 (c /
// 8) .. + 15 of the entry (the piece's two groups among them); window
// piece: 32 E4M3 bytes.
struct HLoads {
  v4u lo, hi;
  int s;
};

__device__ __forceinline__ void issue_hrow_s(const AttnArgs& a, int s, int abs_row, int c32, const uint8_t* win_row0,
                                             HLoads& L) {
  L.s = s;
  const RowPtrs rp = row_ptrs(a, s, win_row0, abs_row, 16 * c32, 16 * (c32 >> 3), 32 * c32);
  L.lo = gld16(rp.p0);
  L.hi = gld16(rp.p1);
}

template <int KP>
__global__ __launch_bounds__(kHThreads) void attn_heads_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) half_t tile[2][kSub * kTileRowHalves];  // double-buffered
  __shared__ __attribute__((aligned(16))) half_t pmat[64 * kPStride];            // P [head][row]
  __shared__ __attribute__((aligned(16))) v4f spart[4][2][64];                   // kh = 1 partial logits
  __shared__ __attribute__((aligned(16))) float salpha[64];
  __shared__ __attribute__((aligned(16))) float sfin[2][64];                     // final m, l
  __shared__ __attribute__((aligned(16))) float sqmax[2][64];
  __shared__ int sgrow[4];
  __shared__ __attribute__((aligned(16))) int rslot[kMaxRows + kSub];

  const int unit = blockIdx.x;  // split + n_splits * (b*T + t)
  if (unit >= a.n_splits * a.BT) return;
  const int split = unit % a.n_splits;
  const int bt = unit / a.n_splits;
  const int b = bt / a.T, t = bt % a.T;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int ht = wave & 3, kh = wave >> 2;  // Q.K role
  int n = a.n_entries[b];
  n = min(n, a.max_pages * kPage);
  const int n_rows = a.topk + kSwa;
  const int row0 = split * a.split_rows;
  const int row1 = min(n_rows, row0 + a.split_rows);
  const int n_sub = (row1 - row0 + kSub - 1) / kSub;
  const int n_rel = n_sub * kSub;
  const int32_t* idx_row = a.topk_idx + (int64_t)bt * a.topk;
  const uint8_t* win_row0 = a.swa + ((int64_t)b * (kSwa - 1 + a.T) + t) * kD;

  // the query of head 16 ht + col, channels 256 kh + 32 s + 8 g .. + 7 (K
  // slice s of the half), goes out first
  v4u qraw[8];
  {
    const uint16_t* qrow = a.q + (((int64_t)bt * a.H) + ht * 16 + col) * kD + 256 * kh + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qraw[s] = *reinterpret_cast<const v4u*>(qrow + 32 * s);
  }

  // ---- resolve the split's rows once (all index loads, then all page loads)
  {
    constexpr int kPer = KP;
    int jj[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int row = row0 + (int)threadIdx.x + k * kHThreads;
      jj[k] = idx_row[max(0, min(row, a.topk - 1))];
    }
    resolve_fence(jj);  // (each batch taken whole, as in the head-tile kernel)
    int pp[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int lp = max(0, min(jj[k] >> 6, a.max_pages - 1));
      pp[k] = a.page_table[(int64_t)b * a.max_pages + lp];
    }
    resolve_fence(pp);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int r = (int)threadIdx.x + k * kHThreads;
      if (r < n_rel) rslot[r] = row_slot(a, row0 + r, row1, n, jj[k], pp[k]);
    }
    resolve_rest(a, idx_row, b, n, row0, row1, kPer * kHThreads, kHThreads, n_rel, rslot);
  }
  // each head's largest |q| over this wave's 256 channels (bf16 bits in the high half)
  {
    uint32_t mx = 0u;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max((qraw[s][e] << 16) & 0x7FFF0000u, qraw[s][e] & 0x7FFF0000u));
    const float m = rows4_max(__uint_as_float(mx));
    if (lane < 16) sqmax[kh][16 * ht + lane] = m;
  }
  __syncthreads();

  // ---- the first sub-chunks' row loads, kh = 1 waves (the ring below keeps
  // two sub-chunks in flight)
  const int dv = wave & 3;
  const int drow = 16 * (dv & 1) + (lane & 15);  // dequant role: this lane's row of a sub-chunk
  const int c32 = 4 * (dv >> 1) + (lane >> 4);   // and its 32-channel pieces c32, c32 + 8
  HLoads buf[2][2];
  // the kh = 0 waves issue the prologue's loads too, of absent rows (the
  // pool's first bytes), so that every path reaches the loops with the same
  // loads in flight and the waits on them count exactly
  const int sc_pro = kh == 1 ? 0 : n_sub + 4;
  // (sub_slot: the slot of this lane's row of sub-chunk sc, read from LDS
  // ahead of the loads it addresses)
  auto sub_slot = [&](int sc) __attribute__((always_inline)) { return row_at(rslot, sc * kSub + drow, n_rel); };
  auto issue_sub_s = [&](int sc, int s, HLoads (&L)[2]) __attribute__((always_inline)) {
    issue_hrow_s(a, s, row0 + sc * kSub + drow, c32, win_row0, L[0]);
    issue_hrow_s(a, s, row0 + sc * kSub + drow, c32 + 8, win_row0, L[1]);
  };
  auto issue_sub = [&](int sc, HLoads (&L)[2]) __attribute__((always_inline)) { issue_sub_s(sc, sub_slot(sc), L); };
  issue_sub(sc_pro, buf[0]);
  issue_sub(sc_pro + 1, buf[1]);

  // ---- the query as the B operand, scaled per head by a power of two that
  // puts its largest |q| in [2^14, 2^15) (fp16 never overflows; the logits
  // take the inverse power back, exact)
  v8h qb[8];
  float lg_scale;
  {
    const float m = fmaxf(sqmax[0][16 * ht + col], sqmax[1][16 * ht + col]);
    const int e = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 : 14;
    const int sh = min(127, 14 - e);
    const float up = __builtin_ldexpf(1.0f, sh);
    lg_scale = a.sm_scale_log2 * __builtin_ldexpf(1.0f, -sh);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v4u pk;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const h2_t h = {(_Float16)(u2f(qraw[s][e2] << 16) * up), (_Float16)(u2f(qraw[s][e2] & 0xFFFF0000u) * up)};
        pk[e2] = __builtin_bit_cast(uint32_t, h);
      }
      asm volatile("" : "+v"(pk));
      qb[s] = __builtin_bit_cast(v8h, pk);
    }
  }

  // LDS addresses (bytes) in tile buffer 0: the dequant stores (row drow,
  // chunks 4 c32 + j), the Q.K operand reads (row 16 rt + col, chunk 4 s + g
  // of the wave's half: slices s and s + 4 lie 256 bytes apart, since the
  // swizzle keeps bits 4, 5 of the chunk), the transposed V reads (rows 8 g +
  // col / 4 and + 4, channels 64 w + 16 ct + 4 (col % 4) .. + 3)
  // (rows r and r + 16 share the swizzle: the second row tile is 16 KB on)
  uint32_t st_addr[2][4], qk_addr[4], pv_addr[4];
#pragma unroll
  for (int pc = 0; pc < 2; ++pc)
#pragma unroll
    for (int j = 0; j < 4; ++j) st_addr[pc][j] = lds_addr(&tile[0][htile_off(drow, 4 * (c32 + 8 * pc) + j)]);
#pragma unroll
  for (int s = 0; s < 4; ++s) qk_addr[s] = lds_addr(&tile[0][htile_off(col, 32 * kh + 4 * s + g)]);
  {
    // K-elements of lane group g: rows 4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3
    // (the second read 16 rows on, where the swizzle repeats; P is stored in
    // the same order)
    const int tr_row = 4 * g + (col >> 2), tq = col & 3;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      pv_addr[ct] = lds_addr(&tile[0][htile_off(tr_row, 8 * wave + 2 * ct + (tq >> 1)) + 4 * (tq & 1)]);
  }
  constexpr uint32_t kBufBytes = kSub * kTileRowHalves * 2;  // 32 KB
  constexpr uint32_t kRows16 = 16 * kTileRowHalves * 2;      // 16 rows, bytes
  // P row of a head holds its weights in the K order of the P.V product: row
  // 16 rt + 4 g + i at 8 g + 4 rt + i.  Stores: head 16 ht + col, rows 16 rt
  // + 4 g ..; reads: head 16 h4 + col, places 8 g .. 8 g + 7; head tiles lie
  // 16 P rows apart
  const uint32_t p_st = lds_addr(&pmat[(16 * ht + col) * kPStride + 8 * g]);
  const uint32_t p_rd = lds_addr(&pmat[col * kPStride + 8 * g]);
  constexpr uint32_t kPTile = 16 * kPStride * 2;

  float m_run = -__builtin_inff();  // kh = 0: running reference (log2) of head 16 ht + col
  float l_run = 0.0f;
  v4f o_acc[4][4];                  // [head tile][channel tile]: heads 16 h4 + 4 g + i
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o_acc[h4][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  // kh = 1 waves: dequantize this lane's two row pieces (32 channels each)
  // of sub-chunk sc into tile buffer sc % 2.  One code path for every
  // sub-chunk: each lane's row is an FP4 entry, a window row or absent
  // (lanes branch apart only in the one sub-chunk that holds both kinds)
  auto dequant = [&](int sc, const HLoads (&LL)[2]) __attribute__((always_inline)) {
    const uint32_t tb = (uint32_t)(sc & 1) * kBufBytes;
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      const HLoads& L = LL[pc];
      v8h d[4];
      const int s = L.s;
      auto fp4_row = [&](bool present) {
        uint32_t pm = present ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(pm));
        // groups 2 c, 2 c + 1 of piece c (c = c32 + 8 pc): bytes 2 (c % 8),
        // + 1 of the 16 loaded scale bytes (c % 8 = c32 % 8), picked by selects (a lane-dependent element index
        // would put the load buffers in scratch memory)
        const int wsel = (c32 & 7) >> 1;
        const uint32_t w01 = (wsel & 1) ? L.hi[1] : L.hi[0];
        const uint32_t w23 = (wsel & 1) ? L.hi[3] : L.hi[2];
        const uint32_t sw = (((wsel & 2) ? w23 : w01) >> (16 * (c32 & 1))) & 0xFFFFu;
        const uint32_t s0 = (sw & 0xFFu) * 0x101u & pm, s1 = (sw >> 8) * 0x101u & pm;
        const h2_t sc0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, false);
        const h2_t sc1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, false);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const h2_t scq = q < 2 ? sc0 : sc1;
          const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(L.lo[q], 1.0f, 0) * scq;
          const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(L.lo[q], 1.0f, 1) * scq;
          const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(L.lo[q], 1.0f, 2) * scq;
          const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(L.lo[q], 1.0f, 3) * scq;
          d[q] = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        }
      };
      auto fp8_row = [&](bool w) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t c0 = w ? (q < 2 ? L.lo[2 * q] : L.hi[2 * q - 4]) : 0u;
          const uint32_t c1 = w ? (q < 2 ? L.lo[2 * q + 1] : L.hi[2 * q - 3]) : 0u;
          const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, false);
          const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c0, 1.0f, true);
          const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, false);
          const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c1, 1.0f, true);
          d[q] = v8h{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
        }
      };
      if (s != kRowWindow) fp4_row(s >= 0);
      else fp8_row(true);
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_st16(st_addr[pc][j] + tb, d[j]);
    }
  };

  // slot: the ring slot of sub-chunk sc + 1 (its loads in, sub-chunk sc + 3's
  // loads out); the loop below alternates the slots, so that no load result
  // is copied (a copy would wait for the load)
  // The two roles run their own copies of the loop (KH1: the wave's channel
  // half, known at compile time), so that the kh = 1 waves issue their loads
  // in every pass and each wait on them counts exactly the newer loads.
  auto process = [&](auto kh_c, int sc, HLoads (&slot)[2]) __attribute__((always_inline)) {
    constexpr bool KH1 = decltype(kh_c)::value;
    const uint32_t tb = (uint32_t)(sc & 1) * kBufBytes;
    // (kh = 1: the slot of sub-chunk sc + 3's row, read now, long before its
    // loads go out after the dequant)
    const int s_next = KH1 ? sub_slot(sc + 3) : 0;
    // ---- Q.K role: partial logits of rows 16 rt + 4 g + i, head 16 ht + col,
    // over this wave's channel half
    v4f sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8h ka[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = lds_ld16(qk_addr[s] + tb + kRows16 * (uint32_t)rt + 256u * (uint32_t)h);
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[rt] = mfma16(ka[s], qb[4 * h + s], sacc[rt]);
      }
    }
    if constexpr (KH1) {
      spart[ht][0][lane] = sacc[0];
      spart[ht][1][lane] = sacc[1];
    }
    lds_barrier();  // 1: the second halves' partial logits
    if constexpr (!KH1) {
      // ---- logits (fixed order: first half + second half), online softmax
      // with the lazy reference of the head-tile kernel above
      const int sub0 = sc * kSub;
      const v4i pr0 = *reinterpret_cast<const v4i*>(&rslot[sub0 + 4 * g]);
      const v4i pr1 = *reinterpret_cast<const v4i*>(&rslot[sub0 + 16 + 4 * g]);
      const v4f o0 = spart[ht][0][lane], o1 = spart[ht][1][lane];
      float lg[8];
      float mx = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lg[i] = __builtin_fmaf(sacc[0][i] + o0[i], lg_scale, pr0[i] != kRowAbsent ? 0.0f : -__builtin_inff());
        lg[4 + i] = __builtin_fmaf(sacc[1][i] + o1[i], lg_scale, pr1[i] != kRowAbsent ? 0.0f : -__builtin_inff());
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = fmaxf(mx, lg[k]);
      mx = rows4_max(mx);
      const bool grow = mx > m_run + 8.0f;
      const float m_new = grow ? mx : m_run;
      const float m_sub = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
      const bool rescale = __ballot(grow && m_run != -__builtin_inff()) != 0;
      float psum = 0.0f;
      v4h pq[2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(lg[k] - m_sub);
        pq[k >> 2][k & 3] = p;
        psum += (float)p;
      }
      psum = rows4_sum(psum);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) *(__attribute__((address_space(3))) v4h*)(uintptr_t)(p_st + 8u * rt) = pq[rt];
      if (lane < 16) salpha[16 * ht + lane] = alpha;
      if (lane == 0) sgrow[ht] = rescale ? 1 : 0;
    } else {
      // ---- the next sub-chunk's tile (its buffer was last read by the
      // P.V of sub-chunk sc - 1, which every wave finished before barrier
      // 1); past the last sub-chunk the rows are absent (zeros into a
      // buffer no wave reads again, loads of the pool's first bytes)
      dequant(sc + 1, slot);
      issue_sub_s(sc + 3, s_next, slot);
    }
    lds_barrier();  // 2: P, the rescale factors and the next tile
    // ---- P.V role: rescale, then O[heads][64 w + 16 ct ..] += P . V
    if ((sgrow[0] | sgrow[1] | sgrow[2] | sgrow[3]) != 0) {
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) {
        const v4f al = *reinterpret_cast<const v4f*>(&salpha[16 * h4 + 4 * g]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_acc[h4][ct][i] *= al[i];
      }
    }
    v8h vb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v4h v0 = lds_ld_tr(pv_addr[ct] + tb);
      const v4h v1 = lds_ld_tr(pv_addr[ct] + tb + kRows16);
      vb[ct] = v8h{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
      const v8h pa = lds_ld16(p_rd + kPTile * (uint32_t)h4);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) o_acc[h4][ct] = mfma16(pa, vb[ct], o_acc[h4][ct]);
    }
  };

  // the first tile, then one pass per sub-chunk (ring slot s % 2 holds
  // sub-chunk s's loads)
  if (kh == 1) dequant(0, buf[0]);
  issue_sub(sc_pro + 2, buf[0]);
  lds_barrier();
  auto loop = [&](auto kh_c) __attribute__((always_inline)) {
    int sc = 0;
    for (; sc + 1 < n_sub; sc += 2) {
      process(kh_c, sc, buf[1]);
      process(kh_c, sc + 1, buf[0]);
    }
    if (sc < n_sub) process(kh_c, sc, buf[1]);
  };
  if (kh == 0) loop(std::false_type{});
  else loop(std::true_type{});

  // ---- every head's (m, l) to all waves
  if (kh == 0 && lane < 16) {
    sfin[0][16 * ht + lane] = m_run;
    sfin[1][16 * ht + lane] = l_run;
  }
  __syncthreads();
  // lane (g, col) of wave w holds O[16 h4 + 4 g + i][64 w + 16 ct + col]
  if (a.n_splits == 1) {
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
      const v4f lv = *reinterpret_cast<const v4f*>(&sfin[1][16 * h4 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv = 1.0f / lv[i];
        float* orow = a.out + ((int64_t)bt * a.H + 16 * h4 + 4 * g + i) * kD + 64 * wave + col;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) orow[16 * ct] = o_acc[h4][ct][i] * inv;
      }
    }
    if (a.out_lse && threadIdx.x < 64)
      a.out_lse[(int64_t)bt * a.H + threadIdx.x] =
          (sfin[0][threadIdx.x] + log2f(sfin[1][threadIdx.x])) * 0.69314718055994530942f;
    return;
  }
  // ---- partials in the head-tile kernel's layout: [bt][ht][split][16][512]
#pragma unroll
  for (int h4 = 0; h4 < 4; ++h4) {
    const int64_t pidx = ((int64_t)bt * 4 + h4) * a.n_splits + split;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* po = a.part_o + (pidx * 16 + 4 * g + i) * kD + 64 * wave + col;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) po[16 * ct] = o_acc[h4][ct][i];
    }
  }
  if (threadIdx.x < 64) {
    const int h = threadIdx.x;
    const int64_t pidx = ((int64_t)bt * 4 + (h >> 4)) * a.n_splits + split;
    a.part_ml[pidx * 32 + (h & 15)] = sfin[0][h];
    a.part_ml[pidx * 32 + 16 + (h & 15)] = sfin[1][h];
  }
}

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  int H;
  int n_splits;
  float* out;
  float* out_lse;
};

// One workgroup per (b, t, h), 128 threads of 4 channels: merge the splits'
// (max, sum, output).  Wave 0 loads the (max, sum) pairs first, then every
// thread issues its loads of all splits' output rows; the split weights are
// formed (one wave, in registers) while those are in flight.
constexpr int kMaxSplits = 24;
constexpr int kLoadRing = 3;  // sub-chunks whose row loads are in flight together
constexpr int kStraightSubs = 5;  // splits of at most this many sub-chunks: the loop unrolled whole
constexpr int kStraightBufs = 4;  // with this many load buffers
constexpr int kPairBufs = 3;      // two wave groups: load buffers of each (its whole share)
// Rows per thread that cover a whole list (the longest split)
constexpr int kResolveMax = (kMaxRows + kAttnThreads - 1) / kAttnThreads;  // 9
constexpr int kHResolveMax = (kMaxRows + kHThreads - 1) / kHThreads;       // 5

template <int MAXS>
__global__ __launch_bounds__(128) void attn_combine_kernel(CombineArgs a) {
  __shared__ float wsplit[MAXS];
  __shared__ float inv_l;
  const int h = blockIdx.x % a.H;
  const int bt = blockIdx.x / a.H;
  const int NHT = a.H >> 4, ht = h >> 4, hh = h & 15;
  const int64_t base = ((int64_t)bt * NHT + ht) * a.n_splits;
  const int lane = lane_id();
  const int tid = (int)threadIdx.x;
  // (max, sum) of split `tid` (threads 0..MAXS-1; MAXS <= 128)
  const bool in = tid < a.n_splits;
  float ms = -__builtin_inff(), ls = 0.0f;
  if (in) {
    ms = a.part_ml[(base + tid) * 32 + hh];
    ls = a.part_ml[(base + tid) * 32 + 16 + hh];
  }
  // loads complete in issue order: keep the pairs ahead of the rows
  asm volatile("" ::: "memory");
  const int c = tid * 4;
  // unconditional loads (splits past n_splits re-read the last one and are
  // not used), so that no branch separates them and each waits only for its own
  v4f po[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const int sc = min(s, a.n_splits - 1);
    po[s] = *reinterpret_cast<const v4f*>(a.part_o + ((base + sc) * 16 + hh) * kD + c);
  }
  // every row load is issued before the first wait for the pairs
  asm volatile("" : "+v"(ms), "+v"(ls)::"memory");
  // the global maximum and the weighted sum, over the splits, in thread order
  __shared__ float red[2][2];
  float M = ms;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[0][tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  const float wgt = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - M);
  float L = wgt * ls;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
  if (lane == 0) red[1][tid >> 6] = L;
  if (tid < MAXS) wsplit[tid] = in ? wgt : 0.0f;
  __syncthreads();
  if (tid == 0) {
    const float Lt = red[1][0] + red[1][1];
    inv_l = 1.0f / Lt;
    if (a.out_lse) a.out_lse[(int64_t)bt * a.H + h] = (M + log2f(Lt)) * 0.69314718055994530942f;
  }
  __syncthreads();
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) acc += wsplit[s] * po[s];
  *reinterpret_cast<v4f*>(a.out + ((int64_t)bt * a.H + h) * kD + c) = acc * inv_l;
}

}  // namespace csa2

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// 64 heads with B*T >= 8 take the all-heads kernel (one workgroup per (b,
// t, split)); fewer heads or rows the head-tile kernel (one per (b, t, head
// tile, split)).
// (At B*T = 4, 1M context, the head-tile kernel's 272 workgroups (now one
// round of 256) finished the
// replayed layer step ~4.5 us sooner than the all-heads kernel's 92; from
// B*T = 8 on the all-heads kernel is faster: 62 against 67 us per 128K Full
// layer at B = 8, 56 against 90 us per layer at B*T = 64.)
bool all_heads(int H, int BT) { return H == 64 && BT >= 8; }

// Rows per split (a multiple of 32) and the number of splits of one (b, t)'s
// [top-k | window] row list: about kTargetWorkgroups workgroups in all.
void split_plan(int BT, int H, int topk, int* n_splits, int* split_rows, int* split_base, int* split_extra) {
  const int rows = topk + CSA2_SWA;
  const int subs = (rows + csa2::kSub - 1) / csa2::kSub;
  if (all_heads(H, BT)) {
    const int max_splits = std::min(subs, csa2::kMaxSplits);
    int ns = std::max(1, std::min((csa2::kTargetWorkgroups + BT - 1) / BT, max_splits));
    int per = (rows + ns - 1) / ns;
    per = (per + csa2::kSub - 1) / csa2::kSub * csa2::kSub;
    *split_rows = per;
    *n_splits = (rows + per - 1) / per;
    *split_base = per / csa2::kSub;
    *split_extra = 0;
    return;
  }
  const int units = BT * (H / 16);
  // as many splits as fit the target in one round of workgroups (a second,
  // partly filled round would make its workgroups share compute units); a
  // large batch takes two workgroups per compute unit, so that one's waits
  // hide behind the other's work
  const int target = units >= csa2::kTargetWorkgroups / 2 ? 2 * csa2::kTargetWorkgroups : csa2::kTargetWorkgroups;
  const int ns = std::max(1, std::min(target / units, std::min(subs, csa2::kMaxSplits)));
  // the sub-chunks shared out as evenly as whole sub-chunks allow
  *n_splits = ns;
  *split_base = subs / ns;
  *split_extra = subs % ns;
  *split_rows = (*split_base + (*split_extra > 0 ? 1 : 0)) * csa2::kSub;
}
}  // namespace

extern "C" size_t csa2_attn_ws_bytes(int32_t B, int32_t T, int32_t H, int32_t topk) {
  int ns, per, base, extra;
  split_plan(B * T, H, topk, &ns, &per, &base, &extra);
  if (ns == 1) return 256;  // no partials
  const size_t units = (size_t)B * T * (H / 16) * ns;
  return align256(units * 16 * csa2::kD * 4) + align256(units * 32 * 4);
}

extern "C" int csa2_sparse_attn(const uint16_t* q, float sm_scale, const uint8_t* kv_pool,
                                int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                const int32_t* n_entries, const int32_t* topk_idx, int32_t topk,
                                const uint8_t* swa, int32_t B, int32_t T, int32_t H, float* out,
                                float* out_lse, void* ws, size_t ws_bytes, csa2_stream_t stream) {
  if (!q || !kv_pool || !page_table || !n_entries || !topk_idx || !swa || !out)
    return CSA2_ERR_INVALID_ARG;
  // 16-byte rows of q and of the window are read with aligned loads
  if (((uintptr_t)q & 15) || ((uintptr_t)swa & 15)) return CSA2_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || n_pages <= 0 || max_pages <= 0 || topk <= 0)
    return CSA2_ERR_INVALID_ARG;
  if (topk > CSA2_MAX_TOPK) return CSA2_ERR_INVALID_ARG;
  if (!(H == 16 || H == 32 || H == 64)) return CSA2_ERR_UNSUPPORTED;
  if (T > CSA2_MAX_T) return CSA2_ERR_UNSUPPORTED;
  if ((int64_t)B * T > 65535) return CSA2_ERR_UNSUPPORTED;
  // cache slots (page * 64 + offset) are held as int32
  if (n_pages > (int64_t)INT32_MAX / csa2::kPage) return CSA2_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return CSA2_ERR_INVALID_ARG;
  const size_t need = csa2_attn_ws_bytes(B, T, H, topk);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  csa2::AttnArgs aa{};
  aa.q = q;
  aa.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  aa.kv_pool = kv_pool;
  aa.n_pages = n_pages;
  aa.page_table = page_table;
  aa.max_pages = max_pages;
  aa.n_entries = n_entries;
  aa.topk_idx = topk_idx;
  aa.topk = topk;
  aa.swa = swa;
  aa.T = T;
  aa.H = H;
  aa.BT = B * T;
  split_plan(B * T, H, topk, &aa.n_splits, &aa.split_rows, &aa.split_base, &aa.split_extra);
  const size_t units = (size_t)B * T * (H / 16) * aa.n_splits;
  if (aa.n_splits > 1) {
    aa.part_o = reinterpret_cast<float*>(ws);
    aa.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256(units * 16 * csa2::kD * 4));
  } else {
    aa.out = out;
    aa.out_lse = out_lse;
  }
  const int n_units = aa.n_splits * B * T;
  // rows each thread resolves up front: enough for the split's rows
  if (all_heads(H, B * T)) {
    const int kp = (aa.split_rows + csa2::kHThreads - 1) / csa2::kHThreads;
    if (kp <= 1)
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, csa2::attn_heads_kernel<1>, dim3(n_units), dim3(csa2::kHThreads),
                  (hipStream_t)stream, aa);
    else if (kp <= 2)
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, csa2::attn_heads_kernel<2>, dim3(n_units), dim3(csa2::kHThreads),
                  (hipStream_t)stream, aa);
    else
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, csa2::attn_heads_kernel<csa2::kHResolveMax>, dim3(n_units),
                  dim3(csa2::kHThreads), (hipStream_t)stream, aa);
  } else {
    const int grid = 8 * (H / 16) * ((n_units + 7) / 8);
    const int kp = (aa.split_rows + csa2::kAttnThreads - 1) / csa2::kAttnThreads;
    // two wave groups per workgroup when the splits have two sub-chunks or
    // more and one round of workgroups holds the grid (one per compute unit)
    if (aa.split_rows <= csa2::kStraightSubs * csa2::kSub && aa.split_rows >= 2 * csa2::kSub &&
        grid <= csa2::kTargetWorkgroups)
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, (csa2::attn_split_kernel<csa2::kPairBufs, 1, csa2::kStraightSubs, 2>),
                  dim3(grid), dim3(2 * csa2::kAttnThreads), (hipStream_t)stream, aa);
    else if (aa.split_rows <= csa2::kStraightSubs * csa2::kSub)
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, (csa2::attn_split_kernel<csa2::kStraightBufs, 1, csa2::kStraightSubs, 1>),
                  dim3(grid), dim3(csa2::kAttnThreads), (hipStream_t)stream, aa);
    else if (kp <= 3)
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, (csa2::attn_split_kernel<csa2::kLoadRing, 3, 0, 1>), dim3(grid),
                  dim3(csa2::kAttnThreads), (hipStream_t)stream, aa);
    else
      CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, (csa2::attn_split_kernel<csa2::kLoadRing, csa2::kResolveMax, 0, 1>),
                  dim3(grid), dim3(csa2::kAttnThreads), (hipStream_t)stream, aa);
  }
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  if (aa.n_splits == 1) return CSA2_OK;
  csa2::CombineArgs ca{};
  ca.part_o = aa.part_o;
  ca.part_ml = aa.part_ml;
  ca.H = H;
  ca.n_splits = aa.n_splits;
  ca.out = out;
  ca.out_lse = out_lse;
  CSA2_LAUNCH(CSA2_K_ATTN_COMBINE, csa2::attn_combine_kernel<csa2::kMaxSplits>, dim3(B * T * H), dim3(128),
              (hipStream_t)stream, ca);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
