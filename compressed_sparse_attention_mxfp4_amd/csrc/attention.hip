// Sparse attention over the selected FP4 main-KV entries merged with the
// FP8 sliding window ("Inside DeepSeek V4.1 Flash", section "CSA2: reuse
// memory and reuse selection independently": the main query attends to the
// selected global entries together with the local window; knowledge note
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
// "FP4 main KV": entries are dequantized before attention, the window stays
// FP8).  Each 512-channel row is both key and value; one softmax runs over
// the union of the rows.
//
// Work split: one workgroup per (b, t, 16-head tile, 128-row split of the
// row list [top-k slots | 128 window rows]); its 4 waves own 128 channels
// each.  The split's rows are resolved once (index, page) and all their code
// bytes are loaded up front.  Per 32-row sub-chunk a wave converts its
// channel slice to fp16 (hardware FP4 / E4M3 conversion, exact) into a
// swizzled row-major LDS tile, computes partial logits over its channels
// with f16 MFMA; the four partials are summed in fixed order through LDS,
// every wave runs the same online softmax and accumulates P.V for its
// channels, reading V transposed from the same tile.  Splits write (max,
// sum, unnormalised output) and a combine kernel merges them.
#include "common.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kRowsPerSplit = 128;
constexpr int kSub = 32;               // rows per sub-chunk
constexpr int kRowHalves = 128;        // a wave's 128-channel slice of one row (256 B, 16 chunks of 16 B)

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
template <int M>
struct ModeTag {
  static constexpr int value = M;
};

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
  float* part_o;   // [B*T][H/16][n_splits][16][512]
  float* part_ml;  // [B*T][H/16][n_splits][32]  (m[16] in log2 units, l[16])
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
// Row loads through global-address-space pointers: the row pointers are
// passed through LDS, and plain (flat) loads of them would also count on the
// LDS wait counter, so every LDS wait would wait for the row loads as well.
typedef const __attribute__((address_space(1))) v2u gbl_v2u_t;
typedef const __attribute__((address_space(1))) uint32_t gbl_u32_t;
__device__ __forceinline__ v2u gld8(const uint8_t* p) { return *(gbl_v2u_t*)p; }
__device__ __forceinline__ uint32_t gld4(const uint8_t* p) { return *(gbl_u32_t*)p; }
__device__ __forceinline__ void lds_st16(uint32_t addr, v8h v) { *(lds_v8h_t*)(uintptr_t)addr = v; }
__device__ __forceinline__ v8h lds_ld16(uint32_t addr) { return *(const lds_v8h_t*)(uintptr_t)addr; }
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 4 halves that lane 4j + i / 4 points at, for j = 0..3
__device__ __forceinline__ v4h lds_ld_tr(uint32_t addr) {
  return __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(uintptr_t)addr));
}

// Kinds of row content a split can hold (decided per split, the same for
// every wave): only FP4 entries (rows < topk), only window rows, or both.
enum SplitMode { kMixed = 0, kFp4Only = 1, kWindowOnly = 2 };

__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) half_t kr[4][kSub * kRowHalves];
  __shared__ __attribute__((aligned(16))) v4f ssum[2][4][2][64];  // double-buffered by sub-chunk
  __shared__ __attribute__((aligned(16))) float alph[4][16];       // per wave: rescale factor per head
  __shared__ const uint8_t* rptr0[kRowsPerSplit];  // codes (FP4) or window row start
  __shared__ const uint8_t* rptr1[kRowsPerSplit];  // scale row (FP4) or window row start + 8
  __shared__ __attribute__((aligned(16))) int rkind[kRowsPerSplit];
  __shared__ __attribute__((aligned(16))) float rbias[kRowsPerSplit];  // 0 present, -inf absent

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
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  int n = a.n_entries[b];
  n = min(n, a.max_pages * kPage);

  const int n_rows = a.topk + kSwa;
  const int row0 = split * kRowsPerSplit;
  const int row1 = min(n_rows, row0 + kRowsPerSplit);
  const int32_t* idx_row = a.topk_idx + (int64_t)bt * a.topk;

  // ---- resolve the split's rows once: FP4 entry address (index, page
  // lookup) or window row; threads 0..127 take one row each
  if (threadIdx.x < kRowsPerSplit) {
    const int row = row0 + (int)threadIdx.x;
    // absent rows point at the pool's first bytes (read and discarded)
    const uint8_t* p0 = a.kv_pool;
    const uint8_t* p1 = a.kv_pool;
    int kind = 0;
    if (row < row1) {
      if (row < a.topk) {
        const int j = idx_row[row];
        if (j >= 0 && j < n) {
          const int64_t pg = phys_page(a.page_table, a.max_pages, a.n_pages, b, j >> 6);
          if (pg >= 0) {
            const uint8_t* page = a.kv_pool + pg * kPageBytes;
            p0 = page + (j & 63) * kEntryCodes;
            p1 = page + kPage * kEntryCodes + (j & 63) * kEntryScales;
            kind = 1;
          }
        }
      } else {
        p0 = a.swa + ((int64_t)b * (kSwa - 1 + a.T) + t + (row - a.topk)) * kD;
        p1 = p0 + 8;
        kind = 2;
      }
    }
    rptr0[threadIdx.x] = p0;
    rptr1[threadIdx.x] = p1;
    rkind[threadIdx.x] = kind;
    rbias[threadIdx.x] = kind != 0 ? 0.0f : -__builtin_inff();
  }

  // ---- Q slice as the B operand: head ht*16+col, channels 128*wave + 32*s
  // + 8*g .. +8, kept as packed half pairs
  v8h qb[4];
  {
    const uint16_t* qrow = a.q + (((int64_t)bt * a.H) + ht * 16 + col) * kD + 128 * wave + 8 * g;
    v4u raw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const v4u*>(qrow + 32 * s);
    // the packed words pass through an empty asm so that the compiler keeps
    // them packed instead of re-packing the halves before every MFMA
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4u pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t h = {(_Float16)u2f(raw[s][e] << 16), (_Float16)u2f(raw[s][e] & 0xFFFF0000u)};
        pk[e] = __builtin_bit_cast(uint32_t, h);
      }
      asm volatile("" : "+v"(pk));
      qb[s] = __builtin_bit_cast(v8h, pk);
    }
  }

  // lane (rg, cg) of wave w dequantizes rows 4*rg .. 4*rg+3 of each 32-row
  // sub-chunk, channels 128*w + 16*cg .. +16 (16-byte chunks 2cg, 2cg+1 of
  // the wave's tile); odd channel groups store their two chunks in the other
  // order (keeps each store instruction conflict-free)
  const int rg = lane >> 3, cg = lane & 7;
  const int odd = cg & 1;
  const int ch0 = 128 * wave + 16 * cg;
  half_t* my_kr = kr[wave];
  uint32_t st_addr[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st_addr[i][0] = lds_addr(&my_kr[tile_off(4 * rg + i, 2 * cg + odd)]);
    st_addr[i][1] = lds_addr(&my_kr[tile_off(4 * rg + i, 2 * cg + (odd ^ 1))]);
  }
  // Q.K operand rows: lane (g, col) reads row col (+16), channels 32s + 8g
  uint32_t qk_addr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qk_addr[s] = lds_addr(&my_kr[tile_off(col, 4 * s + g)]);
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
  // LDS-only barriers throughout: the row loads stay in flight across them
  lds_barrier();

  // The whole sub-chunk loop, specialised by what the split's rows can be.
  auto run = [&](auto mode_tag) {
    constexpr int kMode = decltype(mode_tag)::value;
    constexpr int kSubs = kRowsPerSplit / kSub;  // 4
    // ---- issue every code load of the split up front: per row 8 code
    // bytes + the dword holding the scale byte (FP4) or 16 bytes (window);
    // absent rows read the pool's first bytes, discarded
    const int off_fp4_0 = ch0 / 2, off_fp4_1 = (ch0 / 16) & ~3;
    v2u lo8[kSubs][4], hi8[kSubs][4];
    bool present[kSubs][4];
#pragma unroll
    for (int sc = 0; sc < kSubs; ++sc) {
      const v4i k4 = *reinterpret_cast<const v4i*>(&rkind[sc * kSub + 4 * rg]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = sc * kSub + 4 * rg + i;
        if (kMode == kFp4Only) {
          lo8[sc][i] = gld8(rptr0[rr] + off_fp4_0);
          hi8[sc][i][0] = gld4(rptr1[rr] + off_fp4_1);
          hi8[sc][i][1] = 0u;
          present[sc][i] = k4[i] == 1;
        } else if (kMode == kWindowOnly) {
          lo8[sc][i] = gld8(rptr0[rr] + ch0);
          hi8[sc][i] = gld8(rptr1[rr] + ch0);
          present[sc][i] = k4[i] == 2;
        } else {
          const bool fp4 = k4[i] == 1;
          lo8[sc][i] = gld8(rptr0[rr] + (fp4 ? off_fp4_0 : ch0));
          hi8[sc][i] = gld8(rptr1[rr] + (fp4 ? off_fp4_1 : ch0));
          present[sc][i] = k4[i] != 0;
        }
      }
      // keep the loads in sub-chunk order: the wait counter retires them in
      // issue order, so sub-chunk 0 then waits only for its own rows
      asm volatile("" ::: "memory");
    }

    float m_run = -__builtin_inff();  // running reference (log2 units) of head `col`
    float l_run = 0.0f;               // running sum of head `col`
    v4f o_acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o_acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int sc = 0; sc < kSubs; ++sc) {
      const int sub = row0 + sc * kSub;
      if (sub >= row1) break;
      // ---- dequantize 4 rows x 16 channels into the swizzled tile.
      // Hardware conversions with unit scale are exact for every FP4 and
      // E4M3 code (element 0 = low nibble / low byte); the E4M3 block scale
      // is applied by one packed fp16 multiply per channel pair, exact since
      // the product has at most 6 significant bits and lies in fp16 range.
      // Odd channel groups convert their two 8-channel halves in the other
      // order, to match their store order.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h2_t v[8];
        const v2u lo = lo8[sc][i], hi = hi8[sc][i];
        auto fp4_row = [&]() {
          // absent row: zero scale, zero row (FP4 codes are all finite).  The
          // mask is opaque so that the scale load stays unconditional (a
          // select on `present` would let the compiler sink the load into a
          // branch and wait for it there).
          uint32_t pm = present[sc][i] ? 0xFFFFFFFFu : 0u;
          asm volatile("" : "+v"(pm));
          const uint32_t scode = (hi[0] >> (8 * (cg & 3))) & 0xFFu;  // group ch0/16 = 8w + cg
          const uint32_t spair = (scode * 0x101u) & pm;
          const h2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(spair, 1.0f, false);
          const uint32_t half[2] = {odd ? lo[1] : lo[0], odd ? lo[0] : lo[1]};
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            v[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(half[d], 1.0f, 0) * s2;
            v[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(half[d], 1.0f, 1) * s2;
            v[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(half[d], 1.0f, 2) * s2;
            v[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(half[d], 1.0f, 3) * s2;
          }
        };
        auto fp8_row = [&](bool w) {
          // window row: 16 E4M3 codes; absent row: zeros (its bytes may hold
          // NaN codes, and its V must be 0 to meet p = 0)
          const v2u x = odd ? hi : lo, y = odd ? lo : hi;
          const uint32_t c4[4] = {w ? x[0] : 0u, w ? x[1] : 0u, w ? y[0] : 0u, w ? y[1] : 0u};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            v[2 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c4[d], 1.0f, false);
            v[2 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c4[d], 1.0f, true);
          }
        };
        if (kMode == kFp4Only) {
          fp4_row();
        } else if (kMode == kWindowOnly) {
          fp8_row(present[sc][i]);
        } else {
          const int kind = rkind[sc * kSub + 4 * rg + i];
          if (kind == 1) fp4_row();
          else fp8_row(kind == 2);
        }
        v8h r0, r1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          r0[2 * e] = v[e][0];
          r0[2 * e + 1] = v[e][1];
          r1[2 * e] = v[4 + e][0];
          r1[2 * e + 1] = v[4 + e][1];
        }
        lds_st16(st_addr[i][0], r0);
        lds_st16(st_addr[i][1], r1);
      }
      wave_lds_order();

      // ---- partial logits S^T (32 rows x 16 heads) over this wave's 128 channels
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        v4f sacc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc = mfma16(lds_ld16(qk_addr[s] + rt * kRowBytes16), qb[s], sacc);
        ssum[sc & 1][wave][rt][lane] = sacc;
      }
      // one barrier per sub-chunk: the next sub-chunk writes the other buffer,
      // and this buffer is rewritten only after the next sub-chunk's barrier
      lds_barrier();
      // row biases (0 or -inf) of rows 4g..4g+3 and 16+4g..16+4g+3
      const v4f bias0 = *reinterpret_cast<const v4f*>(&rbias[sc * kSub + 4 * g]);
      const v4f bias1 = *reinterpret_cast<const v4f*>(&rbias[sc * kSub + 16 + 4 * g]);
      v4f part[4][2];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) part[w4][rt] = ssum[sc & 1][w4][rt][lane];
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
        lg[i] = __builtin_fmaf(st[0][i], a.sm_scale_log2, bias0[i]);
        lg[4 + i] = __builtin_fmaf(st[1][i], a.sm_scale_log2, bias1[i]);
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
      float psum = 0.0f;
      v8h pa;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __builtin_amdgcn_exp2f(lg[k] - m_sub);
        psum += p;
        pa[k] = (_Float16)p;
      }
      psum = rows4_sum(psum);
      l_run = l_run * alpha + psum;
      // rescale output rows (heads 4g+i) by their alpha, only when some head
      // with a nonzero accumulator moved its reference (wave-uniform test;
      // every wave of the workgroup takes the same decision)
      // lane (g, col) has head col's factor; output rows are heads 4g..4g+3
      if (__ballot(grow && m_run != -__builtin_inff()) != 0) {
        if (lane < 16) alph[wave][lane] = alpha;
        wave_lds_order();
        const v4f al = *reinterpret_cast<const v4f*>(&alph[wave][4 * g]);
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) o_acc[c][i] *= al[i];
      }
      m_run = m_new;

      // ---- O (16 heads x 128 channels) += P (16 x 32 rows) . V (32 rows x 128)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v4h v0 = lds_ld_tr(pv_addr[c]);
        const v4h v1 = lds_ld_tr(pv_addr[c] + kRowBytes16);
        const v8h vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o_acc[c] = mfma16(pa, vb, o_acc[c]);
      }
      wave_lds_order();
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
  };
  if (row1 <= a.topk) run(ModeTag<kFp4Only>{});
  else if (row0 >= a.topk) run(ModeTag<kWindowOnly>{});
  else run(ModeTag<kMixed>{});
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
constexpr int kMaxSplits = (CSA2_MAX_TOPK + CSA2_SWA + kRowsPerSplit - 1) / kRowsPerSplit;

__global__ __launch_bounds__(128) void attn_combine_kernel(CombineArgs a) {
  __shared__ float wsplit[kMaxSplits];
  __shared__ float inv_l;
  const int h = blockIdx.x % a.H;
  const int bt = blockIdx.x / a.H;
  const int NHT = a.H >> 4, ht = h >> 4, hh = h & 15;
  const int64_t base = ((int64_t)bt * NHT + ht) * a.n_splits;
  const int lane = lane_id();
  const bool in = lane < a.n_splits;
  float ms = -__builtin_inff(), ls = 0.0f;
  if (threadIdx.x < 64 && in) {
    ms = a.part_ml[(base + lane) * 32 + hh];
    ls = a.part_ml[(base + lane) * 32 + 16 + hh];
  }
  // loads complete in issue order: keep the pairs ahead of the rows
  asm volatile("" ::: "memory");
  const int c = threadIdx.x * 4;
  // unconditional loads (splits past n_splits re-read the last one and are
  // not used), so that no branch separates them and each waits only for its own
  v4f po[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    const int sc = min(s, a.n_splits - 1);
    po[s] = *reinterpret_cast<const v4f*>(a.part_o + ((base + sc) * 16 + hh) * kD + c);
  }
  // every row load is issued before the first wait for the pairs
  asm volatile("" : "+v"(ms), "+v"(ls)::"memory");
  if (threadIdx.x < 64) {
    float M = ms;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wgt = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - M);
    float L = wgt * ls;
    // fixed-order sum over the splits (lane order)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) L += __shfl_xor(L, o);
    // splits past n_splits get weight 0 (their re-read rows are finite)
    if (lane < kMaxSplits) wsplit[lane] = in ? wgt : 0.0f;
    if (lane == 0) {
      inv_l = 1.0f / L;
      if (a.out_lse) a.out_lse[(int64_t)bt * a.H + h] = (M + log2f(L)) * 0.69314718055994530942f;
    }
  }
  lds_barrier();
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) acc += wsplit[s] * po[s];
  *reinterpret_cast<v4f*>(a.out + ((int64_t)bt * a.H + h) * kD + c) = acc * inv_l;
}

}  // namespace csa2

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int n_splits_for(int topk) { return (topk + CSA2_SWA + csa2::kRowsPerSplit - 1) / csa2::kRowsPerSplit; }
}  // namespace

extern "C" size_t csa2_attn_ws_bytes(int32_t B, int32_t T, int32_t H, int32_t topk) {
  const size_t ns = (size_t)n_splits_for(topk);
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
  if (B <= 0 || T <= 0 || H <= 0 || n_pages <= 0 || max_pages <= 0 || topk <= 0)
    return CSA2_ERR_INVALID_ARG;
  if (topk > CSA2_MAX_TOPK) return CSA2_ERR_INVALID_ARG;
  if (!(H == 16 || H == 32 || H == 64)) return CSA2_ERR_UNSUPPORTED;
  if (T > CSA2_MAX_T) return CSA2_ERR_UNSUPPORTED;
  if ((int64_t)B * T > 65535) return CSA2_ERR_UNSUPPORTED;
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
  aa.n_splits = n_splits_for(topk);
  aa.BT = B * T;
  const size_t units = (size_t)B * T * (H / 16) * aa.n_splits;
  aa.part_o = reinterpret_cast<float*>(ws);
  aa.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256(units * 16 * csa2::kD * 4));
  const int n_units = aa.n_splits * B * T;
  const int grid = 8 * (H / 16) * ((n_units + 7) / 8);
  CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, csa2::attn_split_kernel, dim3(grid),
              dim3(csa2::kAttnThreads), (hipStream_t)stream, aa);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  csa2::CombineArgs ca{};
  ca.part_o = aa.part_o;
  ca.part_ml = aa.part_ml;
  ca.H = H;
  ca.n_splits = aa.n_splits;
  ca.out = out;
  ca.out_lse = out_lse;
  CSA2_LAUNCH(CSA2_K_ATTN_COMBINE, csa2::attn_combine_kernel, dim3(B * T * H), dim3(128),
              (hipStream_t)stream, ca);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
