// FP4 main-KV cache write (knowledge note "DeepSeek-V4.1-Flash: Pushing the
// Limits of KV Cache Compression", section "FP4 main KV: trade precision for
// bytes"; "Inside DeepSeek V4.1 Flash", section "Reconstructing the 890-byte
// cache budget": 512 x 4/8 + 512/16 = 288 B per entry).
//
// One thread per 16-channel group: 32 threads cover one 1 KiB bf16 row with
// two 16 B loads each (a wave reads 2 KiB contiguous), write 8 B of E2M1
// nibbles each (256 B contiguous per row) and one E4M3 scale byte, gathered
// four at a time into a dword store.  1,024 B read + 288 B written per row.
//
// The elements are rounded in pairs on packed 16-bit integers: a non-negative
// bf16 bit pattern orders like its value, and every E2M1 decision boundary
// mid * scale (mid in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, scale an E4M3
// value) has at most 7 significant bits, so it is itself a bf16 value and
// "|x| >= boundary" is an exact integer comparison of bit patterns (a strict
// boundary compares against the next pattern up).  Three such comparisons
// per element, a binary search over the 8 magnitudes, give the code.
#include "common.h"

namespace csa2 {

// E4M3 code (positive, saturating at 448 = 0x7E) nearest to t, ties to even.
// t >= 0 is a correctly rounded binary32 quotient amax / 6; rounding that
// quotient to binary32 cannot move it onto or across an E4M3 midpoint
// (amax has 8 significant bits, so amax / 6 is either exact or at least
// 2^-10 relative away from every midpoint), so this equals the E4M3
// rounding of the exact quotient.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
// Per 16-bit half: all ones where a > t1, else zero (a, t1 below 2^15: the
// sign of the 16-bit difference t1 - a, spread by an arithmetic shift).
// `sh15` holds 15 in both halves, as a value the compiler cannot see: with a
// constant shift it turns the sign test into a compare and a select per half.
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t reach_mask(uint32_t a, uint32_t t1, i16x2 sh15) {
  const i16x2 d = __builtin_bit_cast(i16x2, as_u32(as_u16x2(t1) - as_u16x2(a)));
  return __builtin_bit_cast(uint32_t, (i16x2)(d >> sh15));
}
// Logical shift right by 12 of each 16-bit half.
__device__ __forceinline__ uint32_t pk_shr12(uint32_t x) { return as_u32(as_u16x2(x) >> (u16x2){12, 12}); }
// Bits of x where m is set, of y elsewhere.
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t x, uint32_t y) { return (m & x) | (~m & y); }


__device__ __forceinline__ uint32_t e4m3_rne_pos(float t) {
  if (t >= 448.0f) return 0x7Eu;
  if (t < 0.015625f) {  // below the smallest normal 2^-6: steps of 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);  // 0..8 (8 is the normal 2^-6)
  }
  uint32_t u = f2u(t);
  uint32_t lsb = (u >> 20) & 1u;
  u += 0x7FFFFu + lsb;                 // round the 23-bit mantissa to 3 bits
  uint32_t e = (u >> 23) - 120u;       // E4M3 exponent field (bias 7)
  uint32_t code = (e << 3) | ((u >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of a positive E4M3 code as binary32 (exact).
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
  uint32_t e = c >> 3, m = c & 7u;
  return e ? u2f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// FP4 group of 16 bf16 channels (h[j]: channels 2j low, 2j + 1 high):
// E2M1 nibbles in w0 (channels 0..7) and w1 (channels 8..15), scale code sc.
struct Fp4Group {
  uint32_t w0, w1, sc;
};
__device__ __forceinline__ Fp4Group fp4_group(const uint32_t (&h)[8]) {
  // amax over 16 bf16 magnitudes (pairs of bit patterns)
  u16x2 mag[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mag[i] = as_u16x2(h[i] & 0x7FFF7FFFu);
  u16x2 mx2 = mag[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx2 = max(mx2, mag[i]);
  const uint32_t amax_bits = max((uint32_t)mx2.x, (uint32_t)mx2.y);
  const float amax = u2f(amax_bits << 16);
  const uint32_t sc = e4m3_rne_pos(__fdiv_rn(amax, 6.0f));
  const float sv = e4m3_value_pos(sc);
  // decision boundaries as bf16 bit patterns in both halves: |x| >= t (ties
  // at 0.75, 1.75, 3.5 go up to the even code) or |x| > t, i.e. >= t + 1
  // (ties at 0.25, 1.25, 2.5, 5 go down to the even code).  A zero scale
  // (every |x| < 0.006) takes the scale 2^100 instead: every boundary lies
  // above every |x|, and the magnitudes are 0.
  const float svb = sc != 0u ? sv : 0x1p100f;
  // (each boundary is kept minus one: "|x| >= t" is "t - 1 - |x| < 0")
  auto bnd = [&](float mid, uint32_t strict) -> uint32_t {
    const uint32_t p = f2u(mid * svb);
    return __builtin_amdgcn_perm(p, p, 0x03020302u) + strict * 0x10001u - 0x10001u;  // high half, twice
  };
  const uint32_t T0 = bnd(0.25f, 1u), T1 = bnd(0.75f, 0u), T2 = bnd(1.25f, 1u), T3 = bnd(1.75f, 0u);
  const uint32_t T4 = bnd(2.5f, 1u), T5 = bnd(3.5f, 0u), T6 = bnd(5.0f, 1u);
  // binary search, with masks G = all ones where |x| reaches the boundary:
  //   level 1: 1.75; level 2: 3.5 or 0.75; level 3: 5, 2.5, 1.25 or 0.25;
  //   magnitude = 4 [G1] + 2 [G2] + [G3].  Codes of elements 2j (low half)
  //   and 2j + 1 (high half): sign << 3 | magnitude.
  // constants as values the compiler cannot see, so that each select stays
  // one v_bfi_b32 and each shift one packed shift
  i16x2 sh15 = {15, 15};
  uint32_t K4 = 0x00040004u, K2 = 0x00020002u, K7 = 0x00070007u;
  asm("" : "+v"(sh15), "+v"(K4), "+v"(K2), "+v"(K7));
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = h[j] & 0x7FFF7FFFu;
    const uint32_t g1 = reach_mask(a, T3, sh15);
    const uint32_t g2 = reach_mask(a, bitsel(g1, T5, T1), sh15);
    const uint32_t g3 = reach_mask(a, bitsel(g2, bitsel(g1, T6, T2), bitsel(g1, T4, T0)), sh15);
    // magnitude bit 2 from G1, bit 1 from G2, bit 0 from G3; bit 3 is the
    // sign: h >> 12 per half is sign << 3 | three exponent bits
    const uint32_t mag = bitsel(K4, g1, bitsel(K2, g2, g3));
    c[j] = bitsel(K7, mag, pk_shr12(h[j]));
  }
  // nibble packing: perm gathers the low bytes of the halves of two pairs,
  // x | x >> 4 puts each odd byte's code in the high nibble below it, and a
  // final perm keeps bytes 0 and 2 of two such words
  auto pack4 = [&](int j0) -> uint32_t {
    const uint32_t x01 = __builtin_amdgcn_perm(c[j0 + 1], c[j0], 0x06040200u);  // c0.b0 c0.b2 c1.b0 c1.b2
    const uint32_t x23 = __builtin_amdgcn_perm(c[j0 + 3], c[j0 + 2], 0x06040200u);
    const uint32_t y01 = x01 | (x01 >> 4), y23 = x23 | (x23 >> 4);
    return __builtin_amdgcn_perm(y23, y01, 0x06040200u);
  };
  return {pack4(0), pack4(4), sc};
}

// Stores one row's group (lanes g = 0..31 of a row, all executing): 8 code
// bytes per lane, and the scale bytes of four neighbouring groups as one
// dword from the first of them.
__device__ __forceinline__ void store_fp4_group(const Fp4Group& q, int g, bool ok, int64_t s,
                                                uint8_t* __restrict__ pool) {
  const uint32_t s1 = __shfl_down(q.sc, 1, 4), s2 = __shfl_down(q.sc, 2, 4), s3 = __shfl_down(q.sc, 3, 4);
  if (ok) {
    const int64_t page = s >> 6, off = s & 63;
    uint8_t* base = pool + page * kPageBytes;
    v2u cw = {q.w0, q.w1};
    __builtin_nontemporal_store(cw, reinterpret_cast<v2u*>(base + off * kEntryCodes + g * 8));
    if ((g & 3) == 0) {
      uint32_t sw = q.sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
      __builtin_nontemporal_store(sw, reinterpret_cast<uint32_t*>(base + kPage * kEntryCodes +
                                                                  off * kEntryScales + g));
    }
  }
}

__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ x,
                                                          int64_t rows,
                                                          const int64_t* __restrict__ slot,
                                                          uint8_t* __restrict__ pool,
                                                          int64_t n_pages) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = gid >> 5;      // row
  const int g = (int)(gid & 31);   // 16-channel group
  const bool live = r < rows;
  uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t s = -1;
  if (live) {
    const v4u* src = reinterpret_cast<const v4u*>(x + r * kD + g * 16);
    v4u a = __builtin_nontemporal_load(src);
    v4u b = __builtin_nontemporal_load(src + 1);
    h[0] = a.x; h[1] = a.y; h[2] = a.z; h[3] = a.w;
    h[4] = b.x; h[5] = b.y; h[6] = b.z; h[7] = b.w;
    s = slot[r];
  }
  const Fp4Group q = fp4_group(h);
  store_fp4_group(q, g, live && s >= 0 && s < n_pages * kPage, s, pool);
}

// ---------------------------------------------------------------------------
// Fused RoPE + cache writes (knowledge note "FP4 main KV": the main KV is
// quantized after RoPE; the indexer keys are E4M3).  The rotary channels and
// angles are the caller's: the last 64 channels of each main-KV row and of
// each indexer key turn in pairs (2i, 2i + 1) by the angle of pair i at the
// row's position, cs[pos][i] = (cos, sin) in binary32.  Each product and
// each sum is its own binary32 operation, the results are rounded to bf16
// (nearest, ties to even), then written as by the FP4 cache write (main KV)
// and as E4M3 nearest-even codes saturating at 448 (indexer keys).
//
// Two rows per wave: lanes 0..31 serve the first row, lanes 32..63 the
// second, and every lane g (0..31 within its half) does the same work:
//  - main-KV group g (16 channels), quantized as by the cache write;
//  - rotary main-KV pair g (channels 448 + 2g, 449 + 2g), loaded once more as
//    one dword (a cache hit) and turned there; groups 28..31 then collect
//    their eight turned pairs from lanes 8 (g - 28) .. 8 (g - 28) + 7 by
//    lane permutes before quantizing;
//  - indexer-key channels 4g .. 4g + 3, turned in place where rotary
//    (g >= 16: pairs 2 (g - 16), + 1), rounded to E4M3 and stored as a dword.
// Spreading the turns and the E4M3 rounding over all lanes, rather than over
// the 8 lanes that hold the rotary main-KV groups and the 16 that hold
// indexer-key groups, is what keeps the vector instruction count per row
// below the time the row's bytes take.  Per row 1,280 B of bf16 and 16 B of
// position and slot are read, 256 B of angles (from HBM once), 416 B written.

// bf16 bit pattern nearest to a finite binary32 value, ties to even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Rotates one pair (x = low half, y = high half of xy, bf16) by (c, s).
__device__ __forceinline__ uint32_t rope_pair(uint32_t xy, float c, float s) {
#pragma clang fp contract(off)
  const float x = u2f(xy << 16), y = u2f(xy & 0xFFFF0000u);
  const float xr = x * c - y * s;
  const float yr = x * s + y * c;
  return bf16_rne_bits(xr) | (bf16_rne_bits(yr) << 16);
}

// E4M3 code of a bf16 value (bit pattern b): sign copied, magnitude nearest
// with ties to even, saturating at 448, without branches.  From 2^-6 up the
// 7-bit bf16 mantissa is rounded to 3 bits on the bit pattern (a carry moves
// into the exponent, as it should), and the exponent is rebased from bias
// 127 to bias 7; below 2^-6 the E4M3 steps are 2^-9 and the code is the
// value times 2^9 rounded to an integer (exact product, rint ties to even).
__device__ __forceinline__ uint32_t e4m3_of_bf16(uint32_t b) {
  const uint32_t m = b & 0x7FFFu;
  const uint32_t nrm = min(((m + 7u + ((m >> 4) & 1u)) >> 4) - (120u << 3), 0x7Eu);
  const uint32_t sub = (uint32_t)__builtin_rintf(u2f(min(m, 121u << 7) << 16) * 512.0f);
  return ((b >> 8) & 0x80u) | (m >= (121u << 7) ? nrm : sub);
}

__global__ __launch_bounds__(256) void rope_write_kernel(
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ kidx, int64_t rows,
    const int64_t* __restrict__ pos, const float* __restrict__ cs, int64_t max_pos,
    const int64_t* __restrict__ slot, uint8_t* __restrict__ kv_pool,
    uint8_t* __restrict__ kidx_pool, int64_t n_pages) {
  const int lane = (int)(threadIdx.x & 63);
  const int half = lane >> 5, g = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * 2;  // the wave's first row (uniform)
  // rows past the end are loaded clamped and not stored: no branch ahead of
  // the loads, so all of them are in flight at once
  const int64_t ra = min(r0, rows - 1), rb = min(r0 + 1, rows - 1);
  const int64_t r = half ? rb : ra;
  const uint16_t* krow = kv + r * kD;
  const v4u* src = reinterpret_cast<const v4u*>(krow + g * 16);
  const v4u a = __builtin_nontemporal_load(src);
  const v4u b = __builtin_nontemporal_load(src + 1);
  const uint32_t kv_pair = *reinterpret_cast<const uint32_t*>(krow + kD - 64 + 2 * g);
  const v2u kk = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(kidx + r * kDI + g * 4));
  const int64_t pa = pos[ra], pb = pos[rb], sa = slot[ra], sb = slot[rb];
  const int64_t p = half ? pb : pa, s = half ? sb : sa;
  // a row that is skipped is turned at position 0 (max_pos > 0), not stored
  const bool ok = (r0 + half < rows) & (p >= 0) & (p < max_pos) & (s >= 0) & (s < n_pages * kPage);
  const float* crow = cs + (ok ? p : 0) * (2 * 32);
  const v2f t1 = *reinterpret_cast<const v2f*>(crow + 2 * g);          // pair g
  const v4f t2 = *reinterpret_cast<const v4f*>(crow + 4 * (g & 15));   // pairs 2 (g & 15), + 1
  const uint32_t kv_turned = rope_pair(kv_pair, t1.x, t1.y);
  const uint32_t k0r = rope_pair(kk.x, t2.x, t2.y), k1r = rope_pair(kk.y, t2.z, t2.w);
  const uint32_t k0 = g >= 16 ? k0r : kk.x, k1 = g >= 16 ? k1r : kk.y;
  uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int from = (half << 5) + ((g & 3) << 3);  // lanes 28..31: pairs 8 (g - 28) ..
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t v = (uint32_t)__shfl((int)kv_turned, from + j, 64);
    h[j] = g >= 28 ? v : h[j];
  }
  store_fp4_group(fp4_group(h), g, ok, s, kv_pool);
  if (ok) {
    const uint32_t w = e4m3_of_bf16(k0 & 0xFFFFu) | (e4m3_of_bf16(k0 >> 16) << 8) |
                       (e4m3_of_bf16(k1 & 0xFFFFu) << 16) | (e4m3_of_bf16(k1 >> 16) << 24);
    uint8_t* dst = kidx_pool + (s >> 6) * (int64_t)(kPage * kDI) + (s & 63) * kDI + g * 4;
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(dst));
  }
}

}  // namespace csa2

extern "C" int csa2_quantize_kv(const uint16_t* kv_bf16, int64_t rows, const int64_t* dst_slot,
                                uint8_t* kv_pool, int64_t n_pages, csa2_stream_t stream) {
  if (rows < 0 || n_pages < 0) return CSA2_ERR_INVALID_ARG;
  if (rows == 0) return CSA2_OK;
  if (!kv_bf16 || !dst_slot || !kv_pool) return CSA2_ERR_INVALID_ARG;
  if (n_pages > ((int64_t)1 << 40) / csa2::kPageBytes) return CSA2_ERR_UNSUPPORTED;
  const int64_t threads = rows * 32;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  CSA2_LAUNCH(CSA2_K_QUANTIZE, csa2::quantize_kv_kernel, dim3((uint32_t)blocks), dim3(256),
              (hipStream_t)stream, kv_bf16, rows, dst_slot, kv_pool, n_pages);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}

extern "C" int csa2_rope_write_caches(const uint16_t* kv_bf16, const uint16_t* kidx_bf16,
                                      int64_t rows, const int64_t* pos, const float* rope_cs,
                                      int64_t max_pos, const int64_t* dst_slot, uint8_t* kv_pool,
                                      uint8_t* kidx_pool, int64_t n_pages, csa2_stream_t stream) {
  if (rows < 0 || n_pages < 0 || max_pos < 0) return CSA2_ERR_INVALID_ARG;
  if (rows == 0) return CSA2_OK;
  if (max_pos == 0) return CSA2_OK;  // every row skipped
  if (!kv_bf16 || !kidx_bf16 || !pos || !rope_cs || !dst_slot || !kv_pool || !kidx_pool)
    return CSA2_ERR_INVALID_ARG;
  if (((uintptr_t)kv_bf16 & 15) || ((uintptr_t)kidx_bf16 & 7) || ((uintptr_t)rope_cs & 15) ||
      ((uintptr_t)kv_pool & 7) || ((uintptr_t)kidx_pool & 3))
    return CSA2_ERR_INVALID_ARG;
  if (n_pages > ((int64_t)1 << 40) / csa2::kPageBytes) return CSA2_ERR_UNSUPPORTED;
  if (max_pos > ((int64_t)1 << 40) / 256) return CSA2_ERR_UNSUPPORTED;
  const int64_t blocks = (rows + 7) / 8;  // two rows per wave, four waves per block
  CSA2_LAUNCH(CSA2_K_ROPE_WRITE, csa2::rope_write_kernel, dim3((uint32_t)blocks), dim3(256),
              (hipStream_t)stream, kv_bf16, kidx_bf16, rows, pos, rope_cs, max_pos, dst_slot,
              kv_pool, kidx_pool, n_pages);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
