// FP4 group quantization shared by the cache-write kernels: one thread per
// 16-channel group of a bf16 main-KV row (knowledge note "FP4 main KV":
// E2M1 elements, one E4M3 scale per 16 channels).
//
// The elements are rounded in pairs on packed 16-bit integers: a non-negative
// bf16 bit pattern orders like its value, and every E2M1 decision boundary
// mid * scale (mid in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, scale an E4M3
// value) has at most 7 significant bits, so it is itself a bf16 value and
// "|x| >= boundary" is an exact integer comparison of bit patterns (a strict
// boundary compares against the next pattern up).  Three such comparisons
// per element, a binary search over the 8 magnitudes, give the code.
#pragma once
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

}  // namespace csa2
