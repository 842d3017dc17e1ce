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
// Per 16-bit half: all ones where a < t, else zero (a, t below 2^15: the
// sign of the 16-bit difference, spread by an arithmetic shift).
// Written as two packed instructions: the compiler would otherwise turn the
// sign test into a compare and a select per half.
__device__ __forceinline__ uint32_t below_mask(uint32_t a, uint32_t t) {
  uint32_t d, m;
  asm("v_pk_sub_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(t));
  asm("v_pk_ashrrev_i16 %0, %1, %2" : "=v"(m) : "v"(0x000F000Fu), "v"(d));  // shift 15 in both halves
  return m;
}
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
  // decision boundaries as bf16 bit patterns: |x| >= t (ties at 0.75, 1.75,
  // 3.5 go up to the even code) or |x| > t, i.e. >= t + 1 (ties at 0.25,
  // 1.25, 2.5, 5 go down to the even code); a zero scale takes no boundary
  auto bnd = [&](float mid, uint32_t strict) -> uint32_t {
    return sc != 0u ? (f2u(mid * sv) >> 16) + strict : 0x7FFFu;
  };
  const uint32_t t0 = bnd(0.25f, 1u), t1 = bnd(0.75f, 0u), t2 = bnd(1.25f, 1u), t3 = bnd(1.75f, 0u);
  const uint32_t t4 = bnd(2.5f, 1u), t5 = bnd(3.5f, 0u), t6 = bnd(5.0f, 1u);
  // binary search, with masks M = all ones where |x| is below the boundary:
  //   level 1: 1.75; level 2: 3.5 or 0.75; level 3: 5, 2.5, 1.25 or 0.25;
  //   magnitude = 7 - (4 [M1] + 2 [M2] + [M3])
  const uint32_t T3 = t3 * 0x10001u, T1 = t1 * 0x10001u, T5 = t5 * 0x10001u;
  const uint32_t T0 = t0 * 0x10001u, T2 = t2 * 0x10001u, T4 = t4 * 0x10001u, T6 = t6 * 0x10001u;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t a = h[j] & 0x7FFF7FFFu;
    const uint32_t m1 = below_mask(a, T3);
    const uint32_t m2 = below_mask(a, bitsel(m1, T1, T5));
    const uint32_t m3 = below_mask(a, bitsel(m1, bitsel(m2, T0, T2), bitsel(m2, T4, T6)));
    const uint32_t nb = bitsel(0x00040004u, m1, bitsel(0x00020002u, m2, m3)) & 0x00070007u;
    // codes of elements 2j (low half) and 2j + 1: sign << 3 | magnitude
    const uint32_t c = (nb ^ 0x00070007u) | ((h[j] >> 12) & 0x00080008u);
    w[j >> 2] |= ((c | (c >> 12)) & 0xFFu) << (8 * (j & 3));
  }
  const uint32_t w0 = w[0], w1 = w[1];
  // four neighbouring groups' scale bytes -> one dword store
  const uint32_t s1 = __shfl_down(sc, 1, 4), s2 = __shfl_down(sc, 2, 4), s3 = __shfl_down(sc, 3, 4);
  const bool ok = live && s >= 0 && s < n_pages * kPage;
  if (ok) {
    const int64_t page = s >> 6, off = s & 63;
    uint8_t* base = pool + page * kPageBytes;
    v2u cw = {w0, w1};
    __builtin_nontemporal_store(cw, reinterpret_cast<v2u*>(base + off * kEntryCodes + g * 8));
    if ((g & 3) == 0) {
      uint32_t sw = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
      __builtin_nontemporal_store(sw, reinterpret_cast<uint32_t*>(base + kPage * kEntryCodes +
                                                                  off * kEntryScales + g));
    }
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
