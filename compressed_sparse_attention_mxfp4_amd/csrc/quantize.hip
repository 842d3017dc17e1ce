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
// The group quantization itself (fp4.h) is shared with the indexer's fused
// cache write.
#include "common.h"
#include "fp4.h"

namespace csa2 {

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
