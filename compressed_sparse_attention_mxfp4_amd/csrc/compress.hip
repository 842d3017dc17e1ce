// Non-overlapping sequence compressor ("Inside DeepSeek V4.1 Flash", deep
// dive "Causal Encoder-Decoder", its symbol table and equation 1; the
// section on CSA2 simplifying sequence compression).  Every m consecutive
// source positions of C (main KV per position) form one entry, weighted by
// the positions' compression weights Z: per channel, a softmax over the m
// positions of Z, applied to C elementwise, with no positional term.
//
// One wave per entry, eight channels per lane (a 16-byte load of C and of Z
// per position): the m positions' loads are issued together, then per
// channel the maximum of Z, the weights exp(Z - max) by v_exp_f32 on a base-2
// argument, their sum and the weighted sum of C (fused multiply-add), all in
// binary32, and the quotient rounded to bf16 (nearest, ties to even).  Per
// entry 2 m KiB read and 1 KiB written: bound by HBM.
#include "common.h"

namespace csa2 {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int M>
__global__ __launch_bounds__(256) void compress_kernel(const uint16_t* __restrict__ c,
                                                       const uint16_t* __restrict__ z,
                                                       int64_t groups, uint16_t* __restrict__ out) {
  const int64_t gi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // entry (one per wave)
  if (gi >= groups) return;                                         // whole waves
  const int lane = (int)(threadIdx.x & 63);
  const int64_t base = gi * M * kD + lane * 8;
  v4u cv[M], zv[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    cv[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(c + base + (int64_t)i * kD));
    zv[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(z + base + (int64_t)i * kD));
  }
  float zf[M][8], cf[M][8];
#pragma unroll
  for (int i = 0; i < M; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      zf[i][2 * q] = bf16_lo(zv[i][q]);
      zf[i][2 * q + 1] = bf16_hi(zv[i][q]);
      cf[i][2 * q] = bf16_lo(cv[i][q]);
      cf[i][2 * q + 1] = bf16_hi(cv[i][q]);
    }
  }
  constexpr float kLog2e = 1.4426950408889634f;
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t half[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = 2 * q + k;
      float mx = zf[0][j];
#pragma unroll
      for (int i = 1; i < M; ++i) mx = fmaxf(mx, zf[i][j]);
      float s = 0.f, acc = 0.f;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const float e = __builtin_amdgcn_exp2f((zf[i][j] - mx) * kLog2e);
        s += e;
        acc = __builtin_fmaf(e, cf[i][j], acc);
      }
      half[k] = bf16_bits_rne(__fdiv_rn(acc, s));
    }
    o[q] = half[0] | (half[1] << 16);
  }
  __builtin_nontemporal_store((v4u){o[0], o[1], o[2], o[3]},
                              reinterpret_cast<v4u*>(out + gi * kD + lane * 8));
}

}  // namespace csa2

extern "C" int csa2_compress(const uint16_t* c_bf16, const uint16_t* z_bf16, int64_t rows,
                             int32_t m, uint16_t* out_bf16, csa2_stream_t stream) {
  if (rows < 0 || m <= 0) return CSA2_ERR_INVALID_ARG;
  if (m != 1 && m != 2 && m != 4 && m != 8) return CSA2_ERR_UNSUPPORTED;
  const int64_t groups = rows / m;  // a trailing partial group forms no entry
  if (groups == 0) return CSA2_OK;
  if (!c_bf16 || !z_bf16 || !out_bf16) return CSA2_ERR_INVALID_ARG;
  if (((uintptr_t)c_bf16 & 15) || ((uintptr_t)z_bf16 & 15) || ((uintptr_t)out_bf16 & 15))
    return CSA2_ERR_INVALID_ARG;
  const int64_t blocks = (groups + 3) / 4;  // one entry per wave, four waves per block
  if (blocks > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  const dim3 grid((uint32_t)blocks), block(256);
  const hipStream_t st = (hipStream_t)stream;
  switch (m) {
    case 1: CSA2_LAUNCH(CSA2_K_COMPRESS, csa2::compress_kernel<1>, grid, block, st, c_bf16, z_bf16, groups, out_bf16); break;
    case 2: CSA2_LAUNCH(CSA2_K_COMPRESS, csa2::compress_kernel<2>, grid, block, st, c_bf16, z_bf16, groups, out_bf16); break;
    case 4: CSA2_LAUNCH(CSA2_K_COMPRESS, csa2::compress_kernel<4>, grid, block, st, c_bf16, z_bf16, groups, out_bf16); break;
    default: CSA2_LAUNCH(CSA2_K_COMPRESS, csa2::compress_kernel<8>, grid, block, st, c_bf16, z_bf16, groups, out_bf16); break;
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
