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
// each.  Per 32-row sub-chunk a wave dequantizes its channel slice into LDS
// (row-major for Q.K, channel-major for P.V; FP4 and FP8 values are exact in
// fp16), computes partial logits over its channels with f16 MFMA, the four
// partials are summed in fixed order through LDS, and every wave runs the
// same online softmax and accumulates P.V for its channels.  Splits write
// (max, sum, unnormalised output) and a combine kernel merges them.
#include "common.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kRowsPerSplit = 128;
constexpr int kSub = 32;               // rows per sub-chunk
constexpr int kKrStride = 128 + 8;     // halves per row-major row (136 -> 68 dwords)
constexpr int kKtStride = kSub + 4;    // halves per channel-major row (36 -> 18 dwords)

typedef _Float16 half_t;

__device__ __forceinline__ v4f mfma16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// E2M1 magnitude codes 0..7 as the high byte of fp16(256 * value); the low
// byte of every such fp16 is zero, and code 0 (value 0) selects 0x00.
// 256 * {0, .5, 1, 1.5, 2, 3, 4, 6} = {0, 128, 256, 384, 512, 768, 1024, 1536}.
constexpr uint32_t kE2M1HiLo = 0x5E5C5800u;  // bytes for codes 0..3
constexpr uint32_t kE2M1HiHi = 0x66646260u;  // bytes for codes 4..7

// 8 E2M1 nibbles (one dword, channel 2i in the low nibble of byte i) times
// a scale given as fp16(scale / 256) -> 8 fp16 values, exactly.
__device__ __forceinline__ void fp4x8_to_f16(uint32_t x, _Float16 s256, half_t* out) {
  const uint32_t lo_n = x & 0x07070707u;
  const uint32_t hi_n = (x >> 4) & 0x07070707u;
  const uint32_t sgn0 = (x & 0x08080808u) << 4;  // channel 2i sign at bit 7 of byte i
  const uint32_t sgn1 = x & 0x80808080u;         // channel 2i+1 sign at bit 7 of byte i
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // perm selector bytes [0x0C, k, 0x0C, 4+k]: [0, lo_n.byte k, 0, hi_n.byte k]
    const uint32_t pick = 0x000C000Cu | ((uint32_t)k << 8) | ((uint32_t)(4 + k) << 24);
    const uint32_t sel = __builtin_amdgcn_perm(hi_n, lo_n, pick);
    uint32_t h2 = __builtin_amdgcn_perm(kE2M1HiHi, kE2M1HiLo, sel);
    h2 |= __builtin_amdgcn_perm(sgn1, sgn0, pick);
    _Float16 v0 = __builtin_bit_cast(_Float16, (uint16_t)(h2 & 0xFFFFu));
    _Float16 v1 = __builtin_bit_cast(_Float16, (uint16_t)(h2 >> 16));
    out[2 * k] = v0 * s256;
    out[2 * k + 1] = v1 * s256;
  }
}

// fp16 bits of (E4M3 value / 256) for a scale code (sign ignored: scales are >= 0).
__device__ __forceinline__ _Float16 e4m3_div256_f16(uint32_t code) {
  return __builtin_bit_cast(_Float16, (uint16_t)((code & 0x7Fu) << 7));
}

// 4 E4M3 codes -> 4 fp16 values, exactly (fp16 bits of value/256, times 256).
__device__ __forceinline__ void fp8x4_to_f16(uint32_t x, half_t* out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t c = (x >> (8 * k)) & 0xFFu;
    const uint16_t hb = (uint16_t)(((c & 0x7Fu) << 7) | ((c & 0x80u) << 8));
    out[k] = __builtin_bit_cast(_Float16, hb) * (_Float16)256.0f;
  }
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
  int n_splits;
  float* part_o;   // [B*T][H/16][n_splits][16][512]
  float* part_ml;  // [B*T][H/16][n_splits][32]  (m[16] in log2 units, l[16])
};

__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) half_t kr[4][kSub * kKrStride];
  __shared__ __attribute__((aligned(16))) half_t kt[4][128 * kKtStride];
  __shared__ __attribute__((aligned(16))) v4f ssum[4][2][64];

  const int split = blockIdx.x;
  const int ht = blockIdx.y;
  const int bt = blockIdx.z;
  const int b = bt / a.T, t = bt % a.T;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int NHT = a.H >> 4;
  int n = a.n_entries[b];
  n = min(n, a.max_pages * kPage);

  // ---- Q slice as the B operand: head ht*16+col, channels 128*wave + 32*s + 8*g .. +8
  v8h qb[4];
  {
    const uint16_t* qrow = a.q + (((int64_t)bt * a.H) + ht * 16 + col) * kD + 128 * wave + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4u raw = *reinterpret_cast<const v4u*>(qrow + 32 * s);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = u2f(raw[e] << 16), f1 = u2f(raw[e] & 0xFFFF0000u);
        qb[s][2 * e] = (_Float16)f0;
        qb[s][2 * e + 1] = (_Float16)f1;
      }
    }
  }

  const int n_rows = a.topk + kSwa;
  const int row0 = split * kRowsPerSplit;
  const int row1 = min(n_rows, row0 + kRowsPerSplit);
  const int32_t* idx_row = a.topk_idx + (int64_t)bt * a.topk;

  float m_run = -__builtin_inff();  // running max (log2 units) of head `col`
  float l_run = 0.0f;               // running sum of head `col`
  v4f o_acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o_acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  half_t* my_kr = kr[wave];
  half_t* my_kt = kt[wave];

  for (int sub = row0; sub < row1; sub += kSub) {
    // ---- dequantize rows sub .. sub+31, channels 128*wave + 64*hc .. +64
    const int r = lane & 31, hc = lane >> 5;
    const int row = sub + r;
    const int cbase = 128 * wave + 64 * hc;
    half_t vals[64];
    bool valid = false;
    if (row < row1) {
      if (row < a.topk) {
        const int j = idx_row[row];
        if (j >= 0 && j < n) {
          const int64_t pg = phys_page(a.page_table, a.max_pages, a.n_pages, b, j >> 6);
          if (pg >= 0) {
            valid = true;
            const uint8_t* base = a.kv_pool + pg * kPageBytes;
            const uint8_t* cp = base + (j & 63) * kEntryCodes + cbase / 2;
            const v4u c0 = *reinterpret_cast<const v4u*>(cp);
            const v4u c1 = *reinterpret_cast<const v4u*>(cp + 16);
            const uint32_t sc = *reinterpret_cast<const uint32_t*>(
                base + kPage * kEntryCodes + (j & 63) * kEntryScales + cbase / 16);
#pragma unroll
            for (int d = 0; d < 8; ++d) {
              const uint32_t x = d < 4 ? c0[d] : c1[d - 4];
              const _Float16 s256 = e4m3_div256_f16((sc >> (8 * (d >> 1))) & 0xFFu);
              fp4x8_to_f16(x, s256, vals + 8 * d);
            }
          }
        }
      } else {
        valid = true;
        const uint8_t* sp = a.swa + ((int64_t)b * (kSwa - 1 + a.T) + t + (row - a.topk)) * kD + cbase;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const v4u c = *reinterpret_cast<const v4u*>(sp + 16 * d);
#pragma unroll
          for (int e = 0; e < 4; ++e) fp8x4_to_f16(c[e], vals + 16 * d + 4 * e);
        }
      }
    }
    if (!valid) {
#pragma unroll
      for (int i = 0; i < 64; ++i) vals[i] = (_Float16)0.0f;
    }
    const uint64_t vmask_all = __ballot(valid);
    const uint32_t vmask = (uint32_t)vmask_all;  // bit r: row sub+r is present
    // row-major and channel-major copies of this wave's slice
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v8h v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = vals[8 * i + e];
      *reinterpret_cast<v8h*>(&my_kr[r * kKrStride + 64 * hc + 8 * i]) = v;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) my_kt[(64 * hc + i) * kKtStride + r] = vals[i];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();

    // ---- partial logits S^T (32 rows x 16 heads) over this wave's 128 channels
    v4f sacc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      sacc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8h ka = *reinterpret_cast<const v8h*>(&my_kr[(rt * 16 + col) * kKrStride + 32 * s + 8 * g]);
        sacc[rt] = mfma16(ka, qb[s], sacc[rt]);
      }
      ssum[wave][rt][lane] = sacc[rt];
    }
    __syncthreads();
    v4f st[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      st[rt] = ssum[0][rt][lane];
      st[rt] = st[rt] + ssum[1][rt][lane];
      st[rt] = st[rt] + ssum[2][rt][lane];
      st[rt] = st[rt] + ssum[3][rt][lane];
    }
    __syncthreads();

    // ---- online softmax for head `col` over rows 4g+i (+16)
    float lg[8];
    float mx = -__builtin_inff();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = rt * 16 + 4 * g + i;
        const bool ok = (vmask >> rr) & 1u;
        const float v = ok ? st[rt][i] * a.sm_scale_log2 : -__builtin_inff();
        lg[rt * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
    v8h pa;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = (lg[k] == -__builtin_inff()) ? 0.0f : exp2f(lg[k] - m_new);
      psum += p;
      pa[k] = (_Float16)p;
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale output rows (heads 4g+i) by their alpha
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) o_acc[c][i] *= al[i];

    // ---- O (16 heads x 128 channels) += P (16 x 32 rows) . V (32 rows x 128)
    // P's K slice for lane l is rows {4g..4g+3, 16+4g..16+4g+3}; V matches it.
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const half_t* vt = &my_kt[(c * 16 + col) * kKtStride];
      const v4h v0 = *reinterpret_cast<const v4h*>(vt + 4 * g);
      const v4h v1 = *reinterpret_cast<const v4h*>(vt + 16 + 4 * g);
      const v8h vb = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o_acc[c] = mfma16(pa, vb, o_acc[c]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
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

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  int H;
  int n_splits;
  float* out;
  float* out_lse;
};

// One workgroup per (b, t, h): merge the splits' (max, sum, output).
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
  const int h = blockIdx.x % a.H;
  const int bt = blockIdx.x / a.H;
  const int NHT = a.H >> 4, ht = h >> 4, hh = h & 15;
  const int64_t base = ((int64_t)bt * NHT + ht) * a.n_splits;
  float M = -__builtin_inff();
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, a.part_ml[(base + s) * 32 + hh]);
  float L = 0.0f;
  float acc0 = 0.0f, acc1 = 0.0f;
  const int c = threadIdx.x * 2;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = a.part_ml[(base + s) * 32 + hh];
    const float wgt = (ms == -__builtin_inff()) ? 0.0f : exp2f(ms - M);
    L += wgt * a.part_ml[(base + s) * 32 + 16 + hh];
    const float* po = a.part_o + ((base + s) * 16 + hh) * kD;
    acc0 += wgt * po[c];
    acc1 += wgt * po[c + 1];
  }
  const float inv = 1.0f / L;
  float* o = a.out + ((int64_t)bt * a.H + h) * kD;
  o[c] = acc0 * inv;
  o[c + 1] = acc1 * inv;
  if (a.out_lse && threadIdx.x == 0)
    a.out_lse[(int64_t)bt * a.H + h] = (M + log2f(L)) * 0.69314718055994530942f;
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
  const size_t units = (size_t)B * T * (H / 16) * aa.n_splits;
  aa.part_o = reinterpret_cast<float*>(ws);
  aa.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256(units * 16 * csa2::kD * 4));
  CSA2_LAUNCH(CSA2_K_ATTN_SPLIT, csa2::attn_split_kernel, dim3(aa.n_splits, H / 16, B * T),
              dim3(csa2::kAttnThreads), (hipStream_t)stream, aa);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  csa2::CombineArgs ca{};
  ca.part_o = aa.part_o;
  ca.part_ml = aa.part_ml;
  ca.H = H;
  ca.n_splits = aa.n_splits;
  ca.out = out;
  ca.out_lse = out_lse;
  CSA2_LAUNCH(CSA2_K_ATTN_COMBINE, csa2::attn_combine_kernel, dim3(B * T * H), dim3(256),
              (hipStream_t)stream, ca);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
