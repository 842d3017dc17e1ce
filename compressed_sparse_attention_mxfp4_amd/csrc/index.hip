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
constexpr int kChunk = 32;                // entries folded together per wave
constexpr int kEntriesPerWG = 1024;
constexpr int kMaxRT = 4;                 // row tiles of 16 heads (HI <= 64)
constexpr int kFoldStride = kMaxRT * 16 + 4;

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

struct Limbs {
  v4i lo, mid, top;
  uint32_t top_any;
};

// 16 FP8 codes (one v4u) -> their three limb planes (16 int8 each).
__device__ __forceinline__ void to_limbs(const uint8_t* lut_bytes, uint32_t lane4, v4u codes,
                                         Limbs& out) {
  uint32_t lo[4], mid[4], top[4];
  uint32_t any = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t x = codes[d];
    uint32_t L[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t addr = __builtin_amdgcn_perm(x, lane4, 0x0C0C0000u | ((4u + k) << 8));
      L[k] = *reinterpret_cast<const uint32_t*>(lut_bytes + addr);
    }
    uint32_t t01 = __builtin_amdgcn_perm(L[1], L[0], 0x05010400u);
    uint32_t t23 = __builtin_amdgcn_perm(L[3], L[2], 0x05010400u);
    lo[d] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    mid[d] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    uint32_t u01 = __builtin_amdgcn_perm(L[1], L[0], 0x0C0C0602u);
    uint32_t u23 = __builtin_amdgcn_perm(L[3], L[2], 0x0C0C0602u);
    top[d] = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
    any |= top[d];
  }
  out.lo = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
  out.mid = v4i{(int)mid[0], (int)mid[1], (int)mid[2], (int)mid[3]};
  out.top = v4i{(int)top[0], (int)top[1], (int)top[2], (int)top[3]};
  out.top_any = any;
}

__device__ __forceinline__ v4i mfma8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Sum over 128 channels of |M| for the lane's 32 channels (both K-slices).
__device__ __forceinline__ uint32_t abs_limb_sum(const Limbs& s0, const Limbs& s1) {
  uint32_t acc = 0;
  const v4i* planes[6] = {&s0.lo, &s0.mid, &s0.top, &s1.lo, &s1.mid, &s1.top};
#pragma unroll
  for (int p = 0; p < 6; ++p) {
    const uint32_t w = (p % 3 == 0) ? 1u : (p % 3 == 1) ? 128u : 16384u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t x = (uint32_t)(*planes[p])[d];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int v = (int)(int8_t)((x >> (8 * k)) & 0xFFu);
        acc += (uint32_t)(v < 0 ? -v : v) * w;
      }
    }
  }
  return acc;
}

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
};

// POOL = false: Full scan; blockIdx.y = b, the 8 waves split T tokens x
//               entry slices of this workgroup's 1,024 positions.
// POOL = true : Reindex scan; blockIdx.y = b * T + t, positions are the
//               entries of the pool blocks of (b, t).
template <bool POOL>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 64];
  __shared__ __attribute__((aligned(16))) float fold[kWaves][kChunk * kFoldStride];

  build_lut(lut);
  __syncthreads();
  const uint8_t* lut_bytes = reinterpret_cast<const uint8_t*>(lut);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int g = lane >> 4;   // 16-byte K slice within a 64-deep step
  const int col = lane & 15;

  int b, t, slice, n_slices;
  if (POOL) {
    b = blockIdx.y / a.T;
    t = blockIdx.y % a.T;
    slice = wave;
    n_slices = kWaves;
  } else {
    b = blockIdx.y;
    t = wave % a.T;
    slice = wave / a.T;
    n_slices = kWaves / a.T;
    if (t >= a.T || slice >= n_slices) return;  // idle waves when T does not divide 8
  }
  int n = a.n_entries[b];
  n = min(n, a.max_n);
  n = min(n, a.max_pages * kPage);
  int n_pos;            // positions handled in this row
  const int32_t* pool_row = nullptr;
  if (POOL) {
    pool_row = a.pool + ((int64_t)b * a.T + t) * a.pool_blocks;
    int pn = a.pool_n[(int64_t)b * a.T + t];
    pn = max(0, min(pn, a.pool_blocks));
    n_pos = pn * kBlock;
  } else {
    n_pos = n;
  }
  const int wg_base = blockIdx.x * kEntriesPerWG;
  if (wg_base >= n_pos && !POOL) return;

  const int HI = a.HI;
  const int NRT = (HI + 15) >> 4;

  // ---- query limbs (A operands) and head weights for token t
  Limbs qa[kMaxRT][2];
  float wq[kMaxRT][4];
  uint32_t q_top = 0, q_abs_max = 0;
  const int64_t qrow0 = ((int64_t)b * a.T + t) * HI;
#pragma unroll
  for (int rt = 0; rt < kMaxRT; ++rt) {
    const int h = rt * 16 + col;
    v4u c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
    if (rt < NRT && h < HI) {
      const v4u* src = reinterpret_cast<const v4u*>(a.q_idx + (qrow0 + h) * kDI + 16 * g);
      c0 = src[0];
      c1 = src[4];
    }
    to_limbs(lut_bytes, lane4, c0, qa[rt][0]);
    to_limbs(lut_bytes, lane4, c1, qa[rt][1]);
    q_top |= qa[rt][0].top_any | qa[rt][1].top_any;
    uint32_t s = abs_limb_sum(qa[rt][0], qa[rt][1]);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    q_abs_max = max(q_abs_max, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = rt * 16 + 4 * g + i;
      // w * 2^-18 is exact for 2^-100 <= |w| (and w = 0), see csa2.h
      wq[rt][i] = (rt < NRT && hh < HI) ? a.w[qrow0 + hh] * 0x1p-18f : 0.0f;
    }
  }
  // q_abs_max = sum_c |Mq| of the lane's head; the fast path needs the
  // wave maximum below 2^17 so that sum_c |Mq||Mk| < 2^17 * 2^14 = 2^31.
  uint32_t qmax = q_abs_max;
  for (int o = 1; o < 64; o <<= 1) qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, o));
  const bool fast_q = (__ballot(q_top != 0) == 0) && (qmax < (1u << 17));

  float* my_fold = fold[wave];
  float* out_s_row = a.out_s + ((int64_t)b * a.T + t) * (POOL ? (int64_t)a.pool_blocks * kBlock
                                                                 : (int64_t)a.max_n);
  const int n_chunks = (min(kEntriesPerWG, max(0, n_pos - wg_base)) + kChunk - 1) / kChunk;
  for (int ch = slice; ch < n_chunks; ch += n_slices) {
    const int chunk_base = wg_base + ch * kChunk;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int p = chunk_base + st * 16 + col;   // position index in this row's list
      int j = -1;
      if (p < n_pos) {
        if (POOL) {
          const int blk = pool_row[p >> 3];
          const bool blk_ok = blk >= 0 && blk < (n + kBlock - 1) / kBlock;
          const int jj = blk_ok ? blk * kBlock + (p & 7) : n;
          j = jj < n ? jj : -1;
        } else {
          j = p;
        }
      }
      v4u k0 = {0, 0, 0, 0}, k1 = {0, 0, 0, 0};
      if (j >= 0) {
        const int64_t pg = phys_page(a.page_table, a.max_pages, a.n_pages, b, j >> 6);
        if (pg >= 0) {
          const v4u* src =
              reinterpret_cast<const v4u*>(a.kidx + pg * (kPage * kDI) + (j & 63) * kDI + 16 * g);
          k0 = src[0];
          k1 = src[4];
        }
      }
      Limbs kb0, kb1;
      to_limbs(lut_bytes, lane4, k0, kb0);
      to_limbs(lut_bytes, lane4, k1, kb1);
      const bool fast = fast_q && (__ballot((kb0.top_any | kb1.top_any) != 0) == 0);
#pragma unroll
      for (int rt = 0; rt < kMaxRT; ++rt) {
        if (rt >= NRT) break;
        float r4[4];
        if (fast) {
          v4i z = {0, 0, 0, 0};
          v4i a0 = mfma8(qa[rt][0].lo, kb0.lo, z);
          a0 = mfma8(qa[rt][1].lo, kb1.lo, a0);
          v4i a1 = mfma8(qa[rt][0].lo, kb0.mid, z);
          a1 = mfma8(qa[rt][0].mid, kb0.lo, a1);
          a1 = mfma8(qa[rt][1].lo, kb1.mid, a1);
          a1 = mfma8(qa[rt][1].mid, kb1.lo, a1);
          v4i a2 = mfma8(qa[rt][0].mid, kb0.mid, z);
          a2 = mfma8(qa[rt][1].mid, kb1.mid, a2);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // |each weighted term| <= sum |Mq||Mk| < 2^31: exact in wrapping int32
            uint32_t D = (uint32_t)a0[i] + ((uint32_t)a1[i] << 7) + ((uint32_t)a2[i] << 14);
            r4[i] = (float)(int32_t)D;
          }
        } else {
          v4i z = {0, 0, 0, 0};
          v4i acc[5] = {z, z, z, z, z};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const Limbs& Q = qa[rt][s];
            const Limbs& K = s ? kb1 : kb0;
            acc[0] = mfma8(Q.lo, K.lo, acc[0]);
            acc[1] = mfma8(Q.lo, K.mid, acc[1]);
            acc[1] = mfma8(Q.mid, K.lo, acc[1]);
            acc[2] = mfma8(Q.lo, K.top, acc[2]);
            acc[2] = mfma8(Q.mid, K.mid, acc[2]);
            acc[2] = mfma8(Q.top, K.lo, acc[2]);
            acc[3] = mfma8(Q.mid, K.top, acc[3]);
            acc[3] = mfma8(Q.top, K.mid, acc[3]);
            acc[4] = mfma8(Q.top, K.top, acc[4]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // each term and the sum are integers below 2^53: exact, one rounding below
            double D = (double)acc[0][i] + (double)acc[1][i] * 128.0 +
                       (double)acc[2][i] * 16384.0 + (double)acc[3][i] * 2097152.0 +
                       (double)acc[4][i] * 268435456.0;
            r4[i] = (float)D;
          }
        }
        v4f pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = r4[i] > 0.0f ? r4[i] : 0.0f;
          pv[i] = wq[rt][i] * r;
        }
        *reinterpret_cast<v4f*>(&my_fold[(st * 16 + col) * kFoldStride + rt * 16 + 4 * g]) = pv;
      }
    }
    // the fold reads what other lanes of this wave wrote
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // ---- sequential head fold: lane e < 32 folds entry e of this chunk
    float s = 0.0f;
    if (lane < kChunk) {
      const float* row = &my_fold[lane * kFoldStride];
      for (int h = 0; h < HI; h += 4) {
        const v4f v = *reinterpret_cast<const v4f*>(row + h);
        s = s + v[0];
        if (h + 1 < HI) s = s + v[1];
        if (h + 2 < HI) s = s + v[2];
        if (h + 3 < HI) s = s + v[3];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // positions whose page is unusable are not visible: NaN marker (key 0)
    const int p = chunk_base + lane;
    bool valid = false;
    if (lane < kChunk && p < n_pos) {
      int jj = p;
      if (POOL) {
        const int blk = pool_row[p >> 3];
        jj = (blk >= 0 && blk < (n + kBlock - 1) / kBlock) ? blk * kBlock + (p & 7) : n;
      }
      valid = jj < n && phys_page(a.page_table, a.max_pages, a.n_pages, b, jj >> 6) >= 0;
      out_s_row[p] = valid ? s : u2f(0xFFFFFFFFu);
    }
    if (!POOL) {
      // block maxima over the visible entries of blocks of 8
      float m = valid ? s : -__builtin_inff();
      m = fmaxf(m, __shfl_xor(m, 1));
      m = fmaxf(m, __shfl_xor(m, 2));
      m = fmaxf(m, __shfl_xor(m, 4));
      if (lane < kChunk && (lane & 7) == 0 && p < n_pos) {
        const int nb_row = (a.max_n + kBlock - 1) / kBlock;
        a.out_bm[((int64_t)b * a.T + t) * nb_row + (p >> 3)] =
            (m == -__builtin_inff()) ? u2f(0xFFFFFFFFu) : m;
      }
    }
  }
}

// ---------------------------------------------------------------- selection
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct SelShared {
  uint32_t hist[8][256];
  int wave_tot[kSelWaves];
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
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    int wt = sh.wave_tot[i];
    if (i < wave) before += wt;
    tot += wt;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Top-K selection among keys held KPT per thread (thread i owns list
// positions [i*KPT, i*KPT + KPT)), order (key desc, position asc); key 0
// marks an empty slot.  Writes, in ascending position order, out(rank, pos)
// for every selected position.  Returns the number selected.
template <int KPT, typename Emit>
__device__ int block_topk(const uint32_t (&key)[KPT], int K, SelShared& sh, Emit emit) {
  const int lane = lane_id();
  int valid = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) valid += key[r] != 0;
  int n_valid;
  (void)block_excl_scan(valid, sh, &n_valid);
  uint32_t tau = 1;      // select all valid keys (key >= 1)
  int need_eq = 0x7FFFFFFF;
  if (n_valid > K) {
    uint32_t prefix = 0, mask = 0;
    int rem = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 8 * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const uint32_t k = key[r];
        if (k != 0 && (k & mask) == prefix) atomicAdd(&sh.hist[lane & 7][(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        // lane l owns bins 255-4l .. 252-4l (descending)
        uint32_t c[4];
        uint32_t sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bin = 255 - 4 * lane - q;
          uint32_t v = 0;
#pragma unroll
          for (int cp = 0; cp < 8; ++cp) v += sh.hist[cp][bin];
          c[q] = v;
          sum += v;
        }
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        uint32_t above = incl - sum;   // count in bins above this lane's bins
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above < (uint32_t)rem && (uint32_t)rem <= above + c[q]) {
            sh.misc[0] = 255 - 4 * lane - q;
            sh.misc[1] = (int)above;
          }
          above += c[q];
        }
      }
      __syncthreads();
      const uint32_t d = (uint32_t)sh.misc[0];
      rem -= sh.misc[1];
      prefix |= d << shift;
      mask |= 255u << shift;
      __syncthreads();
    }
    tau = prefix;
    need_eq = rem;
  }
  // compaction in position order
  int gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    gt += key[r] != 0 && key[r] > tau;
    eq += key[r] != 0 && key[r] == tau;
  }
  int eq_tot;
  const int eq_before = block_excl_scan(eq, sh, &eq_tot);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  int sel_tot;
  int off = block_excl_scan(gt + take_eq, sh, &sel_tot);
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
    const int nb_row = (a.max_n + kBlock - 1) / kBlock;
    const float* bm = a.bm + (int64_t)row * nb_row;
    constexpr int KPT = 32;  // 32,768 blocks = 262,144 entries
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int blk = threadIdx.x * KPT + r;
      key[r] = blk < nb ? score_key(bm[blk]) : 0u;
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
  const float* srow = FULL ? a.s + (int64_t)row * a.max_n : a.s + (int64_t)row * P * kBlock;
#pragma unroll
  for (int r = 0; r < KPT2; ++r) {
    const int p = threadIdx.x * KPT2 + r;
    const int slot = p >> 3;
    uint32_t k = 0;
    if (slot < pool_n) {
      const int blk = sh.pool_blk[slot];
      if (blk >= 0 && blk < (n + kBlock - 1) / kBlock) {
        const int j = blk * kBlock + (p & 7);
        if (j < n) k = FULL ? score_key(srow[j]) : score_key(srow[p]);
      }
    }
    key2[r] = k;
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
    const size_t nb = ((size_t)max_n + 7) / 8;
    return align256((size_t)B * T * max_n * 4) + align256((size_t)B * T * nb * 4);
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
                                       align256((size_t)B * T * max_n_entries * 4));
  const int gx = (max_n_entries + csa2::kEntriesPerWG - 1) / csa2::kEntriesPerWG;
  CSA2_LAUNCH(CSA2_K_SCORE_FULL, csa2::score_kernel<false>, dim3(gx, B), dim3(csa2::kScoreThreads),
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
  const int gx = (pool_blocks * csa2::kBlock + csa2::kEntriesPerWG - 1) / csa2::kEntriesPerWG;
  CSA2_LAUNCH(CSA2_K_SCORE_REINDEX, csa2::score_kernel<true>, dim3(gx, B * T),
              dim3(csa2::kScoreThreads), (hipStream_t)stream, sa);
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
