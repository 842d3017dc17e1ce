// Selection of the hierarchical sparse indexer: the block pool and the
// top-k entries of each (b, t) row from the scan's scores (knowledge note
// "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
// "Hierarchical Sparse Indexer": keep the blocks with the largest maxima,
// then the top-k entries inside them; "Inside DeepSeek V4.1 Flash", section
// "Hierarchical indexing bounds later searches, not every search").
//
// Order: key descending, list position ascending among equal keys, where a
// key is the order-preserving uint32 image of a score (0 = empty).  The
// selected positions are written in ascending list order.
//
// Fast path: the scan has left, per row and list, segments of candidate
// keys (every key of a workgroup's part at or above a local threshold).  The
// top K of their union is the exact top K of the list when no key left out
// could rank in it: either no segment dropped a key and the union is the
// whole list, or the union's K-th key tau is at or above every dropping
// segment's threshold (each dropped key lies strictly below its segment's
// threshold, hence below tau).  Otherwise the selection falls back to the
// whole lists.
//
// A workgroup is 512 threads, two waves per SIMD.  Each step is a chain of
// dependent instructions over the keys a thread owns (stage writes, radix
// digits, ranks), so halving the keys per thread shortens every step, and
// the second wave on each SIMD fills the first one's latencies; 1,024
// threads measured no faster (the block-wide steps and barriers grow).
// The keys being ranked sit in LDS, thread t owning a contiguous range.
#include <algorithm>

#include "common.h"
#include "fp4.h"
#include "index_common.h"

namespace csa2 {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kDigit = 12;
constexpr int kBins = 1 << kDigit;         // radix digits: 64 bins per lane of one wave
constexpr int kStage = 32768;              // LDS key slots: a whole list of block maxima
constexpr int kPosOff = kStage / 2;        // segment path: candidate positions from here
// Segment path: at most 64 candidates per thread, 16,384 per row and list
// (the ranking's reads then end inside the key half)
constexpr int kSegE = 32;
constexpr int kCandCap = kSegE * kSelThreads;
static_assert(kCandCap <= kPosOff, "key reads inside the key half");
constexpr int kSegFail = CSA2_ROW_UNRANKED;  // the segments cannot give the exact result
constexpr int kSegBad = CSA2_ROW_BAD_SCALE;

struct SelShared {
  uint32_t stage[kStage];
  uint32_t bins[kBins + 64];  // one radix level's histogram, then a spare bin per lane
  int red_n[kSelWaves];
  uint32_t red_max[kSelWaves], red_min[kSelWaves];
  int scan_a[kSelWaves], scan_b[kSelWaves];
  int hdr_sum[kSelWaves], hdr_flags[kSelWaves];
  uint32_t hdr_thr[kSelWaves], hdr_cmax[kSelWaves], hdr_kmax[kSelWaves], hdr_kmin[kSelWaves];
  int misc[4];
  uint32_t gath[kSelWaves][64];  // per wave: keys of a radix level's crossing bin, when few
  int gath_n[kSelWaves];
  uint32_t dummy[64];            // target of the writes a lane does not need (no branch)
  int pool_blk[CSA2_MAX_POOL_BLOCKS];
  int seg_off[kMaxSegs + 1];
};

// Maximum over the 64 lanes (DPP, unsigned; every lane gets it).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = std::max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Exclusive prefix sums of a and b over the workgroup in thread order, and
// their totals.  scan_a / scan_b are written again only after later barriers.
__device__ __forceinline__ void block_excl_scan2(int a, int b, SelShared& sh, int* pa, int* pb, int* ta, int* tb) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int xa = (int)wave_incl_scan((uint32_t)a), xb = (int)wave_incl_scan((uint32_t)b);
  if (lane == 63) {
    sh.scan_a[wave] = xa;
    sh.scan_b[wave] = xb;
  }
  lds_barrier();
  const int wa = (int)wave_incl_scan(lane < kSelWaves ? (uint32_t)sh.scan_a[lane] : 0u);
  const int wb = (int)wave_incl_scan(lane < kSelWaves ? (uint32_t)sh.scan_b[lane] : 0u);
  *pa = (wave > 0 ? __builtin_amdgcn_readlane(wa, wave - 1) : 0) + xa - a;
  *pb = (wave > 0 ? __builtin_amdgcn_readlane(wb, wave - 1) : 0) + xb - b;
  *ta = __builtin_amdgcn_readlane(wa, kSelWaves - 1);
  *tb = __builtin_amdgcn_readlane(wb, kSelWaves - 1);
}

// One wave, histogram h of 4,096 bins (lane l owns bins [4096 - 64(l+1),
// 4096 - 64l), lane 0 has the highest digits).  For the rank x >= 1 (counted
// from the top) returns the bin holding it (-1 if the histogram holds fewer
// than x keys) and writes the count above that bin.
__device__ __forceinline__ int wave_crossing(const uint32_t* h, uint32_t x, uint32_t* above_bin, uint32_t* in_bin,
                                             int lane) {
  const v4u* hv = reinterpret_cast<const v4u*>(h + kBins - 64 * (lane + 1));
  uint32_t sum = 0;
  // lane l reads its 16 quads starting at quad l % 16, so that 16 lanes read
  // 16 different bank groups (the lanes' ranges lie 256 bytes apart)
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const v4u v = hv[(q + lane) & 15];
    sum += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const uint64_t who = __ballot(incl - sum < x && x <= incl);
  if (who == 0) {
    *above_bin = 0;
    *in_bin = 0;
    return -1;
  }
  const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(who));
  const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), src);
  // lane j takes the j-th highest bin of lane src
  const int top_bin = kBins - 64 * src - 1;
  const uint32_t c = h[top_bin - lane];
  const uint32_t ci = wave_incl_scan(c);
  const uint64_t hit = __ballot(above + ci >= x);
  const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  *above_bin = above + (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), j);
  *in_bin = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
  return top_bin - j;
}

// Top K of the keys keys[0 .. n) (LDS, list order, key 0 = empty), order
// (key desc, position asc).  Thread t owns positions E t .. E t + E - 1,
// E = ceil(n / 512) rounded up to 8 (at most EMAX), and reads them into
// registers at once (with PAY, also the payload words pay[E t ..]), so every
// later step works on registers, in chunks of 8 (only the E / 8 chunks in
// use are processed); the reads end below 512 E, which the callers keep
// inside their arrays.
// The K-th largest key tau comes from radix levels over v = key - (smallest
// key), the first over the top 12 bits that vary among the keys; then every
// key above tau and the first keys equal to tau, up to K, are written as
// out[rank] = val(position, payload), rank = place in ascending position
// order: into LDS (out), or with GOUT straight to global memory (gout; the
// stores need no barrier and no copy pass after them).
// The keys may be part of a larger list whose top K is wanted: with more
// than K keys, tau must be at least min_tau; with K or fewer, `complete`
// must hold.  Otherwise nothing is emitted and the result is -1.  Returns
// the number selected.
// What the caller may already know of the keys: their count and extremes.
struct KeyStats {
  bool known;
  int n_valid;
  uint32_t kmin, kmax;
};

template <int EMAX, bool PAY, bool GOUT = false, typename Val>
__device__ __forceinline__ int lds_topk(const uint32_t* keys, const uint32_t* pay, int n, int K, uint32_t min_tau,
                                        bool complete, KeyStats ks, SelShared& sh, uint32_t* out, Val val,
                                        int32_t* gout = nullptr) {
  static_assert(EMAX % 8 == 0, "chunks of 8");
  constexpr int NC = EMAX / 8;
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int E = ((n + kSelThreads - 1) / kSelThreads + 7) & ~7;
  const int nch = E / 8;  // chunks in use (the same for every thread)
  const int i0 = E * tid;
  const int cnt = std::max(0, std::min(E, n - i0));
  uint32_t k[EMAX];
  uint32_t pv[PAY ? EMAX : 1];
  // body(r) for every slot r of the chunks in use
  auto each = [&](auto&& body) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c < nch) {
#pragma unroll
        for (int j = 0; j < 8; ++j) body(8 * c + j);
      }
    }
  };
  // the keys pass through an empty asm at the start of every pass, so that
  // the compiler keeps no per-key value (a digit, a predicate) from one pass
  // to the next
  auto fresh = [&]() {
#pragma unroll
    for (int r = 0; r < EMAX; ++r) asm volatile("" : "+v"(k[r]));
  };
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c < nch) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4u v = *reinterpret_cast<const v4u*>(keys + i0 + 8 * c + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) k[8 * c + 4 * h + e] = v[e];
        if (PAY) {
          const v4u w = *reinterpret_cast<const v4u*>(pay + i0 + 8 * c + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[PAY ? 8 * c + 4 * h + e : 0] = w[e];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) k[8 * c + j] = 0u;
    }
  }
  each([&](int r) { k[r] = r < cnt ? k[r] : 0u; });
  // ---- valid keys, smallest and largest (unless known)
  int n_valid = ks.n_valid;
  uint32_t kmin = ks.kmin, kmax = ks.kmax;
  if (!ks.known) {
    int nv = 0;
    uint32_t lmax = 0u, lmin_inv = 0u;
    each([&](int r) {
      nv += k[r] != 0u ? 1 : 0;
      lmax = std::max(lmax, k[r]);
      lmin_inv = std::max(lmin_inv, k[r] != 0u ? ~k[r] : 0u);
    });
    const int s = wave_sum(nv);
    const uint32_t mx = wave_max_u32(lmax), mn = wave_max_u32(lmin_inv);
    if (lane == 0) {
      sh.red_n[wave] = s;
      sh.red_max[wave] = mx;
      sh.red_min[wave] = mn;
    }
    lds_barrier();
    n_valid = wave_sum(lane < kSelWaves ? sh.red_n[lane] : 0);
    kmax = wave_max_u32(lane < kSelWaves ? sh.red_max[lane] : 0u);
    kmin = ~wave_max_u32(lane < kSelWaves ? sh.red_min[lane] : 0u);
  }
  uint32_t tau = 0u;  // with tau = 0 every valid key is selected
  int need_eq = 0;
  if (n_valid > K) {
    const uint32_t range = kmax - kmin;
    const int nbits = range ? 32 - __builtin_clz(range) : 0;
    int shift = std::max(nbits - kDigit, 0), width = nbits - shift;
    uint32_t prefix = 0u;  // digits found so far, in v = key - kmin
    int rem = K;
    for (;;) {
      fresh();
#pragma unroll
      for (int q = 0; q < kBins / kSelThreads; ++q) sh.bins[tid + q * kSelThreads] = 0u;
      lds_barrier();
      // keys whose digits above this level match the prefix count in their
      // digit's bin, the others in a spare bin of their lane (no branch)
      const int top_shift = shift + width;
      const uint32_t hmask = top_shift >= 32 ? 0u : ~0u << top_shift;
      const uint32_t hval = prefix & hmask;
      const uint32_t dmask = (1u << width) - 1u;
      each([&](int r) {
        const uint32_t d = k[r] - kmin;
        const bool m = k[r] != 0u && (d & hmask) == hval;
        atomicAdd(&sh.bins[m ? (d >> shift) & dmask : (uint32_t)(kBins + lane)], 1u);
      });
      lds_barrier();
      if (threadIdx.x < 64) {
        uint32_t ab, ib;
        const int d = wave_crossing(sh.bins, (uint32_t)rem, &ab, &ib, lane);
        if (lane == 0) {
          sh.misc[0] = d;
          sh.misc[1] = (int)ab;
          sh.misc[3] = (int)ib;
        }
      }
      lds_barrier();
      prefix |= (uint32_t)sh.misc[0] << shift;
      rem -= sh.misc[1];
      if (shift == 0) break;
      if (sh.misc[3] <= 64) {
        // ---- few keys share the crossing bin: one wave ranks them among
        // themselves (the rem-th largest is tau) instead of further levels
        const uint32_t hm = ~0u << shift, hv = prefix & hm;
        fresh();
        uint32_t* gw = sh.gath[wave];
        int wn = 0;  // this wave's keys so far
        each([&](int r) {
          const bool m = k[r] != 0u && ((k[r] - kmin) & hm) == hv;
          const uint64_t bal = __ballot(m);
          const int at = wn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          *(m ? gw + at : sh.dummy + lane) = k[r];
          wn += __builtin_popcountll(bal);
        });
        if (lane == 0) sh.gath_n[wave] = wn;
        lds_barrier();
        if (threadIdx.x < 64) {
          const int c1 = sh.misc[3];
          // lane l takes key l of the waves' lists, in wave order
          uint32_t kl = 0u;
          int base = 0;
#pragma unroll
          for (int w = 0; w < kSelWaves; ++w) {
            const int nw = sh.gath_n[w];
            if (lane >= base && lane < base + nw) kl = sh.gath[w][lane - base];
            base += nw;
          }
          int gt = 0, ge = 0;
          for (int j = 0; j < c1; ++j) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kl, j);
            gt += kj > kl ? 1 : 0;
            ge += kj >= kl ? 1 : 0;
          }
          // the key with gt < rem <= ge (one value; several lanes may hold it)
          const uint64_t hit = __ballot(lane < c1 && gt < rem && rem <= ge);
          const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
          if (lane == l) {
            sh.misc[0] = (int)kl;
            sh.misc[1] = rem - gt;
          }
        }
        lds_barrier();
        prefix = (uint32_t)sh.misc[0] - kmin;
        rem = sh.misc[1];
        break;
      }
      width = std::min(shift, kDigit);
      shift -= width;
    }
    tau = kmin + prefix;
    need_eq = rem;
    if (tau < min_tau) return -1;
  } else if (!complete) {
    return -1;
  }

  // ---- emission: counts, their prefix over the threads, then the keys again
  fresh();
  int ngt = 0, neq = 0;
  each([&](int r) {
    ngt += k[r] > tau ? 1 : 0;
    neq += (k[r] != 0u && k[r] == tau) ? 1 : 0;
  });
  int gt_before, eq_before, gt_tot, eq_tot;
  block_excl_scan2(ngt, neq, sh, &gt_before, &eq_before, &gt_tot, &eq_tot);
  const int got = gt_tot + std::min(eq_tot, need_eq);
  if (ngt + neq > 0) {
    fresh();
    int rank = gt_before + std::min(eq_before, need_eq);
    int eq_seen = eq_before;
    each([&](int r) {
      const bool eq = k[r] != 0u && k[r] == tau;
      const bool take = (k[r] > tau || (eq && eq_seen < need_eq)) && rank < K;
      if (GOUT) {
        if (take) gout[rank] = (int32_t)val(i0 + r, pv[PAY ? r : 0]);
      } else {
        *(take ? out + rank : sh.dummy + lane) = val(i0 + r, pv[PAY ? r : 0]);
      }
      rank += take ? 1 : 0;
      eq_seen += eq ? 1 : 0;
    });
  }
  return std::min(got, K);
}

// Candidates of one (row, list), loaded ahead of the headers that say how
// many there are, for the usual segment count W (segs_guess): thread t
// covers segment t / tps, slots (t % tps) + tps r (r < kSegR), with tps =
// 512 / W threads per segment; thread t also reads header t (t < max_segs)
// and every thread the row's segment count.
constexpr int kSegR = 16;
struct SegCands {
  v2u c[kSegR];
  SegHeader h;    // header t
  SegHeader own;  // header of segment t / tps
  int nseg;       // the row's segments
};

__device__ __forceinline__ void seg_issue(const SelectArgs& a, int64_t bt, int list, SegCands& L) {
  const int tid = (int)threadIdx.x;
  const int W = a.segs_guess, tps = kSelThreads / W;
  const int64_t seg0 = (bt * 2 + list) * a.max_segs;
  // every load is issued, with clamped indices (masked later), so that none
  // waits for another
  L.nseg = a.seg_n[bt];
  const v2u hv = *reinterpret_cast<const v2u*>(a.seg_hdr + seg0 + std::min(tid, a.max_segs - 1));
  L.h = SegHeader{hv[0], hv[1]};
  const int s = std::min(tid / tps, W - 1), j0 = tid % tps;
  // (only the count of the own header is used: a 4-byte load, since a dead
  // half of a wider load's destination could be reused early, and that
  // reuse would wait for the load)
  L.own = SegHeader{reinterpret_cast<const uint32_t*>(a.seg_hdr + seg0 + s)[0], 0u};
  const Cand* base = a.seg_cand + (bt * 2 + list) * a.seg_region + seg_off_at(a.seg_k, s);
  const int cap = seg_cap_at(a.seg_k, s);
#pragma unroll
  for (int r = 0; r < kSegR; ++r) L.c[r] = *reinterpret_cast<const v2u*>(base + std::min(j0 + tps * r, cap - 1));
}

// Top K of a (row, list) from its segments (seg_issue): returns kSegBad when
// a segment reports an out-of-range MXFP4 scale; else, with `use`, the
// number selected (gout[rank] = val(list position), global memory; nothing
// is written otherwise), or kSegFail when the segments cannot give the
// exact top K (or `use` is false).
template <typename Val>
__device__ __forceinline__ int seg_finish(const SelectArgs& a, int64_t bt, int list, int K, bool use,
                                          const SegCands& L, SelShared& sh, int32_t* gout, Val val) {
  const int tid = (int)threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // the row's segments; the early loads are of use when it has the usual count
  const int W = std::max(1, std::min(L.nseg, a.max_segs)), tps = kSelThreads / W;
  const bool early = W == a.segs_guess;
  // ---- headers: offsets, total, flags, the highest threshold of a segment
  // that dropped keys, the largest count (one round through LDS)
  const bool mine = tid < W;
  const int c = mine ? (int)(L.h.count_flags & 0xFFFFFFu) : 0;
  const uint32_t f = mine ? L.h.count_flags >> 24 : 0u;
  const int x = (int)wave_incl_scan((uint32_t)c);
  const uint32_t fw = (__ballot(f & kSegDropped) ? 1u : 0u) | (__ballot(f & kSegOverflow) ? 2u : 0u) |
                      (__ballot(f & kSegBadScale) ? 4u : 0u);
  const uint32_t tw = wave_max_u32((f & kSegDropped) ? L.h.thr : 0u);
  const uint32_t cw = wave_max_u32((uint32_t)c);
  // extremes of the candidates loaded ahead (the slots below their
  // segment's count)
  uint32_t lmax = 0u, lmin_inv = 0u;
  {
    const bool in_seg = early && tid / tps < W;
    const int own_cnt = in_seg ? (int)(L.own.count_flags & 0xFFFFFFu) : 0;
    const int j0 = tid % tps;
#pragma unroll
    for (int r = 0; r < kSegR; ++r) {
      const bool in = j0 + tps * r < own_cnt;
      lmax = std::max(lmax, in ? L.c[r][0] : 0u);
      lmin_inv = std::max(lmin_inv, in ? ~L.c[r][0] : 0u);
    }
  }
  const uint32_t mxw = wave_max_u32(lmax), mnw = wave_max_u32(lmin_inv);
  if (lane == 63) sh.hdr_sum[wave] = x;
  if (lane == 0) {
    sh.hdr_flags[wave] = (int)fw;
    sh.hdr_thr[wave] = tw;
    sh.hdr_cmax[wave] = cw;
    sh.hdr_kmax[wave] = mxw;
    sh.hdr_kmin[wave] = mnw;
  }
  lds_barrier();
  const int wt = (int)wave_incl_scan(lane < kSelWaves ? (uint32_t)sh.hdr_sum[lane] : 0u);
  const int before = wave > 0 ? __builtin_amdgcn_readlane(wt, wave - 1) : 0;
  const int tot = __builtin_amdgcn_readlane(wt, kSelWaves - 1);
  const uint32_t fr = lane < kSelWaves ? (uint32_t)sh.hdr_flags[lane] : 0u;
  const uint32_t fl = (__ballot(fr & 1u) ? 1u : 0u) | (__ballot(fr & 2u) ? 2u : 0u) | (__ballot(fr & 4u) ? 4u : 0u);
  const uint32_t thr_max = wave_max_u32(lane < kSelWaves ? sh.hdr_thr[lane] : 0u);
  const int cmax = (int)wave_max_u32(lane < kSelWaves ? sh.hdr_cmax[lane] : 0u);
  KeyStats ks;
  ks.known = early && cmax <= tps * kSegR;  // every candidate was among the early loads
  ks.n_valid = tot;
  ks.kmax = wave_max_u32(lane < kSelWaves ? sh.hdr_kmax[lane] : 0u);
  ks.kmin = ~wave_max_u32(lane < kSelWaves ? sh.hdr_kmin[lane] : 0u);
  if (mine) sh.seg_off[tid] = before + x - c;
  if (tid == W - 1) sh.seg_off[W] = before + x;
  lds_barrier();
  if (fl & 4u) return kSegBad;
  if (!use || (fl & 2u) || tot > kCandCap) return kSegFail;
  const bool complete = (fl & 1u) == 0u;
  if (tot <= K && !complete) return kSegFail;

  // ---- the candidates in list order into the stage (keys, then positions
  // at kPosOff); slots past the early loads' reach (all of them when the row
  // has an unusual segment count) are loaded here
  {
    const int s = tid / tps, j0 = tid % tps;
    const int off_s = s < W ? sh.seg_off[s] : 0;
    const int cnt_s = s < W ? sh.seg_off[s + 1] - off_s : 0;
    int j_from = j0;
    if (early) {
      const int rmax = (cmax + tps - 1) / tps;  // slots any segment fills (the same for every thread)
#pragma unroll
      for (int r0 = 0; r0 < kSegR; r0 += 8) {
        if (r0 < rmax) {
#pragma unroll
          for (int r = r0; r < r0 + 8; ++r) {
            const int j = j0 + tps * r;
            const bool in = j < cnt_s;
            *(in ? sh.stage + off_s + j : sh.dummy + lane) = L.c[r][0];
            *(in ? sh.stage + kPosOff + off_s + j : sh.dummy + lane) = L.c[r][1];
          }
        }
      }
      j_from = j0 + tps * kSegR;
    }
    if (!early || cmax > tps * kSegR) {
      const int sc = std::min(s, W - 1);
      const Cand* base = a.seg_cand + (bt * 2 + list) * a.seg_region + seg_off_at(a.seg_k, sc);
      const int cap = seg_cap_at(a.seg_k, sc);
      for (int j = j_from; j < cnt_s; j += 4 * tps) {
        v2u c4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c4[u] = *reinterpret_cast<const v2u*>(base + std::min(j + u * tps, cap - 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (j + u * tps < cnt_s) {
            sh.stage[off_s + j + u * tps] = c4[u][0];
            sh.stage[kPosOff + off_s + j + u * tps] = c4[u][1];
          }
        }
      }
    }
  }
  lds_barrier();
  const int got = lds_topk<kSegE, true, true>(sh.stage, sh.stage + kPosOff, tot, K, thr_max, complete, ks, sh,
                                              nullptr, [&](int, uint32_t pos) { return val(pos); }, gout);
  return got < 0 ? kSegFail : got;
}

// The pool of a Full-mode row from the whole list of block maxima: the
// blocks with the P largest maxima, in ascending block order in
// sh.pool_blk (-1 past the count).  Returns the count.
__device__ __forceinline__ int pool_whole(const SelectArgs& a, int row, int nb, SelShared& sh) {
  const int tid = (int)threadIdx.x;
  const int P = a.pool_blocks;
  static_assert(kStage * kBlock >= CSA2_MAX_ENTRIES, "blocks per row");
  for (int i = tid; i < P; i += kSelThreads) sh.pool_blk[i] = -1;
  const float* bm = a.bm + (int64_t)row * bm_stride(a.max_n);
  // reads past the row return zero; blocks >= nb are masked
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)bm, 0, bm_stride(a.max_n) * 4, kBufferFlags);
  const int n4 = (nb + 3) / 4;
  for (int q0 = 0; q0 < n4; q0 += 16 * kSelThreads) {
    v4u raw[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      raw[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(q0 + tid + u * kSelThreads) * 16u, 0, 0);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int p0 = 4 * (q0 + tid + u * kSelThreads);
      if (p0 < nb) {
        v4u k;
#pragma unroll
        for (int e = 0; e < 4; ++e) k[e] = p0 + e < nb ? score_key(__uint_as_float(raw[u][e])) : 0u;
        *reinterpret_cast<v4u*>(&sh.stage[p0]) = k;
      }
    }
  }
  lds_barrier();
  const int n = lds_topk<kStage / kSelThreads, false>(sh.stage, nullptr, nb, P, 0u, true, KeyStats{}, sh,
                                                     reinterpret_cast<uint32_t*>(sh.pool_blk),
                                                     [&](int i, uint32_t) { return (uint32_t)i; });
  lds_barrier();
  return n;
}

// Top-k over the pool's positions (list position p = 8 * slot + e): thread t
// gathers slots t + 512 q with 16-byte loads into the stage.  Full mode:
// the entries of the pool's blocks from the entry scores; Reindex mode: the
// pool-order scores.
template <bool FULL>
__device__ __forceinline__ int pool_topk(const SelectArgs& a, int row, int n, int pool_n, SelShared& sh,
                                         uint32_t* out) {
  const int tid = (int)threadIdx.x;
  const int P = a.pool_blocks;
  const int nb = (n + kBlock - 1) / kBlock;
  static_assert(kStage >= CSA2_MAX_POOL_BLOCKS * kBlock, "pool positions");
  const float* srow = FULL ? a.s + (int64_t)row * s_stride(a.max_n) : a.s + (int64_t)row * P * kBlock;
  const uint32_t row_bytes = FULL ? (uint32_t)s_stride(a.max_n) * 4u : (uint32_t)P * kBlock * 4u;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)srow, 0, row_bytes, kBufferFlags);
  constexpr int kSlots = CSA2_MAX_POOL_BLOCKS / kSelThreads;  // 4
  v4u g[kSlots][2];
  int blk[kSlots];
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int slot = tid + u * kSelThreads;
    blk[u] = slot < pool_n ? sh.pool_blk[slot] : -1;
    const bool ok = blk[u] >= 0 && blk[u] < nb;
    // an offset past the row reads zeros (masked below)
    const uint32_t off = ok ? (uint32_t)(FULL ? blk[u] : slot) * kBlock * 4u : row_bytes;
    g[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    g[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kSlots; ++u) {
    const int slot = tid + u * kSelThreads;
    if (slot < pool_n) {
      const bool ok = blk[u] >= 0 && blk[u] < nb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4u k;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          k[e] = (ok && blk[u] * kBlock + 4 * h + e < n) ? score_key(__uint_as_float(g[u][h][e])) : 0u;
        *reinterpret_cast<v4u*>(&sh.stage[8 * slot + 4 * h]) = k;
      }
    }
  }
  lds_barrier();
  return lds_topk<CSA2_MAX_POOL_BLOCKS * kBlock / kSelThreads, false>(
      sh.stage, nullptr, pool_n * kBlock, a.topk, 0u, true, KeyStats{}, sh, out,
      [&](int p, uint32_t) { return (uint32_t)(sh.pool_blk[p >> 3] * kBlock + (p & 7)); });
}

// FULL: two workgroups per (b, t) row: the even one writes the pool, the odd
// one the top-k, which lies inside the pool since topk <= pool_blocks (each
// block holding a key of the top-k has a maximum that ranks at least as
// high, and fewer than topk blocks rank above it), so it is the top-k of the
// whole list.  Its fallback recomputes the pool.  REINDEX: one workgroup
// per row, top-k over the pool-order scores.
template <bool FULL>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ SelShared sh;
  const int tid = (int)threadIdx.x;
  const int row = FULL ? (int)(blockIdx.x >> 1) : (int)blockIdx.x;  // b * T + t
  const int list = FULL ? 1 - (int)(blockIdx.x & 1) : 0;
  // the row's visible entries: both counts are read unconditionally, first
  // (a load waited for later retires every load issued before it)
  const int b = row / a.T;
  const int ne = a.n_entries[b];
  const int nvis = (a.n_vis != nullptr ? a.n_vis + row : a.n_entries + b)[0];
  // FP4 cache write of wr_n rows (Full mode), 32 threads (16-channel
  // groups) per row, spread over the workgroups: whole rows per wave, so the
  // four lanes of each scale dword are active together.  Nothing the indexer
  // reads is written; the attention that reads these entries runs after this
  // kernel.  When every thread has at most one item (the usual case), its
  // loads go out first and its stores right after the segment loads are
  // issued, where the selection waits for memory anyway.
  const int64_t wr_items = FULL ? a.wr_n * 32 : 0;
  const int64_t wr_stride = (int64_t)gridDim.x * kSelThreads;
  const int64_t wr_t0 = (int64_t)blockIdx.x * kSelThreads + tid;
  const bool wr_one = wr_items <= wr_stride;
  auto write_item = [&](int64_t t, const v4u& x0, const v4u& x1, int64_t s) {
    const uint32_t h[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    store_fp4_group(fp4_group(h), (int)(t & 31), s >= 0 && s < a.wr_pages * kPage, s, a.wr_pool);
  };
  v4u wx0 = {0u, 0u, 0u, 0u}, wx1 = wx0;
  int64_t wslot = -1;
  const bool wr_mine = FULL && wr_one && wr_t0 < wr_items;
  if (wr_mine) {
    const v4u* src = reinterpret_cast<const v4u*>(a.wr_rows + (wr_t0 >> 5) * kD + (wr_t0 & 31) * 16);
    wx0 = src[0];
    wx1 = src[1];
    wslot = a.wr_slots[wr_t0 >> 5];
  }
  SegCands L;
  seg_issue(a, row, list, L);
  if (wr_mine) write_item(wr_t0, wx0, wx1, wslot);

  const int n = std::max(0, std::min(std::min(ne, nvis), std::min(a.max_n, a.max_pages * kPage)));
  const int nb = (n + kBlock - 1) / kBlock;
  const int P = a.pool_blocks;
  // one call site for each path (the paths of the two lists share them)
  const bool pool_list = FULL && list == 1;
  const int K = pool_list ? P : a.topk;
  int32_t* out = a.out_topk + (int64_t)row * a.topk;
  int pool_n = 0;
  if (!FULL) {
    // the pool, for the emission (and the fallback)
    pool_n = std::max(0, std::min(a.pool_n_in[row], P));
    for (int i = tid; i < P; i += kSelThreads) sh.pool_blk[i] = i < pool_n ? a.pool_in[(int64_t)row * P + i] : -1;
  } else if (pool_list) {
    for (int i = tid; i < P; i += kSelThreads) sh.pool_blk[i] = -1;
  }
  // (the LDS writes above are ordered before the emission by the selection's barriers)
  // the segments' selection goes straight to the output (rank order); the
  // whole-list fallback ranks into LDS (the top-k into the stage's first
  // slots, the keys being ranked are in registers by then), then out to
  // memory in one coalesced pass
  uint32_t* topk_buf = sh.stage;
  int32_t* const gout = pool_list ? a.out_pool + (int64_t)row * P : out;
  int got = seg_finish(a, row, list, K, a.mode != 1, L, sh, gout, [&](uint32_t pos) {
    return (FULL || pool_list) ? pos : (uint32_t)(sh.pool_blk[pos >> 3] * kBlock + (pos & 7));
  });
  if (got >= 0) {
    for (int i = got + tid; i < K; i += kSelThreads) gout[i] = -1;
    if (pool_list && tid == 0) a.out_pool_n[row] = got;
  } else {
    if (got == kSegFail && a.mode != 2) {
      // the whole lists (the top-k's fallback recomputes the pool)
      lds_barrier();
      if (FULL) pool_n = pool_whole(a, row, nb, sh);
      got = pool_list ? pool_n : pool_topk<FULL>(a, row, n, pool_n, sh, topk_buf);
    }
    lds_barrier();
    if (pool_list) {
      for (int i = tid; i < P; i += kSelThreads) a.out_pool[(int64_t)row * P + i] = got < 0 ? got : sh.pool_blk[i];
      if (tid == 0) a.out_pool_n[row] = got;
    } else {
      for (int i = tid; i < a.topk; i += kSelThreads) out[i] = i < got ? (int32_t)topk_buf[i] : (got < 0 ? got : -1);
    }
  }
  if (FULL && !wr_one) {
    for (int64_t t = wr_t0; t < wr_items; t += wr_stride) {
      const v4u* src = reinterpret_cast<const v4u*>(a.wr_rows + (t >> 5) * kD + (t & 31) * 16);
      write_item(t, src[0], src[1], a.wr_slots[t >> 5]);
    }
  }
}

int& select_mode() {
  static int mode = 0;
  return mode;
}

}  // namespace csa2

int csa2_launch_select(bool full, const csa2::SelectArgs& se, int rows, hipStream_t stream) {
  if (se.max_segs < 1 || se.max_segs > csa2::kMaxSegs || se.segs_guess < 1 || se.segs_guess > se.max_segs)
    return CSA2_ERR_LAUNCH;
  csa2::SelectArgs args = se;
  args.mode = csa2::select_mode();
  if (full)
    CSA2_LAUNCH(CSA2_K_SELECT_FULL, csa2::select_kernel<true>, dim3(2 * rows), dim3(csa2::kSelThreads), stream,
                args);
  else
    CSA2_LAUNCH(CSA2_K_SELECT_REINDEX, csa2::select_kernel<false>, dim3(rows), dim3(csa2::kSelThreads), stream,
                args);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}
