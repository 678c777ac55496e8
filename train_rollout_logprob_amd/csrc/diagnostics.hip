// Drift diagnostics over the active rows ("WS2 Cross-Config Logprob Drift Contract",
// Diagnostics table): ratio0, clipfrac0, approx_kl0, mean |dlogp|, and p95/p99/max
// |dlogp| as exact nearest-rank order statistics (the ceil(q*n)-th smallest value).
//
// Two launches:
//   diag_tile      one block per tile of kDiagTile rows (G tiles): fp64 sums of |d|,
//                  exp(d), expm1(d) - d and d in a fixed order, the active / clipped /
//                  non-finite counts and the largest key with its first row, written as
//                  one partial per tile;
//   diag_select    one block of kSelThreads: folds the tile partials in a fixed order (lane
//                  j of wave 0 takes tiles j, j + 64, ... in ascending order, then the 64
//                  lane results by the lane butterfly) into the statistics, derives the
//                  nearest ranks and runs the three-digit radix select over all keys with
//                  LDS histograms, one per quantile; the first 16 keys of each thread are
//                  read once into registers (the later digits count only those whose first
//                  digit matches), any further keys are re-read per digit (they stay in L2).
// diag_segments (drift_segment_diagnostics) computes the same statistics per segment of
// rows (per sequence, per batch row or per rank) in one launch, one block per segment.
// Every statistics record also carries mismatch_kl = -mean(d), the k1 estimator of
// KL(rollout || train) ("Attention Debug Matrix", Metrics); approx_kl0 is its k3 form.
// Keys are the IEEE bit patterns of |d| (fabs clears the sign bit), whose unsigned order
// is the order of the values, so the selection is an MSB-first radix select with digits
// of 11, 11 and 10 bits. Counts and digit choices are integer work whose result does not
// depend on scheduling; the sums are fp64 in an order that depends only on N.
#include <math.h>

#include <atomic>
#include <mutex>

#include "common.h"

namespace drift {
namespace {

constexpr int kDiagThreads = 256;
constexpr int kRowsPerThread = 4;
constexpr int kDiagTile = kDiagThreads * kRowsPerThread;
constexpr int kBins = 2048;
constexpr int kNumQ = 2;                         // p95, p99
constexpr int kQNum[kNumQ] = {95, 99};
constexpr int kShift[3] = {21, 10, 0};
constexpr int kBitsOf[3] = {11, 11, 10};

struct TilePartial {
  double s_abs, s_exp, s_kl, s_d;
  long long n, lo, hi, nonfinite;
  unsigned long long best;  // (key << 32) | (0xffffffff - row): max = largest key, first row
  long long pad[7];
};
static_assert(sizeof(TilePartial) == 128, "partial size");

constexpr int kSelThreads = 1024;                // the selection block

struct SelState {
  drift_stats stats;                // the result copied to the host
};
static_assert(sizeof(SelState) <= 512, "state size");

// Batches above this many rows select the order statistics with one multi-block launch per
// digit (integer histograms in the workspace) instead of re-reading every row three times
// in one block.
constexpr int64_t kSelSingleMax = 65536;
constexpr int kPassThreads = 256;
constexpr int kPassRowsPerBlock = 8192;

constexpr size_t up256(size_t x) { return (x + 255) / 256 * 256; }

struct DiagLayout {
  size_t partial_off = 0, hist_off = 0, total = 0;
  int G = 0;
  __host__ __device__ static constexpr DiagLayout make(int64_t N) {
    DiagLayout l;
    l.G = (int)((N + kDiagTile - 1) / kDiagTile);
    l.partial_off = 512;
    l.hist_off = l.partial_off + up256((size_t)(l.G > 0 ? l.G : 1) * sizeof(TilePartial));
    // digit histograms: [3 digits][2 quantiles][kBins] u32 (the first digit uses quantile 0)
    l.total = l.hist_off + (N > kSelSingleMax ? up256(3 * kNumQ * kBins * 4) : 0);
    return l;
  }
};

// Scratch of drift_diagnostics_noalloc: the workspace of its largest batch
// (DRIFT_NOALLOC_MAX_ROWS rows: state, tile partials, digit histograms), one copy per GPU,
// held until the process ends. Host code uses the per-device address from
// diag_noalloc_scratch, never this name.
constexpr size_t kNoAllocScratchBytes = DiagLayout::make(DRIFT_NOALLOC_MAX_ROWS).total;
static_assert(kNoAllocScratchBytes < (size_t{1} << 20), "modest scratch");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__device__ __forceinline__ unsigned int key_of(float d) { return __float_as_uint(fabsf(d)); }
constexpr unsigned int kNoKey = 0xffffffffu;  // no row (keys have bit 31 clear)

template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ unsigned long long wave_max(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Wave 0 of the block: for each quantile q, finds in histogram h[q] (kBins counts in LDS;
// bins past the digit's range are zero) the bin holding the 1-based rank s_rank[q], i.e.
// the digit d with below < rank <= below + h[q][d], where below counts the keys in bins
// before d; appends d to s_prefix[q] at bit `shift` and leaves rank - below in s_rank[q].
// Two levels: lane l sums bins [32 l, 32 l + 32) and a wave scan of the sums finds the
// block of 32 bins holding the rank; then lanes 0-31 take one bin each of that block and
// a second wave scan finds the bin. Counts are 32-bit (a total never exceeds the number
// of rows, below 2^31). The caller separates this from the histogram writes and from the
// next reads of s_prefix / s_rank with block barriers.
// Inclusive prefix sum over the 64 lanes of a fully active wave: Hillis-Steele steps of
// 1, 2, 4 and 8 lanes inside each row of 16 lanes (DPP row_shr; a lane with no source lane
// adds 0), then each row adds the totals of the rows before it (lanes 15, 31, 47, read as
// wave-uniform values). All ALU and no LDS round trip.
template <int kCtrl>
__device__ __forceinline__ unsigned int row_shr_or_zero(unsigned int v) {
  return (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xf, 0xf, false);
}
__device__ __forceinline__ unsigned int wave_incl_scan(unsigned int v, int lane) {
  v += row_shr_or_zero<0x111>(v);  // row_shr:1
  v += row_shr_or_zero<0x112>(v);  // row_shr:2
  v += row_shr_or_zero<0x114>(v);  // row_shr:4
  v += row_shr_or_zero<0x118>(v);  // row_shr:8
  const unsigned int t0 = (unsigned int)__builtin_amdgcn_readlane((int)v, 15);
  const unsigned int t1 = (unsigned int)__builtin_amdgcn_readlane((int)v, 31);
  const unsigned int t2 = (unsigned int)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? t0 : 0u) + (row > 1 ? t1 : 0u) + (row > 2 ? t2 : 0u);
}

__device__ void pick_digits(const unsigned int* h0, const unsigned int* h1, int shift,
                            long long* s_rank, unsigned int* s_prefix) {
  constexpr int PER = kBins / 64;
  const int lane = threadIdx.x;
  if (lane >= 64) return;
  const unsigned int* h[kNumQ] = {h0, h1};
  unsigned int mine[kNumQ], inc[kNumQ];
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) {
    unsigned int m = 0;
    // rotated order: at step j the 32 lanes of a half-wave read 32 distinct banks
#pragma unroll
    for (int j = 0; j < PER; ++j) m += h[q][lane * PER + ((j + lane) & (PER - 1))];
    mine[q] = m;
  }
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) inc[q] = wave_incl_scan(mine[q], lane);
  unsigned int rank[kNumQ], blk[kNumQ], cnt[kNumQ], inc2[kNumQ];
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) {
    const unsigned int rk = (unsigned int)s_rank[q];  // 1 <= rank <= total < 2^31
    const unsigned int ex = inc[q] - mine[q];
    const unsigned long long own = __ballot(ex < rk && rk <= inc[q]);  // exactly one lane
    blk[q] = own ? (unsigned int)(__ffsll((long long)own) - 1) : 0u;
    rank[q] = rk - (unsigned int)__builtin_amdgcn_readlane((int)ex, (int)blk[q]);
    cnt[q] = lane < PER ? h[q][blk[q] * PER + lane] : 0u;
  }
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) inc2[q] = wave_incl_scan(cnt[q], lane);
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) {
    const unsigned int ex = inc2[q] - cnt[q];
    if (ex < rank[q] && rank[q] <= inc2[q]) {  // exactly one lane below PER
      s_prefix[q] |= (blk[q] * PER + (unsigned int)lane) << shift;
      s_rank[q] = (long long)(rank[q] - ex);
    }
  }
}

// Running statistics of a set of active rows. Thread partials are combined by
// block_reduce in a fixed order (lane butterfly, then waves in index order), tile partials
// in tile order.
struct RowStats {
  double s_abs, s_exp, s_kl, s_d;
  long long n, lo, hi, nf;
  unsigned long long best;  // (key << 32) | (0xffffffff - row): max = largest key, first row
};

__device__ __forceinline__ void add_row(RowStats& a, float df, int64_t r, double lo_edge,
                                        double hi_edge) {
  const double v = (double)df;
  const double e = exp(v);
  ++a.n;
  a.s_abs += fabs(v);
  a.s_exp += e;
  a.s_kl += expm1(v) - v;
  a.s_d += v;
  // lo_edge <= hi_edge, so at most one of the two holds (NaN: neither); counted without a
  // branch, which keeps both counters in registers
  a.lo += e < lo_edge ? 1 : 0;
  a.hi += e > hi_edge ? 1 : 0;
  if (!isfinite(df)) ++a.nf;
  const unsigned long long cand = ((unsigned long long)key_of(df) << 32) |
                                  (unsigned long long)(0xffffffffu - (unsigned int)r);
  a.best = cand > a.best ? cand : a.best;
}

__device__ __forceinline__ void add_stats(RowStats& a, const RowStats& b) {
  a.s_abs += b.s_abs;
  a.s_exp += b.s_exp;
  a.s_kl += b.s_kl;
  a.s_d += b.s_d;
  a.n += b.n;
  a.lo += b.lo;
  a.hi += b.hi;
  a.nf += b.nf;
  a.best = b.best > a.best ? b.best : a.best;
}

// Lane butterfly (xor 32, 16, ..., 1) over a fully active wave; every lane ends with the
// total, the fp64 sums in an order fixed by the lane count.
__device__ __forceinline__ RowStats wave_reduce(RowStats a) {
  a.s_abs = wave_sum(a.s_abs);
  a.s_exp = wave_sum(a.s_exp);
  a.s_kl = wave_sum(a.s_kl);
  a.s_d = wave_sum(a.s_d);
  a.n = wave_sum(a.n);
  a.lo = wave_sum(a.lo);
  a.hi = wave_sum(a.hi);
  a.nf = wave_sum(a.nf);
  a.best = wave_max(a.best);
  return a;
}

// Block-cooperative; the total is returned in thread 0.
__device__ RowStats block_reduce(RowStats a) {
  __shared__ RowStats s_w[kDiagThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  a = wave_reduce(a);
  if (lane == 0) s_w[wave] = a;
  __syncthreads();
  RowStats t = {};
  if (tid == 0)
    for (int w = 0; w < kDiagThreads / 64; ++w) add_stats(t, s_w[w]);
  __syncthreads();
  return t;
}

// Fills everything but the percentiles; `lp` (nullable) is a logprob workspace header
// whose status outranks the diagnostics status.
__device__ void finish_stats(drift_stats& s, const RowStats& a, const WsHeader* lp) {
  s.n_active = a.n;
  s.n_clip_low = a.lo;
  s.n_clip_high = a.hi;
  s.n_nonfinite = a.nf;
  if (a.n == 0) {
    s.argmax_row = -1;
    s.ratio0 = s.clipfrac0 = s.approx_kl0 = s.mean_abs_dlogp = s.mean_dlogp = NAN;
    s.mismatch_kl = NAN;
    s.p95_abs_dlogp = s.p99_abs_dlogp = s.max_abs_dlogp = NAN;
    s.status = DRIFT_ENOACTIVE;
  } else {
    const double dn = (double)a.n;
    s.ratio0 = a.s_exp / dn;
    s.approx_kl0 = a.s_kl / dn;
    s.clipfrac0 = (double)(a.lo + a.hi) / dn;
    s.mean_abs_dlogp = a.s_abs / dn;
    s.mean_dlogp = a.s_d / dn;
    s.mismatch_kl = -s.mean_dlogp;  // k1: mean of log pi_rollout - log pi_train
    s.max_abs_dlogp = __uint_as_float((unsigned int)(a.best >> 32));
    s.argmax_row = (long long)(0xffffffffu - (unsigned int)(a.best & 0xffffffffull));
    s.status = a.nf ? DRIFT_ENONFINITE : DRIFT_OK;
  }
  if (lp) {
    const int lst = header_status(lp->magic, lp->err_bits);
    if (lst != DRIFT_OK) s.status = lst;
  }
}

__device__ __forceinline__ long long quantile_rank(int q, long long n) {
  const long long k = (kQNum[q] * n + 99) / 100;  // ceil(q * n), exact
  return k < 1 ? 1 : (k > n ? n : k);
}

__global__ void __launch_bounds__(kDiagThreads) diag_tile(DiagParams p) {
  const int tid = threadIdx.x;
  const DiagLayout lay = DiagLayout::make(p.N);
  const double lo_edge = 1.0 - p.eps_low, hi_edge = 1.0 + p.eps_high;
  RowStats acc = {};
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
  // all loads first (one round trip), then the rows in the same order as ever
  uint8_t act[kRowsPerThread];
  float dv[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    act[j] = r < p.N ? p.active[r] : (uint8_t)0;
    dv[j] = r < p.N ? p.d[r] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    if (act[j]) add_row(acc, dv[j], r, lo_edge, hi_edge);
  }
  if (p.N > kSelSingleMax && blockIdx.x == 0) {  // read by the digit launches that follow
    unsigned int* h = (unsigned int*)(p.ws + lay.hist_off);
    for (int i = tid; i < 3 * kNumQ * kBins; i += kDiagThreads) h[i] = 0;
  }
  const RowStats t = block_reduce(acc);
  if (tid == 0) {
    TilePartial o = {};
    o.s_abs = t.s_abs;
    o.s_exp = t.s_exp;
    o.s_kl = t.s_kl;
    o.s_d = t.s_d;
    o.n = t.n;
    o.lo = t.lo;
    o.hi = t.hi;
    o.nonfinite = t.nf;
    o.best = t.best;
    ((TilePartial*)(p.ws + lay.partial_off))[blockIdx.x] = o;
  }
}

constexpr int kSelBatch = 8;                  // rows per thread per batch of loads
static_assert(kPassRowsPerBlock % (4 * kPassThreads) == 0 &&
                  (kPassRowsPerBlock / kPassThreads) % kSelBatch == 0,
              "a pass block's rows split evenly into batches");
static_assert(kBins % kPassThreads == 0 && (kNumQ * kBins) % kPassThreads == 0 &&
                  (kNumQ * kBins) % kSelThreads == 0,
              "histogram copies split evenly over the threads");

// Keys of rows r0 .. r0 + 3 (kNoKey for inactive rows and rows past hi): one 16-byte load
// of d and one 4-byte load of the mask when all four rows exist; d and active must then be
// 16- and 4-byte aligned at r0.
__device__ __forceinline__ void keys4(const float* d, const uint8_t* active, int64_t r0,
                                      int64_t hi, unsigned int (&k)[4]) {
  if (r0 + 3 < hi) {
    const float4 v = *(const float4*)(d + r0);
    const uint32_t a = *(const uint32_t*)(active + r0);
    k[0] = (a & 0xffu) ? key_of(v.x) : kNoKey;
    k[1] = (a & 0xff00u) ? key_of(v.y) : kNoKey;
    k[2] = (a & 0xff0000u) ? key_of(v.z) : kNoKey;
    k[3] = (a & 0xff000000u) ? key_of(v.w) : kNoKey;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t r = r0 + e;
      k[e] = (r < hi && active[r]) ? key_of(d[r]) : kNoKey;
    }
  }
}

// Block-cooperative (NT threads) three-digit radix select: the nearest-rank keys of both
// quantiles among the active rows [lo, hi), given their 1-based ranks in s_rank (updated in
// place); the keys end in s_prefix (zero on entry). Rows lo + tid + k NT, k < KC, are read
// once into registers; rows past lo + KC NT are re-read for every digit in batches of
// kSelBatch per thread (all loads of a batch issued before any count). When the rows start
// 16-byte aligned (lo = 0 and aligned arrays; the whole-batch call), thread t instead takes
// groups of four consecutive rows with one vector load each (the same rows in total), so a
// pass issues a quarter of the load instructions. Digit h of a
// quantile counts, in LDS, the keys whose upper digits match the ones chosen so far; the
// first digit's histogram is shared by both quantiles.
// select_keys issues the loads of the cached keys (a caller may overlap them with other
// work) and returns whether the vector path applies; radix_select then runs the digits.
template <int NT, int KC>
__device__ __forceinline__ bool select_keys(const float* d, const uint8_t* active, int64_t lo,
                                            int64_t hi, unsigned int (&ck)[KC]) {
  static_assert(KC % 4 == 0, "the vector path caches groups of four rows");
  const int tid = threadIdx.x;
  const bool vec = lo == 0 && ((uintptr_t)d & 15) == 0 && ((uintptr_t)active & 3) == 0;
  if (vec) {  // block-uniform
#pragma unroll
    for (int k = 0; k < KC / 4; ++k) {
      unsigned int k4[4];
      keys4(d, active, 4 * ((int64_t)k * NT + tid), hi, k4);
#pragma unroll
      for (int e = 0; e < 4; ++e) ck[4 * k + e] = k4[e];
    }
  } else {
    uint8_t a[KC];
    float x[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int64_t r = lo + tid + (int64_t)k * NT;
      a[k] = r < hi ? active[r] : (uint8_t)0;
      x[k] = r < hi ? d[r] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) ck[k] = a[k] ? key_of(x[k]) : kNoKey;
  }
  return vec;
}

//
// With `s_list` (64 KC keys per wave in LDS), after the first digit each wave packs the
// cached keys whose first digit matches either quantile's into its own list (ballot and
// lane count, in lane order), and the later digits count that list instead of every cached
// key: far fewer LDS atomics when few keys share the selected bins. The counts, and so the
// result, are the same.
template <int NT, int KC>
__device__ void radix_select(const float* d, const uint8_t* active, int64_t lo, int64_t hi,
                             const unsigned int (&ck)[KC], bool vec,
                             unsigned int (*s_hist)[kBins], long long* s_rank,
                             unsigned int* s_prefix, unsigned int* s_list) {
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned int* wl = s_list ? s_list + (tid >> 6) * (64 * KC) : nullptr;
  unsigned int nl = 0;  // wave-uniform length of wl
  const int64_t rest = lo + (int64_t)KC * NT;
  for (int pass = 0; pass < 3; ++pass) {
    for (int b = tid; b < kNumQ * kBins; b += NT) (&s_hist[0][0])[b] = 0;
    __syncthreads();
    const int shift = kShift[pass];
    const unsigned int mask = (1u << kBitsOf[pass]) - 1u;
    const int hi_shift = pass > 0 ? kShift[pass - 1] : 31;
    const unsigned int pre0 = s_prefix[0] >> hi_shift, pre1 = s_prefix[1] >> hi_shift;
    auto count = [&](unsigned int key) {
      if (key == kNoKey) return;
      if (pass == 0) {
        atomicAdd(&s_hist[0][key >> shift], 1u);
      } else {
        if ((key >> hi_shift) == pre0) atomicAdd(&s_hist[0][(key >> shift) & mask], 1u);
        if ((key >> hi_shift) == pre1) atomicAdd(&s_hist[1][(key >> shift) & mask], 1u);
      }
    };
    if (pass == 0 || !wl) {
#pragma unroll
      for (int k = 0; k < KC; ++k) count(ck[k]);
    } else {
      for (unsigned int i = lane; i < nl; i += 64) count(wl[i]);
    }
    if (vec) {
      for (int64_t base = rest; base < hi; base += (int64_t)NT * kSelBatch) {
        unsigned int kk[kSelBatch / 4][4];
#pragma unroll
        for (int u = 0; u < kSelBatch / 4; ++u)
          keys4(d, active, base + 4 * ((int64_t)u * NT + tid), hi, kk[u]);
#pragma unroll
        for (int u = 0; u < kSelBatch / 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) count(kk[u][e]);
      }
    } else for (int64_t base = rest; base < hi; base += (int64_t)NT * kSelBatch) {
      uint8_t a[kSelBatch];
      float x[kSelBatch];
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {
        const int64_t r = base + tid + (int64_t)u * NT;
        a[u] = r < hi ? active[r] : (uint8_t)0;
        x[u] = r < hi ? d[r] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) count(a[u] ? key_of(x[u]) : kNoKey);
    }
    __syncthreads();
    pick_digits(s_hist[0], s_hist[pass == 0 ? 0 : 1], shift, s_rank, s_prefix);
    __syncthreads();
    if (pass == 0 && wl) {  // wl is block-uniform; the next pass's barrier orders the list
      const unsigned int q0 = s_prefix[0] >> kShift[0], q1 = s_prefix[1] >> kShift[0];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const unsigned int key = ck[k];
        const bool m = key != kNoKey && ((key >> kShift[0]) == q0 || (key >> kShift[0]) == q1);
        const unsigned long long bm = __ballot(m);
        const unsigned int below = __builtin_amdgcn_mbcnt_hi(
            (unsigned int)(bm >> 32), __builtin_amdgcn_mbcnt_lo((unsigned int)bm, 0u));
        if (m) wl[nl + below] = key;
        nl += (unsigned int)__popcll(bm);
      }
    }
  }
}

// The whole batch after diag_tile: folds the tile partials, finishes the statistics and
// selects p95 / p99 (MULTI: from the digit histograms of the multi-block launches, taken
// above kSelSingleMax rows; else from the keys themselves).
template <bool MULTI>
__global__ void __launch_bounds__(kSelThreads) diag_select(DiagParams p) {
  __shared__ unsigned int s_hist[kNumQ][kBins];
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  __shared__ long long s_n;
  __shared__ unsigned int s_list[MULTI ? 1 : kSelThreads * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const DiagLayout lay = DiagLayout::make(p.N);
  const TilePartial* tp = (const TilePartial*)(p.ws + lay.partial_off);
  drift_stats& S = p.out ? *p.out : ((SelState*)p.ws)->stats;
  // The selection's inputs are loaded first, so that their latency overlaps the fold: the
  // digit histograms of the multi-block launches, or the keys this block selects from.
  constexpr int kHistPer = kNumQ * kBins / kSelThreads;
  unsigned int hreg[MULTI ? 3 : 1][kHistPer];
  unsigned int ck[MULTI ? 4 : 16];
  bool vec = false;
  if constexpr (MULTI) {
    const unsigned int* gh = (const unsigned int*)(p.ws + lay.hist_off);
#pragma unroll
    for (int pass = 0; pass < 3; ++pass)
#pragma unroll
      for (int i = 0; i < kHistPer; ++i)
        hreg[pass][i] = gh[(pass * kNumQ) * kBins + tid + i * kSelThreads];
  } else {
    vec = select_keys<kSelThreads, 16>(p.d, p.active, 0, p.N, ck);
  }
  if (wave == 0) {
    RowStats a = {};
    // lane j folds tiles j, j + 64, ... in ascending order, loading four at a time
    for (int g0 = lane; g0 < lay.G; g0 += 4 * 64) {
      RowStats bs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int g = g0 + 64 * u;
        if (g < lay.G) {
          const TilePartial& b = tp[g];
          bs[u] = {b.s_abs, b.s_exp, b.s_kl, b.s_d, b.n, b.lo, b.hi, b.nonfinite, b.best};
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (g0 + 64 * u < lay.G) add_stats(a, bs[u]);
    }
    // then the 64 lane results by the lane butterfly
    a = wave_reduce(a);
    if (lane == 0) {
      finish_stats(S, a, p.lp);
      for (int q = 0; q < kNumQ; ++q) {
        s_rank[q] = quantile_rank(q, a.n);
        s_prefix[q] = 0;
      }
      s_n = a.n;
    }
  }
  __syncthreads();
  if (s_n == 0) return;  // block-uniform
  if constexpr (MULTI) {
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int i = 0; i < kHistPer; ++i) (&s_hist[0][0])[tid + i * kSelThreads] = hreg[pass][i];
      __syncthreads();
      pick_digits(s_hist[0], s_hist[pass == 0 ? 0 : 1], kShift[pass], s_rank, s_prefix);
      __syncthreads();
    }
  } else {
    radix_select<kSelThreads, 16>(p.d, p.active, 0, p.N, ck, vec, s_hist, s_rank, s_prefix,
                                  s_list);
  }
  if (tid == 0) {
    S.p95_abs_dlogp = __uint_as_float(s_prefix[0]);
    S.p99_abs_dlogp = __uint_as_float(s_prefix[1]);
  }
}

// One digit of the multi-block selection (batches above kSelSingleMax rows). Every block
// first rebuilds the digits chosen so far from the histograms of the earlier launches (the
// active count is the first histogram's total, so the ranks follow as in diag_select),
// then counts the keys of its rows whose upper digits match into LDS histograms and adds
// its non-zero bins to the launch's global histogram. All counts are integers: the result
// does not depend on how rows or blocks are scheduled.
template <int PASS>
__global__ void __launch_bounds__(kPassThreads) diag_pass(DiagParams p) {
  __shared__ unsigned int s_hist[kNumQ][kBins];
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  __shared__ unsigned int s_w[kPassThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const DiagLayout lay = DiagLayout::make(p.N);
  unsigned int* gh = (unsigned int*)(p.ws + lay.hist_off);
  if (tid < kNumQ) s_prefix[tid] = 0;
  if (PASS > 0) {
#pragma unroll
    for (int i = 0; i < kBins / kPassThreads; ++i)
      s_hist[0][tid + i * kPassThreads] = gh[tid + i * kPassThreads];
    __syncthreads();
    unsigned int c = 0;
#pragma unroll
    for (int i = 0; i < kBins / kPassThreads; ++i) c += s_hist[0][tid + i * kPassThreads];
    c = (unsigned int)__builtin_amdgcn_readlane((int)wave_incl_scan(c, lane), 63);
    if (lane == 0) s_w[wave] = c;
    __syncthreads();
    if (tid < kNumQ) {
      long long n = 0;
      for (int w = 0; w < kPassThreads / 64; ++w) n += s_w[w];
      s_rank[tid] = quantile_rank(tid, n);
    }
    __syncthreads();
    for (int pass = 0; pass < PASS; ++pass) {
      if (pass > 0) {
#pragma unroll
        for (int i = 0; i < kNumQ * kBins / kPassThreads; ++i) {
          const int b = tid + i * kPassThreads;
          (&s_hist[0][0])[b] = gh[(pass * kNumQ) * kBins + b];
        }
        __syncthreads();
      }
      pick_digits(s_hist[0], s_hist[pass == 0 ? 0 : 1], kShift[pass], s_rank, s_prefix);
      __syncthreads();
    }
  }
  for (int b = tid; b < kNumQ * kBins; b += kPassThreads) (&s_hist[0][0])[b] = 0;
  __syncthreads();
  constexpr int shift = kShift[PASS];
  constexpr unsigned int mask = (1u << kBitsOf[PASS]) - 1u;
  constexpr int hi_shift = PASS > 0 ? kShift[PASS > 0 ? PASS - 1 : 0] : 31;
  const unsigned int pre0 = s_prefix[0] >> hi_shift, pre1 = s_prefix[1] >> hi_shift;
  auto count = [&](unsigned int key) {
    if (key == kNoKey) return;
    if (PASS == 0) {
      atomicAdd(&s_hist[0][key >> shift], 1u);
    } else {
      if ((key >> hi_shift) == pre0) atomicAdd(&s_hist[0][(key >> shift) & mask], 1u);
      if ((key >> hi_shift) == pre1) atomicAdd(&s_hist[1][(key >> shift) & mask], 1u);
    }
  };
  const int64_t lo = (int64_t)blockIdx.x * kPassRowsPerBlock;
  const int64_t hi = lo + kPassRowsPerBlock < p.N ? lo + kPassRowsPerBlock : p.N;
  const bool vec = ((uintptr_t)p.d & 15) == 0 && ((uintptr_t)p.active & 3) == 0;
  // every load of the block's rows is issued before any count
  if (vec) {  // block-uniform; lo is a multiple of 4
    constexpr int kIt = kPassRowsPerBlock / (4 * kPassThreads);
    unsigned int kk[kIt][4];
#pragma unroll
    for (int it = 0; it < kIt; ++it)
      keys4(p.d, p.active, lo + 4 * ((int64_t)it * kPassThreads + tid), hi, kk[it]);
#pragma unroll
    for (int it = 0; it < kIt; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) count(kk[it][e]);
  } else {
    constexpr int kIt = kPassRowsPerBlock / kPassThreads;
    for (int i0 = 0; i0 < kIt; i0 += kSelBatch) {
      unsigned int kb[kSelBatch];
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) {
        const int64_t r = lo + tid + (int64_t)(i0 + u) * kPassThreads;
        kb[u] = (r < hi && p.active[r]) ? key_of(p.d[r]) : kNoKey;
      }
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) count(kb[u]);
    }
  }
  __syncthreads();
  for (int b = tid; b < kNumQ * kBins; b += kPassThreads) {
    const unsigned int c = (&s_hist[0][0])[b];
    if (c) atomicAdd(&gh[(PASS * kNumQ) * kBins + b], c);
  }
}

// Per-segment statistics ("Diagnostics" table, per-sequence and per-rank views): one block
// per segment [off[s], off[s+1]) does the sums, counts and the whole three-digit radix
// select in LDS, reading the segment's rows once per digit. Thread t takes rows lo + t,
// lo + t + 256, ..., so the fixed-order sums depend only on the segment's own rows.
__global__ void __launch_bounds__(kDiagThreads) diag_segments(SegParams p) {
  __shared__ unsigned int s_hist[kNumQ][kBins];
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  __shared__ long long s_n;
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x;
  const int64_t lo = p.off[seg], hi = p.off[seg + 1];
  drift_stats* out = p.out + seg;
  if (!(0 <= lo && lo <= hi && hi <= p.N)) {  // bad segment metadata
    if (tid == 0) {
      const RowStats none = {};
      finish_stats(*out, none, nullptr);
      out->status = DRIFT_EMASK;
    }
    return;
  }
  const double lo_edge = 1.0 - p.eps_low, hi_edge = 1.0 + p.eps_high;
  RowStats acc = {};
  for (int64_t r = lo + tid; r < hi; r += kDiagThreads) {
    if (!p.active[r]) continue;
    add_row(acc, p.d[r], r, lo_edge, hi_edge);
  }
  const RowStats t = block_reduce(acc);
  drift_stats s;
  if (tid == 0) {
    finish_stats(s, t, p.lp);
    for (int q = 0; q < kNumQ; ++q) {
      s_rank[q] = quantile_rank(q, t.n);
      s_prefix[q] = 0;
    }
    s_n = t.n;
  }
  __syncthreads();
  if (s_n == 0) {  // block-uniform
    if (tid == 0) *out = s;
    return;
  }
  unsigned int ck[8];
  const bool vec = select_keys<kDiagThreads, 8>(p.d, p.active, lo, hi, ck);
  radix_select<kDiagThreads, 8>(p.d, p.active, lo, hi, ck, vec, s_hist, s_rank, s_prefix,
                                nullptr);
  if (tid == 0) {
    s.p95_abs_dlogp = __uint_as_float(s_prefix[0]);
    s.p99_abs_dlogp = __uint_as_float(s_prefix[1]);
    *out = s;
  }
}

}  // namespace

size_t diag_ws_bytes(int64_t N) { return DiagLayout::make(N).total; }

hipError_t diag_noalloc_scratch(char** ptr, size_t* bytes) {
  // the device address of `scratch`, looked up once per device with that device current
  constexpr int kMaxDevices = 64;
  static std::atomic<char*> cache[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  char* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = cache[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = (char*)q;
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}
size_t diag_stats_offset() { return offsetof(SelState, stats); }

hipError_t launch_segment_diagnostics(const SegParams& p, hipStream_t s) {
  if (p.S == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_segments, dim3((unsigned)p.S), dim3(kDiagThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_diagnostics(const DiagParams& p, hipStream_t s) {
  const DiagLayout lay = DiagLayout::make(p.N);
  const int G = lay.G > 0 ? lay.G : 1;  // one (empty) tile when N = 0
  hipLaunchKernelGGL(diag_tile, dim3(G), dim3(kDiagThreads), 0, s, p);
  if (p.N > kSelSingleMax) {
    const unsigned nb = (unsigned)((p.N + kPassRowsPerBlock - 1) / kPassRowsPerBlock);
    hipLaunchKernelGGL(diag_pass<0>, dim3(nb), dim3(kPassThreads), 0, s, p);
    hipLaunchKernelGGL(diag_pass<1>, dim3(nb), dim3(kPassThreads), 0, s, p);
    hipLaunchKernelGGL(diag_pass<2>, dim3(nb), dim3(kPassThreads), 0, s, p);
  }
  if (p.N > kSelSingleMax)
    hipLaunchKernelGGL(diag_select<true>, dim3(1), dim3(kSelThreads), 0, s, p);
  else
    hipLaunchKernelGGL(diag_select<false>, dim3(1), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace drift
