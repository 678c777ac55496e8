// Drift diagnostics over the active rows ("WS2 Cross-Config Logprob Drift Contract",
// Diagnostics table): ratio0, clipfrac0, approx_kl0, mean |dlogp|, and p95/p99/max
// |dlogp| as exact nearest-rank order statistics (the ceil(q*n)-th smallest value).
//
// Four launches over tiles of kDiagTile rows (G tiles):
//   diag_init      zeroes the three digit histograms and the tile tickets;
//   diag_tile      per tile: fp64 sums of |d|, exp(d), expm1(d) - d and d in a fixed
//                  order, the active / clipped / non-finite counts, the largest key with
//                  its first row, and the histogram of the top 11 bits of the keys
//                  (integer atomics into one global histogram). The last tile to finish
//                  (atomic ticket) folds the tile partials in tile order into the
//                  statistics, derives the nearest ranks and picks the top digit;
//   diag_hist 1,2  histogram of the next digit among keys whose upper digits match the
//                  ones chosen so far, one histogram per quantile; the last tile picks the
//                  digit, and after the third digit the keys are exact.
// diag_segments (drift_segment_diagnostics) computes the same statistics per segment of
// rows (per sequence, per batch row or per rank) in one launch, one block per segment.
// Every statistics record also carries mismatch_kl = -mean(d), the k1 estimator of
// KL(rollout || train) ("Attention Debug Matrix", Metrics); approx_kl0 is its k3 form.
// Keys are the IEEE bit patterns of |d| (fabs clears the sign bit), whose unsigned order
// is the order of the values, so the selection is an MSB-first radix select with digits
// of 11, 11 and 10 bits. Counts and digit choices are integer work whose result does not
// depend on scheduling; the sums are fp64 in an order that depends only on N.
#include <math.h>

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

struct SelState {
  drift_stats stats;                // the result copied to the host
  unsigned int prefix[kNumQ];       // selected key bits so far
  long long rank[kNumQ];            // remaining 1-based rank inside the current bucket
  long long n;
  unsigned int ticket[3];           // tiles finished, per pass
};
static_assert(sizeof(SelState) <= 512, "state size");

struct DiagLayout {
  size_t hist_off, partial_off, total;
  int G;
  __host__ __device__ static DiagLayout make(int64_t N) {
    DiagLayout l;
    l.G = (int)((N + kDiagTile - 1) / kDiagTile);
    l.hist_off = 512;
    l.partial_off = l.hist_off + (size_t)3 * kNumQ * kBins * 4;
    l.total = l.partial_off + align_up((size_t)(l.G > 0 ? l.G : 1) * sizeof(TilePartial), 256);
    return l;
  }
};

__device__ __forceinline__ unsigned int key_of(float d) { return __float_as_uint(fabsf(d)); }

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

__device__ __forceinline__ unsigned int* hist_of(const DiagParams& p, int pass, int q) {
  return (unsigned int*)(p.ws + DiagLayout::make(p.N).hist_off) + ((size_t)pass * kNumQ + q) * kBins;
}

// Adds a block's LDS histogram into the global one (integer atomics; order-independent).
__device__ __forceinline__ void flush_hist(const unsigned int* sh, unsigned int* gh, int nbins) {
  for (int b = threadIdx.x; b < nbins; b += kDiagThreads)
    if (sh[b]) atomicAdd(gh + b, sh[b]);
}

// Every block calls this after its global writes; returns true in the last block to
// arrive, which then sees all of them.
__device__ __forceinline__ bool last_block(unsigned int* ticket, unsigned int G) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(ticket, 1u) == G - 1);
  __syncthreads();
  if (!s_last) return false;
  __threadfence();
  return true;
}

// Block-cooperative: in histogram h (nbins <= kBins counts, global or LDS), finds the bin
// holding the 1-based rank `rank`, i.e. the digit d with below < rank <= below + h[d],
// where below counts the keys in bins before d. Each thread owns kBins / kDiagThreads
// adjacent bins; an inclusive scan over threads locates the bin. Every thread gets the
// result.
__device__ void pick_digit(const unsigned int* h, int nbins, long long rank, int& digit,
                           long long& below) {
  constexpr int PER = kBins / kDiagThreads;
  __shared__ long long s_scan[kDiagThreads / 64];
  __shared__ int s_digit;
  __shared__ long long s_below;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long c[PER];
  long long mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = tid * PER + i;
    c[i] = b < nbins ? (long long)h[b] : 0;
    mine += c[i];
  }
  long long inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_scan[wave] = inc;
  __syncthreads();
  long long run = inc - mine;
  for (int w = 0; w < wave; ++w) run += s_scan[w];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < rank && rank <= run + c[i]) {
      s_digit = tid * PER + i;
      s_below = run;
    }
    run += c[i];
  }
  __syncthreads();
  digit = s_digit;
  below = s_below;
  __syncthreads();  // s_scan / s_digit are reused by the next call
}

// Picks the digit of pass `pass` for both quantiles from the global histograms and
// updates the selection state (read and written by thread 0).
__device__ void select_digit(SelState* st, const DiagParams& p, int pass) {
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  const int tid = threadIdx.x;
  if (tid == 0) {
    for (int q = 0; q < kNumQ; ++q) {
      s_rank[q] = st->rank[q];
      s_prefix[q] = st->prefix[q];
    }
  }
  __syncthreads();
  const int nbins = 1 << kBitsOf[pass];
  for (int q = 0; q < kNumQ; ++q) {
    int digit;
    long long below;
    pick_digit(hist_of(p, pass, pass == 0 ? 0 : q), nbins, s_rank[q], digit, below);
    if (tid == 0) {
      s_prefix[q] |= (unsigned int)digit << kShift[pass];
      s_rank[q] -= below;
    }
    __syncthreads();
  }
  if (tid == 0) {
    for (int q = 0; q < kNumQ; ++q) {
      st->prefix[q] = s_prefix[q];
      st->rank[q] = s_rank[q];
    }
  }
}

__global__ void __launch_bounds__(1024) diag_init(DiagParams p) {
  SelState* st = (SelState*)p.ws;
  unsigned int* h = hist_of(p, 0, 0);
  for (int i = threadIdx.x; i < 3 * kNumQ * kBins; i += 1024) h[i] = 0;
  if (threadIdx.x < 3) st->ticket[threadIdx.x] = 0;
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
  if (e < lo_edge) ++a.lo;
  else if (e > hi_edge) ++a.hi;
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

// Block-cooperative; the total is returned in thread 0.
__device__ RowStats block_reduce(RowStats a) {
  __shared__ RowStats s_w[kDiagThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  a.s_abs = wave_sum(a.s_abs);
  a.s_exp = wave_sum(a.s_exp);
  a.s_kl = wave_sum(a.s_kl);
  a.s_d = wave_sum(a.s_d);
  a.n = wave_sum(a.n);
  a.lo = wave_sum(a.lo);
  a.hi = wave_sum(a.hi);
  a.nf = wave_sum(a.nf);
  a.best = wave_max(a.best);
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
  __shared__ unsigned int s_hist[kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const DiagLayout lay = DiagLayout::make(p.N);
  for (int b = tid; b < kBins; b += kDiagThreads) s_hist[b] = 0;
  __syncthreads();
  const double lo_edge = 1.0 - p.eps_low, hi_edge = 1.0 + p.eps_high;
  RowStats acc = {};
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    if (r >= p.N || !p.active[r]) continue;
    const float df = p.d[r];
    add_row(acc, df, r, lo_edge, hi_edge);
    atomicAdd(&s_hist[key_of(df) >> kShift[0]], 1u);
  }
  const RowStats t = block_reduce(acc);
  TilePartial* tp = (TilePartial*)(p.ws + lay.partial_off);
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
    tp[blockIdx.x] = o;
  }
  flush_hist(s_hist, hist_of(p, 0, 0), kBins);
  SelState* st = (SelState*)p.ws;
  if (!last_block(&st->ticket[0], gridDim.x)) return;

  // last tile: lane j of wave 0 folds tiles j, j + 64, ... in order; thread 0 then folds
  // the 64 lane results in lane order (a tree fixed by the tile count)
  __shared__ long long s_n;
  __shared__ RowStats s_lane[64];
  if (wave == 0) {
    RowStats a = {};
    for (int g = lane; g < lay.G; g += 64) {
      const TilePartial b = tp[g];
      const RowStats bs = {b.s_abs, b.s_exp, b.s_kl, b.s_d, b.n, b.lo, b.hi, b.nonfinite, b.best};
      add_stats(a, bs);
    }
    s_lane[lane] = a;
  }
  __syncthreads();
  if (tid == 0) {
    RowStats a = {};
    for (int g = 0; g < 64; ++g) add_stats(a, s_lane[g]);
    finish_stats(st->stats, a, p.lp);
    st->n = a.n;
    for (int q = 0; q < kNumQ; ++q) {
      st->rank[q] = quantile_rank(q, a.n);
      st->prefix[q] = 0;
    }
    s_n = a.n;
  }
  __syncthreads();
  if (s_n == 0) return;  // block-uniform
  select_digit(st, p, 0);
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
  for (int b = tid; b < kBins; b += kDiagThreads) s_hist[0][b] = 0;
  __syncthreads();
  RowStats acc = {};
  for (int64_t r = lo + tid; r < hi; r += kDiagThreads) {
    if (!p.active[r]) continue;
    const float df = p.d[r];
    add_row(acc, df, r, lo_edge, hi_edge);
    atomicAdd(&s_hist[0][key_of(df) >> kShift[0]], 1u);
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
  for (int pass = 0; pass < 3; ++pass) {
    if (pass > 0) {  // histogram of this digit among keys that match the digits so far
      for (int b = tid; b < kNumQ * kBins; b += kDiagThreads) (&s_hist[0][0])[b] = 0;
      __syncthreads();
      const int hi_shift = kShift[pass - 1], shift = kShift[pass];
      const unsigned int mask = (1u << kBitsOf[pass]) - 1u;
      const unsigned int pre0 = s_prefix[0] >> hi_shift, pre1 = s_prefix[1] >> hi_shift;
      for (int64_t r = lo + tid; r < hi; r += kDiagThreads) {
        if (!p.active[r]) continue;
        const unsigned int key = key_of(p.d[r]);
        if ((key >> hi_shift) == pre0) atomicAdd(&s_hist[0][(key >> shift) & mask], 1u);
        if ((key >> hi_shift) == pre1) atomicAdd(&s_hist[1][(key >> shift) & mask], 1u);
      }
      __syncthreads();
    }
    for (int q = 0; q < kNumQ; ++q) {
      int digit;
      long long below;
      pick_digit(s_hist[pass == 0 ? 0 : q], 1 << kBitsOf[pass], s_rank[q], digit, below);
      if (tid == 0) {
        s_prefix[q] |= (unsigned int)digit << kShift[pass];
        s_rank[q] -= below;
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    s.p95_abs_dlogp = __uint_as_float(s_prefix[0]);
    s.p99_abs_dlogp = __uint_as_float(s_prefix[1]);
    *out = s;
  }
}

__global__ void __launch_bounds__(kDiagThreads) diag_hist(DiagParams p, int pass) {
  __shared__ unsigned int s_hist[kNumQ][kBins];
  const int tid = threadIdx.x;
  SelState* st = (SelState*)p.ws;
  if (st->n == 0) return;  // written by the previous launch; uniform
  for (int b = tid; b < kNumQ * kBins; b += kDiagThreads) (&s_hist[0][0])[b] = 0;
  __syncthreads();
  const int hi_shift = kShift[pass - 1];
  const int shift = kShift[pass];
  const unsigned int mask = (1u << kBitsOf[pass]) - 1u;
  unsigned int pre[kNumQ];
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) pre[q] = st->prefix[q] >> hi_shift;
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    if (r >= p.N || !p.active[r]) continue;
    const unsigned int key = key_of(p.d[r]);
#pragma unroll
    for (int q = 0; q < kNumQ; ++q)
      if ((key >> hi_shift) == pre[q]) atomicAdd(&s_hist[q][(key >> shift) & mask], 1u);
  }
  __syncthreads();
  for (int q = 0; q < kNumQ; ++q) flush_hist(s_hist[q], hist_of(p, pass, q), 1 << kBitsOf[pass]);
  if (!last_block(&st->ticket[pass], gridDim.x)) return;
  select_digit(st, p, pass);
  if (pass == 2 && tid == 0) {
    st->stats.p95_abs_dlogp = __uint_as_float(st->prefix[0]);
    st->stats.p99_abs_dlogp = __uint_as_float(st->prefix[1]);
  }
}

}  // namespace

size_t diag_ws_bytes(int64_t N) { return DiagLayout::make(N).total; }
size_t diag_stats_offset() { return offsetof(SelState, stats); }

hipError_t launch_segment_diagnostics(const SegParams& p, hipStream_t s) {
  if (p.S == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_segments, dim3((unsigned)p.S), dim3(kDiagThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_diagnostics(const DiagParams& p, hipStream_t s) {
  const DiagLayout lay = DiagLayout::make(p.N);
  const int G = lay.G > 0 ? lay.G : 1;
  hipLaunchKernelGGL(diag_init, dim3(1), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(diag_tile, dim3(G), dim3(kDiagThreads), 0, s, p);
  for (int pass = 1; pass < 3; ++pass)
    hipLaunchKernelGGL(diag_hist, dim3(G), dim3(kDiagThreads), 0, s, p, pass);
  return hipGetLastError();
}

}  // namespace drift
