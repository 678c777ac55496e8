// Drift diagnostics over the active rows ("WS2 Cross-Config Logprob Drift Contract",
// Diagnostics table): ratio0, clipfrac0, approx_kl0, mean |dlogp|, and p95/p99/max
// |dlogp| as exact nearest-rank order statistics (the ceil(q*n)-th smallest value).
//
// Launch sequence over tiles of kDiagTile rows (G tiles):
//   diag_tile      per tile: fp64 sums of |d|, exp(d), expm1(d) - d and d in a fixed
//                  order, the active / clipped / non-finite counts, the largest key
//                  with its first row, and a histogram of the top 11 bits of the keys;
//   diag_select 0  folds the tiles in index order into the statistics, derives the
//                  nearest ranks and picks the top digit of each selected key;
//   diag_hist 1,2  per tile histograms of the next digit among keys that match the
//                  digits chosen so far, one histogram per quantile;
//   diag_select 1,2  pick the next digit; after the last one the keys are exact.
// Keys are the IEEE bit patterns of |d| (fabs clears the sign bit), whose unsigned order
// is the order of the values, so the selection is an MSB-first radix select with digits
// of 11, 11 and 10 bits. Counts and digit choices are integer work; the sums are fp64
// in an order that depends only on N.
#include <math.h>

#include "common.h"

namespace drift {
namespace {

constexpr int kDiagThreads = 256;
constexpr int kDiagTile = 4096;
constexpr int kRowsPerThread = kDiagTile / kDiagThreads;
constexpr int kBins = 2048;
constexpr int kSelThreads = 1024;
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
};

struct DiagLayout {
  size_t partial_off, hist_off, total;
  int G;
  __host__ __device__ static DiagLayout make(int64_t N) {
    DiagLayout l;
    l.G = (int)((N + kDiagTile - 1) / kDiagTile);
    l.partial_off = 512;
    l.hist_off = l.partial_off + align_up((size_t)(l.G > 0 ? l.G : 1) * sizeof(TilePartial), 256);
    l.total = l.hist_off + align_up((size_t)(l.G > 0 ? l.G : 1) * kNumQ * kBins * 4, 256);
    return l;
  }
};
static_assert(sizeof(SelState) <= 512, "state size");

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

__global__ void __launch_bounds__(kDiagThreads) diag_tile(DiagParams p) {
  __shared__ unsigned int s_hist[kBins];
  __shared__ double s_sum[4][kDiagThreads / 64];
  __shared__ long long s_cnt[4][kDiagThreads / 64];
  __shared__ unsigned long long s_best[kDiagThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = tid; b < kBins; b += kDiagThreads) s_hist[b] = 0;
  __syncthreads();
  const double lo_edge = 1.0 - p.eps_low, hi_edge = 1.0 + p.eps_high;
  double s_abs = 0, s_exp = 0, s_kl = 0, s_d = 0;
  long long n = 0, lo = 0, hi = 0, nf = 0;
  unsigned long long best = 0;
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    if (r >= p.N || !p.active[r]) continue;
    const float df = p.d[r];
    const double v = (double)df;
    const double e = exp(v);
    ++n;
    s_abs += fabs(v);
    s_exp += e;
    s_kl += expm1(v) - v;
    s_d += v;
    if (e < lo_edge) ++lo;
    else if (e > hi_edge) ++hi;
    if (!isfinite(df)) ++nf;
    const unsigned int key = key_of(df);
    const unsigned long long cand =
        ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (unsigned int)r);
    best = cand > best ? cand : best;
    atomicAdd(&s_hist[key >> kShift[0]], 1u);
  }
  s_abs = wave_sum(s_abs);
  s_exp = wave_sum(s_exp);
  s_kl = wave_sum(s_kl);
  s_d = wave_sum(s_d);
  n = wave_sum(n);
  lo = wave_sum(lo);
  hi = wave_sum(hi);
  nf = wave_sum(nf);
  best = wave_max(best);
  if (lane == 0) {
    s_sum[0][wave] = s_abs;
    s_sum[1][wave] = s_exp;
    s_sum[2][wave] = s_kl;
    s_sum[3][wave] = s_d;
    s_cnt[0][wave] = n;
    s_cnt[1][wave] = lo;
    s_cnt[2][wave] = hi;
    s_cnt[3][wave] = nf;
    s_best[wave] = best;
  }
  __syncthreads();
  const DiagLayout lay = DiagLayout::make(p.N);
  if (tid == 0) {
    TilePartial t = {};
    for (int w = 0; w < kDiagThreads / 64; ++w) {
      t.s_abs += s_sum[0][w];
      t.s_exp += s_sum[1][w];
      t.s_kl += s_sum[2][w];
      t.s_d += s_sum[3][w];
      t.n += s_cnt[0][w];
      t.lo += s_cnt[1][w];
      t.hi += s_cnt[2][w];
      t.nonfinite += s_cnt[3][w];
      t.best = s_best[w] > t.best ? s_best[w] : t.best;
    }
    ((TilePartial*)(p.ws + lay.partial_off))[blockIdx.x] = t;
  }
  unsigned int* gh = (unsigned int*)(p.ws + lay.hist_off) + (size_t)blockIdx.x * kNumQ * kBins;
  for (int b = tid; b < kBins; b += kDiagThreads) gh[b] = s_hist[b];
}

__global__ void __launch_bounds__(kDiagThreads) diag_hist(DiagParams p, int pass) {
  __shared__ unsigned int s_hist[kNumQ][kBins];
  const int tid = threadIdx.x;
  const SelState* st = (const SelState*)p.ws;
  if (st->n == 0) return;
  for (int b = tid; b < kNumQ * kBins; b += kDiagThreads) (&s_hist[0][0])[b] = 0;
  __syncthreads();
  const int hi_shift = kShift[pass - 1];
  const int shift = kShift[pass];
  const unsigned int mask = (1u << kBitsOf[pass]) - 1u;
  unsigned int pre[kNumQ];
#pragma unroll
  for (int q = 0; q < kNumQ; ++q) pre[q] = st->prefix[q] >> hi_shift;
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kDiagThreads + tid;
    if (r >= p.N || !p.active[r]) continue;
    const unsigned int key = key_of(p.d[r]);
#pragma unroll
    for (int q = 0; q < kNumQ; ++q)
      if ((key >> hi_shift) == pre[q]) atomicAdd(&s_hist[q][(key >> shift) & mask], 1u);
  }
  __syncthreads();
  const DiagLayout lay = DiagLayout::make(p.N);
  unsigned int* gh = (unsigned int*)(p.ws + lay.hist_off) + (size_t)blockIdx.x * kNumQ * kBins;
  for (int b = tid; b < kNumQ * kBins; b += kDiagThreads) gh[b] = (&s_hist[0][0])[b];
}

__global__ void __launch_bounds__(kSelThreads) diag_select(DiagParams p, int pass) {
  __shared__ long long s_scan[kSelThreads / 64];
  __shared__ int s_digit;
  __shared__ long long s_below;
  __shared__ long long s_n;
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  SelState* st = (SelState*)p.ws;
  const DiagLayout lay = DiagLayout::make(p.N);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    if (pass == 0) {
      const TilePartial* tp = (const TilePartial*)(p.ws + lay.partial_off);
      double s_abs = 0, s_exp = 0, s_kl = 0, s_d = 0;
      long long n = 0, lo = 0, hi = 0, nf = 0;
      unsigned long long best = 0;
      for (int g = 0; g < lay.G; ++g) {  // tile index order
        s_abs += tp[g].s_abs;
        s_exp += tp[g].s_exp;
        s_kl += tp[g].s_kl;
        s_d += tp[g].s_d;
        n += tp[g].n;
        lo += tp[g].lo;
        hi += tp[g].hi;
        nf += tp[g].nonfinite;
        best = tp[g].best > best ? tp[g].best : best;
      }
      drift_stats& s = st->stats;
      s.n_active = n;
      s.n_clip_low = lo;
      s.n_clip_high = hi;
      s.n_nonfinite = nf;
      st->n = n;
      if (n == 0) {
        s.argmax_row = -1;
        s.ratio0 = s.clipfrac0 = s.approx_kl0 = s.mean_abs_dlogp = s.mean_dlogp = NAN;
        s.p95_abs_dlogp = s.p99_abs_dlogp = s.max_abs_dlogp = NAN;
        s.status = DRIFT_ENOACTIVE;
      } else {
        const double dn = (double)n;
        s.ratio0 = s_exp / dn;
        s.approx_kl0 = s_kl / dn;
        s.clipfrac0 = (double)(lo + hi) / dn;
        s.mean_abs_dlogp = s_abs / dn;
        s.mean_dlogp = s_d / dn;
        s.max_abs_dlogp = __uint_as_float((unsigned int)(best >> 32));
        s.argmax_row = (long long)(0xffffffffu - (unsigned int)(best & 0xffffffffull));
        s.status = nf ? DRIFT_ENONFINITE : DRIFT_OK;
      }
      for (int q = 0; q < kNumQ; ++q) {
        const long long k = (kQNum[q] * n + 99) / 100;  // ceil(q * n), exact
        s_rank[q] = k < 1 ? 1 : (k > n ? n : k);
        s_prefix[q] = 0;
      }
      s_n = n;
    } else {
      s_n = st->n;
      for (int q = 0; q < kNumQ; ++q) {
        s_rank[q] = st->rank[q];
        s_prefix[q] = st->prefix[q];
      }
    }
  }
  __syncthreads();
  if (s_n == 0) return;  // block-uniform
  const unsigned int* gh = (const unsigned int*)(p.ws + lay.hist_off);
  const int nbins = 1 << kBitsOf[pass];
  for (int q = 0; q < kNumQ; ++q) {
    const int hq = pass == 0 ? 0 : q;  // the first histogram is shared by both quantiles
    // each thread owns two adjacent bins; counts summed over tiles (integers)
    long long c0 = 0, c1 = 0;
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    if (b0 < nbins) {
      for (int g = 0; g < lay.G; ++g) {
        const unsigned int* h = gh + ((size_t)g * kNumQ + hq) * kBins;
        c0 += h[b0];
        c1 += h[b1];
      }
    }
    // inclusive scan of the per-thread pair sums across the block
    const long long mine = c0 + c1;
    long long inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) s_scan[wave] = inc;
    __syncthreads();
    long long wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_scan[w];
    const long long before = wbase + inc - mine;  // keys in bins below b0
    const long long rank = s_rank[q];
    if (b0 < nbins) {
      if (before < rank && rank <= before + c0) {
        s_digit = b0;
        s_below = before;
      } else if (before + c0 < rank && rank <= before + mine) {
        s_digit = b1;
        s_below = before + c0;
      }
    }
    __syncthreads();
    if (tid == 0) {
      s_prefix[q] |= (unsigned int)s_digit << kShift[pass];
      s_rank[q] = rank - s_below;
    }
    __syncthreads();
  }
  if (tid == 0) {
    for (int q = 0; q < kNumQ; ++q) {
      st->prefix[q] = s_prefix[q];
      st->rank[q] = s_rank[q];
    }
    if (pass == 2) {
      st->stats.p95_abs_dlogp = __uint_as_float(s_prefix[0]);
      st->stats.p99_abs_dlogp = __uint_as_float(s_prefix[1]);
    }
  }
}

}  // namespace

size_t diag_ws_bytes(int64_t N) { return DiagLayout::make(N).total; }
size_t diag_stats_offset() { return offsetof(SelState, stats); }

hipError_t launch_diagnostics(const DiagParams& p, hipStream_t s) {
  const DiagLayout lay = DiagLayout::make(p.N);
  const int G = lay.G > 0 ? lay.G : 1;
  hipLaunchKernelGGL(diag_tile, dim3(G), dim3(kDiagThreads), 0, s, p);
  hipLaunchKernelGGL(diag_select, dim3(1), dim3(kSelThreads), 0, s, p, 0);
  for (int pass = 1; pass < 3; ++pass) {
    hipLaunchKernelGGL(diag_hist, dim3(G), dim3(kDiagThreads), 0, s, p, pass);
    hipLaunchKernelGGL(diag_select, dim3(1), dim3(kSelThreads), 0, s, p, pass);
  }
  return hipGetLastError();
}

}  // namespace drift
