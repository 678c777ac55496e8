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

// Picks the digit of pass `pass` for both quantiles from the global histograms
// (block of kDiagThreads threads; each owns kBins / kDiagThreads adjacent bins). The
// selection state is read by thread 0, shared through LDS, and written back by thread 0.
__device__ void select_digit(SelState* st, const DiagParams& p, int pass) {
  constexpr int PER = kBins / kDiagThreads;
  __shared__ long long s_scan[kDiagThreads / 64];
  __shared__ int s_digit;
  __shared__ long long s_below;
  __shared__ long long s_rank[kNumQ];
  __shared__ unsigned int s_prefix[kNumQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    for (int q = 0; q < kNumQ; ++q) {
      s_rank[q] = st->rank[q];
      s_prefix[q] = st->prefix[q];
    }
  }
  __syncthreads();
  const int nbins = 1 << kBitsOf[pass];
  for (int q = 0; q < kNumQ; ++q) {
    const unsigned int* gh = hist_of(p, pass, pass == 0 ? 0 : q);
    long long c[PER];
    long long mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = tid * PER + i;
      c[i] = b < nbins ? (long long)gh[b] : 0;
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
    long long before = inc - mine;
    for (int w = 0; w < wave; ++w) before += s_scan[w];
    const long long rank = s_rank[q];
    long long run = before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run < rank && rank <= run + c[i]) {
        s_digit = tid * PER + i;
        s_below = run;
      }
      run += c[i];
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
  }
}

__global__ void __launch_bounds__(1024) diag_init(DiagParams p) {
  SelState* st = (SelState*)p.ws;
  unsigned int* h = hist_of(p, 0, 0);
  for (int i = threadIdx.x; i < 3 * kNumQ * kBins; i += 1024) h[i] = 0;
  if (threadIdx.x < 3) st->ticket[threadIdx.x] = 0;
}

__global__ void __launch_bounds__(kDiagThreads) diag_tile(DiagParams p) {
  __shared__ unsigned int s_hist[kBins];
  __shared__ double s_sum[4][kDiagThreads / 64];
  __shared__ long long s_cnt[4][kDiagThreads / 64];
  __shared__ unsigned long long s_best[kDiagThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const DiagLayout lay = DiagLayout::make(p.N);
  for (int b = tid; b < kBins; b += kDiagThreads) s_hist[b] = 0;
  __syncthreads();
  const double lo_edge = 1.0 - p.eps_low, hi_edge = 1.0 + p.eps_high;
  double s_abs = 0, s_exp = 0, s_kl = 0, s_d = 0;
  long long n = 0, lo = 0, hi = 0, nf = 0;
  unsigned long long best = 0;
  const int64_t tile0 = (int64_t)blockIdx.x * kDiagTile;
#pragma unroll
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
  TilePartial* tp = (TilePartial*)(p.ws + lay.partial_off);
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
    tp[blockIdx.x] = t;
  }
  flush_hist(s_hist, hist_of(p, 0, 0), kBins);
  SelState* st = (SelState*)p.ws;
  if (!last_block(&st->ticket[0], gridDim.x)) return;

  // last tile: lane j of wave 0 folds tiles j, j + 64, ... in order; thread 0 then folds
  // the 64 lane results in lane order (a tree fixed by the tile count)
  __shared__ long long s_n;
  __shared__ TilePartial s_lane[64];
  if (wave == 0) {
    TilePartial a = {};
    for (int g = lane; g < lay.G; g += 64) {
      const TilePartial b = tp[g];
      a.s_abs += b.s_abs;
      a.s_exp += b.s_exp;
      a.s_kl += b.s_kl;
      a.s_d += b.s_d;
      a.n += b.n;
      a.lo += b.lo;
      a.hi += b.hi;
      a.nonfinite += b.nonfinite;
      a.best = b.best > a.best ? b.best : a.best;
    }
    s_lane[lane] = a;
  }
  __syncthreads();
  if (tid == 0) {
    double a_abs = 0, a_exp = 0, a_kl = 0, a_d = 0;
    long long an = 0, alo = 0, ahi = 0, anf = 0;
    unsigned long long abest = 0;
    for (int g = 0; g < 64; ++g) {
      a_abs += s_lane[g].s_abs;
      a_exp += s_lane[g].s_exp;
      a_kl += s_lane[g].s_kl;
      a_d += s_lane[g].s_d;
      an += s_lane[g].n;
      alo += s_lane[g].lo;
      ahi += s_lane[g].hi;
      anf += s_lane[g].nonfinite;
      abest = s_lane[g].best > abest ? s_lane[g].best : abest;
    }
    drift_stats& s = st->stats;
    s.n_active = an;
    s.n_clip_low = alo;
    s.n_clip_high = ahi;
    s.n_nonfinite = anf;
    st->n = an;
    if (an == 0) {
      s.argmax_row = -1;
      s.ratio0 = s.clipfrac0 = s.approx_kl0 = s.mean_abs_dlogp = s.mean_dlogp = NAN;
      s.p95_abs_dlogp = s.p99_abs_dlogp = s.max_abs_dlogp = NAN;
      s.status = DRIFT_ENOACTIVE;
    } else {
      const double dn = (double)an;
      s.ratio0 = a_exp / dn;
      s.approx_kl0 = a_kl / dn;
      s.clipfrac0 = (double)(alo + ahi) / dn;
      s.mean_abs_dlogp = a_abs / dn;
      s.mean_dlogp = a_d / dn;
      s.max_abs_dlogp = __uint_as_float((unsigned int)(abest >> 32));
      s.argmax_row = (long long)(0xffffffffu - (unsigned int)(abest & 0xffffffffull));
      s.status = anf ? DRIFT_ENONFINITE : DRIFT_OK;
    }
    if (p.lp) {  // the logprob call's own status outranks the diagnostics status
      const int lst = header_status(p.lp->magic, p.lp->err_bits);
      if (lst != DRIFT_OK) s.status = lst;
    }
    for (int q = 0; q < kNumQ; ++q) {
      const long long k = (kQNum[q] * an + 99) / 100;  // ceil(q * n), exact
      st->rank[q] = k < 1 ? 1 : (k > an ? an : k);
      st->prefix[q] = 0;
    }
    s_n = an;
  }
  __syncthreads();
  if (s_n == 0) return;  // block-uniform
  select_digit(st, p, 0);
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
