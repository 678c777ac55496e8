// Active-row classification, logical-input validation and stable compaction.
//
// Active rows are the attended response/action rows ("WS2 Cross-Config Logprob Drift
// Contract", Measurement Contract); a logical-input violation (mask shape, padding side,
// out-of-range selected id) makes the comparison invalid rather than noisy (same page,
// "Logical Input and Metadata Drift"), so it is recorded as an error class.
//
// Two launches over tiles of kClassifyTile rows:
//   classify_count   validates every row, writes the `active` output and zeros the
//                    per-row outputs of inactive rows, and stores per tile: the active
//                    count, the error bits and the first offending rows;
//   compact_scatter  turns the counts into offsets and writes the ascending list of
//                    active row indices; tile 0 also folds the per-tile error records and
//                    the total count into the workspace header.
// Integer work only: the results do not depend on scheduling.
#include "common.h"

namespace drift {
namespace {

struct TileRec {          // 32 bytes per tile in the workspace
  int32_t count;
  uint32_t err_bits;
  unsigned long long first_bad_mask;
  unsigned long long first_bad_token;
  int64_t pad;
};

constexpr int kRowsPerThread = kClassifyTile / kClassifyThreads;  // 8

__device__ __forceinline__ int64_t load_id(const void* ids, int64_t r, int32_t i64) {
  return i64 ? ((const int64_t*)ids)[r] : (int64_t)((const int32_t*)ids)[r];
}

__global__ void __launch_bounds__(kClassifyThreads)
classify_count(ClassifyParams p) {
  __shared__ int s_count[kClassifyThreads / 64];
  __shared__ uint32_t s_err;
  __shared__ unsigned long long s_bad_mask, s_bad_token;
  __shared__ int64_t s_end;
  const int tid = threadIdx.x;
  const int64_t tile0 = (int64_t)blockIdx.x * kClassifyTile;
  if (tid == 0) {
    s_err = 0;
    s_bad_mask = ~0ull;
    s_bad_token = ~0ull;
    int64_t end = p.N;
    if (p.layout == DRIFT_PACKED) {
      end = (int64_t)p.cu[p.nseq];
      end = end < 0 ? 0 : (end > p.N ? p.N : end);
    }
    s_end = end;
  }
  __syncthreads();

  // Packed metadata: cu_seqlens starts at 0, never decreases and ends inside the buffer.
  if (p.layout == DRIFT_PACKED && blockIdx.x == 0) {
    for (int64_t i = tid; i <= p.nseq; i += kClassifyThreads) {
      int64_t c = p.cu[i];
      bool bad = (i == 0 && c != 0) || (i > 0 && c < (int64_t)p.cu[i - 1]) || c > p.N;
      if (bad) {
        atomicOr(&s_err, 1u << kErrMask);
        atomicMin(&s_bad_mask, 0ull);
      }
    }
  }

  int my_count = 0;
  uint32_t my_err = 0;
  unsigned long long bad_mask = ~0ull, bad_token = ~0ull;
  const int64_t end = s_end;
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kClassifyThreads + tid;
    if (r >= p.N) break;
    const uint8_t a = p.att ? p.att[r] : (uint8_t)1;
    const uint8_t c = p.act ? p.act[r] : (uint8_t)1;
    bool emask = (a > 1) || (c > 1);
    bool real;
    if (p.layout == DRIFT_PACKED) {
      real = r < end;
      if (p.att && ((a != 0) != real)) emask = true;
    } else {
      real = a != 0;
      if (p.att) {
        const int64_t t = r % p.L;
        if (t + 1 < p.L) {
          const uint8_t a2 = p.att[r + 1];
          if (p.layout == DRIFT_PAD_RIGHT && a == 0 && a2 != 0) emask = true;
          if (p.layout == DRIFT_PAD_LEFT && a != 0 && a2 == 0) emask = true;
        }
      }
    }
    if (c != 0 && !real) emask = true;
    const bool act_row = real && (c != 0);
    if (act_row) {
      const int64_t y = load_id(p.ids, r, p.ids_i64);
      if (y < 0 || y >= p.V) {
        my_err |= 1u << kErrToken;
        bad_token = bad_token < (unsigned long long)r ? bad_token : (unsigned long long)r;
      }
      ++my_count;
    } else {
      p.out_t[r] = 0.0f;
      p.out_r[r] = 0.0f;
      p.out_d[r] = 0.0f;
    }
    if (emask) {
      my_err |= 1u << kErrMask;
      bad_mask = bad_mask < (unsigned long long)r ? bad_mask : (unsigned long long)r;
    }
    p.active[r] = act_row ? 1 : 0;
  }

  // Block totals: the count by wave sums, errors by LDS atomics (order-independent).
  int wc = my_count;
  for (int off = 32; off > 0; off >>= 1) wc += __shfl_xor(wc, off);
  if ((tid & 63) == 0) s_count[tid >> 6] = wc;
  if (my_err) {
    atomicOr(&s_err, my_err);
    if (bad_mask != ~0ull) atomicMin(&s_bad_mask, bad_mask);
    if (bad_token != ~0ull) atomicMin(&s_bad_token, bad_token);
  }
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kClassifyThreads / 64; ++w) tot += s_count[w];
    TileRec* rec = (TileRec*)(p.ws + LogprobWs::make(p.N).counts_off) + blockIdx.x;
    rec->count = tot;
    rec->err_bits = s_err;
    rec->first_bad_mask = s_bad_mask;
    rec->first_bad_token = s_bad_token;
  }
}

__global__ void __launch_bounds__(kClassifyThreads)
compact_scatter(ClassifyParams p, int nblk) {
  __shared__ long long s_part[kClassifyThreads / 64];
  __shared__ int s_wave[kClassifyThreads / 64];
  __shared__ long long s_base;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const LogprobWs lay = LogprobWs::make(p.N);
  const TileRec* recs = (const TileRec*)(p.ws + lay.counts_off);
  int32_t* rows = (int32_t*)(p.ws + lay.rows_off);

  // Offset of this tile = sum of the counts of earlier tiles.
  long long part = 0;
  for (int j = tid; j < (int)blockIdx.x; j += kClassifyThreads) part += recs[j].count;
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) s_part[wave] = part;
  __syncthreads();
  if (tid == 0) {
    long long b = 0;
    for (int w = 0; w < kClassifyThreads / 64; ++w) b += s_part[w];
    s_base = b;
  }
  __syncthreads();
  long long base = s_base;

  const int64_t tile0 = (int64_t)blockIdx.x * kClassifyTile;
  for (int j = 0; j < kRowsPerThread; ++j) {
    const int64_t r = tile0 + (int64_t)j * kClassifyThreads + tid;
    const bool a = (r < p.N) && p.active[r];
    const unsigned long long m = __ballot(a);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int woff = 0, tot = 0;
    for (int w = 0; w < kClassifyThreads / 64; ++w) {
      woff += (w < wave) ? s_wave[w] : 0;
      tot += s_wave[w];
    }
    if (a) rows[base + woff + before] = (int32_t)r;
    base += tot;
    __syncthreads();
  }

  // Tile 0 folds the per-tile records into the header.
  if (blockIdx.x == 0) {
    __shared__ uint32_t s_err;
    __shared__ unsigned long long s_bm, s_bt;
    __shared__ long long s_tot[kClassifyThreads / 64];
    if (tid == 0) { s_err = 0; s_bm = ~0ull; s_bt = ~0ull; }
    __syncthreads();
    long long tot = 0;
    for (int j = tid; j < nblk; j += kClassifyThreads) {
      const TileRec rc = recs[j];
      tot += rc.count;
      if (rc.err_bits) {
        atomicOr(&s_err, rc.err_bits);
        atomicMin(&s_bm, rc.first_bad_mask);
        atomicMin(&s_bt, rc.first_bad_token);
      }
    }
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane == 0) s_tot[wave] = tot;
    __syncthreads();
    if (tid == 0) {
      long long t = 0;
      for (int w = 0; w < kClassifyThreads / 64; ++w) t += s_tot[w];
      WsHeader* h = (WsHeader*)p.ws;
      h->err_bits = s_err;
      h->magic = kWsMagic;
      h->n_active = t;
      h->first_bad[kErrMask] = s_bm;
      h->first_bad[kErrToken] = s_bt;
      h->first_bad[kErrNonfinite] = ~0ull;
      h->first_bad[3] = ~0ull;
    }
  }
}

}  // namespace

hipError_t launch_classify(const ClassifyParams& p, hipStream_t s) {
  const int nblk = (int)((p.N + kClassifyTile - 1) / kClassifyTile);
  if (nblk > 0) {
    hipLaunchKernelGGL(classify_count, dim3(nblk), dim3(kClassifyThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compact_scatter, dim3(nblk > 0 ? nblk : 1), dim3(kClassifyThreads), 0, s,
                     p, nblk);
  return hipGetLastError();
}

}  // namespace drift
