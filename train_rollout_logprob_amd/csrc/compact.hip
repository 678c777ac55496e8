// Stable compaction of the active rows: rows[0 .. n) = the indices r with active[r] != 0,
// ascending ("WS2 Cross-Config Logprob Drift Contract", Measurement Contract: only the
// active response/action tokens enter the comparison). Callers use the list to gather or
// scatter per-token results of the active rows only.
//
// Launches over tiles of kCompactTile rows:
//   compact_count    one block per tile: the tile's active count;
//   compact_scan     above kCompactDirectTiles tiles only: one block forms every tile's
//                    offset (the exclusive prefix of the counts, int64);
//   compact_scatter  one block per tile: takes its offset from compact_scan, or with
//                    fewer tiles adds the counts of the tiles before it itself (at most
//                    4 loads per thread; integer, exact), then walks its tile in 16 rounds
//                    of 256 consecutive rows; a round ranks its active rows with wave
//                    ballots and a 4-entry LDS prefix, so rows are written in ascending
//                    order. The last tile also writes n.
#include "common.h"

namespace drift {
namespace {

constexpr int kCompactThreads = 256;
constexpr int kCompactRounds = 16;
constexpr int kCompactTile = kCompactThreads * kCompactRounds;
constexpr int kCompactWaves = kCompactThreads / 64;
constexpr int64_t kCompactDirectTiles = 1024;  // in-block prefix up to this many tiles
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kCompactThreads) compact_count(const uint8_t* __restrict__ active,
                                                                 int64_t N,
                                                                 int32_t* __restrict__ counts) {
  __shared__ int s_w[kCompactWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * kCompactTile;
  uint8_t f[kCompactRounds];
#pragma unroll
  for (int j = 0; j < kCompactRounds; ++j) {
    const int64_t r = base + (int64_t)j * kCompactThreads + tid;
    f[j] = r < N ? active[r] : (uint8_t)0;
  }
  int c = 0;
#pragma unroll
  for (int j = 0; j < kCompactRounds; ++j) c += __popcll(__ballot(f[j] != 0));
  if (lane == 0) s_w[wave] = c;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kCompactWaves; ++w) t += s_w[w];
    counts[blockIdx.x] = t;
  }
}

// One block: offs[g] = counts[0] + ... + counts[g - 1]. Thread t owns the contiguous run
// of tiles [t·per, (t+1)·per): it sums the run, a block scan of the run sums gives the
// run's first offset, and the thread walks the run again writing offsets.
__global__ void __launch_bounds__(kScanThreads) compact_scan(const int32_t* __restrict__ counts,
                                                             int64_t G,
                                                             long long* __restrict__ offs) {
  __shared__ long long s_w[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = (G + kScanThreads - 1) / kScanThreads;
  const int64_t lo = (int64_t)tid * per < G ? (int64_t)tid * per : G;
  const int64_t hi = lo + per < G ? lo + per : G;
  long long sum = 0;
  for (int64_t g = lo; g < hi; ++g) sum += counts[g];
  long long x = sum;  // inclusive scan over the wave's lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  long long run = x - sum;
  for (int w = 0; w < wave; ++w) run += s_w[w];
  for (int64_t g = lo; g < hi; ++g) {
    offs[g] = run;
    run += counts[g];
  }
}

__global__ void __launch_bounds__(kCompactThreads) compact_scatter(
    const uint8_t* __restrict__ active, int64_t N, const int32_t* __restrict__ counts,
    const long long* __restrict__ offs, int32_t* __restrict__ rows,
    int64_t* __restrict__ n_out) {
  __shared__ long long s_part[kCompactWaves];
  __shared__ int s_w[kCompactWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * kCompactTile;
  uint8_t f[kCompactRounds];
#pragma unroll
  for (int j = 0; j < kCompactRounds; ++j) {
    const int64_t r = base + (int64_t)j * kCompactThreads + tid;
    f[j] = r < N ? active[r] : (uint8_t)0;
  }
  // rows of the tiles before this one
  long long off = 0;
  if (offs) {
    off = offs[blockIdx.x];
  } else {
    long long part = 0;
    for (int g = tid; g < (int)blockIdx.x; g += kCompactThreads) part += counts[g];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) s_part[wave] = part;
    __syncthreads();
    for (int w = 0; w < kCompactWaves; ++w) off += s_part[w];
  }
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kCompactRounds; ++j) {
    const bool a = f[j] != 0;
    const unsigned long long m = __ballot(a);
    if (lane == 0) s_w[wave] = __popcll(m);
    __syncthreads();
    long long before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kCompactWaves; ++w) {
      before += w < wave ? s_w[w] : 0;
      total += s_w[w];
    }
    if (a) rows[off + before + __popcll(m & below)] = (int32_t)(base + (int64_t)j * kCompactThreads + tid);
    off += total;
    __syncthreads();  // s_w is rewritten by the next round
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) *n_out = off;
}

}  // namespace

int64_t compact_tiles(int64_t N) {
  const int64_t g = (N + kCompactTile - 1) / kCompactTile;
  return g > 0 ? g : 1;
}

// per-tile counts (int32), then above kCompactDirectTiles tiles the offsets (int64)
size_t compact_ws_bytes(int64_t N) {
  const int64_t G = compact_tiles(N);
  return align_up((size_t)G * 4, 256) + (G > kCompactDirectTiles ? align_up((size_t)G * 8, 256)
                                                                  : 0);
}

hipError_t launch_compact(const uint8_t* active, int64_t N, int32_t* rows, int64_t* n_out,
                          char* ws, hipStream_t s) {
  const int64_t G = compact_tiles(N);
  int32_t* counts = (int32_t*)ws;
  long long* offs = nullptr;
  hipLaunchKernelGGL(compact_count, dim3((unsigned)G), dim3(kCompactThreads), 0, s, active, N,
                     counts);
  if (G > kCompactDirectTiles) {
    offs = (long long*)(ws + align_up((size_t)G * 4, 256));
    hipLaunchKernelGGL(compact_scan, dim3(1), dim3(kScanThreads), 0, s, (const int32_t*)counts,
                       G, offs);
  }
  hipLaunchKernelGGL(compact_scatter, dim3((unsigned)G), dim3(kCompactThreads), 0, s, active, N,
                     (const int32_t*)counts, (const long long*)offs, rows, n_out);
  return hipGetLastError();
}

}  // namespace drift
