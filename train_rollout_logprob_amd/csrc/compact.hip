// Stable compaction of the active rows: rows[0 .. n) = the indices r with active[r] != 0,
// ascending ("WS2 Cross-Config Logprob Drift Contract", Measurement Contract: only the
// active response/action tokens enter the comparison). Callers use the list to gather or
// scatter per-token results of the active rows only.
//
// Two launches over tiles of kCompactTile rows:
//   compact_count    one block per tile: the tile's active count;
//   compact_scatter  one block per tile: adds the counts of the tiles before it (integer,
//                    exact), then walks its tile in 16 rounds of 256 consecutive rows; a
//                    round ranks its active rows with wave ballots and a 4-entry LDS
//                    prefix, so rows are written in ascending order. The last tile also
//                    writes n.
#include "common.h"

namespace drift {
namespace {

constexpr int kCompactThreads = 256;
constexpr int kCompactRounds = 16;
constexpr int kCompactTile = kCompactThreads * kCompactRounds;
constexpr int kCompactWaves = kCompactThreads / 64;

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

__global__ void __launch_bounds__(kCompactThreads) compact_scatter(
    const uint8_t* __restrict__ active, int64_t N, const int32_t* __restrict__ counts,
    int32_t* __restrict__ rows, int64_t* __restrict__ n_out) {
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
  long long part = 0;
  for (int g = tid; g < (int)blockIdx.x; g += kCompactThreads) part += counts[g];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) s_part[wave] = part;
  __syncthreads();
  long long off = 0;
  for (int w = 0; w < kCompactWaves; ++w) off += s_part[w];
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

size_t compact_ws_bytes(int64_t N) { return align_up((size_t)compact_tiles(N) * 4, 256); }

hipError_t launch_compact(const uint8_t* active, int64_t N, int32_t* rows, int64_t* n_out,
                          char* ws, hipStream_t s) {
  const int64_t G = compact_tiles(N);
  int32_t* counts = (int32_t*)ws;
  hipLaunchKernelGGL(compact_count, dim3((unsigned)G), dim3(kCompactThreads), 0, s, active, N,
                     counts);
  hipLaunchKernelGGL(compact_scatter, dim3((unsigned)G), dim3(kCompactThreads), 0, s, active, N,
                     (const int32_t*)counts, rows, n_out);
  return hipGetLastError();
}

}  // namespace drift
