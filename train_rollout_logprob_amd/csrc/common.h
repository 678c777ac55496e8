// Internal definitions shared by the HIP sources of the drift library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drift.h"

namespace drift {

// Device error classes recorded in the workspace header (bit i = class i).
enum ErrClass : uint32_t { kErrMask = 0, kErrToken = 1, kErrNonfinite = 2, kNumErr = 3 };

// Workspace header of drift_selected_logprob / drift_lmhead_logprob. 256 bytes, at the
// start of the workspace; rewritten by every call.
struct WsHeader {
  uint32_t err_bits;
  uint32_t magic;
  int64_t n_active;
  unsigned long long first_bad[4];  // smallest offending row per class, ~0 if none
  int64_t reserved[26];
};
static_assert(sizeof(WsHeader) == 256, "header size");
constexpr uint32_t kWsMagic = 0x44524654u;  // "DRFT"

// Classification tiles: a block of 256 threads covers kClassifyTile consecutive rows.
constexpr int kClassifyThreads = 256;
constexpr int kClassifyTile = 2048;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout of drift_selected_logprob.
struct LogprobWs {
  size_t rows_off, counts_off, total;
  __host__ __device__ static LogprobWs make(int64_t N) {
    LogprobWs w;
    size_t nblk = (size_t)((N + kClassifyTile - 1) / kClassifyTile);
    w.rows_off = 256;
    w.counts_off = w.rows_off + align_up((size_t)N * 4, 256);
    w.total = w.counts_off + align_up(nblk * 32 + 32, 256);
    return w;
  }
};

__device__ __forceinline__ void record_error(WsHeader* h, ErrClass c, int64_t row) {
  atomicOr(&h->err_bits, 1u << c);
  atomicMin(&h->first_bad[c], (unsigned long long)row);
}

// ---- launchers (each defined next to its kernels) --------------------------------
struct ClassifyParams {
  int64_t N, V, B, L, nseq;
  int32_t layout, ids_i64;
  const void* ids;
  const uint8_t* att;
  const uint8_t* act;
  const int32_t* cu;
  float* out_t;
  float* out_r;
  float* out_d;
  uint8_t* active;
  char* ws;
};
hipError_t launch_classify(const ClassifyParams& p, hipStream_t s);

struct ScoreParams {
  int64_t N, V, stride;
  int32_t dtype, ids_i64;
  const void* train;
  const void* rollout;
  const void* ids;
  float* out_t;
  float* out_r;
  float* out_d;
  char* ws;
};
hipError_t launch_score(const ScoreParams& p, hipStream_t s);

struct DiagParams {
  int64_t N;
  double eps_low, eps_high;
  const float* d;
  const uint8_t* active;
  char* ws;
};
size_t diag_ws_bytes(int64_t N);
size_t diag_stats_offset();
hipError_t launch_diagnostics(const DiagParams& p, hipStream_t s);

struct LmheadParams {
  int64_t T, H, V;
  const void* hidden;
  const void* weight;
  const int32_t* ids;
  const uint8_t* active;
  float* logp;
  char* ws;
};
size_t lmhead_ws_bytes(int64_t T, int64_t V);
hipError_t launch_lmhead(const LmheadParams& p, hipStream_t s);

}  // namespace drift
