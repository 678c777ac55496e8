// Internal definitions shared by the HIP sources of the drift library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drift.h"
#include "rowio.h"

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

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of drift_selected_logprob: the header only.
constexpr size_t kLogprobWsBytes = sizeof(WsHeader);

__device__ __forceinline__ void record_error(WsHeader* h, ErrClass c, int64_t row) {
  atomicOr(&h->err_bits, 1u << c);
  atomicMin(&h->first_bad[c], (unsigned long long)row);
}

// ---- launchers (each defined next to its kernels) --------------------------------
struct ScoreParams {
  int64_t N, V, stride, L, nseq;  // V: columns of the row that enter the log-sum-exp
  int64_t Vid;                    // selected ids must lie in [0, Vid)
  int32_t dtype, ids_i64, layout;
  Chain xf[2];                    // transform chain per side (train, rollout)
  const void* train;
  const void* rollout;
  const void* ids;
  const uint8_t* att;
  const uint8_t* act;
  const int32_t* cu;
  float* out_t;
  float* out_r;
  float* out_d;
  uint8_t* active;
  float* ent[2];   // optional per-row entropy of each side's softmax
  double* lse[2];  // optional per-row natural-log LSE of each side
  char* ws;
  // exact mode / vocab shards: global column of the row's first column, and (shard
  // export) the per-side partial outputs; null = finalize the row here
  int64_t vstart;
  drift_lse_partial* part[2];
  int64_t row0;  // first row of the launch (set by the launcher)
};
// Launches the header initialisation and the scoring kernel; `ev` (nullable) are recorded
// right before and after the scoring kernel.
hipError_t launch_score(const ScoreParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// The exact-mode scoring kernel (order-independent sums), finalizing or exporting shard
// partials.
hipError_t launch_score_exact(const ScoreParams& p, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1);
constexpr int kMaxShards = 64;
struct MergeParams {
  ScoreParams p;  // classification inputs and the outputs
  const drift_lse_partial* part[2];  // [S][N] per side
  int32_t S;
  int64_t bound[kMaxShards + 1];     // shard s owns global columns [bound[s], bound[s+1])
};
hipError_t launch_merge_shards(const MergeParams& m, hipStream_t s);

struct DiagParams {
  int64_t N;
  double eps_low, eps_high;
  const float* d;
  const uint8_t* active;
  const WsHeader* lp;  // nullable: header of the drift_selected_logprob call that made d
  char* ws;
  drift_stats* out;    // nullable: where the statistics go (null = the workspace's record)
};

// Status recorded in a logprob workspace header (priority mask > token > non-finite).
__host__ __device__ inline int header_status(uint32_t magic, uint32_t err_bits) {
  if (magic != kWsMagic) return DRIFT_EWORKSPACE;
  if (err_bits & (1u << kErrMask)) return DRIFT_EMASK;
  if (err_bits & (1u << kErrToken)) return DRIFT_ETOKEN;
  if (err_bits & (1u << kErrNonfinite)) return DRIFT_ENONFINITE;
  return DRIFT_OK;
}
struct SegParams {
  int64_t N, S;
  double eps_low, eps_high;
  const float* d;
  const uint8_t* active;
  const int32_t* off;  // [S + 1] segment row offsets
  const WsHeader* lp;  // nullable
  drift_stats* out;    // [S], device
};
hipError_t launch_segment_diagnostics(const SegParams& p, hipStream_t s);
size_t diag_ws_bytes(int64_t N);
// The diagnostics scratch of the current device for drift_diagnostics_noalloc (a
// file-scope device array of the diagnostics source; its address is looked up once per
// device).
hipError_t diag_noalloc_scratch(char** ptr, size_t* bytes);
size_t diag_stats_offset();
hipError_t launch_diagnostics(const DiagParams& p, hipStream_t s);

struct LmheadParams {
  int64_t T, H, V;
  bool w_vh;  // weight stored [V, H] (K contiguous) instead of [H, V]
  Chain xf;   // transform chain of the head's logits (n = 0: none)
  const void* hidden;
  const void* weight;
  const int32_t* ids;
  const uint8_t* active;
  float* logp;
  char* ws;
};
size_t lmhead_ws_bytes(int64_t T, int64_t H, int64_t V, bool w_vh);
bool lmhead_shape_ok(int64_t T, int64_t V);  // the GEMM grid fits one dispatch
hipError_t launch_lmhead(const LmheadParams& p, hipStream_t s);

struct DlogitsParams {
  int64_t N, V, Vr, stride, out_stride;  // Vr: columns that entered the log-sum-exp
  int32_t dtype, ids_i64, out_dtype;
  Chain xf;
  const void* logits;
  const void* ids;
  const double* lse;
  const uint8_t* active;
  const float* grad;  // nullable: 1 on every active row
  void* out;
  int64_t row0;  // first row of the launch (set by the launcher)
};
hipError_t launch_dlogits(const DlogitsParams& p, hipStream_t s);

int64_t compact_tiles(int64_t N);
size_t compact_ws_bytes(int64_t N);
hipError_t launch_compact(const uint8_t* active, int64_t N, int32_t* rows, int64_t* n_out,
                          char* ws, hipStream_t s);

}  // namespace drift
