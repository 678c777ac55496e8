// Per-row classification and logical-input validation (device code, header-only).
//
// Active rows are the attended response/action rows ("WS2 Cross-Config Logprob Drift
// Contract", Measurement Contract); a logical-input violation (mask shape, padding side,
// out-of-range selected id) makes the comparison invalid rather than noisy (same page,
// "Logical Input and Metadata Drift"), so it is recorded as an error class instead of
// being scored as drift.
#pragma once

#include "common.h"

namespace drift {

struct RowClass {
  bool active;     // attended and action row
  bool score;      // active with a selected id inside [0, V)
  int64_t y;       // selected id (valid when score)
  uint32_t err;    // error-class bits found on this row
};

__device__ __forceinline__ int64_t load_id(const void* ids, int64_t r, int32_t i64) {
  return i64 ? ((const int64_t*)ids)[r] : (int64_t)((const int32_t*)ids)[r];
}

// `end` is the packed-buffer end (cu_seqlens[num_seqs] clamped to [0, N]); unused otherwise.
__device__ __forceinline__ RowClass classify_row(const ScoreParams& p, int64_t r, int64_t end) {
  RowClass c;
  c.err = 0;
  const uint8_t a = p.att ? p.att[r] : (uint8_t)1;
  const uint8_t m = p.act ? p.act[r] : (uint8_t)1;
  bool emask = (a > 1) || (m > 1);
  bool real;
  if (p.layout == DRIFT_PACKED) {
    real = r < end;
    if (p.att && ((a != 0) != real)) emask = true;
  } else {
    real = a != 0;
    if (p.att) {  // one contiguous attended block on the declared side of each sequence
      const int64_t t = r % p.L;
      if (t + 1 < p.L) {
        const uint8_t a2 = p.att[r + 1];
        if (p.layout == DRIFT_PAD_RIGHT && a == 0 && a2 != 0) emask = true;
        if (p.layout == DRIFT_PAD_LEFT && a != 0 && a2 == 0) emask = true;
      }
    }
  }
  if (m != 0 && !real) emask = true;  // an action row must be attended
  if (emask) c.err |= 1u << kErrMask;
  c.active = real && (m != 0);
  c.score = false;
  c.y = -1;
  if (c.active) {
    c.y = load_id(p.ids, r, p.ids_i64);
    if (c.y < 0 || c.y >= p.Vid) {
      c.err |= 1u << kErrToken;
    } else {
      c.score = true;
    }
  }
  return c;
}

}  // namespace drift
