// Order-independent log-sum-exp accumulation: the exact mode of the scoring kernel and the
// vocab-shard partials ("[WS2] Framework for ablation experiment", LogProb knobs rows 3-5:
// shard ownership, partial reduction, merge order; the tp-partition control of the
// "Attention Debug Matrix" page's Metrics section).
//
// The fixed-tree mode (lse.h) sums fp64 partials in an order fixed by V, so a row's bits
// depend on how its columns are split. Here the sum is exact integer arithmetic, so any
// split of a row into pieces, reduced in any order and merged in any order, gives the
// same bits:
//   * a group of VEC consecutive columns (aligned to VEC in the global column index) gives
//     one value G * 2^n, with n = ceil(x * log2 e) of the group's first logit (of its
//     largest where the first does not serve, group_piece) and G = sum of
//     exp2(x * log2 e - n) in fp32, pairwise: a function of the group alone;
//   * the value's 24 mantissa bits are cut at absolute bit positions that are multiples
//     of 32 ("bins") and added as integers into the bins;
//   * an accumulator keeps the three highest bins it has seen (top, top-1, top-2) in
//     uint64, dropping lower ones. A bin never carries into another, so the final bins
//     are the sums, over all groups, of each group's pieces in bins >= top_final - 2,
//     whatever the order of the additions.
// The kept window spans at least 55 bits below the largest group's leading bit: the
// truncation costs less than #groups * 2^-55 relative (about 1e-12 at V = 151936).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lse.h"

namespace drift {

constexpr int32_t kEmptyTop = -(1 << 28);         // top of an accumulator that saw nothing
constexpr float kMaxGroupExp = 16777216.0f;       // |n| limit (|x| < 1.16e7): else fail closed

struct AccX {
  int32_t top;   // bin index of b2; kEmptyTop while empty
  uint32_t bad;  // a NaN or +inf logit, or an exponent out of range
  uint64_t b2, b1, b0;
};

__device__ __forceinline__ AccX accx_empty() {
  AccX a;
  a.top = kEmptyTop;
  a.bad = 0;
  a.b2 = a.b1 = a.b0 = 0;
  return a;
}

// Moves the window up to T >= a.top, dropping the bins that fall out.
__device__ __forceinline__ void accx_shift(AccX& a, int32_t T) {
  const int32_t d = T - a.top;
  if (d <= 0) return;
  if (d == 1) {
    a.b0 = a.b1;
    a.b1 = a.b2;
    a.b2 = 0;
  } else if (d == 2) {
    a.b0 = a.b2;
    a.b1 = 0;
    a.b2 = 0;
  } else {
    a.b0 = a.b1 = a.b2 = 0;
  }
  a.top = T;
}

__device__ __forceinline__ AccX merge(AccX a, AccX b) {
  const int32_t T = a.top > b.top ? a.top : b.top;
  accx_shift(a, T);
  accx_shift(b, T);
  a.b2 += b.b2;
  a.b1 += b.b1;
  a.b0 += b.b0;
  a.bad |= b.bad;
  return a;
}

// The integer pieces of one group: value = hi * 2^(32 (bin + 1)) + lo * 2^(32 bin).
struct GroupPiece {
  int32_t bin;    // meaningless when live == 0 (the pieces are 0 then)
  uint32_t hi, lo;
  uint32_t live;  // 0: every logit of the group is -inf (adds nothing)
  uint32_t bad;
};

// sum of exp2(x * log2e - n) over the group in fp32, pairwise
template <int VEC>
__device__ __forceinline__ float group_exp_sum(const float (&x)[VEC], float n) {
  float e[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, -n));
#pragma unroll
  for (int st = 1; st < VEC; st *= 2) {
#pragma unroll
    for (int i = 0; i + st < VEC; i += 2 * st) e[i] = e[i] + e[i + st];
  }
  return e[0];
}

// The group's exponent n is taken from its first logit: that term is then in (1/2, 1], so
// G >= 1/2, and G stays finite while no logit of the group exceeds the first by more than
// about 88. Otherwise (first logit -inf or out of range, G overflowing, a NaN or +inf
// logit) n comes from the group's maximum, where G is in [1, 8] for finite logits. Either
// way G * 2^n is a function of the group alone. Only the maximum-based exponent decides
// failure: the first-logit path requires |n| <= 2^24 - 128, and a finite G there bounds
// the maximum's exponent by n + 128.
template <int VEC>
__device__ __forceinline__ GroupPiece group_piece(const float (&x)[VEC]) {
  GroupPiece g;
  float n = ceilf(x[0] * kLog2e);
  float G = group_exp_sum<VEC>(x, n);
  bool live = true;
  bool ok = fabsf(n) <= kMaxGroupExp - 128.0f && G <= 3.4028235e38f;  // false for NaN
  if (!ok) {
    float m = x[0];
#pragma unroll
    for (int i = 1; i < VEC; ++i) m = fmaxf(m, x[i]);  // NaN-ignoring
    live = m != -INFINITY;
    n = live ? ceilf(m * kLog2e) : 0.0f;
    G = group_exp_sum<VEC>(x, n);
    // NaN, +inf or a huge exponent fail closed
    ok = fabsf(n) <= kMaxGroupExp && G >= 0.125f && G <= 64.0f;
  }
  g.bad = (live && !ok) ? 1u : 0u;
  g.live = (live && ok) ? 1u : 0u;
  const uint32_t bits = __float_as_uint(G);
  const int32_t eg = (int32_t)((bits >> 23) & 0xffu) - 127;
  const uint64_t mant = (uint64_t)((bits & 0x7fffffu) | 0x800000u);
  const int32_t p = (int32_t)n + eg - 23;  // exponent of the mantissa's lowest bit
  g.bin = p >> 5;                          // floor(p / 32)
  const uint64_t v = mant << (uint32_t)(p & 31);
  g.lo = g.live ? (uint32_t)v : 0u;
  g.hi = g.live ? (uint32_t)(v >> 32) : 0u;
  return g;
}

// Adds a group's pieces to an accumulator whose window already reaches bin + 1 (a group
// that is not live has zero pieces). Branch-free: each bin takes the piece that lands in it.
__device__ __forceinline__ void accx_add(AccX& a, const GroupPiece& g) {
  a.bad |= g.bad;
  const int32_t rel = a.top - (g.bin + 1);
  a.b2 += (uint64_t)(rel == 0 ? g.hi : 0u);
  a.b1 += (uint64_t)(rel == 0 ? g.lo : (rel == 1 ? g.hi : 0u));
  a.b0 += (uint64_t)(rel == 1 ? g.lo : (rel == 2 ? g.hi : 0u));
}

// log2 of the accumulated value (-inf when empty). The three bins are combined into one
// 128-bit integer, normalised to 64 bits (a sticky bit keeps the rounding direction) and
// converted once.
__device__ __forceinline__ double accx_log2(const AccX& a) {
  const uint64_t lo = a.b0 + (a.b1 << 32);
  const uint64_t carry = lo < a.b0 ? 1u : 0u;
  const uint64_t hi = a.b2 + (a.b1 >> 32) + carry;
  if (hi == 0 && lo == 0) return -INFINITY;
  double mant;
  int e;
  if (hi == 0) {
    mant = (double)lo;
    e = 0;
  } else {
    const int lz = __clzll((long long)hi);
    uint64_t top = lz ? ((hi << lz) | (lo >> (64 - lz))) : hi;
    const uint64_t rest = lz ? (lo << lz) : lo;
    top |= rest != 0 ? 1u : 0u;
    mant = (double)top;
    e = 64 - lz;
  }
  return log2(mant) + (double)e + 32.0 * (double)(a.top - 2);
}

}  // namespace drift
