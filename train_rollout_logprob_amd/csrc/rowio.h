// Row access shared by the streaming kernels: 16-byte groups of stored logits widened to
// fp32, and the per-side logit transform chain ("[WS2] Framework for ablation
// experiment", LogProb knobs row 7) with its derivative (row 11, dlogits).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "drift.h"

namespace drift {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // logits per 16-byte group
  __device__ static __forceinline__ void unpack(const u32x4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return ((const float*)p)[i];
  }
};
template <> struct Elem<uint16_t> {  // bf16 bit patterns
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void unpack(const u32x4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return __uint_as_float(((uint32_t)((const uint16_t*)p)[i]) << 16);
  }
};

// One side's transform chain as the kernels read it: steps in order, each multiplying by
// v (SCALE: the value, TEMPERATURE: its reciprocal) or, for SOFTCAP, x -> v * tanh(x * inv)
// with inv = 1 / v.
//
// The same chain folded into one step for the log-sum-exp terms of the scoring kernels
// (tree and exact reductions) and for the gradient (dlogits) (kind != 0): z = fa + fb g(x),
// with
//   kind 1 (multiplying steps only): g(x) = x, fa = 0, fb = the product of the factors;
//   kind 2 (one SOFTCAP step of value c, factor p before it and q after it):
//     g(x) = 1 / (1 + 2^(fc * x)), fc = 2 log2(e) p / c, fa = q c, fb = -2 q c,
//   from tanh(u) = 1 - 2 / (e^(2u) + 1) (the logistic form of tanh), so that
//   q c tanh(p x / c) = fa + fb g(x); g takes one hardware exp2 and one reciprocal, and
//   fa + fb g is within 3.6e-7 |fa| of the exact value (measured over every bf16 input
//   with both instructions off by one ulp either way); used when |fa| <= 40;
//   kind 0: two or more SOFTCAP steps, or a fold out of those bounds (no fold).
// The selected logit always takes the step-by-step chain (apply_chain).
// fal = fa log2(e) and fbl = fb log2(e) make the exponent z log2(e) - k one FMA of g.
struct Chain {
  int32_t n;
  int32_t op[DRIFT_MAX_TRANSFORMS];
  float v[DRIFT_MAX_TRANSFORMS];
  float inv[DRIFT_MAX_TRANSFORMS];
  int32_t kind;
  float fc, fa, fb, fal, fbl;
  // kind 2: |z| <= |fa|, so a fixed exponent offset ceil(|fa| log2 e) + 1 keeps every term
  // in [2^-118, 2^-1] (|fa| <= 40) and the running maximum is not needed
  float kfix;
  // the gradient's form (dlogits): fa log2(e) and fb log2(e) in fp64, and the slope
  // dz/dx = fb (kind 1) or fdz g (1 - g) with fdz = 4 p q (kind 2: the derivative of
  // q c tanh(p x / c) is p q (1 - tanh^2) and 1 - tanh^2 = 4 g (1 - g))
  double fald, fbld;
  float fdz;
  // the log-sum-exp of the folded terms back in natural log: terms 2^(fbl g + fal - k)
  // sum to 2^L with L = k + log2 s, and LSE(z) = fa + (L - fal) * lse_scale with
  // lse_scale = fb / fbl in fp64 (ln 2 when fb = 0), which undoes the fp32 rounding of
  // fbl and fal instead of assuming fbl = fb log2(e) exactly
  double lse_scale;
};

// g(x) of the folded chain, in place (kind 1: unchanged). The chain is a kernel argument,
// so the branch is uniform. 2^(fc x) overflows to +inf for large fc x, and g is then 0:
// the soft-cap's saturation; fc x = -inf gives g = 1.
template <int VEC>
__device__ __forceinline__ void fold_values(float (&x)[VEC], const Chain& c) {
  if (c.kind == 2) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      x[e] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x[e] * c.fc) + 1.0f);
  }
}

// Applies the chain to a group in place. Branches are uniform (the chain is a kernel
// argument).
template <int VEC>
__device__ __forceinline__ void apply_chain(float (&x)[VEC], const Chain& c) {
#pragma unroll
  for (int i = 0; i < DRIFT_MAX_TRANSFORMS; ++i) {
    if (i >= c.n) break;
    const float v = c.v[i];
    if (c.op[i] == DRIFT_XF_SOFTCAP) {
      const float inv = c.inv[i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = v * tanhf(x[e] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[e] = x[e] * v;
    }
  }
}

// The same chain, also returning dz/dx per element: the product of the step derivatives
// (v for a multiplying step, 1 - tanh^2 for SOFTCAP) taken at each step's input.
template <int VEC>
__device__ __forceinline__ void apply_chain_grad(float (&x)[VEC], float (&dz)[VEC],
                                                 const Chain& c) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) dz[e] = 1.0f;
#pragma unroll
  for (int i = 0; i < DRIFT_MAX_TRANSFORMS; ++i) {
    if (i >= c.n) break;
    const float v = c.v[i];
    if (c.op[i] == DRIFT_XF_SOFTCAP) {
      const float inv = c.inv[i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float t = tanhf(x[e] * inv);
        dz[e] = dz[e] * fmaf(-t, t, 1.0f);
        x[e] = v * t;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        dz[e] = dz[e] * v;
        x[e] = x[e] * v;
      }
    }
  }
}

}  // namespace drift
