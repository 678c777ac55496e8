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
struct Chain {
  int32_t n;
  int32_t op[DRIFT_MAX_TRANSFORMS];
  float v[DRIFT_MAX_TRANSFORMS];
  float inv[DRIFT_MAX_TRANSFORMS];
};

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
