// Log-sum-exp partials in the power-of-two form used by every kernel of the library.
//
// A partial (k, s) stands for 2^k * s = sum_i 2^(x_i*kLog2e) over the logits it covers,
// with s = sum_i 2^(x_i*kLog2e - k) accumulated in fp64 and k an integer-valued float
// (-inf while empty). Merging rescales by exact powers of two (ldexp), so the only
// roundings are the fp64 adds; merges happen in a fixed order chosen by each kernel (the
// online-softmax merge of "[WS2] Framework for ablation experiment", LogProb knobs rows 5
// and 10, and Attention knobs row 7). LSE is exported in the natural-log domain:
// lse = (k + log2 s) / kLog2e (Attention knobs row 6). kLog2e is log2(e) rounded to fp32,
// so the terms are exponentials of x * kLog2e * ln2 = x (1 - 1.3e-8); dividing by the same
// kLog2e returns LSE(x) up to 1.3e-8 (ln V + the spread of the logits), where multiplying
// by ln 2 would leave LSE(x (1 - 1.3e-8)), 1.3e-5 off at logits of 1000.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace drift {

constexpr float kLog2e = 1.44269504088896340736f;          // log2(e), rounded to fp32
constexpr double kLn2 = 0.693147180559945309417232121458;  // ln(2), rounded to fp64
constexpr double kInvLog2e = 1.0 / (double)kLog2e;          // 1 / the fp32 log2(e)

// Exponent range of the partials. k = ceil(m * log2e) is taken from the fp32 product, so it
// can sit half an fp32 ulp of that product away from the exact exponent of the largest
// logit m, and each term 2^(fma(x, log2e, -k)) carries that offset: at most 32 below
// |k| = 2^30, which the fp32 terms and the fp64 sums absorb. A row whose largest exponent
// reaches 2^30 in magnitude (|max logit| above about 7.4e8) fails closed: a kernel raising
// k to 2^30 or beyond poisons the partial with NaN, and one whose maximum lies below -2^30
// clamps k at -2^30, which the row's final check rejects.
constexpr float kMaxK = 1073741824.0f;  // 2^30
__device__ __forceinline__ bool k_ok(float k) { return fabsf(k) < kMaxK; }

struct Acc {
  float k;   // -inf while empty, else an integer
  double s;  // sum of 2^(x*log2e - k); 0 or NaN while empty
};

__device__ __forceinline__ double rescale(double s, float k, float K) {
  // s * 2^(k - K) for k <= K; empty partials keep their 0 (or NaN).
  return (k == -INFINITY) ? s : ldexp(s, (int)fmaxf(k - K, -2048.0f));
}

__device__ __forceinline__ Acc merge(const Acc& a, const Acc& b) {
  Acc r;
  r.k = fmaxf(a.k, b.k);
  if (r.k == -INFINITY) {
    r.s = a.s + b.s;
  } else {
    r.s = rescale(a.s, a.k, r.k) + rescale(b.s, b.k, r.k);
  }
  return r;
}

__device__ __forceinline__ double lse_of(const Acc& a) {
  return ((double)a.k + log2(a.s)) * kInvLog2e;
}

// A finite, non-empty partial (some logit finite, none NaN or +inf).
__device__ __forceinline__ bool lse_ok(const Acc& a) { return a.s > 0.0 && a.s < INFINITY; }

// Partial with the first moment of the exponent, for the entropy of the softmax:
// s2 = sum_i 2^(a_i) a_i with a_i = x_i*log2e - k. Then, with p_i = 2^(a_i) / s,
//   H = -sum_i p_i ln p_i = ln2 (log2 s - s2 / s)
// ("[WS2] Framework for ablation experiment", LogProb knobs row 11, entropy). Moving the
// reference from k to K >= k shifts every a_i by k - K, so
//   s2 -> 2^(k-K) (s2 - (K - k) s),   s -> 2^(k-K) s.
struct AccE {
  float k;
  double s;
  double s2;
};

__device__ __forceinline__ double rescale2(double s2, double s, float k, float K) {
  return (k == -INFINITY) ? s2
                          : ldexp(s2 - (double)(K - k) * s, (int)fmaxf(k - K, -2048.0f));
}

__device__ __forceinline__ AccE merge(const AccE& a, const AccE& b) {
  AccE r;
  r.k = fmaxf(a.k, b.k);
  if (r.k == -INFINITY) {
    r.s = a.s + b.s;
    r.s2 = a.s2 + b.s2;
  } else {
    r.s2 = rescale2(a.s2, a.s, a.k, r.k) + rescale2(b.s2, b.s, b.k, r.k);
    r.s = rescale(a.s, a.k, r.k) + rescale(b.s, b.k, r.k);
  }
  return r;
}

__device__ __forceinline__ double lse_of(const AccE& a) {
  return ((double)a.k + log2(a.s)) * kInvLog2e;
}
__device__ __forceinline__ bool lse_ok(const AccE& a) { return a.s > 0.0 && a.s < INFINITY; }
__device__ __forceinline__ double entropy_of(const AccE& a) {
  return (log2(a.s) - a.s2 / a.s) * kLn2;
}

}  // namespace drift
