// Gradient of the selected-token logprob with respect to the stored logits
// ("[WS2] Framework for ablation experiment", LogProb knobs row 11: dlogits).
//
// For an active row with selected id y, upstream gradient g = dL/dlogp and logits z =
// chain(x) (the side's transform chain; identity when empty):
//   dL/dx_v = g * ([v == y] - p_v) * dz_v/dx_v,   p_v = exp(z_v - LSE(z)),  v < Vr,
// and 0 for columns Vr <= v < V, which never entered the log-sum-exp. LSE comes from the
// forward scoring pass of the same logits, so a row is read once here and written once:
// an elementwise, HBM-bound pass. The exponent z_v - LSE is formed in fp64 and rounded
// once to fp32 before exp2, so p_v carries the error of one exp2 and one rounding.
// Inactive rows are written with zeros; an active row whose LSE is NaN (an id the
// forward pass rejected) comes out NaN over [0, Vr). A chain with at most one soft-cap step
// is taken in its folded form (rowio.h), as the scoring pass forms its log-sum-exp terms
// when both sides' chains fold.
#include <math.h>

#include "classify.h"
#include "common.h"
#include "rowio.h"

namespace drift {
namespace {

constexpr double kLog2eD = 1.44269504088896340736;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Gradient rows are written once and not read back by this pass. A lane's output group
// that one 16-byte store covers goes out as a streaming (nontemporal) store; a wider group
// (bf16 logits -> fp32 gradient: two 16-byte halves from two store instructions) uses
// plain stores, so that L2 merges the halves into whole lines before they reach HBM
// (measured on MI355X: 4.9 TB/s with plain stores, 3.4 TB/s with streaming ones).
template <bool kStream, typename V_>
__device__ __forceinline__ void put(V_ v, V_* p) {
  if constexpr (kStream) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename O> struct Out;
template <> struct Out<float> {
  template <int VEC>
  __device__ static __forceinline__ void group(void* row, int64_t g, const float (&v)[VEC]) {
    u32x4* q = (u32x4*)row + g * (VEC / 4);
    constexpr bool kStream = VEC == 4;
#pragma unroll
    for (int j = 0; j < VEC / 4; ++j) {
      u32x4 w;
      w.x = __float_as_uint(v[4 * j]);
      w.y = __float_as_uint(v[4 * j + 1]);
      w.z = __float_as_uint(v[4 * j + 2]);
      w.w = __float_as_uint(v[4 * j + 3]);
      put<kStream>(w, q + j);
    }
  }
  __device__ static __forceinline__ void one(void* row, int64_t i, float v) {
    ((float*)row)[i] = v;
  }
};
template <> struct Out<uint16_t> {  // bf16 bit patterns
  template <int VEC>
  __device__ static __forceinline__ void group(void* row, int64_t g, const float (&v)[VEC]) {
    uint32_t w[VEC / 2];
#pragma unroll
    for (int j = 0; j < VEC / 2; ++j) w[j] = bf16_bits(v[2 * j]) | (bf16_bits(v[2 * j + 1]) << 16);
    if constexpr (VEC == 8) {
      u32x4 q;
      q.x = w[0];
      q.y = w[1];
      q.z = w[2];
      q.w = w[3];
      put<true>(q, (u32x4*)row + g);
    } else {
      u32x2 q;
      q.x = w[0];
      q.y = w[1];
      put<true>(q, (u32x2*)row + g);
    }
  }
  __device__ static __forceinline__ void one(void* row, int64_t i, float v) {
    ((uint16_t*)row)[i] = (uint16_t)bf16_bits(v);
  }
};

// dL/dx for the VEC logits of group g (columns c0 .. c0+VEC-1). XF: 0 no chain, 1 the
// chain step by step, 2 the folded chain (rowio.h): z = fa + fb v with v = g(x) for a
// soft-cap (slope fdz g (1 - g)) or v = x for multiplying steps (slope fb), the same
// values the scoring pass's log-sum-exp terms were formed from; the exponent
// z log2(e) - LSE log2(e) is then one fp64 FMA of v.
template <int VEC, int XF>
__device__ __forceinline__ void grad_group(float (&x)[VEC], int64_t c0, int64_t y, int64_t Vr,
                                           double L2, float g, const Chain& c) {
  float dz[VEC];
  double sl = kLog2eD, base = -L2;  // exponent = v * sl + base
  if constexpr (XF == 2) {
    if (c.kind == 2) {
      fold_values<VEC>(x, c);
#pragma unroll
      for (int e = 0; e < VEC; ++e) dz[e] = c.fdz * fmaf(-x[e], x[e], x[e]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) dz[e] = c.fb;
    }
    sl = c.fbld;
    base = c.fald - L2;
  } else if constexpr (XF == 1) {
    apply_chain_grad<VEC>(x, dz, c);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) dz[e] = 1.0f;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int64_t col = c0 + e;
    const float a = (float)fma((double)x[e], sl, base);
    const float pv = __builtin_amdgcn_exp2f(a);
    const float oh = col == y ? 1.0f : 0.0f;
    const float gv = (g * dz[e]) * (oh - pv);
    x[e] = col < Vr ? gv : 0.0f;
  }
}

template <typename T, typename O, int NT, int U, int XF>
__global__ void __launch_bounds__(NT) dlogits_rows(DlogitsParams p) {
  constexpr int VEC = Elem<T>::kVec;
  const int64_t r = p.row0 + blockIdx.x;
  const int tid = threadIdx.x;
  const char* row = (const char*)p.logits + (size_t)r * (size_t)p.stride * sizeof(T);
  char* orow = (char*)p.out + (size_t)r * (size_t)p.out_stride * sizeof(O);
  const int64_t V = p.V;
  const bool act = p.active[r] != 0;
  const int64_t y = act ? load_id(p.ids, r, p.ids_i64) : -1;
  const double L2 = act ? p.lse[r] * kLog2eD : 0.0;
  const float g = act ? (p.grad ? p.grad[r] : 1.0f) : 0.0f;
  const int64_t Vr = act ? p.Vr : 0;  // inactive rows: every column is written as 0
  const int64_t nfull = V / VEC;
  const int64_t ngroups = (V + VEC - 1) / VEC;
  const bool vec = ((((uintptr_t)row) | ((uintptr_t)orow)) & 15) == 0;
  int64_t gi = tid;
  if (vec) {
    const u32x4* src = (const u32x4*)row;
    for (; gi + (U - 1) * NT < nfull; gi += U * NT) {
      u32x4 b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = act ? __builtin_nontemporal_load(src + gi + u * NT) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elem<T>::unpack(b[u], x);
        grad_group<VEC, XF>(x, (gi + u * NT) * VEC, y, Vr, L2, g, p.xf);
        Out<O>::template group<VEC>(orow, gi + u * NT, x);
      }
    }
    for (; gi < nfull; gi += NT) {
      float x[VEC];
      Elem<T>::unpack(act ? __builtin_nontemporal_load(src + gi) : u32x4{0, 0, 0, 0}, x);
      grad_group<VEC, XF>(x, gi * VEC, y, Vr, L2, g, p.xf);
      Out<O>::template group<VEC>(orow, gi, x);
    }
  }
  for (; gi < ngroups; gi += NT) {  // unaligned rows, and the ragged last group
    float x[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int64_t i = gi * VEC + e;
      x[e] = (act && i < V) ? Elem<T>::load1(row, i) : 0.0f;
    }
    grad_group<VEC, XF>(x, gi * VEC, y, Vr, L2, g, p.xf);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int64_t i = gi * VEC + e;
      if (i < V) Out<O>::one(orow, i, x[e]);
    }
  }
}

#ifndef DRIFT_DLOGITS_THREADS
#define DRIFT_DLOGITS_THREADS 256
#endif
#ifndef DRIFT_DLOGITS_UNROLL
#define DRIFT_DLOGITS_UNROLL 4
#endif

template <typename T, typename O>
void launch_typed(const DlogitsParams& p, hipStream_t s) {
  constexpr int NT = DRIFT_DLOGITS_THREADS, U = DRIFT_DLOGITS_UNROLL;
  // at most 2^32 - 1 work-items per dispatch: larger batches take several launches over
  // consecutive row ranges (p.row0 = first row of the launch)
  const int64_t per = (int64_t)(0xffffffffu / (unsigned)NT);
  DlogitsParams q = p;
  for (int64_t r0 = 0; r0 < p.N; r0 += per) {
    q.row0 = r0;
    const dim3 grid((unsigned)(p.N - r0 < per ? p.N - r0 : per));
    if (p.xf.n == 0)
      hipLaunchKernelGGL((dlogits_rows<T, O, NT, U, 0>), grid, dim3(NT), 0, s, q);
    else if (p.xf.kind != 0)
      hipLaunchKernelGGL((dlogits_rows<T, O, NT, U, 2>), grid, dim3(NT), 0, s, q);
    else
      hipLaunchKernelGGL((dlogits_rows<T, O, NT, U, 1>), grid, dim3(NT), 0, s, q);
  }
}

}  // namespace

hipError_t launch_dlogits(const DlogitsParams& p, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  if (p.dtype == DRIFT_BF16) {
    if (p.out_dtype == DRIFT_BF16) launch_typed<uint16_t, uint16_t>(p, s);
    else launch_typed<uint16_t, float>(p, s);
  } else {
    if (p.out_dtype == DRIFT_BF16) launch_typed<float, uint16_t>(p, s);
    else launch_typed<float, float>(p, s);
  }
  return hipGetLastError();
}

}  // namespace drift
