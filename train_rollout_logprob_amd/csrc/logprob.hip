// Paired one-pass selected-token log-softmax for the train and rollout logits.
//
// For an active row r with selected id y, each side computes
//   logp = x_y - LSE(x),  LSE(x) = log(sum_i exp(x_i))
// and dlogp = train_logp - rollout_logp ("WS2 Cross-Config Logprob Drift Contract",
// Measurement Contract). Both rows are streamed once from HBM.
//
// Arithmetic (precision and downcast points, "[WS2] Framework for ablation experiment",
// LogProb knobs row 6):
//   * stored logits (fp32, or bf16 widened exactly) are read as fp32;
//   * each lane keeps (k, s): k an integer-valued float, a power-of-two running maximum
//     k = ceil(max_i x_i * log2e); s = sum_i 2^(x_i*log2e - k) in fp64. A vector of
//     16 bytes of logits contributes fp32 terms exp2(fma(x, log2e, -k)) summed in fp32,
//     then added to s in fp64. Raising k rescales s by an exact power of two (ldexp);
//   * lanes, waves and the block merge (k, s) pairs in a fixed order; the online
//     softmax tiling of LogProb knobs row 10 with the merge in a fixed global order of
//     row 5. The element -> lane -> wave mapping depends only on V and the compile-time
//     block shape, so a row's bits never depend on the batch it is in (the
//     batch-composition control of the "Attention Debug Matrix" page);
//   * LSE is exported in the natural-log domain: lse = (k + log2 s) * ln2 in fp64
//     (Attention knobs row 6, LSE domain); logp and dlogp are formed in fp64 and rounded
//     once to fp32.
// The selected logit is read once by its single owner (LogProb knobs row 8).
#include <math.h>

#include "common.h"

namespace drift {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;      // log2(e), rounded to fp32
constexpr double kLn2 = 0.693147180559945309417232121458;  // ln(2), rounded to fp64

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Adds one group of VEC logits to a lane's partial, in a fixed order.
template <int VEC>
__device__ __forceinline__ void push(Acc& a, const float (&x)[VEC]) {
  float m = x[0];
#pragma unroll
  for (int i = 1; i < VEC; ++i) m = fmaxf(m, x[i]);
  const float kn = ceilf(m * kLog2e);
  if (kn > a.k) {
    if (kn == INFINITY) {
      a.s = NAN;  // +inf logit, or |x| too large for the fp32 exponent: fail closed
    } else {
      a.s = rescale(a.s, a.k, kn);
      a.k = kn;
    }
  }
  float e[VEC];
  if (a.k == -INFINITY) {
    // Every logit seen so far is -inf (probability zero) or NaN.
#pragma unroll
    for (int i = 0; i < VEC; ++i) e[i] = (x[i] == -INFINITY) ? 0.0f : NAN;
  } else {
    const float nk = -a.k;
#pragma unroll
    for (int i = 0; i < VEC; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, nk));
  }
  // pairwise fp32 sum of the group, then one fp64 add
#pragma unroll
  for (int w = 1; w < VEC; w *= 2) {
#pragma unroll
    for (int i = 0; i + w < VEC; i += 2 * w) e[i] = e[i] + e[i + w];
  }
  a.s += (double)e[0];
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;
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

__device__ __forceinline__ int64_t load_id(const void* ids, int64_t r, int32_t i64) {
  return i64 ? ((const int64_t*)ids)[r] : (int64_t)((const int32_t*)ids)[r];
}

// Lane `tid` owns the 16-byte groups v = tid, tid + NT, tid + 2NT, ... of the row and
// pushes them in ascending order; the last partial group (V % VEC logits, padded with
// -inf) belongs to the lane that would own group V / VEC. U groups per side are loaded
// ahead for memory-level parallelism; U does not change the arithmetic.
template <typename T, int NT, int U, bool kAligned>
__device__ __forceinline__ void stream_row(const void* rt, const void* rr, int64_t V, int tid,
                                           Acc& at, Acc& ar) {
  constexpr int VEC = Elem<T>::kVec;
  const int64_t nvec = V / VEC;
  int64_t v = tid;
  if constexpr (kAligned) {
    const u32x4* vt = (const u32x4*)rt;
    const u32x4* vr = (const u32x4*)rr;
    const int64_t nround = nvec / ((int64_t)NT * U);
    for (int64_t it = 0; it < nround; ++it) {
      u32x4 bt[U], br[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bt[u] = __builtin_nontemporal_load(vt + v + u * NT);
        br[u] = __builtin_nontemporal_load(vr + v + u * NT);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elem<T>::unpack(bt[u], x);
        push<VEC>(at, x);
        Elem<T>::unpack(br[u], x);
        push<VEC>(ar, x);
      }
      v += (int64_t)NT * U;
    }
    for (; v < nvec; v += NT) {
      const u32x4 bt = __builtin_nontemporal_load(vt + v);
      const u32x4 br = __builtin_nontemporal_load(vr + v);
      float x[VEC];
      Elem<T>::unpack(bt, x);
      push<VEC>(at, x);
      Elem<T>::unpack(br, x);
      push<VEC>(ar, x);
    }
  } else {
    for (; v < nvec; v += NT) {
      float xt[VEC], xr[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        xt[e] = Elem<T>::load1(rt, v * VEC + e);
        xr[e] = Elem<T>::load1(rr, v * VEC + e);
      }
      push<VEC>(at, xt);
      push<VEC>(ar, xr);
    }
  }
  if (v == nvec && nvec * VEC < V) {  // the ragged tail group
    float xt[VEC], xr[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int64_t i = nvec * VEC + e;
      xt[e] = (i < V) ? Elem<T>::load1(rt, i) : -INFINITY;
      xr[e] = (i < V) ? Elem<T>::load1(rr, i) : -INFINITY;
    }
    push<VEC>(at, xt);
    push<VEC>(ar, xr);
  }
}

template <typename T, int NT, int U>
__global__ void __launch_bounds__(NT) score_rows(ScoreParams p) {
  constexpr int NW = NT / 64;
  __shared__ float s_k[2][NW];
  __shared__ double s_s[2][NW];
  WsHeader* h = (WsHeader*)p.ws;
  const int64_t i = blockIdx.x;
  if (i >= h->n_active) return;
  const int32_t* rows = (const int32_t*)(p.ws + LogprobWs::make(p.N).rows_off);
  const int64_t r = rows[i];
  const int64_t y = load_id(p.ids, r, p.ids_i64);
  const int tid = threadIdx.x;
  if (y < 0 || y >= p.V) {  // recorded as a token error by the classification pass
    if (tid == 0) {
      p.out_t[r] = NAN;
      p.out_r[r] = NAN;
      p.out_d[r] = NAN;
    }
    return;
  }
  const size_t off = (size_t)r * (size_t)p.stride * sizeof(T);
  const char* rt = (const char*)p.train + off;
  const char* rr = (const char*)p.rollout + off;

  Acc at = {-INFINITY, 0.0}, ar = {-INFINITY, 0.0};
  if ((((uintptr_t)rt | (uintptr_t)rr) & 15) == 0) {
    stream_row<T, NT, U, true>(rt, rr, p.V, tid, at, ar);
  } else {
    stream_row<T, NT, U, false>(rt, rr, p.V, tid, at, ar);
  }

  // wave butterfly, then waves in index order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Acc bt, br;
    bt.k = __shfl_xor(at.k, o);
    bt.s = __shfl_xor(at.s, o);
    br.k = __shfl_xor(ar.k, o);
    br.s = __shfl_xor(ar.s, o);
    at = merge(at, bt);
    ar = merge(ar, br);
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    s_k[0][wave] = at.k;
    s_s[0][wave] = at.s;
    s_k[1][wave] = ar.k;
    s_s[1][wave] = ar.s;
  }
  __syncthreads();
  if (tid == 0) {
    Acc T_ = {s_k[0][0], s_s[0][0]}, R_ = {s_k[1][0], s_s[1][0]};
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      T_ = merge(T_, Acc{s_k[0][w], s_s[0][w]});
      R_ = merge(R_, Acc{s_k[1][w], s_s[1][w]});
    }
    const float xty = Elem<T>::load1(rt, y);
    const float xry = Elem<T>::load1(rr, y);
    const double lse_t = ((double)T_.k + log2(T_.s)) * kLn2;
    const double lse_r = ((double)R_.k + log2(R_.s)) * kLn2;
    p.out_t[r] = (float)((double)xty - lse_t);
    p.out_r[r] = (float)((double)xry - lse_r);
    p.out_d[r] = (float)(((double)xty - (double)xry) - (lse_t - lse_r));
    const bool ok = (T_.s > 0.0) && (T_.s < INFINITY) && (R_.s > 0.0) && (R_.s < INFINITY) &&
                    (xty > -INFINITY) && (xry > -INFINITY);
    if (!ok) record_error(h, kErrNonfinite, r);
  }
}

constexpr int kScoreThreads = 256;
constexpr int kScoreUnroll = 4;

}  // namespace

hipError_t launch_score(const ScoreParams& p, hipStream_t s) {
  if (p.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)p.N), block(kScoreThreads);
  if (p.dtype == DRIFT_BF16) {
    hipLaunchKernelGGL((score_rows<uint16_t, kScoreThreads, kScoreUnroll>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((score_rows<float, kScoreThreads, kScoreUnroll>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace drift
