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
//   * each lane keeps (k, s) with s = sum_i 2^(x_i*log2e - k) in fp64 and k an integer
//     shared by the 64 lanes of a wave: a power-of-two running maximum. A group of 16
//     bytes of logits contributes fp32 terms exp2(fma(x, log2e, -k)) summed in fp32,
//     then added to s in fp64. When some lane's group sum reaches 16 (a term above 2^4,
//     the first group, or a non-finite logit) the wave raises k to ceil(max x * log2e)
//     over the wave's group and rescales s by an exact power of two (ldexp). Terms
//     therefore never exceed 2^4 and the running maximum costs one compare per group;
//   * lanes, waves and the block merge (k, s) pairs in a fixed order; the online
//     softmax tiling of LogProb knobs row 10 with the merge in a fixed global order of
//     row 5. The element -> lane -> wave mapping depends only on V and the compile-time
//     block shape, so a row's bits never depend on the batch it is in (the
//     batch-composition control of the "Attention Debug Matrix" page);
//   * LSE is exported in the natural-log domain: lse = (k + log2 s) / log2e in fp64, with
//     the same fp32 log2e the exponents used (lse.h; Attention knobs row 6, LSE domain);
//     logp and dlogp are formed in fp64 and rounded once to fp32;
//   * a per-side transform chain (LogProb knobs row 7) with at most one soft-cap step is
//     folded for the log-sum-exp terms (rowio.h): the exponent is one FMA of the value
//     g(x), and a soft-capped side, whose logits are bounded by the cap, keeps a fixed k
//     instead of the running maximum. The selected logit takes the chain step by step.
// The selected logit is read once by its single owner (LogProb knobs row 8).
//
// The same file holds the kernels of the optional outputs and modes, which share the row
// streaming above: the entropy instantiation of score_rows (a second fp64 moment per
// partial, LogProb knobs row 11), and score_rows_exact with merge_shards, the
// order-independent reduction (exact.h) used unsharded or for vocabulary shards whose
// partials are merged in global shard order (LogProb knobs rows 3-5).
#include <math.h>

#include <type_traits>

#include "classify.h"
#include "common.h"
#include "exact.h"
#include "lse.h"
#include "rowio.h"

namespace drift {
namespace {

constexpr float kRaise = 16.0f;  // a group sum at or above this raises the wave's k

// A group's values as the log-sum-exp reads them, with z(i) the logit and expo(i, base(nk))
// the exponent z log2e - k for nk = -k: the logits themselves (Plain), or the values g of a
// folded chain with z = fa + fb g (Folded; rowio.h), whose exponent is one FMA of g.
template <int VEC> struct Plain {
  const float (&x)[VEC];
  __device__ __forceinline__ float z(int i) const { return x[i]; }
  __device__ __forceinline__ float base(float nk) const { return nk; }
  __device__ __forceinline__ float expo(int i, float c) const { return fmaf(x[i], kLog2e, c); }
};
template <int VEC> struct Folded {
  const float (&g)[VEC];
  const Chain& ch;
  __device__ __forceinline__ float z(int i) const { return fmaf(ch.fb, g[i], ch.fa); }
  __device__ __forceinline__ float base(float nk) const { return ch.fal + nk; }
  __device__ __forceinline__ float expo(int i, float c) const { return fmaf(g[i], ch.fbl, c); }
};

// Natural-log LSE of a side whose terms 2^(fbl g + fal - k) came from the folded chain c:
// fa + (log2 of the sum - fal) * fb / fbl (rowio.h).
template <typename A>
__device__ __forceinline__ double lse_folded(const A& a, const Chain& c) {
  return (double)c.fa + (((double)a.k + log2(a.s)) - (double)c.fal) * c.lse_scale;
}

// exp2 terms of one group in fp32, summed pairwise; with ENT also the first moment of
// the exponent, sum of 2^a * a over the group (a = x*log2e - k) as a chain of fp32 FMAs in
// element order; -inf exponents contribute 0. The moment is first taken without a guard: a
// -inf exponent then gives 0 * -inf = NaN, and only such groups (masked or -inf columns)
// take it again with the exponent clamped to -1e30. Both give the same bits wherever the
// first is not NaN (a term with a below -1e30 has 2^a = 0 and adds a signed zero to the
// chain either way).
template <int VEC, bool ENT, typename G>
__device__ __forceinline__ void group_sums(const G& grp, float nk, float& t, float& t2) {
  const float c = grp.base(nk);
  float e[VEC];
  float w = 0.0f;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const float a = grp.expo(i, c);
    e[i] = __builtin_amdgcn_exp2f(a);
    if constexpr (ENT) w = fmaf(e[i], a, w);
  }
  if constexpr (ENT) {
    if (w != w) {
      w = 0.0f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) w = fmaf(e[i], fmaxf(grp.expo(i, c), -1.0e30f), w);
    }
  }
#pragma unroll
  for (int st = 1; st < VEC; st *= 2) {
#pragma unroll
    for (int i = 0; i + st < VEC; i += 2 * st) e[i] = e[i] + e[i + st];
  }
  t = e[0];
  t2 = w;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  return m;
}

// Adds one group of VEC logits to a lane's partial (Acc, or AccE with the entropy moment).
// Every lane of the wave calls it at the same point (groups past the end of the row are all
// -inf), so k stays wave-uniform.
template <int VEC, typename A, typename G>
__device__ __forceinline__ void push_group(A& a, const G& grp) {
  constexpr bool ENT = std::is_same<A, AccE>::value;
  float t, t2;
  group_sums<VEC, ENT>(grp, -a.k, t, t2);
  if (__ballot(!(t < kRaise))) {  // wave-uniform: raise k
    float m = grp.z(0);
#pragma unroll
    for (int i = 1; i < VEC; ++i) m = fmaxf(m, grp.z(i));
    m = wave_max(m);  // NaN-ignoring; -inf if every logit in the wave's group is -inf/NaN
    const float kn = ceilf(m * kLog2e);
    if (kn > a.k) {
      if (!(kn < kMaxK)) {
        a.s = NAN;  // +inf logit, or a maximum beyond the exponent range (lse.h): fail closed
        if constexpr (ENT) a.s2 = NAN;
      } else {
        // a maximum below -2^30 clamps k (lse.h); the row's final check rejects such a k
        const float kc = fmaxf(kn, -kMaxK);
        if (kc > a.k) {
          if constexpr (ENT) a.s2 = rescale2(a.s2, a.s, a.k, kc);
          a.s = rescale(a.s, a.k, kc);
          a.k = kc;
        }
      }
    }
    if (a.k == -INFINITY) {
      // every logit seen so far by the wave is -inf (probability zero) or NaN
      t = 0.0f;
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        if (!(grp.z(i) == -INFINITY)) t = NAN;
      t2 = t;
    } else {
      group_sums<VEC, ENT>(grp, -a.k, t, t2);
    }
  }
  a.s += (double)t;
  if constexpr (ENT) a.s2 += (double)t2;
}

template <int VEC, typename A>
__device__ __forceinline__ void push(A& a, const float (&x)[VEC]) {
  push_group<VEC>(a, Plain<VEC>{x});
}

// A group of a folded soft-cap chain (kind 2) with the fixed offset k = kfix: every term is
// within [2^-118, 2^-1], so there is nothing to raise; a NaN value makes the sum NaN.
template <int VEC, typename A, typename G>
__device__ __forceinline__ void push_fixed(A& a, const G& grp) {
  constexpr bool ENT = std::is_same<A, AccE>::value;
  float t, t2;
  group_sums<VEC, ENT>(grp, -a.k, t, t2);
  a.s += (double)t;
  if constexpr (ENT) a.s2 += (double)t2;
}

// Exact mode: one group's integer pieces into the lane's bins. The window top is raised
// for the whole wave at once (ballot + max), as k is in the fixed-tree mode.
template <int VEC>
__device__ __forceinline__ void push(AccX& a, const float (&x)[VEC]) {
  const GroupPiece g = group_piece<VEC>(x);
  const int32_t need = g.live ? g.bin + 1 : kEmptyTop;
  if (__ballot(need > a.top)) {
    int32_t T = need;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int32_t u = __shfl_xor(T, o);
      T = u > T ? u : T;
    }
    accx_shift(a, T);
  }
  accx_add(a, g);
}

// Lane `tid` owns the 16-byte groups g = tid, tid + NT, tid + 2NT, ... of the row and
// pushes them in ascending order; the last partial group (V % VEC logits, padded with
// -inf) belongs to the lane that would own group V / VEC. All lanes run the same number
// of pushes (missing groups are all -inf and add exactly 0). U groups per side are
// loaded ahead for memory-level parallelism; U does not change the arithmetic. XF: 0 no
// chain, 1 chains applied step by step, 2 both chains folded (rowio.h).
template <typename T, int NT, int U, bool kAligned, int XF, typename A>
__device__ __forceinline__ void stream_row(const char* rt, const char* rr, int64_t V, int tid,
                                           A& at, A& ar, const ScoreParams& p) {
  constexpr int VEC = Elem<T>::kVec;
  const int64_t nfull = V / VEC;                      // complete groups
  const int64_t ngroups = (V + VEC - 1) / VEC;        // including the ragged one
  const int64_t full_iters = nfull / NT;              // iterations where every lane is full
  const int64_t iters = (ngroups + NT - 1) / NT;
  int64_t j = 0;
  if constexpr (XF == 2 && !std::is_same<A, AccX>::value) {
    // a folded soft-cap side starts at its fixed offset (rowio.h)
    if (p.xf[0].kind == 2) at.k = p.xf[0].kfix;
    if (p.xf[1].kind == 2) ar.k = p.xf[1].kfix;
  }
  if constexpr (kAligned) {
    const u32x4* vt = (const u32x4*)rt;
    const u32x4* vr = (const u32x4*)rr;
    for (; j + U <= full_iters; j += U) {
      u32x4 bt[U], br[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t g = (j + u) * NT + tid;
        bt[u] = __builtin_nontemporal_load(vt + g);
        br[u] = __builtin_nontemporal_load(vr + g);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[VEC];
        if constexpr (XF == 2 && std::is_same<A, AccX>::value) {
          // exact mode, folded chains: the logits z = fa + fb g, as in the ragged group
          Elem<T>::unpack(bt[u], x);
          fold_values<VEC>(x, p.xf[0]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) x[e] = fmaf(p.xf[0].fb, x[e], p.xf[0].fa);
          push<VEC>(at, x);
          Elem<T>::unpack(br[u], x);
          fold_values<VEC>(x, p.xf[1]);
#pragma unroll
          for (int e = 0; e < VEC; ++e) x[e] = fmaf(p.xf[1].fb, x[e], p.xf[1].fa);
          push<VEC>(ar, x);
        } else if constexpr (XF == 2) {  // both chains folded: the terms from g (rowio.h)
          Elem<T>::unpack(bt[u], x);
          fold_values<VEC>(x, p.xf[0]);
          if (p.xf[0].kind == 2)
            push_fixed<VEC>(at, Folded<VEC>{x, p.xf[0]});
          else
            push_group<VEC>(at, Folded<VEC>{x, p.xf[0]});
          Elem<T>::unpack(br[u], x);
          fold_values<VEC>(x, p.xf[1]);
          if (p.xf[1].kind == 2)
            push_fixed<VEC>(ar, Folded<VEC>{x, p.xf[1]});
          else
            push_group<VEC>(ar, Folded<VEC>{x, p.xf[1]});
        } else {
          Elem<T>::unpack(bt[u], x);
          if constexpr (XF == 1) apply_chain<VEC>(x, p.xf[0]);
          push<VEC>(at, x);
          Elem<T>::unpack(br[u], x);
          if constexpr (XF == 1) apply_chain<VEC>(x, p.xf[1]);
          push<VEC>(ar, x);
        }
      }
    }
  }
  for (; j < iters; ++j) {
    const int64_t g = j * NT + tid;
    float xt[VEC], xr[VEC];
    if (kAligned && g < nfull) {
      Elem<T>::unpack(__builtin_nontemporal_load((const u32x4*)rt + g), xt);
      Elem<T>::unpack(__builtin_nontemporal_load((const u32x4*)rr + g), xr);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int64_t i = g * VEC + e;
        xt[e] = (i < V) ? Elem<T>::load1(rt, i) : 0.0f;
        xr[e] = (i < V) ? Elem<T>::load1(rr, i) : 0.0f;
      }
    }
    if constexpr (XF == 2) {  // the folded chain's logits, z = fa + fb g
      fold_values<VEC>(xt, p.xf[0]);
      fold_values<VEC>(xr, p.xf[1]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        xt[e] = fmaf(p.xf[0].fb, xt[e], p.xf[0].fa);
        xr[e] = fmaf(p.xf[1].fb, xr[e], p.xf[1].fa);
      }
    } else if constexpr (XF == 1) {
      apply_chain<VEC>(xt, p.xf[0]);
      apply_chain<VEC>(xr, p.xf[1]);
    }
    // columns past the end are -inf after the chain (a chain may map -inf to a finite value)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (g * VEC + e >= V) {
        xt[e] = -INFINITY;
        xr[e] = -INFINITY;
      }
    }
    push<VEC>(at, xt);
    push<VEC>(ar, xr);
  }
}

// Header initialisation (and the packed-metadata check) before the scoring kernel.
__global__ void __launch_bounds__(256) init_header(ScoreParams p) {
  __shared__ uint32_t s_err;
  WsHeader* h = (WsHeader*)p.ws;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  __syncthreads();
  if (p.layout == DRIFT_PACKED) {  // cu_seqlens starts at 0, never decreases, ends inside
    for (int64_t i = tid; i <= p.nseq; i += 256) {
      const int64_t c = p.cu[i];
      if ((i == 0 && c != 0) || (i > 0 && c < (int64_t)p.cu[i - 1]) || c > p.N)
        atomicOr(&s_err, 1u << kErrMask);
    }
  }
  __syncthreads();
  if (tid == 0) {
    h->err_bits = s_err;
    h->magic = kWsMagic;
    h->n_active = 0;
    h->first_bad[kErrMask] = s_err ? 0ull : ~0ull;
    h->first_bad[kErrToken] = ~0ull;
    h->first_bad[kErrNonfinite] = ~0ull;
    h->first_bad[3] = ~0ull;
  }
}

// One block per row: thread 0 classifies and validates the row; active rows with a valid
// id are streamed by the whole block.
template <typename T, int NT, int U, int XF, bool ENT>
__global__ void __launch_bounds__(NT) score_rows(ScoreParams p) {
  using A = std::conditional_t<ENT, AccE, Acc>;
  constexpr int NW = NT / 64;
  __shared__ float s_k[2][NW];
  __shared__ double s_s[2][NW];
  __shared__ double s_s2[2][ENT ? NW : 1];
  __shared__ int64_t s_y;
  WsHeader* h = (WsHeader*)p.ws;
  const int64_t r = p.row0 + blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int64_t end = p.N;
    if (p.layout == DRIFT_PACKED) {
      end = (int64_t)p.cu[p.nseq];
      end = end < 0 ? 0 : (end > p.N ? p.N : end);
    }
    const RowClass c = classify_row(p, r, end);
    p.active[r] = c.active ? 1 : 0;
    if (c.err & (1u << kErrMask)) record_error(h, kErrMask, r);
    if (c.err & (1u << kErrToken)) record_error(h, kErrToken, r);
    if (!c.score) {  // inactive rows get 0, active rows with a bad id NaN
      const float f = c.active ? NAN : 0.0f;
      p.out_t[r] = f;
      p.out_r[r] = f;
      p.out_d[r] = f;
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        if (p.ent[side]) p.ent[side][r] = f;
        if (p.lse[side]) p.lse[side][r] = (double)f;
      }
    }
    s_y = c.score ? c.y : -1;
  }
  __syncthreads();
  const int64_t y = s_y;
  if (y < 0) return;  // block-uniform

  const size_t off = (size_t)r * (size_t)p.stride * sizeof(T);
  const char* rt = (const char*)p.train + off;
  const char* rr = (const char*)p.rollout + off;
  A at, ar;
  at.k = ar.k = -INFINITY;
  at.s = ar.s = 0.0;
  if constexpr (ENT) at.s2 = ar.s2 = 0.0;
  if ((((uintptr_t)rt | (uintptr_t)rr) & 15) == 0) {
    stream_row<T, NT, U, true, XF>(rt, rr, p.V, tid, at, ar, p);
  } else {
    stream_row<T, NT, U, false, XF>(rt, rr, p.V, tid, at, ar, p);
  }

  // lanes (fixed butterfly), then waves in index order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    A bt, br;
    bt.k = __shfl_xor(at.k, o);
    bt.s = __shfl_xor(at.s, o);
    br.k = __shfl_xor(ar.k, o);
    br.s = __shfl_xor(ar.s, o);
    if constexpr (ENT) {
      bt.s2 = __shfl_xor(at.s2, o);
      br.s2 = __shfl_xor(ar.s2, o);
    }
    at = merge(at, bt);
    ar = merge(ar, br);
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    s_k[0][wave] = at.k;
    s_s[0][wave] = at.s;
    s_k[1][wave] = ar.k;
    s_s[1][wave] = ar.s;
    if constexpr (ENT) {
      s_s2[0][wave] = at.s2;
      s_s2[1][wave] = ar.s2;
    }
  }
  __syncthreads();
  if (tid == 0) {
    auto lds = [&](int side, int w) {
      A v;
      v.k = s_k[side][w];
      v.s = s_s[side][w];
      if constexpr (ENT) v.s2 = s_s2[side][w];
      return v;
    };
    A T_ = lds(0, 0), R_ = lds(1, 0);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      T_ = merge(T_, lds(0, w));
      R_ = merge(R_, lds(1, w));
    }
    float xty = Elem<T>::load1(rt, y);
    float xry = Elem<T>::load1(rr, y);
    if constexpr (XF) {  // the selected logit goes through the same chain
      float one[1] = {xty};
      apply_chain<1>(one, p.xf[0]);
      xty = one[0];
      one[0] = xry;
      apply_chain<1>(one, p.xf[1]);
      xry = one[0];
    }
    // a side whose maximum exponent left the range (lse.h) gives NaN outputs; folded
    // chains take their own way back to natural log (rowio.h)
    const bool kt = k_ok(T_.k), kr = k_ok(R_.k);
    const double lse_t = !kt ? (double)NAN : XF == 2 ? lse_folded(T_, p.xf[0]) : lse_of(T_);
    const double lse_r = !kr ? (double)NAN : XF == 2 ? lse_folded(R_, p.xf[1]) : lse_of(R_);
    p.out_t[r] = (float)((double)xty - lse_t);
    p.out_r[r] = (float)((double)xry - lse_r);
    p.out_d[r] = (float)(((double)xty - (double)xry) - (lse_t - lse_r));
    if (p.lse[0]) p.lse[0][r] = lse_t;
    if (p.lse[1]) p.lse[1][r] = lse_r;
    if constexpr (ENT) {
      if (p.ent[0]) p.ent[0][r] = kt ? (float)entropy_of(T_) : NAN;
      if (p.ent[1]) p.ent[1][r] = kr ? (float)entropy_of(R_) : NAN;
    }
    const bool ok = lse_ok(T_) && lse_ok(R_) && kt && kr && (xty > -INFINITY) &&
                    (xry > -INFINITY);
    if (!ok) record_error(h, kErrNonfinite, r);
  }
}

// ---- exact mode (order-independent sums) and vocabulary shards ----------------------

__device__ __forceinline__ AccX shfl_xor_acc(const AccX& a, int o) {
  AccX b;
  b.top = __shfl_xor(a.top, o);
  b.bad = __shfl_xor(a.bad, o);
  b.b2 = __shfl_xor(a.b2, o);
  b.b1 = __shfl_xor(a.b1, o);
  b.b0 = __shfl_xor(a.b0, o);
  return b;
}

__device__ __forceinline__ AccX from_partial(const drift_lse_partial& q) {
  AccX a;
  a.top = q.top;
  a.bad = (q.flags & DRIFT_PART_BAD) ? 1u : 0u;
  a.b2 = q.bin[0];
  a.b1 = q.bin[1];
  a.b0 = q.bin[2];
  return a;
}

// Outputs of one scored row from its two exact sums and selected logits; shared by the
// unsharded exact kernel and the shard merge, so both give the same bits.
__device__ __forceinline__ void finish_row_exact(const ScoreParams& p, WsHeader* h, int64_t r,
                                                 const AccX& T_, const AccX& R_, float xty,
                                                 float xry) {
  const double lse_t = T_.bad ? (double)NAN : accx_log2(T_) * kInvLog2e;
  const double lse_r = R_.bad ? (double)NAN : accx_log2(R_) * kInvLog2e;
  p.out_t[r] = (float)((double)xty - lse_t);
  p.out_r[r] = (float)((double)xry - lse_r);
  p.out_d[r] = (float)(((double)xty - (double)xry) - (lse_t - lse_r));
  if (p.lse[0]) p.lse[0][r] = lse_t;
  if (p.lse[1]) p.lse[1][r] = lse_r;
  const bool ok = isfinite(lse_t) && isfinite(lse_r) && (xty > -INFINITY) && (xry > -INFINITY);
  if (!ok) record_error(h, kErrNonfinite, r);
}

__device__ __forceinline__ void unscored_outputs(const ScoreParams& p, int64_t r, bool active) {
  const float f = active ? NAN : 0.0f;
  p.out_t[r] = f;
  p.out_r[r] = f;
  p.out_d[r] = f;
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    if (p.lse[side]) p.lse[side][r] = (double)f;
  }
}

// One block per row, as score_rows, with the exact accumulator. The row holds the global
// columns [vstart, vstart + V); with p.part set it writes the shard partials instead of
// finalizing.
template <typename T, int NT, int U, int XF>
__global__ void __launch_bounds__(NT) score_rows_exact(ScoreParams p) {
  constexpr int NW = NT / 64;
  __shared__ AccX s_acc[2][NW];
  __shared__ int64_t s_y;
  WsHeader* h = (WsHeader*)p.ws;
  const int64_t r = p.row0 + blockIdx.x;
  const int tid = threadIdx.x;
  const bool shard = p.part[0] != nullptr;
  if (tid == 0) {
    int64_t end = p.N;
    if (p.layout == DRIFT_PACKED) {
      end = (int64_t)p.cu[p.nseq];
      end = end < 0 ? 0 : (end > p.N ? p.N : end);
    }
    const RowClass c = classify_row(p, r, end);
    if (p.active) p.active[r] = c.active ? 1 : 0;
    if (c.err & (1u << kErrMask)) record_error(h, kErrMask, r);
    if (c.err & (1u << kErrToken)) record_error(h, kErrToken, r);
    if (!c.score) {
      if (shard) {
        for (int side = 0; side < 2; ++side) {
          drift_lse_partial& q = p.part[side][r];
          q.bin[0] = q.bin[1] = q.bin[2] = 0;
          q.top = kEmptyTop;
          q.flags = 0;
          q.x_sel = 0.0f;
          q.reserved = 0.0f;
        }
      } else {
        unscored_outputs(p, r, c.active);
      }
    }
    s_y = c.score ? c.y : -1;
  }
  __syncthreads();
  const int64_t y = s_y;
  if (y < 0) return;  // block-uniform

  const size_t off = (size_t)r * (size_t)p.stride * sizeof(T);
  const char* rt = (const char*)p.train + off;
  const char* rr = (const char*)p.rollout + off;
  AccX at = accx_empty(), ar = accx_empty();
  if ((((uintptr_t)rt | (uintptr_t)rr) & 15) == 0) {
    stream_row<T, NT, U, true, XF>(rt, rr, p.V, tid, at, ar, p);
  } else {
    stream_row<T, NT, U, false, XF>(rt, rr, p.V, tid, at, ar, p);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    at = merge(at, shfl_xor_acc(at, o));
    ar = merge(ar, shfl_xor_acc(ar, o));
  }
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    s_acc[0][wave] = at;
    s_acc[1][wave] = ar;
  }
  __syncthreads();
  if (tid == 0) {
    AccX T_ = s_acc[0][0], R_ = s_acc[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      T_ = merge(T_, s_acc[0][w]);
      R_ = merge(R_, s_acc[1][w]);
    }
    const bool owner = y >= p.vstart && y < p.vstart + p.V;
    float xty = 0.0f, xry = 0.0f;
    if (owner) {  // single owner: the selected logit goes through the same chain
      float one[1] = {Elem<T>::load1(rt, y - p.vstart)};
      if constexpr (XF) apply_chain<1>(one, p.xf[0]);
      xty = one[0];
      one[0] = Elem<T>::load1(rr, y - p.vstart);
      if constexpr (XF) apply_chain<1>(one, p.xf[1]);
      xry = one[0];
    }
    if (shard) {
      auto put = [&](drift_lse_partial& q, const AccX& a, float xs) {
        q.bin[0] = a.b2;
        q.bin[1] = a.b1;
        q.bin[2] = a.b0;
        q.top = a.top;
        q.flags = DRIFT_PART_SCORED | (owner ? DRIFT_PART_OWNER : 0u) |
                  (a.bad ? DRIFT_PART_BAD : 0u);
        q.x_sel = xs;
        q.reserved = 0.0f;
      };
      put(p.part[0][r], T_, xty);
      put(p.part[1][r], R_, xry);
    } else {
      finish_row_exact(p, h, r, T_, R_, xty, xry);
    }
  }
}

// The exact pass for short rows (vocabulary shards, small V): one wave per row, four rows
// per block, with no block barrier. Lane 0 classifies the row and finishes it, the wave
// streams it and merges its lanes. The bins make the sum independent of how a row is
// split among lanes, so the results are bitwise those of score_rows_exact.
template <typename T, int U, int XF>
__global__ void __launch_bounds__(256) score_rows_exact_w(ScoreParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r = p.row0 + (int64_t)blockIdx.x * 4 + wave;
  if (r >= p.N) return;  // wave-uniform: the last block's rows past the batch
  WsHeader* h = (WsHeader*)p.ws;
  const bool shard = p.part[0] != nullptr;
  int64_t y = -1;
  if (lane == 0) {
    int64_t end = p.N;
    if (p.layout == DRIFT_PACKED) {
      end = (int64_t)p.cu[p.nseq];
      end = end < 0 ? 0 : (end > p.N ? p.N : end);
    }
    const RowClass c = classify_row(p, r, end);
    if (p.active) p.active[r] = c.active ? 1 : 0;
    if (c.err & (1u << kErrMask)) record_error(h, kErrMask, r);
    if (c.err & (1u << kErrToken)) record_error(h, kErrToken, r);
    if (!c.score) {
      if (shard) {
        for (int side = 0; side < 2; ++side) {
          drift_lse_partial& q = p.part[side][r];
          q.bin[0] = q.bin[1] = q.bin[2] = 0;
          q.top = kEmptyTop;
          q.flags = 0;
          q.x_sel = 0.0f;
          q.reserved = 0.0f;
        }
      } else {
        unscored_outputs(p, r, c.active);
      }
    }
    y = c.score ? c.y : -1;
  }
  // lane 0's value to the whole wave (lane 0 is its first active lane here)
  const uint32_t ylo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)y);
  const uint32_t yhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)y >> 32));
  y = (int64_t)(((uint64_t)yhi << 32) | ylo);
  if (y < 0) return;  // wave-uniform

  const size_t off = (size_t)r * (size_t)p.stride * sizeof(T);
  const char* rt = (const char*)p.train + off;
  const char* rr = (const char*)p.rollout + off;
  AccX at = accx_empty(), ar = accx_empty();
  if ((((uintptr_t)rt | (uintptr_t)rr) & 15) == 0) {
    stream_row<T, 64, U, true, XF>(rt, rr, p.V, lane, at, ar, p);
  } else {
    stream_row<T, 64, U, false, XF>(rt, rr, p.V, lane, at, ar, p);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    at = merge(at, shfl_xor_acc(at, o));
    ar = merge(ar, shfl_xor_acc(ar, o));
  }
  if (lane == 0) {
    const bool owner = y >= p.vstart && y < p.vstart + p.V;
    float xty = 0.0f, xry = 0.0f;
    if (owner) {  // single owner: the selected logit goes through the same chain
      float one[1] = {Elem<T>::load1(rt, y - p.vstart)};
      if constexpr (XF) apply_chain<1>(one, p.xf[0]);
      xty = one[0];
      one[0] = Elem<T>::load1(rr, y - p.vstart);
      if constexpr (XF) apply_chain<1>(one, p.xf[1]);
      xry = one[0];
    }
    if (shard) {
      auto put = [&](drift_lse_partial& q, const AccX& a, float xs) {
        q.bin[0] = a.b2;
        q.bin[1] = a.b1;
        q.bin[2] = a.b0;
        q.top = a.top;
        q.flags = DRIFT_PART_SCORED | (owner ? DRIFT_PART_OWNER : 0u) |
                  (a.bad ? DRIFT_PART_BAD : 0u);
        q.x_sel = xs;
        q.reserved = 0.0f;
      };
      put(p.part[0][r], at, xty);
      put(p.part[1][r], ar, xry);
    } else {
      finish_row_exact(p, h, r, at, ar, xty, xry);
    }
  }
}

// Shard merge: one thread per row classifies it, folds the S partials of each side in
// shard order and takes the selected logit from the owner shard.
__global__ void __launch_bounds__(256) merge_shards(MergeParams m) {
  const ScoreParams& p = m.p;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= p.N) return;
  WsHeader* h = (WsHeader*)p.ws;
  int64_t end = p.N;
  if (p.layout == DRIFT_PACKED) {
    end = (int64_t)p.cu[p.nseq];
    end = end < 0 ? 0 : (end > p.N ? p.N : end);
  }
  const RowClass c = classify_row(p, r, end);
  p.active[r] = c.active ? 1 : 0;
  if (c.err & (1u << kErrMask)) record_error(h, kErrMask, r);
  if (c.err & (1u << kErrToken)) record_error(h, kErrToken, r);
  if (!c.score) {
    unscored_outputs(p, r, c.active);
    return;
  }
  AccX T_ = accx_empty(), R_ = accx_empty();
  bool consistent = true;
  float xty = 0.0f, xry = 0.0f;
  for (int s = 0; s < m.S; ++s) {
    const drift_lse_partial qt = m.part[0][(int64_t)s * p.N + r];
    const drift_lse_partial qr = m.part[1][(int64_t)s * p.N + r];
    consistent = consistent && (qt.flags & DRIFT_PART_SCORED) && (qr.flags & DRIFT_PART_SCORED);
    T_ = merge(T_, from_partial(qt));
    R_ = merge(R_, from_partial(qr));
    if (c.y >= m.bound[s] && c.y < m.bound[s + 1]) {
      consistent = consistent && (qt.flags & DRIFT_PART_OWNER) && (qr.flags & DRIFT_PART_OWNER);
      xty = qt.x_sel;
      xry = qr.x_sel;
    }
  }
  if (!consistent) {  // a shard did not score the row or does not hold its selected id
    record_error(h, kErrMask, r);
    unscored_outputs(p, r, true);
    return;
  }
  finish_row_exact(p, h, r, T_, R_, xty, xry);
}

// Block shapes of the scoring kernel, per logits dtype (measured on MI355X: bf16 rows
// stream best with 256 threads x 4 groups in flight, fp32 rows with 512 x 4). The
// per-row reduction tree depends on the block width, so a build fixes it once; the unroll
// depth only changes load scheduling.
#ifndef DRIFT_SCORE_THREADS_BF16
#define DRIFT_SCORE_THREADS_BF16 256
#endif
#ifndef DRIFT_SCORE_UNROLL_BF16
#define DRIFT_SCORE_UNROLL_BF16 4
#endif
#ifndef DRIFT_SCORE_THREADS_F32
#define DRIFT_SCORE_THREADS_F32 512
#endif
#ifndef DRIFT_SCORE_UNROLL_F32
#define DRIFT_SCORE_UNROLL_F32 4
#endif
static_assert(DRIFT_SCORE_THREADS_BF16 % 64 == 0 && DRIFT_SCORE_THREADS_BF16 <= 1024, "shape");
static_assert(DRIFT_SCORE_THREADS_F32 % 64 == 0 && DRIFT_SCORE_THREADS_F32 <= 1024, "shape");

// Launches `kernel` (one block of `nt` threads per row) over rows [0, p.N). A dispatch
// holds at most 2^32 - 1 work-items per grid dimension, so larger batches are covered by
// consecutive launches over row ranges (p.row0 = first row of the launch); a row's
// arithmetic does not depend on the launch it falls in.
template <typename K>
void launch_over_rows(K kernel, ScoreParams p, int nt, hipStream_t s) {
  const int64_t per = (int64_t)(0xffffffffu / (unsigned)nt);
  for (int64_t r0 = 0; r0 < p.N; r0 += per) {
    p.row0 = r0;
    const int64_t n = p.N - r0 < per ? p.N - r0 : per;
    hipLaunchKernelGGL(kernel, dim3((unsigned)n), dim3(nt), 0, s, p);
  }
}

// Launches a four-rows-per-block kernel (one wave per row) over rows [0, p.N) in
// consecutive launches over row ranges whose lengths are multiples of 4, so that only the
// last block of the last launch has rows past the batch (it skips them).
template <typename K>
void launch_over_rows_w(K kernel, ScoreParams p, hipStream_t s) {
  const int64_t per = (int64_t)(0xffffffffu / 256u) * 4;
  for (int64_t r0 = 0; r0 < p.N; r0 += per) {
    p.row0 = r0;
    const int64_t n = p.N - r0 < per ? p.N - r0 : per;
    hipLaunchKernelGGL(kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, p);
  }
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  hipLaunchKernelGGL(init_header, dim3(1), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
  if (p.N > 0) {
    // chains: none (0), step by step (1), or both folded (2, rowio.h)
    const int xf = !(p.xf[0].n > 0 || p.xf[1].n > 0) ? 0
                   : (p.xf[0].kind != 0 && p.xf[1].kind != 0) ? 2 : 1;
    const bool ent = p.ent[0] != nullptr || p.ent[1] != nullptr;
    constexpr int NB = DRIFT_SCORE_THREADS_BF16, UB = DRIFT_SCORE_UNROLL_BF16;
    constexpr int NF = DRIFT_SCORE_THREADS_F32, UF = DRIFT_SCORE_UNROLL_F32;
#define DRIFT_SCORE_LAUNCH(T, NT, U, X, E) \
  launch_over_rows(score_rows<T, NT, U, X, E>, p, NT, s)
#define DRIFT_SCORE_LAUNCH_XF(T, NT, U, E)              \
  do {                                                  \
    if (xf == 2) DRIFT_SCORE_LAUNCH(T, NT, U, 2, E);    \
    else if (xf == 1) DRIFT_SCORE_LAUNCH(T, NT, U, 1, E); \
    else DRIFT_SCORE_LAUNCH(T, NT, U, 0, E);            \
  } while (0)
    if (p.dtype == DRIFT_BF16) {
      if (ent) DRIFT_SCORE_LAUNCH_XF(uint16_t, NB, UB, true);
      else DRIFT_SCORE_LAUNCH_XF(uint16_t, NB, UB, false);
    } else {
      if (ent) DRIFT_SCORE_LAUNCH_XF(float, NF, UF, true);
      else DRIFT_SCORE_LAUNCH_XF(float, NF, UF, false);
    }
#undef DRIFT_SCORE_LAUNCH_XF
#undef DRIFT_SCORE_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_score_exact(const ScoreParams& p, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1) {
  hipLaunchKernelGGL(init_header, dim3(1), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
  if (p.N > 0) {
    // The exact sum does not depend on how a row is split among lanes, so the layout
    // follows the row length: a block of 256 threads per row for rows of 4096 or more
    // 16-byte groups, one wave per row (four rows per block) for shorter ones (vocabulary
    // shards), which keeps more rows in flight per CU without block barriers.
    // chains as in launch_score: none (0), step by step (1), both folded (2)
    const int xf = !(p.xf[0].n > 0 || p.xf[1].n > 0) ? 0
                   : (p.xf[0].kind != 0 && p.xf[1].kind != 0) ? 2 : 1;
    const int vec = p.dtype == DRIFT_BF16 ? 8 : 4;
    const bool wide = (p.V + vec - 1) / vec >= 4096;
    auto go = [&](auto kernel, int nt) { launch_over_rows(kernel, p, nt, s); };
    constexpr int U = 4;
    auto by_xf = [&](auto k0, auto k1, auto k2, int nt) {
      if (xf == 2) go(k2, nt);
      else if (xf == 1) go(k1, nt);
      else go(k0, nt);
    };
    auto by_xf_w = [&](auto k0, auto k1, auto k2) {
      if (xf == 2) launch_over_rows_w(k2, p, s);
      else if (xf == 1) launch_over_rows_w(k1, p, s);
      else launch_over_rows_w(k0, p, s);
    };
    if (p.dtype == DRIFT_BF16) {
      if (wide) by_xf(score_rows_exact<uint16_t, 256, U, 0>, score_rows_exact<uint16_t, 256, U, 1>,
                      score_rows_exact<uint16_t, 256, U, 2>, 256);
      else by_xf_w(score_rows_exact_w<uint16_t, U, 0>, score_rows_exact_w<uint16_t, U, 1>,
                   score_rows_exact_w<uint16_t, U, 2>);
    } else {
      if (wide) by_xf(score_rows_exact<float, 256, U, 0>, score_rows_exact<float, 256, U, 1>,
                      score_rows_exact<float, 256, U, 2>, 256);
      else by_xf_w(score_rows_exact_w<float, U, 0>, score_rows_exact_w<float, U, 1>,
                   score_rows_exact_w<float, U, 2>);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_merge_shards(const MergeParams& m, hipStream_t s) {
  hipLaunchKernelGGL(init_header, dim3(1), dim3(256), 0, s, m.p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || m.p.N == 0) return e;
  hipLaunchKernelGGL(merge_shards, dim3((unsigned)((m.p.N + 255) / 256)), dim3(256), 0, s, m);
  return hipGetLastError();
}

}  // namespace drift
