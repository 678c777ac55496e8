// Fused LM-head selected logprob on the matrix cores.
//
// logp[t] = z[t, y_t] - LSE_v(z[t, v]) with z = hidden . W, W stored [H, V] (vocabulary
// contiguous): the head GEMM of "[WS2] Framework for ablation experiment", LogProb knobs
// row 9, fused with the online log-sum-exp of row 10, so the logits never reach memory.
//
// Launches:
//   lm_init          workspace header;
//   lm_transpose_w   W [H, V] -> WT [Vp, Hp] (K contiguous, zero padded) in the workspace,
//                    so both MFMA operands load as 16-byte K-contiguous vectors;
//   lm_pad_hidden    (only when T or H is not a tile multiple) hidden -> [Tp, Hp], zero pad;
//   lm_gemm_lse      C^T tiles: 128 vocab rows x 128 tokens per block, K = H in steps of 64
//                    through double-buffered LDS, v_mfma_f32_32x32x16_bf16 with fp32
//                    accumulation. The epilogue turns each token's 128 logits into a (k, s)
//                    log-sum-exp partial and records z[t, y_t] from the single owning lane;
//   lm_merge         per token, the partials of all vocab tiles in ascending tile order.
// The K order of every product is fixed (k-tiles ascending, 16-wide MFMA steps ascending)
// and independent of T, of the token's position in its tile and of the launch, so a
// token's result is bitwise the same in any batch (the batch-invariance check of the
// "Kernel Integration Contract").
#include <math.h>

#include "common.h"
#include "lse.h"

namespace drift {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBV = 128;        // vocab rows per block (MFMA M)
constexpr int kBT = 128;        // tokens per block (MFMA N)
constexpr int kBK = 64;         // K per LDS stage
constexpr int kPitch = kBK + 8; // LDS row pitch in bf16 (144 B: conflict-free 16-B reads)
constexpr int kThreads = 256;   // 4 waves as 2 (vocab) x 2 (tokens), 64 x 64 each
constexpr int kGroupV = 16;     // vocab tiles per scheduling group
constexpr int kGroupT = 16;     // token tiles per scheduling chunk

struct Partial {  // 16 bytes
  float k;
  float pad;
  double s;
};

struct LmLayout {
  int64_t Vp, Tp, Hp, nVt, nTt;
  size_t wt_off, hid_off, part_off, zsel_off, total;
  bool pad_hidden;
  __host__ __device__ static LmLayout make(int64_t T, int64_t H, int64_t V) {
    LmLayout l;
    l.Vp = (V + kBV - 1) / kBV * kBV;
    l.Tp = (T + kBT - 1) / kBT * kBT;
    l.Hp = (H + kBK - 1) / kBK * kBK;
    l.nVt = l.Vp / kBV;
    l.nTt = l.Tp / kBT;
    l.pad_hidden = (l.Tp != T) || (l.Hp != H);
    l.wt_off = 256;
    l.hid_off = l.wt_off + align_up((size_t)l.Vp * l.Hp * 2, 256);
    const size_t hid_bytes = l.pad_hidden ? (size_t)l.Tp * l.Hp * 2 : 0;
    l.part_off = l.hid_off + align_up(hid_bytes, 256);
    l.zsel_off = l.part_off + align_up((size_t)l.nVt * l.Tp * sizeof(Partial), 256);
    l.total = l.zsel_off + align_up((size_t)l.Tp * 4, 256);
    return l;
  }
};

__global__ void lm_init(char* ws) {
  if (threadIdx.x == 0) {
    WsHeader* h = (WsHeader*)ws;
    h->err_bits = 0;
    h->magic = kWsMagic;
    h->n_active = 0;
    for (int c = 0; c < 4; ++c) h->first_bad[c] = ~0ull;
  }
}

// 64 (k) x 64 (v) tiles through LDS; out-of-range elements become 0.
__global__ void __launch_bounds__(256) lm_transpose_w(const uint16_t* __restrict__ W,
                                                       uint16_t* __restrict__ WT, int64_t H,
                                                       int64_t V, int64_t Hp) {
  __shared__ uint16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  const int64_t v0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int kr = c >> 3, vc = (c & 7) * 8;
    const int64_t k = k0 + kr, v = v0 + vc;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (k < H && v < V) x = __builtin_nontemporal_load((const u32x4*)(W + k * V + v));
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[kr][vc + 2 * e] = (uint16_t)(w[e] & 0xffffu);
      tile[kr][vc + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int vr = c >> 3, kc = (c & 7) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[kc + 2 * e][vr] | ((uint32_t)tile[kc + 2 * e + 1][vr] << 16);
    const u32x4 o = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(WT + (v0 + vr) * Hp + k0 + kc) = o;
  }
}

__global__ void __launch_bounds__(256) lm_pad_hidden(const uint16_t* __restrict__ hid,
                                                      uint16_t* __restrict__ out, int64_t T,
                                                      int64_t H, int64_t Tp, int64_t Hp) {
  const int64_t nvec = Tp * (Hp / 8);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / (Hp / 8), k = (i % (Hp / 8)) * 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (t < T && k < H) x = *(const u32x4*)(hid + t * H + k);
    *(u32x4*)(out + t * Hp + k) = x;
  }
}

// Block id -> (vocab tile, token tile). Groups of kGroupV vocab tiles are walked in order;
// inside a group, chunks of kGroupT token tiles; inside a chunk (256 blocks = one block
// per CU), the 32 blocks that the dispatcher sends to one XCD (ids equal mod 8) form a
// 4 x 8 sub-grid, so they share operand panels in that XCD's L2. Ids past the end map
// outside the grid and exit.
__device__ __forceinline__ void tile_of(int64_t b, int64_t nVt_pad, int64_t nTt_pad,
                                        int64_t& vt, int64_t& tt) {
  const int64_t per_group = (int64_t)kGroupV * nTt_pad;
  const int64_t g = b / per_group, j = b % per_group;
  const int64_t chunk = j / (kGroupV * kGroupT), jj = j % (kGroupV * kGroupT);
  const int xcd = (int)(jj % 8), s = (int)(jj / 8);
  vt = g * kGroupV + 4 * (xcd % 4) + (s % 4);
  tt = chunk * kGroupT + 8 * (xcd / 4) + (s / 4);
}

struct GemmArgs {
  const uint16_t* wt;   // [Vp, Hp]
  const uint16_t* hid;  // [Tp, Hp] (padded copy) or the caller's [T, H] when no pad
  int64_t T, V, Hp, nVt, nTt, nVt_pad, nTt_pad, Tp;
  const int32_t* ids;
  Partial* part;        // [nVt, Tp]
  float* zsel;          // [Tp]
};

__global__ void __launch_bounds__(kThreads) lm_gemm_lse(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBV][kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBT][kPitch];
  __shared__ float s_k[2][64];
  __shared__ double s_s[2][64];
  int64_t vt, tt;
  tile_of(blockIdx.x, a.nVt_pad, a.nTt_pad, vt, tt);
  if (vt >= a.nVt || tt >= a.nTt) return;  // block-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave >> 1, wt = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t v0 = vt * kBV, t0 = tt * kBT;
  const uint16_t* gA = a.wt + v0 * a.Hp;
  const uint16_t* gB = a.hid + t0 * a.Hp;

  // stage loader: 16 KB per operand, 4 x 16 B per thread per operand
  u32x4 ra[4], rb[4];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int row = c >> 3, col = (c & 7) * 8;
      ra[i] = *(const u32x4*)(gA + (int64_t)row * a.Hp + k0 + col);
      rb[i] = *(const u32x4*)(gB + (int64_t)row * a.Hp + k0 + col);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int row = c >> 3, col = (c & 7) * 8;
      *(u32x4*)&sA[buf][row][col] = ra[i];
      *(u32x4*)&sB[buf][row][col] = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int im = 0; im < 2; ++im)
#pragma unroll
    for (int in = 0; in < 2; ++in)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[im][in][r] = 0.0f;

  const int64_t nk = a.Hp / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int koff = kk * 16 + lh * 8;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int im = 0; im < 2; ++im)
        fa[im] = *(const bf16x8*)&sA[buf][64 * wv + 32 * im + lr][koff];
#pragma unroll
      for (int in = 0; in < 2; ++in)
        fb[in] = *(const bf16x8*)&sB[buf][64 * wt + 32 * in + lr][koff];
#pragma unroll
      for (int im = 0; im < 2; ++im)
#pragma unroll
        for (int in = 0; in < 2; ++in)
          acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[im], fb[in], acc[im][in], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // Epilogue. Lane (lr, lh) of wave (wv, wt) holds, for token t = t0 + 64 wt + 32 in + lr,
  // the logits of vocab rows v0 + 64 wv + 32 im + 8 (r / 4) + 4 lh + (r % 4).
#pragma unroll
  for (int in = 0; in < 2; ++in) {
    const int64_t t = t0 + 64 * wt + 32 * in + lr;
    const int64_t y = (t < a.T) ? (int64_t)a.ids[t] : -1;
    float m = -INFINITY;
#pragma unroll
    for (int im = 0; im < 2; ++im)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t v = v0 + 64 * wv + 32 * im + 8 * (r / 4) + 4 * lh + (r % 4);
        if (v < a.V) m = fmaxf(m, acc[im][in][r]);
        if (v == y) a.zsel[t] = acc[im][in][r];  // the single owner of z[t, y_t]
      }
    Acc p = {-INFINITY, 0.0};
    if (m > -INFINITY) {
      const float k = ceilf(m * kLog2e);
      float s = 0.0f;
      if (k == INFINITY) {
        s = NAN;
      } else {
#pragma unroll
        for (int im = 0; im < 2; ++im)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t v = v0 + 64 * wv + 32 * im + 8 * (r / 4) + 4 * lh + (r % 4);
            if (v < a.V) s += __builtin_amdgcn_exp2f(fmaf(acc[im][in][r], kLog2e, -k));
          }
      }
      p.k = (k == INFINITY) ? 0.0f : k;
      p.s = (double)s;
    } else if (!(m == -INFINITY)) {
      p.k = 0.0f;
      p.s = NAN;
    }
    // the other half of the wave holds the other 4-row groups of the same token
    Acc o;
    o.k = __shfl_xor(p.k, 32);
    o.s = __shfl_xor(p.s, 32);
    p = merge(p, o);
    if (wv == 1 && lh == 0) {
      s_k[wt][32 * in + lr] = p.k;
      s_s[wt][32 * in + lr] = p.s;
    }
    __syncthreads();
    if (wv == 0 && lh == 0 && t < a.Tp) {
      const Acc q = merge(p, Acc{s_k[wt][32 * in + lr], s_s[wt][32 * in + lr]});
      Partial out;
      out.k = q.k;
      out.pad = 0.0f;
      out.s = q.s;
      a.part[vt * a.Tp + t] = out;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) lm_merge(const Partial* __restrict__ part,
                                                 const float* __restrict__ zsel,
                                                 const int32_t* __restrict__ ids,
                                                 const uint8_t* __restrict__ active,
                                                 float* __restrict__ logp, int64_t T,
                                                 int64_t Tp, int64_t V, int64_t nVt, char* ws) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  if (active && !active[t]) {
    logp[t] = 0.0f;
    return;
  }
  WsHeader* h = (WsHeader*)ws;
  const int64_t y = ids[t];
  if (y < 0 || y >= V) {
    logp[t] = NAN;
    record_error(h, kErrToken, t);
    return;
  }
  Acc A = {-INFINITY, 0.0};
  for (int64_t j = 0; j < nVt; ++j) {  // vocab tiles in ascending order
    const Partial q = part[j * Tp + t];
    A = merge(A, Acc{q.k, q.s});
  }
  const float z = zsel[t];
  logp[t] = (float)((double)z - lse_of(A));
  if (!lse_ok(A) || !(fabsf(z) < INFINITY)) record_error(h, kErrNonfinite, t);
}

}  // namespace

size_t lmhead_ws_bytes(int64_t T, int64_t H, int64_t V) { return LmLayout::make(T, H, V).total; }

hipError_t launch_lmhead(const LmheadParams& p, hipStream_t s) {
  const LmLayout l = LmLayout::make(p.T, p.H, p.V);
  hipLaunchKernelGGL(lm_init, dim3(1), dim3(64), 0, s, p.ws);
  if (p.T == 0) return hipGetLastError();
  uint16_t* wt = (uint16_t*)(p.ws + l.wt_off);
  hipLaunchKernelGGL(lm_transpose_w, dim3((unsigned)(l.Vp / 64), (unsigned)(l.Hp / 64)), dim3(256),
                     0, s, (const uint16_t*)p.weight, wt, p.H, p.V, l.Hp);
  const uint16_t* hid = (const uint16_t*)p.hidden;
  if (l.pad_hidden) {
    uint16_t* hp = (uint16_t*)(p.ws + l.hid_off);
    const int64_t nvec = l.Tp * (l.Hp / 8);
    const unsigned blocks = (unsigned)((nvec + 255) / 256 < 65536 ? (nvec + 255) / 256 : 65536);
    hipLaunchKernelGGL(lm_pad_hidden, dim3(blocks), dim3(256), 0, s, hid, hp, p.T, p.H, l.Tp,
                       l.Hp);
    hid = hp;
  }
  GemmArgs g;
  g.wt = wt;
  g.hid = hid;
  g.T = p.T;
  g.V = p.V;
  g.Hp = l.Hp;
  g.nVt = l.nVt;
  g.nTt = l.nTt;
  g.nVt_pad = (l.nVt + kGroupV - 1) / kGroupV * kGroupV;
  g.nTt_pad = (l.nTt + kGroupT - 1) / kGroupT * kGroupT;
  g.Tp = l.Tp;
  g.ids = p.ids;
  g.part = (Partial*)(p.ws + l.part_off);
  g.zsel = (float*)(p.ws + l.zsel_off);
  const int64_t nblocks = g.nVt_pad * g.nTt_pad;
  hipLaunchKernelGGL(lm_gemm_lse, dim3((unsigned)nblocks), dim3(kThreads), 0, s, g);
  hipLaunchKernelGGL(lm_merge, dim3((unsigned)((p.T + 255) / 256)), dim3(256), 0, s, g.part,
                     g.zsel, p.ids, p.active, p.logp, p.T, l.Tp, p.V, l.nVt, p.ws);
  return hipGetLastError();
}

}  // namespace drift
