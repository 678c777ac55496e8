// Fused LM-head selected logprob on the matrix cores.
//
// logp[t] = z[t, y_t] - LSE_v(z[t, v]) with z = hidden . W, W stored [H, V] (vocabulary
// contiguous) or [V, H] (hidden contiguous, the layout of a linear layer's weight): the
// head GEMM of "[WS2] Framework for ablation experiment", LogProb knobs row 9, fused with
// the online log-sum-exp of row 10, so the logits never reach memory.
//
// Launches:
//   lm_init          workspace header;
//   lm_transpose_w   (W [H, V]) W -> WT [Vp, Hp] (K contiguous, zero padded) in the
//                    workspace, so both MFMA operands load as 16-byte K-contiguous vectors;
//   lm_pad_rows      (H not a multiple of 64) hidden, or W [V, H], -> [rows, Hp] with K
//                    padding; and the last 256-row panel of an operand read in place
//                    when its row count is not a multiple of 256;
//   lm_gemm_lse      C^T tiles: 256 vocab rows x 256 tokens per block, 8 waves (two per
//                    SIMD) of 128 vocab rows x 64 tokens,
//                    K = H in steps of 64 through two LDS buffers filled by direct-to-LDS
//                    loads, v_mfma_f32_32x32x16_bf16 with fp32 accumulation. The epilogue
//                    turns each token's 256 logits into a (k, s) log-sum-exp partial and
//                    records z[t, y_t] from the single owning lane;
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
typedef __attribute__((address_space(3))) void* lds_ptr;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Block tile and its schedule over the chip. The K order of the products does not depend
// on these shapes; the epilogue tree depends only on the vocab-wave split (2).
constexpr int kBV = 256;        // vocab rows per block (MFMA M)
constexpr int kBT = 256;        // tokens per block (MFMA N)
constexpr int kBK = 64;         // K per LDS stage
constexpr int kPW = 128;        // vocab rows per wave: 2 vocab waves
constexpr int kPN = 64;         // tokens per wave: 4 token waves
constexpr int kPT = kPW / 32;   // 32x32 MFMA tiles per wave along the vocab
constexpr int kPU = kPN / 32;   // and along the tokens
constexpr int kPWaves = 8;      // two waves per SIMD
constexpr int kPThreads = 64 * kPWaves;
static_assert(kBV == kBT && kBK == 64 && kBV == 2 * kPW && kBT == 4 * kPN, "tile shape");
#ifndef DRIFT_LM_GROUP_V
#define DRIFT_LM_GROUP_V 16
#endif
#ifndef DRIFT_LM_GROUP_T
#define DRIFT_LM_GROUP_T 16
#endif
constexpr int kGroupV = DRIFT_LM_GROUP_V;  // vocab tiles per scheduling group
constexpr int kGroupT = DRIFT_LM_GROUP_T;  // token tiles per scheduling chunk
static_assert(kGroupV * kGroupT == 256 && kGroupV % 4 == 0 && kGroupT % 2 == 0,
              "one chunk = one block per CU, 8 XCD sub-grids");

struct Partial {  // 16 bytes
  float k;
  float pad;
  double s;
};

// Workspace of one call. Both GEMM operands are read as K-contiguous [rows, Hp] panels of
// 256 rows. W [H, V] is always transposed into `wt` (all Vp rows); W given as [V, H] is
// read in place when H is a multiple of 64, else copied with K padding into `wt`. Hidden
// is read in place when H is a multiple of 64, else copied with K padding into `hid`. An
// operand read in place whose row count is not a multiple of 256 has its last panel copied
// (rows past the end zero) into a 256-row tail buffer, so that no panel reads past the
// caller's array.
struct LmLayout {
  int64_t Vp, Tp, Hp, nVt, nTt;
  size_t wt_off, hid_off, wtail_off, htail_off, part_off, zsel_off, total;
  bool copy_w, copy_hidden, w_tail, h_tail;
  __host__ __device__ static LmLayout make(int64_t T, int64_t H, int64_t V, bool w_vh) {
    LmLayout l;
    l.Vp = (V + kBV - 1) / kBV * kBV;
    l.Tp = (T + kBT - 1) / kBT * kBT;
    l.Hp = (H + kBK - 1) / kBK * kBK;
    l.nVt = l.Vp / kBV;
    l.nTt = l.Tp / kBT;
    const bool kpad = l.Hp != H;
    l.copy_w = !w_vh || kpad;
    l.copy_hidden = kpad;
    l.w_tail = !l.copy_w && l.Vp != V;
    l.h_tail = !l.copy_hidden && l.Tp != T;
    const size_t panel = (size_t)kBV * l.Hp * 2;
    l.wt_off = 256;
    l.hid_off = l.wt_off + (l.copy_w ? align_up((size_t)l.Vp * l.Hp * 2, 256) : 0);
    l.wtail_off = l.hid_off + (l.copy_hidden ? align_up((size_t)l.Tp * l.Hp * 2, 256) : 0);
    l.htail_off = l.wtail_off + (l.w_tail ? panel : 0);
    l.part_off = l.htail_off + (l.h_tail ? panel : 0);
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

// Rows [0, T) of a row-major [T, H] bf16 array into [Tp, Hp], zero padded in both
// directions (grid-stride over 16-byte groups).
__global__ void __launch_bounds__(256) lm_pad_rows(const uint16_t* __restrict__ hid,
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
// (kGroupV / 4) x (kGroupT / 2) sub-grid, so they share operand panels in that XCD's L2.
// Ids past the end map outside the grid and exit.
__device__ __forceinline__ void tile_of(int64_t b, int64_t nTt_pad, int64_t& vt,
                                        int64_t& tt) {
  const int64_t per_group = (int64_t)kGroupV * nTt_pad;
  const int64_t g = b / per_group, j = b % per_group;
  const int64_t chunk = j / (kGroupV * kGroupT), jj = j % (kGroupV * kGroupT);
  constexpr int SV = kGroupV / 4, ST = kGroupT / 2;  // one XCD's sub-grid: SV x ST
  const int xcd = (int)(jj % 8), s = (int)(jj / 8);
  vt = g * kGroupV + SV * (xcd % 4) + (s % SV);
  tt = chunk * kGroupT + ST * (xcd / 4) + (s / SV);
}

struct GemmArgs {
  const uint16_t* wt;     // W as K-contiguous rows [>= V, Hp]: the transposed or padded copy,
                          // or the caller's [V, H] weight
  const uint16_t* hid;    // [>= T, Hp]: the padded copy or the caller's [T, H]
  const uint16_t* wtail;  // nullable: the last vocab panel (256 rows, zero past V)
  const uint16_t* htail;  // nullable: the last token panel (256 rows, zero past T)
  int64_t T, V, Hp, nVt, nTt, nVt_pad, nTt_pad, Tp;
  const int32_t* ids;
  Partial* part;        // [nVt, Tp]
  float* zsel;          // [Tp]
  Chain xf;             // transform chain of the logits (used by the XF kernel only)
};

// Epilogue of the GEMM kernels: each token's logits of this block become one (k, s)
// log-sum-exp partial; the single owner of z[t, y_t] records it. Lane (lr, lh) of wave
// (wv, wt) holds, for token t = t0 + WT wt + 32 in + lr, the logits of vocab rows
// vb + 32 im + 8 (r / 4) + (r % 4), vb = v0 + WV wv + 4 lh, i.e. the offsets from vb whose
// bit 2 is clear. FULL (every vocab row of the block is real: all tiles but the last) drops
// the per-row range tests; otherwise they compare the compile-time offset against a
// per-lane limit. The owner of y (offset y - vb in [0, WV) with bit 2 clear) takes z[t, y]
// out of its 64 values with a select tree on the offset's bits and stores it once. The two
// vocab waves of a token merge through LDS (wave wv = 1 writes the partials of all its
// tokens, one barrier, wave wv = 0 merges and stores).
template <int TM, int TN, int WV, int WT, bool FULL, bool XF>
__device__ __forceinline__ void lse_epilogue(const f32x16 (&acc)[TM][TN], const GemmArgs& a,
                                             int64_t vt, int64_t v0, int64_t t0, int wv, int wt,
                                             int lr, int lh, float (*s_k)[WT],
                                             double (*s_s)[WT]) {
  static_assert(TM == 4 && WV == 128, "the select tree covers 4 x 16 values per token");
  constexpr int NZ = TM * 16;
  const int64_t vb = v0 + WV * wv + 4 * lh;
  const int64_t vlim64 = a.V - vb;  // offsets below this are real vocab rows
  const int vlim = vlim64 > WV ? WV : (int)vlim64;
  Acc pt[TN];  // this lane's merged partial of each of its tokens
#pragma unroll
  for (int in = 0; in < TN; ++in) {
    const int64_t t = t0 + WT * wt + 32 * in + lr;
    const int64_t y = (t < a.T) ? (int64_t)a.ids[t] : -1;
    const int64_t yr64 = y - vb;
    const int yrel = (y >= 0 && yr64 >= 0 && yr64 < WV) ? (int)yr64 : -1;
    // value i = 16 im + r sits at offset 32 im + 8 (r / 4) + (r % 4); rows past V are -inf
    float z[NZ];
#pragma unroll
    for (int i = 0; i < NZ; ++i) {
      const int off = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + (i & 3);
      z[i] = (XF || FULL || off < vlim) ? acc[i >> 4][in][i & 15] : -INFINITY;
    }
    if (yrel >= 0 && (yrel & 4) == 0) {
      // the owner: i = 16 (bits 5-6) + 4 (bits 3-4) + (bits 0-1) of the offset, picked by a
      // select tree on i's bits (all-ones / zero lane masks, no branches)
      const uint32_t i_sel = (uint32_t)(((yrel >> 5) << 4) | (((yrel >> 3) & 3) << 2) | (yrel & 3));
      uint32_t u[NZ / 2];
      const uint32_t m0 = 0u - (i_sel & 1u);
#pragma unroll
      for (int q = 0; q < NZ / 2; ++q)
        u[q] = (m0 & __float_as_uint(z[2 * q + 1])) | (~m0 & __float_as_uint(z[2 * q]));
#pragma unroll
      for (int b = 1, n = NZ / 4; n >= 1; ++b, n >>= 1) {
        const uint32_t mb = 0u - ((i_sel >> b) & 1u);
#pragma unroll
        for (int q = 0; q < n; ++q) u[q] = (mb & u[2 * q + 1]) | (~mb & u[2 * q]);
      }
      float zs = __uint_as_float(u[0]);
      if constexpr (XF) {  // the selected logit takes the chain step by step
        float one[1] = {zs};
        apply_chain<1>(one, a.xf);
        zs = one[0];
      }
      a.zsel[t] = zs;
    }
    if constexpr (XF) {
      // the logits through the chain: folded (rowio.h) or step by step; rows past V are
      // -inf after it
      if (a.xf.kind == 2) {
        fold_values<NZ>(z, a.xf);
#pragma unroll
        for (int i = 0; i < NZ; ++i) z[i] = fmaf(a.xf.fb, z[i], a.xf.fa);
      } else {  // kind 1 (the entry point takes folded chains only)
#pragma unroll
        for (int i = 0; i < NZ; ++i) z[i] = z[i] * a.xf.fb;
      }
      if constexpr (!FULL) {
#pragma unroll
        for (int i = 0; i < NZ; ++i) {
          const int off = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + (i & 3);
          if (off >= vlim) z[i] = -INFINITY;
        }
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NZ; ++i) m = fmaxf(m, z[i]);
    Acc p = {-INFINITY, 0.0};
    if (m > -INFINITY) {
      // exponent range as in lse.h: fail closed at or above 2^30, clamp below -2^30
      const float kn = ceilf(m * kLog2e);
      const bool big = !(kn < kMaxK);
      const float k = big ? 0.0f : fmaxf(kn, -kMaxK);
      float s = 0.0f;
      if (big) {
        s = NAN;
      } else {
        const float nk = -k;
#pragma unroll
        for (int i = 0; i < NZ; ++i) s += __builtin_amdgcn_exp2f(fmaf(z[i], kLog2e, nk));
      }
      p.k = k;
      p.s = (double)s;
    } else if (!(m == -INFINITY)) {
      p.k = 0.0f;
      p.s = NAN;
    }
  // the other half of the wave holds the other 4-row groups of the same token
    Acc o;
    o.k = __shfl_xor(p.k, 32);
    o.s = __shfl_xor(p.s, 32);
    pt[in] = merge(p, o);
    if (wv == 1 && lh == 0) {
      s_k[wt][32 * in + lr] = pt[in].k;
      s_s[wt][32 * in + lr] = pt[in].s;
    }
  }
  __syncthreads();  // one exchange for all the wave's tokens
  if (wv == 0 && lh == 0) {
#pragma unroll
    for (int in = 0; in < TN; ++in) {
      const int64_t t = t0 + WT * wt + 32 * in + lr;
      const Acc q = merge(pt[in], Acc{s_k[wt][32 * in + lr], s_s[wt][32 * in + lr]});
      Partial out;
      out.k = q.k;
      out.pad = 0.0f;
      out.s = q.s;
      a.part[vt * a.Tp + t] = out;
    }
  }
}

// The head GEMM with its LSE epilogue. 8 waves, two per SIMD (waves w and w + 4 share one),
// in a 2 (vocab) x 4 (tokens) grid each compute 128 vocab rows x 64 tokens (4 x 2 MFMA
// tiles, 128 accumulators). Within a K stage the four 16-wide steps are interleaved by hand
// with the memory work: the MFMAs of a step run while the next step's fragments are read
// from LDS into the other register set, and while one wave of a SIMD waits the other's
// MFMAs can issue. The stage tiles move from global memory into
// LDS with buffer_load_dwordx4 ... lds (lane l of an instruction fills bytes [16 l, 16 l + 16)
// of a 1 KB LDS span, checked on the GPU), so no VGPRs hold them and the LDS fills count
// on vmcnt while the fragment reads alone count on lgkmcnt. Rows are 128 bytes without
// padding; the 16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7), which makes
// the fragment reads (16 lanes = 16 consecutive rows at one logical chunk) hit 16 distinct
// 4-bank groups. The four buffers (A and B, two stages) are separate LDS arrays and the
// stage loop is unrolled by two, so every access names its buffer at compile time.
template <bool XF>
__global__ void __launch_bounds__(kPThreads, 1) lm_gemm_lse(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kBV * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kBV * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[kBT * kBK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[kBT * kBK];
  __shared__ float s_k[4][kPN];
  __shared__ double s_s[4][kPN];
  int64_t vt, tt;
  tile_of(blockIdx.x, a.nTt_pad, vt, tt);
  if (vt >= a.nVt || tt >= a.nTt) return;  // block-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave >> 2, wt = wave & 3;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t v0 = vt * kBV, t0 = tt * kBT;
  const uint16_t* gA = (a.wtail && vt == a.nVt - 1) ? a.wtail : a.wt + v0 * a.Hp;
  const uint16_t* gB = (a.htail && tt == a.nTt - 1) ? a.htail : a.hid + t0 * a.Hp;
  if (a.T < 0) {  // never taken; keeps the LDS arrays from being treated as never written
    sA0[tid] = sA1[tid] = sB0[tid] = sB1[tid] = 0;
  }

  // LDS fills: wave w moves the 8-row blocks 4w .. 4w + 3 of both tiles. Lane l of an
  // instruction for rows r0 .. r0 + 7 takes row r0 + l / 8 and stored chunk l % 8, i.e.
  // logical chunk (l % 8) ^ ((r0 / 2 + l / 16) & 7).
  // The stored chunk of a lane depends on the 8-row block only through its parity (r0 / 2
  // is a multiple of 4), so two per-lane byte offsets serve every instruction; the rest of
  // the address is wave-uniform.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lane_off[2] = {
      (uint32_t)(((lane >> 3) * a.Hp + (((lane & 7) ^ ((lane >> 4) & 7)) * 8)) * 2),
      (uint32_t)(((lane >> 3) * a.Hp + (((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 8)) * 2)};
  // The fills go through buffer resources over the block's two operand panels (256 rows x
  // Hp each, all inside the array the panel comes from): the per-lane byte offset is one
  // of the two constants above and the rest is one scalar offset per instruction, so no
  // address arithmetic or address registers are needed in the loop.
  const uint32_t panel_bytes = (uint32_t)(kBV * a.Hp * 2);
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)gA, (short)0, panel_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rB =
      __builtin_amdgcn_make_buffer_rsrc((void*)gB, (short)0, panel_bytes, 0x00020000);
  // one operand's share of a stage: this wave's 4 blocks of 8 rows (4 instructions of 1 KB)
  auto fill = [&](const __amdgpu_buffer_rsrc_t& r, uint16_t* d, int64_t k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r0 = (wave_u * 4 + j) * 8;
      const uint32_t so = (uint32_t)(((int64_t)r0 * a.Hp + k0) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(d + r0 * kBK), 16, lane_off[j & 1],
                                               so, 0, 0);
    }
  };

  f32x16 acc[kPT][kPU];
#pragma unroll
  for (int i = 0; i < kPT; ++i)
#pragma unroll
    for (int j = 0; j < kPU; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8 fa[2][kPT], fb[2][kPU];
  const int swz = (lr >> 1) & 7;  // rows 128 wv + 32 i + lr share ((row >> 1) & 7)
  auto fread = [&](const uint16_t* bA, const uint16_t* bB, int kk, int set) {
    const int ch = (2 * kk + lh) ^ swz;
#pragma unroll
    for (int i = 0; i < kPT; ++i)
      fa[set][i] = *(const bf16x8*)(bA + (kPW * wv + 32 * i + lr) * kBK + ch * 8);
#pragma unroll
    for (int i = 0; i < kPU; ++i)
      fb[set][i] = *(const bf16x8*)(bB + (kPN * wt + 32 * i + lr) * kBK + ch * 8);
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < kPT; ++i)
#pragma unroll
      for (int j = 0; j < kPU; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j],
                                                            0, 0, 0);
  };
  // the next step's fragment reads go out early in the step, one after each MFMA
  auto interleave_reads = [&]() {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stage kt reads the buffers of parity kt % 2: steps 0-2 read the next step's fragments;
  // then this wave's fills of stage kt + 1 are awaited and the block barrier makes every
  // fill visible and every read of this stage's buffers done; step 3 reads the first
  // fragments of stage kt + 1. A stage's fills go out in two halves of 4 instructions per
  // wave, each interleaved one per MFMA pair with a step: the W half of stage kt + 2 in step 3
  // of stage kt (into this stage's buffer, free after the barrier), the hidden half of
  // stage kt + 1 in step 0 of stage kt (into the other buffer, free since the barrier of
  // stage kt - 1). Issuing a whole stage's fills in one step queued them behind the CU's
  // address unit for about twice the step's length, and the MFMAs behind them in program
  // order waited (the split measured 5-6 % faster per call, bitwise the same). The last stages
  // re-fill with the last stage's data, which nobody reads; stage 0 re-fills the hidden
  // half of stage 1 with the data the prologue put there.
  const int64_t nk = a.Hp / kBK;
  auto stage = [&](const uint16_t* cA, const uint16_t* cB, uint16_t* nA, uint16_t* nB,
                   int64_t kt) {
    const int64_t k1 = (kt + 1 < nk ? kt + 1 : nk - 1) * kBK;
    const int64_t k2 = (kt + 2 < nk ? kt + 2 : nk - 1) * kBK;
    fread(cA, cB, 1, 1);
    fill(rB, nB, k1);
    mfmas(0);
    // per MFMA pair: one or two fragment reads, one fill
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    fread(cA, cB, 2, 0);
    mfmas(1);
    interleave_reads();
    fread(cA, cB, 3, 1);
    mfmas(0);
    interleave_reads();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's fills of stage kt + 1
    __syncthreads();
    fread(nA, nB, 0, 0);
    fill(rA, const_cast<uint16_t*>(cA), k2);
    mfmas(1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  fill(rA, sA0, 0);
  fill(rB, sB0, 0);
  fill(rA, sA1, nk > 1 ? kBK : 0);
  fill(rB, sB1, nk > 1 ? kBK : 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  fread(sA0, sB0, 0, 0);
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    stage(sA0, sB0, sA1, sB1, kt);
    stage(sA1, sB1, sA0, sB0, kt + 1);
  }
  if (kt < nk) stage(sA0, sB0, sA1, sB1, kt);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  if (v0 + kBV <= a.V)  // block-uniform
    lse_epilogue<kPT, kPU, kPW, kPN, true, XF>(acc, a, vt, v0, t0, wv, wt, lr, lh, s_k, s_s);
  else
    lse_epilogue<kPT, kPU, kPW, kPN, false, XF>(acc, a, vt, v0, t0, wv, wt, lr, lh, s_k, s_s);
}

// Four lanes per token: lane q folds the vocab tiles [q*c, (q+1)*c) in ascending order
// (c = ceil(nVt / 4)), then the four results are folded in q order. The tree depends only
// on the number of vocab tiles.
constexpr int kMergeSplit = 4;

__global__ void __launch_bounds__(256) lm_merge(const Partial* __restrict__ part,
                                                 const float* __restrict__ zsel,
                                                 const int32_t* __restrict__ ids,
                                                 const uint8_t* __restrict__ active,
                                                 float* __restrict__ logp, int64_t T,
                                                 int64_t Tp, int64_t V, int64_t nVt, char* ws) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = gid / kMergeSplit;
  const int q = (int)(gid % kMergeSplit);
  const bool live = t < T && (!active || active[t]);
  const int64_t c = (nVt + kMergeSplit - 1) / kMergeSplit;
  const int64_t j0 = (int64_t)q * c, j1 = j0 + c < nVt ? j0 + c : nVt;
  Acc A = {-INFINITY, 0.0};
  if (live) {
    int64_t j = j0;
    for (; j + 8 <= j1; j += 8) {
      Partial b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) b[u] = part[(j + u) * Tp + t];
#pragma unroll
      for (int u = 0; u < 8; ++u) A = merge(A, Acc{b[u].k, b[u].s});
    }
    for (; j < j1; ++j) {
      const Partial b = part[j * Tp + t];
      A = merge(A, Acc{b.k, b.s});
    }
  }
  // fold the four lanes of the token in q order (lanes 4i..4i+3 of the wave)
  Acc P[kMergeSplit];
#pragma unroll
  for (int i = 0; i < kMergeSplit; ++i) {
    P[i].k = __shfl(A.k, (threadIdx.x & ~(kMergeSplit - 1)) + i);
    P[i].s = __shfl(A.s, (threadIdx.x & ~(kMergeSplit - 1)) + i);
  }
  if (q != 0 || t >= T) return;
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
  Acc R = P[0];
#pragma unroll
  for (int i = 1; i < kMergeSplit; ++i) R = merge(R, P[i]);
  const float z = zsel[t];
  const bool kk = k_ok(R.k);
  logp[t] = (float)((double)z - (kk ? lse_of(R) : (double)NAN));
  if (!lse_ok(R) || !kk || !(fabsf(z) < INFINITY)) record_error(h, kErrNonfinite, t);
}

}  // namespace

size_t lmhead_ws_bytes(int64_t T, int64_t H, int64_t V, bool w_vh) {
  return LmLayout::make(T, H, V, w_vh).total;
}

// The GEMM runs one block of kPThreads per (vocab tile, token tile) in one dispatch, which
// holds at most 2^32 - 1 work-items: T is limited by that (3,530,752 tokens at V = 151936).
bool lmhead_shape_ok(int64_t T, int64_t V) {
  const int64_t nVt = (V + kBV - 1) / kBV, nTt = (T + kBT - 1) / kBT;
  const int64_t nVt_pad = (nVt + kGroupV - 1) / kGroupV * kGroupV;
  const int64_t nTt_pad = (nTt + kGroupT - 1) / kGroupT * kGroupT;
  return nVt_pad * nTt_pad <= (int64_t)(0xffffffffu / kPThreads);
}

hipError_t launch_lmhead(const LmheadParams& p, hipStream_t s) {
  const LmLayout l = LmLayout::make(p.T, p.H, p.V, p.w_vh);
  hipLaunchKernelGGL(lm_init, dim3(1), dim3(64), 0, s, p.ws);
  if (p.T == 0) return hipGetLastError();
  // rows [0, rows) of src [rows, H] into dst [rows_p, Hp], zero padded (grid-stride)
  auto pad_copy = [&](const uint16_t* src, uint16_t* dst, int64_t rows, int64_t rows_p) {
    const int64_t nvec = rows_p * (l.Hp / 8);
    const unsigned blocks = (unsigned)((nvec + 255) / 256 < 65536 ? (nvec + 255) / 256 : 65536);
    hipLaunchKernelGGL(lm_pad_rows, dim3(blocks), dim3(256), 0, s, src, dst, rows, p.H, rows_p,
                       l.Hp);
  };
  const uint16_t* wt = (const uint16_t*)p.weight;
  if (l.copy_w) {
    uint16_t* w = (uint16_t*)(p.ws + l.wt_off);
    if (p.w_vh)
      pad_copy((const uint16_t*)p.weight, w, p.V, l.Vp);
    else
      hipLaunchKernelGGL(lm_transpose_w, dim3((unsigned)(l.Vp / 64), (unsigned)(l.Hp / 64)),
                         dim3(256), 0, s, (const uint16_t*)p.weight, w, p.H, p.V, l.Hp);
    wt = w;
  }
  const uint16_t* hid = (const uint16_t*)p.hidden;
  if (l.copy_hidden) {
    uint16_t* h = (uint16_t*)(p.ws + l.hid_off);
    pad_copy(hid, h, p.T, l.Tp);
    hid = h;
  }
  const uint16_t* wtail = nullptr;
  const uint16_t* htail = nullptr;
  if (l.w_tail) {
    uint16_t* d = (uint16_t*)(p.ws + l.wtail_off);
    const int64_t r0 = (l.nVt - 1) * kBV;
    pad_copy(wt + r0 * l.Hp, d, p.V - r0, kBV);
    wtail = d;
  }
  if (l.h_tail) {
    uint16_t* d = (uint16_t*)(p.ws + l.htail_off);
    const int64_t r0 = (l.nTt - 1) * kBT;
    pad_copy(hid + r0 * l.Hp, d, p.T - r0, kBT);
    htail = d;
  }
  GemmArgs g;
  g.wt = wt;
  g.hid = hid;
  g.wtail = wtail;
  g.htail = htail;
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
  g.xf = p.xf;
  if (p.xf.n > 0)
    hipLaunchKernelGGL(lm_gemm_lse<true>, dim3((unsigned)nblocks), dim3(kPThreads), 0, s, g);
  else
    hipLaunchKernelGGL(lm_gemm_lse<false>, dim3((unsigned)nblocks), dim3(kPThreads), 0, s, g);
  hipLaunchKernelGGL(lm_merge, dim3((unsigned)((p.T * kMergeSplit + 255) / 256)), dim3(256), 0, s,
                     g.part,
                     g.zsel, p.ids, p.active, p.logp, p.T, l.Tp, p.V, l.nVt, p.ws);
  return hipGetLastError();
}

}  // namespace drift
