// C entry points of the drift library: argument checks (fail closed, before any launch),
// workspace sizing, dispatch to the kernels, status readback and the backend descriptor.
#include <math.h>
#include <string.h>

#include "common.h"

#ifndef DRIFT_BUILD_FINGERPRINT
#define DRIFT_BUILD_FINGERPRINT "unknown"
#endif

using namespace drift;

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int status_from_header(const WsHeader& h, int64_t* first_bad) {
  const int st = header_status(h.magic, h.err_bits);
  if (first_bad) {
    *first_bad = -1;
    const int cls = st == DRIFT_EMASK ? kErrMask : st == DRIFT_ETOKEN ? kErrToken
                  : st == DRIFT_ENONFINITE ? kErrNonfinite : -1;
    if (cls >= 0) *first_bad = (int64_t)h.first_bad[cls];
  }
  return st;
}

// Transform chain checks: at most DRIFT_MAX_TRANSFORMS known steps with finite values,
// positive for TEMPERATURE and SOFTCAP.
bool chain_ok(const drift_transform& t) {
  if (t.count < 0 || t.count > DRIFT_MAX_TRANSFORMS) return false;
  for (int i = 0; i < t.count; ++i) {
    const float v = t.value[i];
    if (!(v == v) || v == INFINITY || v == -INFINITY) return false;
    if (t.op[i] == DRIFT_XF_SCALE) continue;
    if ((t.op[i] == DRIFT_XF_TEMPERATURE || t.op[i] == DRIFT_XF_SOFTCAP) && v > 0.0f) continue;
    return false;
  }
  return true;
}

// The kernels' form of a checked chain: TEMPERATURE multiplies by the reciprocal.
Chain make_chain(const drift_transform& t) {
  Chain c;
  c.n = t.count;
  for (int i = 0; i < DRIFT_MAX_TRANSFORMS; ++i) {
    const bool used = i < t.count;
    c.op[i] = used ? t.op[i] : 0;
    const float v = used ? t.value[i] : 1.0f;
    c.inv[i] = (float)(1.0 / (double)v);
    c.v[i] = (used && t.op[i] == DRIFT_XF_TEMPERATURE) ? c.inv[i] : v;
  }
  // the folded form (rowio.h): factors before and after the one soft-cap step, in fp64
  const double log2e = 1.44269504088896340736;
  int nsoft = 0;
  double pre = 1.0, post = 1.0, cap = 1.0;
  for (int i = 0; i < t.count; ++i) {
    if (t.op[i] == DRIFT_XF_SOFTCAP) {
      ++nsoft;
      cap = (double)t.value[i];
      continue;
    }
    const double f = t.op[i] == DRIFT_XF_TEMPERATURE ? 1.0 / (double)t.value[i]
                                                     : (double)t.value[i];
    (nsoft == 0 ? pre : post) *= f;
  }
  c.kind = nsoft == 0 ? 1 : (nsoft == 1 ? 2 : 0);
  const double fa = nsoft == 0 ? 0.0 : post * cap;
  const double fb = nsoft == 0 ? pre : -2.0 * post * cap;
  c.fc = nsoft == 1 ? (float)(2.0 * log2e * pre / cap) : 0.0f;
  c.fa = (float)fa;
  c.fb = (float)fb;
  c.fal = (float)(fa * log2e);
  c.fbl = (float)(fb * log2e);
  c.fald = (double)c.fa * log2e;
  c.fbld = (double)c.fb * log2e;
  c.fdz = nsoft == 1 ? (float)(4.0 * pre * post) : 0.0f;
  c.lse_scale = c.fbl != 0.0f ? (double)c.fb / (double)c.fbl : 0.693147180559945309417;
  // factors whose folded form leaves the fp32 range keep the step-by-step chain
  const float f[6] = {c.fc, c.fa, c.fb, c.fal, c.fbl, c.fdz};
  for (float x : f)
    if (!(fabsf(x) < INFINITY)) c.kind = 0;
  if (c.kind == 2 && !(fabsf(c.fc) >= 1.17549435e-38f)) c.kind = 0;  // fc not a normal float
  // g carries at most 3.6e-7 |fa| of error into z (one-ulp exp2 and reciprocal); above
  // |fa| = 40 that would exceed 1.5e-5 and the chain is applied step by step instead
  if (c.kind == 2 && !(fabsf(c.fa) <= 40.0f)) c.kind = 0;
  c.kfix = (float)(ceil(fabs((double)c.fa) * log2e) + 1.0);
  return c;
}

}  // namespace

extern "C" {

size_t drift_workspace_size(int op, int64_t num_rows, int64_t vocab, int64_t hidden_dim,
                            int dtype) {
  if (num_rows < 0 || num_rows > INT32_MAX || vocab < 1) return 0;
  switch (op) {
    case DRIFT_OP_SELECTED_LOGPROB:
      if (dtype != DRIFT_F32 && dtype != DRIFT_BF16) return 0;
      return kLogprobWsBytes;
    case DRIFT_OP_DIAGNOSTICS:
      return diag_ws_bytes(num_rows);
    case DRIFT_OP_LMHEAD:
    case DRIFT_OP_LMHEAD_VH:
      if (dtype != DRIFT_BF16 || hidden_dim < 1 || hidden_dim % 8 || vocab % 8) return 0;
      if (hidden_dim > (int64_t{1} << 22) || !lmhead_shape_ok(num_rows, vocab)) return 0;
      return lmhead_ws_bytes(num_rows, hidden_dim, vocab, op == DRIFT_OP_LMHEAD_VH);
    case DRIFT_OP_ACTIVE_ROWS:
      return compact_ws_bytes(num_rows);
    default:
      return 0;
  }
}

}  // extern "C"

namespace {

// Checks the logical inputs of `a` (ids, masks, layout, chains, vocab_real against
// `vocab_ids`, the global column count) and, with `logits`, the logits description; fills
// the common part of the scoring parameters. Returns a status.
int prepare(const drift_logprob_args* a, bool logits, int64_t vocab_ids, ScoreParams& sp,
            int64_t min_vocab = 1) {
  if (!a) return DRIFT_EINVAL;
  if (a->logits_dtype != DRIFT_F32 && a->logits_dtype != DRIFT_BF16) return DRIFT_EDTYPE;
  if (a->ids_dtype != DRIFT_I32 && a->ids_dtype != DRIFT_I64) return DRIFT_EDTYPE;
  if (a->reduction != DRIFT_REDUCE_TREE && a->reduction != DRIFT_REDUCE_EXACT)
    return DRIFT_EINVAL;
  const int64_t N = a->num_rows, V = a->vocab;
  if (N < 0 || N > INT32_MAX || V < min_vocab || V > INT32_MAX || a->row_stride < V)
    return DRIFT_EINVAL;
  if (vocab_ids < 1 || vocab_ids > INT32_MAX) return DRIFT_EINVAL;
  const size_t esz = a->logits_dtype == DRIFT_F32 ? 4 : 2;
  const size_t isz = a->ids_dtype == DRIFT_I32 ? 4 : 8;
  if (N > 0) {
    if (!a->target_ids || !aligned(a->target_ids, isz)) return DRIFT_EINVAL;
    // an empty shard (V = 0) reads no logits; its pointers may be null
    if (logits && V > 0 &&
        (!a->train_logits || !a->rollout_logits || !aligned(a->train_logits, esz) ||
         !aligned(a->rollout_logits, esz)))
      return DRIFT_EINVAL;
  }
  switch (a->layout) {
    case DRIFT_PAD_RIGHT:
    case DRIFT_PAD_LEFT:
      if (a->batch < 0 || a->seq_len < 1 || a->batch > INT32_MAX || a->seq_len > INT32_MAX ||
          a->batch * a->seq_len != N)  // both below 2^31: the product cannot overflow
        return DRIFT_EINVAL;
      break;
    case DRIFT_PACKED:
      if (!a->cu_seqlens || a->num_seqs < 0 || a->num_seqs > INT32_MAX - 1 ||
          !aligned(a->cu_seqlens, 4))
        return DRIFT_EINVAL;
      break;
    default:
      return DRIFT_EINVAL;
  }
  if (a->vocab_real < 0 || a->vocab_real > vocab_ids) return DRIFT_EINVAL;
  if (!chain_ok(a->transforms[0]) || !chain_ok(a->transforms[1])) return DRIFT_EINVAL;
  for (int side = 0; side < 2; ++side) {
    if ((a->entropy[side] && !aligned(a->entropy[side], 4)) ||
        (a->lse[side] && !aligned(a->lse[side], 8)))
      return DRIFT_EINVAL;
  }
  sp = ScoreParams{};
  sp.N = N;
  sp.Vid = a->vocab_real == 0 ? vocab_ids : a->vocab_real;
  sp.V = sp.Vid < V ? sp.Vid : V;
  sp.xf[0] = make_chain(a->transforms[0]);
  sp.xf[1] = make_chain(a->transforms[1]);
  sp.stride = a->row_stride;
  sp.L = a->layout == DRIFT_PACKED ? 1 : a->seq_len;
  sp.nseq = a->num_seqs;
  sp.dtype = a->logits_dtype;
  sp.ids_i64 = a->ids_dtype == DRIFT_I64;
  sp.layout = a->layout;
  sp.train = a->train_logits;
  sp.rollout = a->rollout_logits;
  sp.ids = a->target_ids;
  sp.att = a->attention_mask;
  sp.act = a->action_mask;
  sp.cu = a->cu_seqlens;
  sp.vstart = 0;
  return DRIFT_OK;
}

int check_outputs(int64_t N, float* t, float* r, float* d, uint8_t* act) {
  if (N > 0 && (!t || !r || !d || !act || !aligned(t, 4) || !aligned(r, 4) || !aligned(d, 4)))
    return DRIFT_EINVAL;
  return DRIFT_OK;
}

}  // namespace

extern "C" {

int drift_selected_logprob(const drift_logprob_args* a, float* train_logp, float* rollout_logp,
                           float* dlogp, uint8_t* active, void* ws, size_t ws_bytes,
                           void* stream) {
  ScoreParams sp;
  int st = prepare(a, true, a ? a->vocab : 0, sp);
  if (st != DRIFT_OK) return st;
  if ((st = check_outputs(a->num_rows, train_logp, rollout_logp, dlogp, active)) != DRIFT_OK)
    return st;
  const bool exact = a->reduction == DRIFT_REDUCE_EXACT;
  if (exact && (a->entropy[0] || a->entropy[1])) return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < kLogprobWsBytes) return DRIFT_EWORKSPACE;
  sp.out_t = train_logp;
  sp.out_r = rollout_logp;
  sp.out_d = dlogp;
  sp.active = active;
  for (int side = 0; side < 2; ++side) {
    sp.ent[side] = a->entropy[side];
    sp.lse[side] = a->lse[side];
  }
  sp.ws = (char*)ws;
  const hipEvent_t e0 = (hipEvent_t)a->prof_events[0], e1 = (hipEvent_t)a->prof_events[1];
  const hipError_t e = exact ? launch_score_exact(sp, (hipStream_t)stream, e0, e1)
                             : launch_score(sp, (hipStream_t)stream, e0, e1);
  return e == hipSuccess ? DRIFT_OK : DRIFT_EHIP;
}

int drift_shard_partials(const drift_logprob_args* local, int64_t vocab_start,
                         int64_t vocab_global, drift_lse_partial* train_part,
                         drift_lse_partial* rollout_part, void* ws, size_t ws_bytes,
                         void* stream) {
  ScoreParams sp;
  int st = prepare(local, true, vocab_global, sp, 0);  // a shard may hold no column
  if (st != DRIFT_OK) return st;
  if (vocab_start < 0 || vocab_start % 8 != 0 || vocab_start + local->vocab > vocab_global)
    return DRIFT_EINVAL;
  if (local->entropy[0] || local->entropy[1] || local->lse[0] || local->lse[1])
    return DRIFT_EINVAL;
  if (local->num_rows > 0 && (!train_part || !rollout_part || !aligned(train_part, 8) ||
                              !aligned(rollout_part, 8)))
    return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < kLogprobWsBytes) return DRIFT_EWORKSPACE;
  // columns of this shard that enter the log-sum-exp
  const int64_t in = sp.Vid - vocab_start;
  sp.V = in < 0 ? 0 : (in < local->vocab ? in : local->vocab);
  sp.vstart = vocab_start;
  sp.part[0] = train_part;
  sp.part[1] = rollout_part;
  sp.ws = (char*)ws;
  const hipEvent_t e0 = (hipEvent_t)local->prof_events[0], e1 = (hipEvent_t)local->prof_events[1];
  return launch_score_exact(sp, (hipStream_t)stream, e0, e1) == hipSuccess ? DRIFT_OK
                                                                          : DRIFT_EHIP;
}

int drift_merge_shards(const drift_logprob_args* global, const drift_lse_partial* train_parts,
                       const drift_lse_partial* rollout_parts, int num_shards,
                       const int64_t* shard_bounds, float* train_logp, float* rollout_logp,
                       float* dlogp, uint8_t* active, void* ws, size_t ws_bytes,
                       void* stream) {
  MergeParams m;
  int st = prepare(global, false, global ? global->vocab : 0, m.p);
  if (st != DRIFT_OK) return st;
  if ((st = check_outputs(global->num_rows, train_logp, rollout_logp, dlogp, active)) != DRIFT_OK)
    return st;
  if (global->entropy[0] || global->entropy[1]) return DRIFT_EINVAL;
  if (num_shards < 1 || num_shards > kMaxShards || !shard_bounds) return DRIFT_EINVAL;
  if (shard_bounds[0] != 0 || shard_bounds[num_shards] != global->vocab) return DRIFT_EINVAL;
  for (int s = 0; s < num_shards; ++s)
    if (shard_bounds[s + 1] < shard_bounds[s]) return DRIFT_EINVAL;
  if (global->num_rows > 0 && (!train_parts || !rollout_parts || !aligned(train_parts, 8) ||
                               !aligned(rollout_parts, 8)))
    return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < kLogprobWsBytes) return DRIFT_EWORKSPACE;
  m.p.out_t = train_logp;
  m.p.out_r = rollout_logp;
  m.p.out_d = dlogp;
  m.p.active = active;
  m.p.lse[0] = global->lse[0];
  m.p.lse[1] = global->lse[1];
  m.p.ws = (char*)ws;
  m.part[0] = train_parts;
  m.part[1] = rollout_parts;
  m.S = num_shards;
  for (int s = 0; s <= kMaxShards; ++s) m.bound[s] = s <= num_shards ? shard_bounds[s] : 0;
  return launch_merge_shards(m, (hipStream_t)stream) == hipSuccess ? DRIFT_OK : DRIFT_EHIP;
}

int drift_get_status(const void* ws, void* stream, int64_t* first_bad_row) {
  if (!ws) return DRIFT_EWORKSPACE;
  WsHeader h;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&h, ws, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess)
    return DRIFT_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DRIFT_EHIP;
  return status_from_header(h, first_bad_row);
}

int drift_diagnostics(const float* dlogp, const uint8_t* active, int64_t num_rows,
                      double eps_low, double eps_high, const void* logprob_ws,
                      drift_stats* out_host, void* ws, size_t ws_bytes, void* stream) {
  if (!out_host || num_rows < 0 || num_rows > INT32_MAX) return DRIFT_EINVAL;
  if (num_rows > 0 && (!dlogp || !active || !aligned(dlogp, 4))) return DRIFT_EINVAL;
  if (!(eps_low >= 0.0 && eps_low < 1.0 && eps_high >= 0.0 && eps_high < 1.0))
    return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < diag_ws_bytes(num_rows)) return DRIFT_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  DiagParams dp{};
  dp.N = num_rows;
  dp.eps_low = eps_low;
  dp.eps_high = eps_high;
  dp.d = dlogp;
  dp.active = active;
  dp.lp = (const WsHeader*)logprob_ws;
  dp.ws = (char*)ws;
  if (launch_diagnostics(dp, s) != hipSuccess) return DRIFT_EHIP;
  // one copy: the device folded the logprob status into stats.status
  if (hipMemcpyAsync(out_host, (const char*)ws + diag_stats_offset(), sizeof(drift_stats),
                     hipMemcpyDeviceToHost, s) != hipSuccess)
    return DRIFT_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DRIFT_EHIP;
  return out_host->status;
}

int drift_diagnostics_async(const float* dlogp, const uint8_t* active, int64_t num_rows,
                            double eps_low, double eps_high, const void* logprob_ws,
                            drift_stats* out, void* ws, size_t ws_bytes, void* stream) {
  if (!out || !aligned(out, 8) || num_rows < 0 || num_rows > INT32_MAX) return DRIFT_EINVAL;
  if (num_rows > 0 && (!dlogp || !active || !aligned(dlogp, 4))) return DRIFT_EINVAL;
  if (!(eps_low >= 0.0 && eps_low < 1.0 && eps_high >= 0.0 && eps_high < 1.0))
    return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < diag_ws_bytes(num_rows)) return DRIFT_EWORKSPACE;
  DiagParams dp{};
  dp.N = num_rows;
  dp.eps_low = eps_low;
  dp.eps_high = eps_high;
  dp.d = dlogp;
  dp.active = active;
  dp.lp = (const WsHeader*)logprob_ws;
  dp.ws = (char*)ws;
  dp.out = out;
  return launch_diagnostics(dp, (hipStream_t)stream) == hipSuccess ? DRIFT_OK : DRIFT_EHIP;
}

int drift_diagnostics_noalloc(const float* dlogp, const uint8_t* active, int64_t num_rows,
                              double eps_low, double eps_high, const void* logprob_ws,
                              drift_stats* out_dev, void* stream) {
  if (!out_dev || !aligned(out_dev, 8) || num_rows < 0) return DRIFT_EINVAL;
  if (num_rows > DRIFT_NOALLOC_MAX_ROWS) return DRIFT_EINVAL;
  if (num_rows > 0 && (!dlogp || !active || !aligned(dlogp, 4))) return DRIFT_EINVAL;
  if (!(eps_low >= 0.0 && eps_low < 1.0 && eps_high >= 0.0 && eps_high < 1.0))
    return DRIFT_EINVAL;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  if (diag_noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return DRIFT_EHIP;
  if (ws_bytes < diag_ws_bytes(num_rows)) return DRIFT_EWORKSPACE;  // cannot happen
  DiagParams dp{};
  dp.N = num_rows;
  dp.eps_low = eps_low;
  dp.eps_high = eps_high;
  dp.d = dlogp;
  dp.active = active;
  dp.lp = (const WsHeader*)logprob_ws;
  dp.ws = ws;
  dp.out = out_dev;
  return launch_diagnostics(dp, (hipStream_t)stream) == hipSuccess ? DRIFT_OK : DRIFT_EHIP;
}

int drift_segment_diagnostics(const float* dlogp, const uint8_t* active, int64_t num_rows,
                              const int32_t* seg_offsets, int64_t num_segments,
                              double eps_low, double eps_high, const void* logprob_ws,
                              drift_stats* out_dev, void* stream) {
  if (num_rows < 0 || num_rows > INT32_MAX || num_segments < 0 || num_segments > INT32_MAX)
    return DRIFT_EINVAL;
  if (!(eps_low >= 0.0 && eps_low < 1.0 && eps_high >= 0.0 && eps_high < 1.0))
    return DRIFT_EINVAL;
  if (num_segments > 0) {
    if (!seg_offsets || !out_dev || !aligned(seg_offsets, 4) || !aligned(out_dev, 8))
      return DRIFT_EINVAL;
    if (num_rows > 0 && (!dlogp || !active || !aligned(dlogp, 4))) return DRIFT_EINVAL;
  }
  SegParams sp;
  sp.N = num_rows;
  sp.S = num_segments;
  sp.eps_low = eps_low;
  sp.eps_high = eps_high;
  sp.d = dlogp;
  sp.active = active;
  sp.off = seg_offsets;
  sp.lp = (const WsHeader*)logprob_ws;
  sp.out = out_dev;
  if (launch_segment_diagnostics(sp, (hipStream_t)stream) != hipSuccess) return DRIFT_EHIP;
  return DRIFT_OK;
}

int drift_active_rows(const uint8_t* active, int64_t num_rows, int32_t* rows, int64_t* n_dev,
                      void* ws, size_t ws_bytes, void* stream) {
  if (num_rows < 0 || num_rows > INT32_MAX) return DRIFT_EINVAL;
  if (!n_dev || !aligned(n_dev, 8)) return DRIFT_EINVAL;
  if (num_rows > 0 && (!active || !rows || !aligned(rows, 4))) return DRIFT_EINVAL;
  if (!ws || !aligned(ws, 256) || ws_bytes < compact_ws_bytes(num_rows)) return DRIFT_EWORKSPACE;
  return launch_compact(active, num_rows, rows, n_dev, (char*)ws, (hipStream_t)stream) ==
                 hipSuccess
             ? DRIFT_OK
             : DRIFT_EHIP;
}

}  // extern "C"

namespace {

int lmhead_call(const void* hidden, const void* weight, bool w_vh, int64_t T, int64_t H,
                int64_t V, const int32_t* target_ids, const uint8_t* active, float* logp,
                void* ws, size_t ws_bytes, void* stream, const drift_transform* chain) {
  if (T < 0 || T > INT32_MAX || H < 1 || V < 1 || V > INT32_MAX) return DRIFT_EINVAL;
  if (H % 8 != 0 || V % 8 != 0 || H > (int64_t{1} << 22)) return DRIFT_EINVAL;
  if (!lmhead_shape_ok(T, V)) return DRIFT_EINVAL;
  if (T > 0 && (!hidden || !weight || !target_ids || !logp)) return DRIFT_EINVAL;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(target_ids, 4) ||
      !aligned(logp, 4))
    return DRIFT_EINVAL;
  LmheadParams lp;
  lp.xf = Chain{};
  if (chain && chain->count > 0) {  // the head takes folded chains only (rowio.h)
    if (!chain_ok(*chain)) return DRIFT_EINVAL;
    lp.xf = make_chain(*chain);
    if (lp.xf.kind == 0) return DRIFT_EINVAL;
  }
  if (!ws || !aligned(ws, 256) || ws_bytes < lmhead_ws_bytes(T, H, V, w_vh))
    return DRIFT_EWORKSPACE;
  lp.T = T;
  lp.H = H;
  lp.V = V;
  lp.w_vh = w_vh;
  lp.hidden = hidden;
  lp.weight = weight;
  lp.ids = target_ids;
  lp.active = active;
  lp.logp = logp;
  lp.ws = (char*)ws;
  if (launch_lmhead(lp, (hipStream_t)stream) != hipSuccess) return DRIFT_EHIP;
  return DRIFT_OK;
}

}  // namespace

extern "C" {

int drift_lmhead_logprob(const void* hidden, const void* weight, int64_t T, int64_t H, int64_t V,
                         const int32_t* target_ids, const uint8_t* active, float* logp,
                         void* ws, size_t ws_bytes, void* stream) {
  return lmhead_call(hidden, weight, false, T, H, V, target_ids, active, logp, ws, ws_bytes,
                     stream, nullptr);
}

int drift_lmhead_logprob_vh(const void* hidden, const void* weight_vh, int64_t T, int64_t H,
                            int64_t V, const int32_t* target_ids, const uint8_t* active,
                            float* logp, void* ws, size_t ws_bytes, void* stream) {
  return lmhead_call(hidden, weight_vh, true, T, H, V, target_ids, active, logp, ws, ws_bytes,
                     stream, nullptr);
}

int drift_lmhead_logprob_chain(const void* hidden, const void* weight, int weight_layout,
                               int64_t T, int64_t H, int64_t V, const int32_t* target_ids,
                               const uint8_t* active, const drift_transform* transform,
                               float* logp, void* ws, size_t ws_bytes, void* stream) {
  if (weight_layout != DRIFT_WEIGHT_HV && weight_layout != DRIFT_WEIGHT_VH) return DRIFT_EINVAL;
  return lmhead_call(hidden, weight, weight_layout == DRIFT_WEIGHT_VH, T, H, V, target_ids,
                     active, logp, ws, ws_bytes, stream, transform);
}

int drift_dlogits(const drift_logprob_args* a, int side, const double* lse,
                  const uint8_t* active, const float* grad_logp, int out_dtype,
                  void* grad_logits, int64_t out_stride, void* stream) {
  if (!a || (side != 0 && side != 1)) return DRIFT_EINVAL;
  if (a->logits_dtype != DRIFT_F32 && a->logits_dtype != DRIFT_BF16) return DRIFT_EDTYPE;
  if (a->ids_dtype != DRIFT_I32 && a->ids_dtype != DRIFT_I64) return DRIFT_EDTYPE;
  if (out_dtype != DRIFT_F32 && out_dtype != DRIFT_BF16) return DRIFT_EDTYPE;
  const int64_t N = a->num_rows, V = a->vocab;
  if (N < 0 || N > INT32_MAX || V < 1 || V > INT32_MAX || a->row_stride < V || out_stride < V)
    return DRIFT_EINVAL;
  if (a->vocab_real < 0 || a->vocab_real > V) return DRIFT_EINVAL;
  const drift_transform& t = a->transforms[side];
  if (!chain_ok(t)) return DRIFT_EINVAL;
  const void* logits = side == 0 ? a->train_logits : a->rollout_logits;
  const size_t esz = a->logits_dtype == DRIFT_F32 ? 4 : 2;
  const size_t isz = a->ids_dtype == DRIFT_I32 ? 4 : 8;
  const size_t osz = out_dtype == DRIFT_F32 ? 4 : 2;
  if (N > 0) {
    if (!logits || !a->target_ids || !lse || !active || !grad_logits) return DRIFT_EINVAL;
    if (!aligned(logits, esz) || !aligned(a->target_ids, isz) || !aligned(lse, 8) ||
        !aligned(grad_logits, osz) || (grad_logp && !aligned(grad_logp, 4)))
      return DRIFT_EINVAL;
  }
  DlogitsParams dp;
  dp.N = N;
  dp.V = V;
  dp.Vr = a->vocab_real == 0 ? V : a->vocab_real;
  dp.stride = a->row_stride;
  dp.out_stride = out_stride;
  dp.dtype = a->logits_dtype;
  dp.ids_i64 = a->ids_dtype == DRIFT_I64;
  dp.out_dtype = out_dtype;
  dp.xf = make_chain(t);
  dp.logits = logits;
  dp.ids = a->target_ids;
  dp.lse = lse;
  dp.active = active;
  dp.grad = grad_logp;
  dp.out = grad_logits;
  if (launch_dlogits(dp, (hipStream_t)stream) != hipSuccess) return DRIFT_EHIP;
  return DRIFT_OK;
}

const drift_backend_desc* drift_backend_descriptor(void) {
  static const drift_backend_desc d = {
      DRIFT_ABI_VERSION,
      "drift.gfx950.v1",
      "selected_token_logprob,dlogp,entropy,lse,exact_reduction,vocab_shard_partials,shard_merge,drift_diagnostics,segment_diagnostics,mismatch_kl,active_rows,lmhead_selected_logprob,dlogits",
      "gfx950",
      "logits:f32,bf16;ids:i32,i64;lmhead:bf16",
      "pad_right,pad_left,packed(cu_seqlens);logits row-major [N,row_stride]",
      "deterministic; fixed-order reductions; per-row results bitwise independent of "
      "batch composition and position; no atomics in value paths",
      "logits widened to fp32; exp2 in fp32 with a power-of-two running max; sums in "
      "fp64; lse/logp/dlogp formed in fp64, rounded once to fp32; diagnostics in fp64; "
      "transform chains with at most one softcap (|cap x later factors| <= 40) folded "
      "for the lse terms and dlogits (softcap as 1 - 2/(1 + 2^(2 log2e x/cap)), one exp2 and one "
      "reciprocal, within 3.6e-7 cap; a fixed exponent offset), others and the selected "
      "logit step by step; lmhead products bf16 x bf16 -> fp32 accumulate, fixed k order",
      "natural log",
      "none: one implementation per (op, dtype, transform chain form: decided by the "
      "caller's chain, never by data or device); unsupported inputs fail closed",
      DRIFT_BUILD_FINGERPRINT,
  };
  return &d;
}

const char* drift_strerror(int status) {
  switch (status) {
    case DRIFT_OK: return "ok";
    case DRIFT_EINVAL: return "invalid argument";
    case DRIFT_EDTYPE: return "unsupported dtype";
    case DRIFT_EWORKSPACE: return "workspace missing, too small, misaligned or not initialised";
    case DRIFT_ETOKEN: return "selected token id outside [0, V) on an active row";
    case DRIFT_EMASK: return "invalid attention/action mask or packed metadata";
    case DRIFT_ENOACTIVE: return "no active rows";
    case DRIFT_ENONFINITE: return "non-finite logit or dlogp on an active row";
    case DRIFT_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
