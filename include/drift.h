/*
 * drift.h - C ABI of the MI355X (gfx950) selected-token logprob drift library.
 *
 * What is computed (the pages' measurement contract):
 *   For every active row r of a teacher-forced batch, the selected-token log-probability
 *   of both sides, logp = x[y_r] - log(sum_i exp(x_i)), and the drift
 *   dlogp = train_recomputed_logp - rollout_old_logp
 *   ("WS2 Cross-Config Logprob Drift Contract", section "Measurement Contract"), then the
 *   diagnostics ratio0, clipfrac0, approx_kl0 and mean/p95/p99/max |dlogp| over the
 *   active rows (same page, "Diagnostics" table), and optionally the logits themselves
 *   from hidden x W_vocab ("[WS2] Framework for ablation experiment", LogProb knobs
 *   row 9, "LM-head GEMM and materialization boundary").
 *
 * Conventions shared by every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller (e.g. torch tensors);
 *     the library never allocates device memory and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void*; every call is stream-ordered. Only
 *     drift_diagnostics and drift_get_status synchronize the stream.
 *   - The caller provides a device workspace of at least drift_workspace_size() bytes,
 *     256-byte aligned. A workspace must not be shared by calls that can overlap.
 *   - Return value: DRIFT_OK (0) or a negative DRIFT_E* status. Argument errors are
 *     detected on the host and returned at once, before any launch. Data-dependent
 *     errors (mask shape, token ids, non-finite logits) are found on the device and
 *     recorded in the workspace; drift_get_status() and drift_diagnostics() report them.
 *     There is exactly one implementation per (operation, dtype); the library never
 *     falls back to another algorithm ("Kernel Integration Contract": no silent
 *     fallback).
 *   - Results are deterministic and each row's results are bitwise independent of the
 *     batch it is scored in (the "Attention Debug Matrix" page, Metrics: the
 *     batch-composition control must be exactly zero).
 */
#ifndef DRIFT_H
#define DRIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRIFT_ABI_VERSION 10

/* ---- status codes ---------------------------------------------------------------- */
#define DRIFT_OK          0
#define DRIFT_EINVAL     -1  /* null/negative/inconsistent argument, misaligned pointer  */
#define DRIFT_EDTYPE     -2  /* unsupported logits or id dtype                           */
#define DRIFT_EWORKSPACE -3  /* workspace missing, too small or misaligned               */
#define DRIFT_ETOKEN     -4  /* an active row's selected id is outside [0, V)            */
#define DRIFT_EMASK      -5  /* mask byte not 0/1, action on a padded row, attention not
                                contiguous on the declared padding side, bad cu_seqlens  */
#define DRIFT_ENOACTIVE  -6  /* diagnostics over zero active rows                        */
#define DRIFT_ENONFINITE -7  /* NaN/+inf logit in an active row, selected logit -inf, a
                                row maximum (after the chain) beyond |z| ~ 7.4e8 (the
                                exponent range, 2^30 / log2 e; the exact mode: 1.16e7),
                                or a non-finite active dlogp; such rows' outputs are NaN */
#define DRIFT_EHIP       -8  /* a HIP runtime call failed                                */

/* ---- element types ---------------------------------------------------------------- */
#define DRIFT_F32  0
#define DRIFT_BF16 1
#define DRIFT_I32  2
#define DRIFT_I64  3

/* ---- batch layouts (the padding side of "Measurement Contract") ------------------- */
#define DRIFT_PAD_RIGHT 0  /* each sequence: attended rows, then padding              */
#define DRIFT_PAD_LEFT  1  /* each sequence: padding, then attended rows              */
#define DRIFT_PACKED    2  /* sequences packed back to back, delimited by cu_seqlens  */

/* ---- logit transforms ("[WS2] Framework for ablation experiment", LogProb knobs row 7:
 *      an ordered chain applied to every logit before the softmax) ---------------------- */
#define DRIFT_XF_SCALE       1  /* x -> x * value        (logit_scale)                   */
#define DRIFT_XF_TEMPERATURE 2  /* x -> x / value        (value > 0; as x * (1/value))   */
#define DRIFT_XF_SOFTCAP     3  /* x -> value * tanh(x * (1/value))  (value > 0)         */
#define DRIFT_MAX_TRANSFORMS 4
/* Arithmetic of a chain in drift_selected_logprob (either reduction): the selected
 * logit takes the steps one by one (tanhf for SOFTCAP). For the log-sum-exp terms a chain
 * with at most one SOFTCAP step is folded into z = a + b g(x): g = x for multiplying
 * steps only, and g = 1 / (1 + 2^(c x)) around one SOFTCAP step (tanh(u) = 1 - 2 /
 * (e^(2u) + 1), one hardware exp2 and one reciprocal per logit), within 3.6e-7 |a| of the
 * exact value, where |a| is the cap times the factors after it; used when |a| <= 40 on
 * both sides, else (and for two SOFTCAP steps) the steps are applied one by one to every
 * logit (DRIFT_REDUCE_EXACT forms each folded logit a + b g(x) before its integer
 * bins). drift_dlogits takes a side's chain in the same folded form when it folds. */

typedef struct drift_transform {
  int32_t count;                       /* steps in use, 0 = identity                     */
  int32_t op[DRIFT_MAX_TRANSFORMS];    /* DRIFT_XF_*, applied in index order             */
  float value[DRIFT_MAX_TRANSFORMS];   /* finite; > 0 for TEMPERATURE and SOFTCAP        */
} drift_transform;

/* ---- reduction of the log-sum-exp ("[WS2] Framework for ablation experiment", LogProb
 *      knobs rows 4-5: reduction topology and merge order) ------------------------------ */
#define DRIFT_REDUCE_TREE  0  /* fp64 partials merged in a tree fixed by V (fastest)      */
#define DRIFT_REDUCE_EXACT 1  /* exact integer sums of per-group values: the same bits for
                                 any split of the vocabulary into shards and any merge
                                 order (the tp-partition control)                         */

/* One side's log-sum-exp partial of one row over one vocabulary shard, in the exact
 * form: the row's value sum_v exp(z_v) over the shard's columns is
 * (bin[0] * 2^64 + bin[1] * 2^32 + bin[2]) * 2^(32 * (top - 2)), accumulated from groups
 * of 8 columns (4 for fp32 logits) aligned in the global column index. Partials of any
 * shards add exactly (bin-wise after aligning `top`), so their merge does not depend on
 * how the vocabulary was split or in which order they are combined. */
typedef struct drift_lse_partial {
  uint64_t bin[3];  /* bins top, top-1, top-2                                       */
  int32_t top;      /* bin index of bin[0]; -2^28 when the shard saw no column      */
  uint32_t flags;   /* DRIFT_PART_* bits                                            */
  float x_sel;      /* the selected logit after the transforms, if this shard owns it */
  float reserved;
} drift_lse_partial;
#define DRIFT_PART_SCORED  1u  /* the row is active with a valid id                      */
#define DRIFT_PART_OWNER   2u  /* the selected id lies in this shard's columns           */
#define DRIFT_PART_BAD     4u  /* a NaN / +inf logit or |logit| >= 1.16e7 in the shard    */
#define DRIFT_MAX_SHARDS  64

/* ---- operations (for drift_workspace_size) ---------------------------------------- */
#define DRIFT_OP_SELECTED_LOGPROB 0
#define DRIFT_OP_DIAGNOSTICS      1
#define DRIFT_OP_LMHEAD           2
#define DRIFT_OP_ACTIVE_ROWS      3
#define DRIFT_OP_LMHEAD_VH        4  /* drift_lmhead_logprob_vh */

/*
 * Arguments of drift_selected_logprob. Logical inputs follow "Measurement Contract"
 * (same token ids, selected ids, attention and action masks, padding layout, packed
 * metadata on both sides).
 *
 *  logits_dtype    DRIFT_F32 or DRIFT_BF16 (both sides share it).
 *  ids_dtype       DRIFT_I32 or DRIFT_I64.
 *  layout          DRIFT_PAD_RIGHT, DRIFT_PAD_LEFT or DRIFT_PACKED.
 *  num_rows        N, rows of the logits tensors (B*L, or the packed capacity). N < 2^31;
 *                  batches beyond one dispatch's 2^32 - 1 work-items are scored by several
 *                  launches over consecutive row ranges, with the same per-row results.
 *  vocab           V >= 1, logits per row; every column enters the log-sum-exp.
 *  row_stride      elements between the starts of consecutive rows, >= V.
 *  train_logits, rollout_logits
 *                  [N, row_stride] row-major, element-aligned. Rows are pre-shifted:
 *                  row r scores target_ids[r] (LogProb knobs row 8). Only active rows
 *                  are read.
 *  target_ids      [N] selected token ids; values on inactive rows are never checked
 *                  (e.g. an ignore_index of -100 is fine there).
 *  attention_mask  [N] bytes 0/1, or NULL = all rows attended (PACKED: all rows before
 *                  cu_seqlens[num_seqs]). RIGHT: every sequence is 1..1 0..0; LEFT:
 *                  0..0 1..1; PACKED: if given, exactly the rows before the end.
 *  action_mask     [N] bytes 0/1, or NULL = every attended row. 0 on prompt rows.
 *  batch, seq_len  RIGHT/LEFT: B and L with B*L == N. Ignored for PACKED.
 *  cu_seqlens      PACKED: device int32 [num_seqs+1], starting at 0, non-decreasing,
 *                  ending <= N; rows at or past the end are packed-buffer padding.
 *  num_seqs        PACKED: number of sequences.
 *  prof_events     optional pair of hipEvent_t (as void*), recorded on `stream` right
 *                  before and after the scoring kernel; NULL entries are skipped.
 *  vocab_real      columns that enter the log-sum-exp: 0 or V = all ("include"), else
 *                  the first vocab_real columns only ("mask": padded vocab rows are
 *                  excluded, LogProb knobs row 2); selected ids must lie below it.
 *  transforms      [0] train side, [1] rollout side: ordered logit transforms applied to
 *                  every logit of that side (the selected one included) before the
 *                  softmax (LogProb knobs row 7). count = 0 on both sides = none.
 *  reduction       DRIFT_REDUCE_TREE or DRIFT_REDUCE_EXACT (see above); entropy needs
 *                  DRIFT_REDUCE_TREE.
 *  entropy         optional outputs ([0] train, [1] rollout; NULL = not computed): fp32
 *                  [N] device arrays, the entropy -sum_v p_v log p_v of the row's softmax
 *                  (after the transforms, over the vocab_real columns), from the same pass
 *                  (LogProb knobs row 11, entropy reduction). 0 on inactive rows, NaN on
 *                  active rows with a rejected id.
 *  lse             optional outputs ([0] train, [1] rollout; NULL = not written): fp64 [N]
 *                  device arrays, the natural-log LSE of the row (the input of
 *                  drift_dlogits). 0 on inactive rows, NaN on active rows with a rejected
 *                  id. Writing it costs no extra pass.
 *
 * A row is active iff attention != 0 and action != 0 (and, PACKED, it is before the end).
 */
typedef struct drift_logprob_args {
  int32_t logits_dtype;
  int32_t ids_dtype;
  int32_t layout;
  int32_t reduction;           /* DRIFT_REDUCE_TREE (0) or DRIFT_REDUCE_EXACT */
  int64_t num_rows;
  int64_t vocab;
  int64_t row_stride;
  const void* train_logits;
  const void* rollout_logits;
  const void* target_ids;
  const uint8_t* attention_mask;
  const uint8_t* action_mask;
  int64_t batch;
  int64_t seq_len;
  const int32_t* cu_seqlens;
  int64_t num_seqs;
  void* prof_events[2];
  int64_t vocab_real;
  drift_transform transforms[2];
  float* entropy[2];
  double* lse[2];
} drift_logprob_args;

/* Statistics of drift_diagnostics ("Diagnostics" table; every metric over active rows).
 *  ratio0          mean over active rows of exp(dlogp)
 *  clipfrac0       (n_clip_low + n_clip_high) / n_active; a ratio is clipped iff
 *                  exp(d) < 1 - eps_low or exp(d) > 1 + eps_high (evaluated in fp64)
 *  approx_kl0      mean of exp(d) - 1 - d, evaluated as expm1(d) - d in fp64: the k3
 *                  estimator of KL(rollout || train) from rollout-sampled tokens
 *                  ("Attention Debug Matrix", Metrics: mismatch_k3_kl)
 *  mismatch_kl     mean of -d = mean of log pi_rollout(y) - log pi_train(y): the k1
 *                  estimator of the same KL (the forward mismatch_kl of that section)
 *  mean_abs_dlogp  mean |d|;   mean_dlogp: mean d
 *  p95/p99_abs_dlogp  nearest rank: the ceil(q*n)-th smallest |d| (exact)
 *  max_abs_dlogp   the largest |d|; argmax_row: smallest row index attaining it
 *  n_nonfinite     active rows whose d is NaN or +-inf (then status ENONFINITE and the
 *                  means and order statistics are not meaningful)
 *  status          the value drift_diagnostics returns
 * Means are fp64 sums in a fixed order divided by n; counts and order statistics are
 * exact. With n_active == 0 the means and order statistics are NaN, argmax_row is -1. */
typedef struct drift_stats {
  int64_t n_active;
  int64_t n_clip_low;
  int64_t n_clip_high;
  int64_t n_nonfinite;
  int64_t argmax_row;
  double ratio0;
  double clipfrac0;
  double approx_kl0;
  double mean_abs_dlogp;
  double mean_dlogp;
  float p95_abs_dlogp;
  float p99_abs_dlogp;
  float max_abs_dlogp;
  int32_t status;
  double mismatch_kl;
} drift_stats;

/* Backend descriptor ("Kernel Integration Contract": stable id, semantic operator,
 * supported architectures/dtypes/layouts, determinism properties, precision and
 * downcast points, build fingerprint). Static storage; never free. */
typedef struct drift_backend_desc {
  int32_t abi_version;
  const char* backend_id;
  const char* semantic_ops;
  const char* archs;
  const char* dtypes;
  const char* layouts;
  const char* determinism;
  const char* precision;
  const char* lse_domain;
  const char* fallback;
  const char* build_fingerprint;
} drift_backend_desc;

/* Workspace bytes for `op` over `num_rows` rows of `vocab` columns of element type
 * `dtype`; `hidden_dim` is H for DRIFT_OP_LMHEAD (num_rows = T there) and ignored
 * otherwise. Returns 0 for invalid arguments. Host only.
 * The "WS2 Cross-Config Logprob Drift Contract" page, Kernel Integration Contract, asks a
 * backend for no hidden long-lived state: the library allocates nothing and keeps nothing
 * between calls, so every device buffer a call needs beyond its inputs and outputs is a
 * caller-owned workspace of this size, and everything in it is rewritten by the call. */
size_t drift_workspace_size(int op, int64_t num_rows, int64_t vocab, int64_t hidden_dim,
                            int dtype);

/* Vocabulary-parallel scoring, one shard's part ("[WS2] Framework for ablation
 * experiment", LogProb knobs rows 3-5 and 8; the allgather_partials_fixed_merge
 * topology). `local` describes this shard's logits: train/rollout_logits point to the
 * [N, row_stride] rows of its `vocab` columns, which are the global columns
 * [vocab_start, vocab_start + vocab); ids, masks and layout are the global ones, and
 * local->vocab_real is the global count of real columns (0 = vocab_global). Requires
 * vocab_start % 8 == 0, vocab_start + vocab <= vocab_global, no entropy / lse outputs.
 * Writes one exact partial per row and side ([N] each; rows that are not scored get
 * flags 0) and the owner's selected logit. Errors of the logical inputs are recorded in
 * `ws` as for drift_selected_logprob. Asynchronous. */
int drift_shard_partials(const drift_logprob_args* local, int64_t vocab_start,
                         int64_t vocab_global, drift_lse_partial* train_part,
                         drift_lse_partial* rollout_part, void* ws, size_t ws_bytes,
                         void* stream);

/* Merge of gathered shard partials in global shard order, then the same finalization as
 * drift_selected_logprob with DRIFT_REDUCE_EXACT: for every shard split the outputs are
 * bitwise those of the unsharded exact call (the tp-partition control).
 *   global        the unsharded arguments (N, vocab = vocab_global, vocab_real, ids, masks,
 *                 layout, lse outputs); logits pointers are not read
 *   train_parts, rollout_parts   device [num_shards][N] partials (an all-gather result)
 *   shard_bounds  host int64 [num_shards + 1]: 0 = b_0 <= b_1 <= ... <= b_S = vocab,
 *                 shard s owns [b_s, b_{s+1}); 1 <= num_shards <= DRIFT_MAX_SHARDS
 * A selected id whose owner shard did not flag it gives EMASK (inconsistent shard
 * metadata). Outputs and status as drift_selected_logprob. Asynchronous. */
int drift_merge_shards(const drift_logprob_args* global, const drift_lse_partial* train_parts,
                       const drift_lse_partial* rollout_parts, int num_shards,
                       const int64_t* shard_bounds, float* train_logp, float* rollout_logp,
                       float* dlogp, uint8_t* active, void* ws, size_t ws_bytes,
                       void* stream);

/* Per-row selected-token logprobs of both sides and their drift
 * ("Measurement Contract"). Outputs, each [N] device arrays:
 *   train_logp, rollout_logp  x_y - LSE(x), fp32 (the fp64 result rounded once)
 *   dlogp                     (x^t_y - x^r_y) - (LSE^t - LSE^r) formed in fp64 from the
 *                             unrounded terms, rounded once to fp32
 *   active                    1 on active rows, 0 elsewhere
 * Inactive rows get 0.0; active rows with an out-of-range id get NaN (status ETOKEN).
 * LSE uses fp32 exp2 terms summed in fp64 with a power-of-two running maximum; the
 * reduction tree depends only on V, so a row's bits do not depend on the batch.
 * Asynchronous: returns after launching; data-dependent errors are read later with
 * drift_get_status(ws) or by passing ws to drift_diagnostics as logprob_ws. */
int drift_selected_logprob(const drift_logprob_args* args, float* train_logp,
                           float* rollout_logp, float* dlogp, uint8_t* active, void* ws,
                           size_t ws_bytes, void* stream);

/* Synchronizes `stream` and returns the data-dependent status recorded by the last
 * drift_selected_logprob or drift_lmhead_logprob call on `ws` (priority EMASK > ETOKEN
 * > ENONFINITE), and, if first_bad_row is not NULL, the smallest row index of that
 * error class (-1 when OK). A workspace that no such call initialised gives
 * DRIFT_EWORKSPACE.
 * Errors found on the device are reported here rather than hidden: the Kernel
 * Integration Contract of "WS2 Cross-Config Logprob Drift Contract" rules out a silent
 * fallback, and the Drift Source Taxonomy of the same page makes a logical-input
 * violation (mask, token id) an invalid comparison, not a noisy one. */
int drift_get_status(const void* ws, void* stream, int64_t* first_bad_row);

/* Diagnostics over the active rows of `dlogp` ("Diagnostics" table). Fills *out_host
 * (host memory) and synchronizes `stream` once. eps_low, eps_high in [0, 1) give the clip
 * range [1 - eps_low, 1 + eps_high]. `logprob_ws` (nullable) is the workspace of the
 * drift_selected_logprob call that produced dlogp: its device status is read in the same
 * synchronization and takes priority in the return value. Returns DRIFT_OK,
 * DRIFT_ENOACTIVE, DRIFT_ENONFINITE, or the logprob status. No threshold is applied:
 * the library reports, it never decides pass/fail. */
int drift_diagnostics(const float* dlogp, const uint8_t* active, int64_t num_rows,
                      double eps_low, double eps_high, const void* logprob_ws,
                      drift_stats* out_host, void* ws, size_t ws_bytes, void* stream);

/* drift_diagnostics without the synchronization, for loops that read a step's statistics
 * while later work runs (a training loop checks step i while step i + 1 is on the GPU).
 *   out   drift_stats [1], caller-owned, writable by the device: device memory, or pinned
 *         host memory (hipHostMalloc) that the host reads once the stream has passed this
 *         call (an event, or a synchronization); its `status` field holds what
 *         drift_diagnostics would return (DRIFT_OK, DRIFT_ENOACTIVE, DRIFT_ENONFINITE, or
 *         the logprob_ws status)
 *   other arguments as drift_diagnostics; ws and out stay in use until the stream has
 *   passed the call
 * The statistics are bitwise those of drift_diagnostics on the same inputs (the same
 * kernels). Returns DRIFT_OK after launching, or EINVAL / EWORKSPACE before any launch,
 * or EHIP when a launch fails. ("Diagnostics" table; the Kernel Integration Contract of
 * "WS2 Cross-Config Logprob Drift Contract": the device status travels with the
 * statistics, nothing is decided or dropped on the host.) */
int drift_diagnostics_async(const float* dlogp, const uint8_t* active, int64_t num_rows,
                            double eps_low, double eps_high, const void* logprob_ws,
                            drift_stats* out, void* ws, size_t ws_bytes, void* stream);

/* Largest batch of drift_diagnostics_noalloc. */
#define DRIFT_NOALLOC_MAX_ROWS (1 << 22)

/* drift_diagnostics for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): no workspace argument,
 * no synchronization, statistics written to device memory.
 *   out_dev   drift_stats [1] device, caller-owned: receives the statistics; its `status`
 *             field holds what drift_diagnostics would return (DRIFT_OK, DRIFT_ENOACTIVE,
 *             DRIFT_ENONFINITE, or the logprob_ws status)
 *   other arguments as drift_diagnostics; num_rows <= DRIFT_NOALLOC_MAX_ROWS, else
 *   DRIFT_EINVAL before any launch
 * The statistics are bitwise those of drift_diagnostics on the same inputs. The kernels'
 * scratch (tile partials and digit histograms, 561 KiB) is a device array inside the
 * library, one copy per GPU, kept until the process ends; the first call on a device looks
 * up its address (hipGetSymbolAddress) with that device current, later calls reuse it.
 * Every call on a GPU shares that GPU's scratch, and the kernels rewrite everything they
 * read from it, so sequential calls are independent; calls that can overlap on one GPU
 * (different streams, threads or processes sharing it) race and must be serialized by
 * the caller. The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine) and records no memset. Asynchronous; returns DRIFT_EHIP if a launch or
 * the address lookup fails. */
int drift_diagnostics_noalloc(const float* dlogp, const uint8_t* active, int64_t num_rows,
                              double eps_low, double eps_high, const void* logprob_ws,
                              drift_stats* out_dev, void* stream);

/* The same statistics per segment of rows ("Diagnostics" table: per-sequence views, and
 * the per-rank versions of a distributed run, each rank's rows being one segment).
 *   seg_offsets   int32 [num_segments + 1] device: segment s is rows
 *                 [seg_offsets[s], seg_offsets[s+1]) (cu_seqlens for packed sequences,
 *                 b * L for batch rows); a segment with bounds outside 0 <= lo <= hi <= N
 *                 gets status EMASK
 *   out_dev       drift_stats [num_segments] device, caller-owned; argmax_row is the
 *                 global row index; status per segment as drift_diagnostics returns it
 *   logprob_ws    nullable, as for drift_diagnostics (its status outranks each segment's)
 * Needs no workspace: each segment's reduction and exact radix select run in one block.
 * Asynchronous; returns EINVAL for bad arguments before any launch. */
int drift_segment_diagnostics(const float* dlogp, const uint8_t* active, int64_t num_rows,
                              const int32_t* seg_offsets, int64_t num_segments,
                              double eps_low, double eps_high, const void* logprob_ws,
                              drift_stats* out_dev, void* stream);

/* The active rows as an ascending list ("Measurement Contract": only active
 * response/action tokens are compared), for callers that gather or scatter per-token
 * results of the active rows.
 *   active      uint8 [N] device, nonzero = active (e.g. the `active` output of
 *               drift_selected_logprob)
 *   rows        int32 [N] device, caller-owned: rows[0 .. n) receives the indices r with
 *               active[r] != 0 in ascending order; entries from n on are not written
 *   n_dev       int64 [1] device: receives n
 *   ws          drift_workspace_size(DRIFT_OP_ACTIVE_ROWS, N, 1, 0, DRIFT_F32) bytes
 *               (per-tile counts of 4096 rows, and above 1024 tiles the tiles' offsets),
 *               256-byte aligned
 * Integer work only: the result is exact and independent of scheduling. Asynchronous;
 * returns EINVAL / EWORKSPACE for bad arguments before any launch, EHIP if a launch
 * fails. */
int drift_active_rows(const uint8_t* active, int64_t num_rows, int32_t* rows, int64_t* n_dev,
                      void* ws, size_t ws_bytes, void* stream);

/* Fused LM-head selected logprob: logits z = hidden x W are formed tile by tile on the
 * matrix cores and never written to memory; logp[t] = z[t, y_t] - LSE(z[t]).
 *   hidden      bf16 [T, H] row-major (16-byte aligned rows: H % 8 == 0; H <= 2^22)
 *   weight      bf16 [H, V] row-major, vocabulary contiguous (V % 8 == 0)
 *   target_ids  int32 [T]; active (nullable) uint8 [T]: inactive rows get 0.0
 *   logp        fp32 [T]
 * The GEMM runs in one dispatch of one 512-thread block per 256 x 256 (vocab, token) tile,
 * so ceil(T/256) * ceil(V/256), each rounded up to a multiple of 16, must not exceed
 * 2^23 - 1 (T up to 3,530,752 at V = 151936); larger T returns DRIFT_EINVAL, and
 * drift_workspace_size returns 0 for it.
 * Products accumulate in fp32 over k = 0..H-1 in a fixed order that does not depend on
 * T or on the row's position, so a row's result is bitwise the same in any batch. */
int drift_lmhead_logprob(const void* hidden, const void* weight, int64_t T, int64_t H,
                         int64_t V, const int32_t* target_ids, const uint8_t* active,
                         float* logp, void* ws, size_t ws_bytes, void* stream);

/* drift_lmhead_logprob with the weight stored [V, H] row-major (hidden contiguous: the
 * layout of a linear layer's [out_features, in_features] weight, as the head's weight is
 * usually kept), the same head GEMM of "[WS2] Framework for ablation experiment", LogProb
 * knobs row 9, and the same results bit for bit: the products run over the same K order
 * on the same values. When H % 64 == 0 the weight is read in place (no transposed copy:
 * the workspace, drift_workspace_size(DRIFT_OP_LMHEAD_VH, T, V, H, DRIFT_BF16), then
 * holds only the partials and at most two 256-row tail panels); otherwise it is copied
 * with K padding. Arguments, alignment, limits and statuses as drift_lmhead_logprob;
 * weight_vh is bf16 [V, H] with 16-byte aligned rows (H % 8 == 0). */
int drift_lmhead_logprob_vh(const void* hidden, const void* weight_vh, int64_t T, int64_t H,
                            int64_t V, const int32_t* target_ids, const uint8_t* active,
                            float* logp, void* ws, size_t ws_bytes, void* stream);

/* The fused LM-head with a transform chain on the head's logits before the softmax
 * ("[WS2] Framework for ablation experiment", LogProb knobs row 7, temperature /
 * logit_scale / soft_cap, applied to the logits that rows 9-10 form and reduce in one
 * pass): logp[t] = chain(z)[t, y_t] - LSE(chain(z)[t]). The logits stay on chip, so a
 * model whose final logits are soft-capped needs the cap here.
 *   weight_layout  DRIFT_WEIGHT_HV (weight bf16 [H, V], as drift_lmhead_logprob) or
 *                  DRIFT_WEIGHT_VH (bf16 [V, H], as drift_lmhead_logprob_vh); the
 *                  workspace is that entry point's
 *   transform      the chain (nullable or count 0: the entry point without a chain, bit
 *                  for bit). It must fold (see the transform arithmetic above: at most one
 *                  SOFTCAP step, |cap x later factors| <= 40), else DRIFT_EINVAL. The
 *                  log-sum-exp terms take the folded form, the selected logit the steps one
 *                  by one; the tile and merge order are those of the entry point without a
 *                  chain, so a row's result is bitwise the same in any batch.
 * Other arguments, limits and statuses as drift_lmhead_logprob. */
#define DRIFT_WEIGHT_HV 0
#define DRIFT_WEIGHT_VH 1
int drift_lmhead_logprob_chain(const void* hidden, const void* weight, int weight_layout,
                               int64_t T, int64_t H, int64_t V, const int32_t* target_ids,
                               const uint8_t* active, const drift_transform* transform,
                               float* logp, void* ws, size_t ws_bytes, void* stream);

/* Gradient of the selected-token logprob of one side with respect to its stored logits
 * ("[WS2] Framework for ablation experiment", LogProb knobs row 11: dlogits), for the
 * backward pass of a loss L over logp. For an active row r with selected id y, upstream
 * gradient g_r = dL/dlogp_r and z = chain(x) (the side's transform chain):
 *   grad_logits[r, v] = g_r * ([v == y] - exp(z_v - lse[r])) * dz_v/dx_v   for v < vocab_real
 *                     = 0                                                  for vocab_real <= v < V
 * Inactive rows (active[r] == 0) are written with zeros; columns past V (up to out_stride)
 * are not touched. NaN lse (a row the forward pass rejected) gives a NaN row.
 *   args        the drift_selected_logprob arguments of the forward pass: logits_dtype,
 *               ids_dtype, num_rows, vocab, row_stride, the side's logits, target_ids,
 *               vocab_real and transforms[side] are read; masks and layout are not (the
 *               forward pass's `active` carries them)
 *   side        0 = train logits, 1 = rollout logits
 *   lse         fp64 [N] device: args->lse[side] written by the forward pass
 *   active      uint8 [N] device: the forward pass's `active`
 *   grad_logp   fp32 [N] device, or NULL = 1 on every row
 *   out_dtype   DRIFT_F32, or DRIFT_BF16 (rounded to nearest even: the gradient
 *               downcast point of row 11)
 *   grad_logits [N, out_stride] of out_dtype, out_stride >= V; caller-owned
 * Elementwise: each row is read once and written once. Asynchronous; returns EINVAL /
 * EDTYPE for bad arguments before any launch, EHIP if the launch fails. */
int drift_dlogits(const drift_logprob_args* args, int side, const double* lse,
                  const uint8_t* active, const float* grad_logp, int out_dtype,
                  void* grad_logits, int64_t out_stride, void* stream);

const drift_backend_desc* drift_backend_descriptor(void);

/* Static description of a status code. */
const char* drift_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DRIFT_H */
