/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse token-choice MoE layer.
 *
 * One process, one GPU.  Every entry point validates its arguments on the
 * host, enqueues hand-written HIP kernels on the given stream and returns; no
 * call synchronises the device and no call allocates or frees device memory.
 * The caller owns every buffer; the library keeps no pointer after a call
 * returns.  Layer outputs that later calls need (logits, top-K, rows, saved
 * activations) are plain caller buffers passed back in.
 *
 * Sources (web pages on the method, cited by title and section):
 *  [P1] "Wrong router gradient with experts_implementation=batched_mm under
 *       expert parallelism": cause section (sentinel slots, proj_out mask).
 *  [P2] MiniMind issue "[Bug] num_experts_per_tok=1: the MoE router receives
 *       no gradient": sections 2 and 3 (renormalised top-1 has a constant
 *       weight).
 *  [P3] "MoE" tutorial chapter (8-MoE): Router/Gating Network, KeepTopK,
 *       Expert Capacity, GShard pseudo-code, Switch Transformers, ST-MoE
 *       (router z-loss), efficient inference (grouping and permutation).
 *  [P4] "MoE training: routing and communication behind sparse compute":
 *       forward data path, load balance, capacity.
 *  [P5] course notes "08 MoE: capacity, routing, gradients, balance and
 *       system implementation": sections 8.1-8.8.
 *
 * Conventions shared by all entry points
 *  - Layouts are row-major.  x, y, dx, dy: [T][D].  logits: [T][E] fp32.
 *    topk_idx, topk_w: [T][K].  Router weight W_r: [E][D] fp32 (s = x W_r^T).
 *    Expert weights (GShard orientation, [P3] GShard pseudo-code):
 *      w_gate, w_up: [G][D][F];  w_down: [G][F][D]
 *    where G = (expert_hi - expert_lo) + n_shared: local routed experts first,
 *    then the shared expert.
 *  - dtype MOE_BF16: x, dy, dx, expert weights and their gradients, x_perm,
 *    act, h, o_perm, y are bf16 (fp32 accumulation everywhere); the router
 *    (logits, W_r, dW_r) stays fp32 ([P3] Switch Transformers: the router is
 *    kept in full precision).  dtype MOE_F32: all of those are fp32.
 *  - "rows": routed rows are expert-major (local expert lo..hi-1), in token
 *    order within an expert; the shared expert's rows follow, one per token.
 *    rows_max (moe_rows_max) bounds every row buffer.
 *  - Routing (cfg->routing).  MOE_TOKEN_CHOICE: slot tables (topk_idx,
 *    topk_w, slot_row) are [T][K], slot t*K+k.  MOE_EXPERT_CHOICE (course
 *    notes 8.4): moe_route_expert_choice replaces moe_route and moe_permute;
 *    slot tables are [T][E], slot t*E+e is the pair (token t, expert e),
 *    topk_w holds p = softmax(s) for every pair and topk_idx is not used (an
 *    implicit identity); K is the average number of experts per token, which
 *    sets the per-expert capacity C; moe_expert_ffn, moe_combine,
 *    aux_balance_loss and moe_backward take the same [T][E] tables.
 *  - Pointers must be 16-byte aligned device pointers (MOE_EALIGN).
 *  - Requirements: T >= 0; D and F positive multiples of 64, at most 2^20
 *    (row buffers of any total size are supported); 1 <= K <= E;
 *    K <= 64 for token choice; E <= 1024; 0 <= expert_lo <= expert_hi <= E;
 *    n_shared in {0,1}; expert choice needs softmax scoring and
 *    MOE_GATE_TRUNCATED (MOE_EINVAL).  T == 0 is a successful no-op.
 *  - Inputs are assumed finite; no entry point checks for NaN or Inf.
 *  - Return value: MOE_OK or a negative MOE_E* code; moe_error_string() gives
 *    text (for MOE_ELAUNCH it includes the HIP error of the failed launch).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* a size, range or enum is out of bounds, or NULL    */
  MOE_EALIGN = -2,     /* a pointer is not 16-byte aligned                   */
  MOE_EDTYPE = -3,     /* dtype not supported for this operation             */
  MOE_ELAUNCH = -4,    /* a HIP launch or runtime call failed                */
  MOE_EWORKSPACE = -5  /* workspace smaller than moe_workspace_size()        */
};

enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_GATE_TRUNCATED = 0, /* gating A: g = p over all E, not renormalised */
       MOE_GATE_RENORM = 1 };  /* gating B: renormalised over the top-K        */
enum { MOE_F32 = 0, MOE_BF16 = 1 };
enum { MOE_ROUTE_LOGITS_GIVEN = 1 }; /* moe_route flag: logits is an input   */
enum { MOE_TOKEN_CHOICE = 0,   /* every token picks its top-K experts            */
       MOE_EXPERT_CHOICE = 1 }; /* every expert picks its top-C tokens          */

/* Plain configuration record, read during the call and never retained. */
typedef struct moe_config {
  int32_t T, D, E, K, F;         /* tokens, model dim, global experts, top-k, FFN width */
  int32_t expert_lo, expert_hi;  /* local experts [lo,hi); slots routed elsewhere are sentinels */
  int32_t n_shared;              /* 0 or 1 always-on shared expert of width F, weight 1 */
  int32_t score_fn;              /* MOE_SCORE_* */
  int32_t gating;                /* MOE_GATE_* */
  int32_t dtype;                 /* MOE_F32 or MOE_BF16 */
  double capacity_factor;        /* <= 0: no capacity (dropless); C = ceil(c*T*K/E) in double */
  int32_t routing;               /* MOE_TOKEN_CHOICE or MOE_EXPERT_CHOICE */
} moe_config;

/* A hipStream_t (NULL: the null stream). */
typedef void* moe_stream_t;

/* Capacity per expert, C = ceil(c*T*K/E) with the global E, evaluated in
 * double ([P5] 8.5; [P3] Switch Transformers capacity factor).  Writes -1
 * when capacity_factor <= 0.  Expert choice: the number of tokens every
 * expert takes, min(ceil(c*T*K/E), T) with c = 1 when capacity_factor <= 0.
 * Host-only. */
int moe_capacity(const moe_config* cfg, int32_t* capacity);

/* rows_max = T*K + n_shared*T (token choice) or (expert_hi - expert_lo)*C +
 * n_shared*T (expert choice, C from moe_capacity).  Host-only. */
int moe_rows_max(const moe_config* cfg, int64_t* rows);

/* Bytes of device workspace needed by moe_permute, moe_route_permute,
 * aux_balance_loss and moe_backward for this configuration.  Host-only. */
int moe_workspace_size(const moe_config* cfg, size_t* bytes);

/*
 * moe_route -- router GEMM, score, top-K and gate weights.
 * [P3] Router/Gating Network (s = x W_g then a score function); [P5] 8.2
 * (token-choice top-K, gating A vs B), 8.6 (sigmoid scores with selection
 * bias b_e used only to select); [P3] KeepTopK.
 *   x        [T][D] (dtype)            in
 *   w_r      [E][D] fp32               in
 *   r_bias   [E] fp32 or NULL          in   router bias, added to the logits
 *   sel_bias [E] fp32 or NULL          in   selection bias (sigmoid only)
 *   logits   [T][E] fp32               out (in with MOE_ROUTE_LOGITS_GIVEN;
 *                                            then x, w_r, r_bias are unused)
 *   topk_idx [T][K] int32              out  in pick order: descending key,
 *                                            equal keys -> lower index first
 *   topk_w   [T][K] fp32               out  gate weights (A or B)
 *   lse      [T] fp32                  out  log-sum-exp of the logits
 * The logits are the binary32 rounding of a double-precision sum of the
 * exact products: another summation order changes a logit only when its
 * double sum lies within double rounding error of a binary32 rounding
 * boundary.  Given identical logits the top-K is bit-exact.  Selection key: softmax -> the logit; sigmoid -> sig32(s) + b, a
 * fixed binary32 sequence (range reduction by ln2 split in two parts, degree-7
 * Taylor polynomial with fma, scaling by 2^n, IEEE division).
 * Token choice only (MOE_EINVAL under expert choice).
 */
int moe_route(const moe_config* cfg, const void* x, const float* w_r, const float* r_bias,
              const float* sel_bias, float* logits, int32_t* topk_idx, float* topk_w, float* lse,
              int32_t flags, moe_stream_t stream);

/*
 * moe_permute -- expert histogram, prefix scan, stable in-expert rank,
 * capacity drops, row maps and the gather of token rows.
 * [P3] efficient inference (sort tokens by expert, gather), GShard
 * pseudo-code (expert buffers filled in token order; overflow dropped),
 * Expert Capacity; [P5] 8.5 (C = ceil(c*T*K/E)), 8.8 (group by expert);
 * [P1] cause section (slots of experts outside [lo,hi) are sentinels).
 *   topk_idx   [T][K] int32  in
 *   x          [T][D] dtype  in
 *   counts_all [E] int32     out  slots per expert over all E, before capacity
 *   offsets    [G+1] int32   out  row offsets of the groups (shared last)
 *   slot_row   [T*K] int32   out  row of slot t*K+k; -1 dropped; -2 sentinel
 *   row_token  [rows_max]    out  token of each row (valid for rows < offsets[G])
 *   row_slot   [rows_max]    out  slot t*K+k of each routed row; -1 for shared rows
 *   n_dropped  [1] int32     out  local assignments dropped by capacity
 *   x_perm     [rows_max][D] out  x rows of the routed rows (shared rows are
 *                                 not copied: the shared expert reads x)
 *   ws, ws_bytes             workspace of moe_workspace_size() bytes
 * Deterministic: the rank inside an expert comes from counts and scans, not
 * from atomic slot grabbing.
 * Token choice only (MOE_EINVAL under expert choice).
 */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* counts_all, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                int32_t* row_slot, int32_t* n_dropped, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/*
 * moe_route_permute -- moe_route (plain routing: no given logits, jitter or
 * noise) followed by moe_permute, in fewer launches: with at most 16 experts
 * and up to 32768 slots the router also ranks every slot among its
 * workgroup's slots of the same expert, and one more kernel forms the
 * offsets, assigns the rows and gathers the token rows (two launches where
 * the separate calls take three); otherwise the two calls' kernels run in
 * sequence.  [P3] Router/Gating Network, efficient inference (group
 * the tokens by expert); [P5] 8.5 (capacity), 8.8.
 *   Arguments and outputs: those of moe_route (flags 0) and moe_permute, with
 *   the same layouts; every output is identical, bit for bit, to the two
 *   separate calls.
 *   ws: the workspace of moe_workspace_size (no initial contents needed).
 * Errors: those of moe_route and moe_permute.
 */
int moe_route_permute(const moe_config* cfg, const void* x, const float* w_r,
                      const float* r_bias, const float* sel_bias, float* logits,
                      int32_t* topk_idx, float* topk_w, float* lse, int32_t* counts_all,
                      int32_t* offsets, int32_t* slot_row, int32_t* row_token, int32_t* row_slot,
                      int32_t* n_dropped, void* x_perm, void* ws, size_t ws_bytes,
                      moe_stream_t stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * results and errors as moe_permute, bit for bit.  Its scratch (the tiled
 * permute's per-tile expert histograms and bases, 2 * ceil(T*K/256) * E
 * int32) lives in a static device array of 8 MiB that every GPU the library
 * runs on holds until the process ends; T*K*E up to about 2^28 fits.  Larger
 * configurations return MOE_EWORKSPACE before any device call.  The call
 * allocates nothing.  It runs on the current device; the first call on a
 * device looks up that device's copy of the array (MOE_ELAUNCH if that
 * fails).  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (on different streams, or from several host threads) race, so
 * order them on one stream.
 */
int moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                        int32_t* row_token, int32_t* row_slot, int32_t* n_dropped, void* x_perm,
                        moe_stream_t stream);

/*
 * moe_expert_ffn -- grouped SwiGLU experts on the permuted rows.
 * [P5] 8.1 (SwiGLU expert, ~3DF parameters), 8.7 (shared expert, weight 1),
 * 8.8 (grouped GEMM instead of a per-expert loop); [P3] efficient inference.
 *   x, x_perm            in   (the shared group reads x directly)
 *   offsets [G+1]        in   from moe_permute
 *   w_gate, w_up, w_down in   expert weights (layouts above)
 *   act   [rows_max][2F] out  saved pre-activations: a = x W_gate in columns
 *                             [0,F), b = x W_up in [F,2F)
 *   h     [rows_max][F]  out  silu(a) * b
 *   o_perm[rows_max][D]  out  expert output h W_down, unweighted (proj_out)
 * Only rows < offsets[G] are written.  No host synchronisation: the grid is
 * sized from rows_max and surplus workgroups exit.
 */
int moe_expert_ffn(const moe_config* cfg, const void* x, const void* x_perm, const int32_t* offsets,
                   const void* w_gate, const void* w_up, const void* w_down, void* act, void* h,
                   void* o_perm, moe_stream_t stream);

/*
 * moe_combine -- weighted scatter-add back to token order.
 * [P5] 8.8 (a token appears K times: accumulate, do not overwrite), 8.7
 * (shared expert added with weight 1); [P3] GShard combine.
 *   y[t] = sum_k [slot_row >= 0] topk_w[t,k] * o_perm[slot_row[t,k]]
 *          + o_perm[offsets[G-1] + t] (shared)          fp32 accumulation
 * Sentinel and dropped slots contribute nothing; a token with all slots
 * dropped gets y = 0 (the residual path is outside the layer).  Expert
 * choice: k runs over the E pairs of the [T][E] tables.
 */
int moe_combine(const moe_config* cfg, const void* o_perm, const int32_t* offsets,
                const int32_t* slot_row, const float* topk_w, void* y, moe_stream_t stream);

/*
 * aux_balance_loss -- Switch load-balance loss and router z-loss.  Defined
 * for softmax scoring only (MOE_EINVAL for sigmoid).
 * [P5] 8.5 (L = alpha*E*sum_e f_e P_e with f held constant), [P4] load
 * balance section; [P3] ST-MoE and [P5] 8.6 (z-loss on log-sum-exp).
 *   f_e = counts_all[e]/(T*K), P_e = mean_t softmax(s_t)_e  (under expert
 *   choice f_e = C/(T*K) for every e, so the balance term is constant and
 *   its gradient zero up to rounding; the z-loss is unchanged)
 *   losses[0] = alpha*E*sum_e f_e P_e;  losses[1] = z_lambda*mean_t lse_t^2;
 *   losses[2] = mean_t lse_t^2 (raw)                         [3] fp32, device
 *   d_logits [T][E] fp32 (NULL: not written) = d(losses[0]+losses[1])/ds
 */
int aux_balance_loss(const moe_config* cfg, const float* logits, const int32_t* counts_all,
                     float alpha, float z_lambda, float* losses, float* d_logits, void* ws,
                     size_t ws_bytes, moe_stream_t stream);

/*
 * moe_backward -- full backward of the layer given dy.
 * [P1] cause section: the gradient of a gate weight is that slot's proj_out,
 * so sentinel (and dropped) slots have proj_out = 0 and dg = 0; [P5] 8.3 and
 * [P2] section 2: gradients reach the router only through the continuous
 * gate weights (top-K indices are piecewise constant).
 *   saved forward tensors: x, w_r, logits, topk_idx, topk_w, offsets,
 *   slot_row, x_perm, act, h, o_perm; weights w_gate, w_up, w_down.
 *   Expert choice: topk_idx may be NULL (the [T][E] tables are indexed by
 *   expert); the gating gradient is that of softmax A over all E pairs,
 *   ds_i = p_i (dg_i - sum_j p_j dg_j), dg = 0 for pairs not taken.
 *   dy [T][D]               in
 *   d_logits_extra [T][E]   in, NULL = none (e.g. from aux_balance_loss)
 *   dx [T][D]               out  through the experts and the router
 *   dw_r [E][D] fp32        out
 *   d_rbias [E] fp32        out, may be NULL
 *   dw_gate, dw_up [G][D][F], dw_down [G][F][D]   out (experts with no rows
 *                                                     get zeros)
 *   d_logits_out [T][E]     out, may be NULL: the logit gradient ds
 * Gating backward (centred forms, G = sum_k g_k dg_k): softmax A:
 * ds_i = p_i(sum_{k:i_k=i} dg_k - G); softmax B: ds_{i_k} = g_k(dg_k - G),
 * other ds = 0; sigmoid A: ds = dg sig(1-sig); sigmoid B:
 * ds = ((dg - G)/sum sig) sig(1-sig).  With K = 1 and B the result is exactly 0.
 */
int moe_backward(const moe_config* cfg, const void* x, const float* w_r, const float* logits,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                 const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                 const void* o_perm, const void* w_gate, const void* w_up, const void* w_down,
                 const void* dy, const float* d_logits_extra, void* dx, float* dw_r,
                 float* d_rbias, void* dw_gate, void* dw_up, void* dw_down, float* d_logits_out,
                 void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Routing with router-logit jitter and noisy top-K selection ("MoE" tutorial
 * chapter, sections ST-MoE and KeepTopK; course notes section 8.6).
 *   jitter: fp32 [T][E] factors u (the tutorial draws them from
 *     [0.99, 1.01]) or NULL; s~ = s * u (one binary32 multiply) is written to
 *     `logits` and replaces the logits everywhere downstream (selection,
 *     weights, lse, losses, backward).  With MOE_ROUTE_LOGITS_GIVEN the
 *     given logits are jittered in place.
 *   w_noise: fp32 [E][D] or NULL.  With it, n = x W_noise^T (binary32 from a
 *     double sum) is written to noise_logits [T][E] and the selection key is
 *     fl32(s~ + eps * softplus(n)), evaluated in double, with eps =
 *     noise_eps [T][E] (standard-normal draws, one per token and expert);
 *     the gate weights and lse stay on s~: the noise only selects.  Noise
 *     requires softmax scoring (MOE_EINVAL otherwise).
 * The random draws are inputs: the library draws nothing.  Every other
 * argument is as in moe_route, which is this call with no jitter or noise.
 */
int moe_route_ex(const moe_config* cfg, const void* x, const float* w_r, const float* r_bias,
                 const float* sel_bias, const float* jitter, const float* w_noise,
                 const float* noise_eps, float* noise_logits, float* logits, int32_t* topk_idx,
                 float* topk_w, float* lse, int32_t flags, moe_stream_t stream);

/*
 * moe_backward with router-logit jitter: `logits` are the jittered s~ that
 * moe_route_ex wrote and `jitter` the same u ([T][E] fp32, or NULL: this is
 * moe_backward).  The gating gradient w.r.t. s~ (plus d_logits_extra, which
 * is taken w.r.t. s~ as well) is multiplied by u, so dx, dw_r, d_rbias and
 * d_logits_out are gradients w.r.t. the raw logits s = x W_r^T + r_b.  The
 * noise logits get no gradient: the noise only selects.
 */
int moe_backward_ex(const moe_config* cfg, const void* x, const float* w_r, const float* logits,
                    const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                    const void* o_perm, const void* w_gate, const void* w_up, const void* w_down,
                    const void* dy, const float* d_logits_extra, const float* jitter, void* dx,
                    float* dw_r, float* d_rbias, void* dw_gate, void* dw_up, void* dw_down,
                    float* d_logits_out, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Load-driven selection-bias step ("Course notes 08 MoE", section 8.6: the
 * experts select on s_e + b_e; an overloaded expert lowers b_e, an
 * underloaded one raises it, by a fixed step; the gate weights keep using the
 * raw scores).  For every expert e:
 *   counts_all[e] * E > T * K  ->  sel_bias[e] -= gamma
 *   counts_all[e] * E < T * K  ->  sel_bias[e] += gamma    (binary32 add)
 *   otherwise unchanged.
 * counts_all: int32 [E] as written by moe_permute (all E, before capacity);
 * sel_bias: fp32 [E], updated in place, caller-owned device memory.  Meant
 * to run once per training step after the routing has consumed sel_bias.
 * Token choice only (expert choice has no selection bias).
 * Errors: MOE_EINVAL (bad config, non-finite gamma, null), MOE_EALIGN.
 */
int moe_bias_update(const moe_config* cfg, const int32_t* counts_all, float gamma,
                    float* sel_bias, moe_stream_t stream);

/*
 * Sequence-wise balance loss (course notes section 8.5's balance loss
 * applied to each sequence of seq_len consecutive tokens and averaged over
 * the T / seq_len sequences; section 8.6 keeps such a term beside the bias
 * rule):
 *   f_{b,e} = (slots of sequence b that chose e) / (seq_len * K)
 *   P_{b,e} = mean over the tokens t of b of p_{t,e}
 *   loss    = alpha * E * (seq_len / T) * sum_b sum_e f_{b,e} P_{b,e}
 * with p = softmax(s) for softmax scoring and sigma(s_e) / sum_j sigma(s_j)
 * for sigmoid scoring; the gradient holds f constant:
 *   d_logits[t,i] = w_{t,i} (u_{b,i} - sum_e p_{t,e} u_{b,e}),
 *   u_{b,e} = alpha * E / T * f_{b,e},  w = p (softmax) or
 *   sigma_i (1 - sigma_i) / sum_j sigma_j (sigmoid).
 * logits: fp32 [T][E]; topk_idx: int32 [T][K] (moe_route); loss: fp32 [1]
 * out; d_logits: fp32 [T][E] out (NULL: loss only), overwritten, or added to
 * when accumulate != 0 (to combine with aux_balance_loss's gradient before
 * moe_backward); ws: the layer workspace.  seq_len must divide T.
 * Token choice only (every expert's load is fixed under expert choice).
 * Errors: MOE_EINVAL (bad config, seq_len, non-finite alpha, null),
 * MOE_EALIGN, MOE_EWORKSPACE.
 */
int aux_seq_loss(const moe_config* cfg, const float* logits, const int32_t* topk_idx,
                 int32_t seq_len, float alpha, float* loss, float* d_logits, int32_t accumulate,
                 void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Expert-choice routing ("Course notes 08 MoE", section 8.4: each expert
 * takes a fixed number of tokens from the batch, so a token can be served by
 * several experts or by none; every expert's load is exactly C).  Replaces
 * moe_route + moe_permute when cfg->routing == MOE_EXPERT_CHOICE.
 *   x [T][D] dtype, w_r [E][D] fp32, r_bias [E] fp32 or NULL   in
 *   logits   [T][E] fp32  out (in with MOE_ROUTE_LOGITS_GIVEN: then x is
 *                              still read by the gather, w_r and r_bias not)
 *   gate_w   [T][E] fp32  out  p_{t,e} = softmax(s_t)_e for every pair
 *   lse      [T] fp32     out  log-sum-exp of the logits (may be NULL)
 *   counts_all [E] int32  out  C for every expert (each takes exactly C)
 *   offsets  [G+1] int32  out  g*C for the local experts, then the shared block
 *   slot_row [T][E] int32 out  row of pair (t,e); -1 not taken; -2 expert
 *                              outside [expert_lo, expert_hi)
 *   row_token, row_slot [rows_max] int32  out  token t and pair t*E+e of
 *                              each routed row (row_slot -1 for shared rows)
 *   x_perm   [rows_max][D] dtype  out  x rows of the routed rows
 *   ws, ws_bytes             workspace of moe_workspace_size() bytes
 * Selection: every local expert e takes the C tokens with the largest key
 * fl32(s_{t,e} - lse_t), s and lse evaluated in double and rounded once, equal
 * keys going to the lower token; its rows are e's block of C rows in token
 * order.  C = min(ceil(c*T*K/E), T), c = capacity_factor or 1 when <= 0.
 * The layer output is y_t = sum over the experts that took t of
 * p_{t,e} FFN_e(x_t) (plus the shared expert): moe_combine with these tables.
 * Deterministic; bit-identical selection for identical logits.
 * Errors: MOE_EINVAL (config not expert choice, NULL, flags), MOE_EALIGN,
 * MOE_EWORKSPACE, MOE_ELAUNCH.
 */
int moe_route_expert_choice(const moe_config* cfg, const void* x, const float* w_r,
                            const float* r_bias, float* logits, float* gate_w, float* lse,
                            int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                            int32_t* row_token, int32_t* row_slot, void* x_perm, int32_t flags,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/* Text for an error code (thread-local detail for MOE_ELAUNCH). */
const char* moe_error_string(int code);

/*
 * Environment variables read at every call (measurement and tests only):
 *   MOE_GEMM_CFG        forces the grouped-GEMM kernel variant: a number
 *                       0..11 for every GEMM (9 to 11 are weight-gradient
 *                       kernels; the other GEMMs then take 1), or
 *                       "name=cfg,..." pairs
 *                       (gemm_gate_up_fwd, gemm_down_fwd, gemm_down_dgrad,
 *                       gemm_down_wgrad, gemm_gate_up_dgrad, gemm_gate_up_wgrad).
 *   MOE_SERIAL_STREAMS  when set, moe_backward runs every kernel on the
 *                       caller's stream instead of overlapping independent
 *                       parts on the library's side streams.
 * MOE_SERIAL_STREAMS does not change any result; every MOE_GEMM_CFG variant
 * meets the same tolerances (each is tested against the oracle).
 *
 * Kernel timing for measurement: while enabled, every kernel the library
 * launches is bracketed by HIP events recorded on its own stream.
 * moe_timing_report() waits for those events and writes one line per kernel
 * name, "name<TAB>launches<TAB>total_ms\n", into buf (NUL-terminated,
 * truncated to len), then clears the records.  Not for concurrent use from
 * several host threads.
 */
int moe_timing_enable(int32_t on);
int moe_timing_report(char* buf, size_t len);
/*
 * Restrict timing to launches of one kernel name (as reported by
 * moe_timing_report); NULL or "" times every launch again.  Timing one
 * kernel adds two event records per launch of it and nothing to the others,
 * so it can stay on inside a timed run.  Events come from a pool that is
 * reused after each report.
 */
int moe_timing_select(const char* kernel_name);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
