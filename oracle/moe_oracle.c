/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle of the sparse
 * token-choice MoE layer (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library) never links, calls or imports it, and this file shares no
 * code, header, table or constant with it.
 *
 * Arithmetic: every floating-point input is widened to double and every step
 * is computed in double precision with plain loops.  The only fp32 results
 * are (a) the router logits, rounded once from the double sum, and (b) the
 * sigmoid selection key, which follows a fixed fp32 operation sequence so
 * that a top-K decision taken on it is reproducible (see sig32 below).
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "Wrong router gradient with experts_implementation=batched_mm under
 *       expert parallelism" -- sections on the cause (sentinel slots) and on
 *       verification (per-parameter gradient comparison).
 *  [P2] MiniMind issue "[Bug] num_experts_per_tok=1: the MoE router receives no
 *       gradient" -- sections 2 (root cause) and 3 (minimal repro).
 *  [P3] "MoE" tutorial chapter (formulaic.cloudchewie.com, 8-MoE) -- sections
 *       Router/Gating Network, KeepTopK, Expert Capacity, GShard pseudo-code,
 *       Switch Transformers (capacity factor), ST-MoE (router z-loss),
 *       efficient inference (token grouping and permutation).
 *  [P4] "MoE training: routing and communication behind sparse compute" --
 *       sections on the forward data path, load balance, capacity.
 *  [P5] Course notes "08 MoE: capacity, routing, gradients, balance and
 *       system implementation" -- sections 8.1 to 8.8.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py against
 * values printed on the pages, closed forms, special cases that reduce to
 * textbook routines, brute force on tiny inputs and finite differences.
 *
 * Threading: a static parallel-for over disjoint outputs; results do not
 * depend on the thread count (each output element is summed in one fixed
 * order by one thread).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* configuration (own definition; not shared with the HIP library)          */
/* ------------------------------------------------------------------------ */
typedef struct {
  int T, D, E, K, F;   /* tokens, model dim, global experts, top-k, FFN width */
  int lo, hi;          /* experts [lo,hi) are local; the rest are sentinels   */
  int n_shared;        /* 0 or 1 always-on shared expert (width F)            */
  int score;           /* 0: softmax, 1: sigmoid                              */
  int gating;          /* 0: A (truncate), 1: B (renormalise over the top-K)  */
  double cap;          /* capacity factor; <= 0 means no capacity             */
  int bug_mode;        /* 1: negative control, sentinel proj_out NOT masked   */
} orc_cfg;

enum { DT_F32 = 0, DT_BF16 = 1, DT_F64 = 2 };

static double ld(const void* p, size_t i, int dt) {
  if (dt == DT_F64) return ((const double*)p)[i];
  if (dt == DT_F32) return (double)((const float*)p)[i];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* tiny static parallel-for                                                  */
/* ------------------------------------------------------------------------ */
typedef void (*body_fn)(void* ctx, long i);
typedef struct { body_fn fn; void* ctx; long n, t, nt; } pf_arg;

static void* pf_run(void* a_) {
  pf_arg* a = (pf_arg*)a_;
  long chunk = (a->n + a->nt - 1) / a->nt;
  long b = a->t * chunk, e = b + chunk;
  if (e > a->n) e = a->n;
  for (long i = b; i < e; ++i) a->fn(a->ctx, i);
  return NULL;
}

/* Default thread count: the CPUs this process may run on (its affinity
 * mask), at most 64 (the parallel-for's limit); callers may set their own. */
static int g_threads = 0;
void orc_set_threads(int n) { g_threads = n; }
int orc_get_threads(void) {
  if (g_threads > 0) return g_threads;
  long n = 0;
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0) n = CPU_COUNT(&set);
  if (n < 1) n = sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 64) n = 64;
  return (int)n;
}

static void parallel_for(long n, body_fn fn, void* ctx) {
  int nt = orc_get_threads();
  if (nt > n) nt = (int)(n > 0 ? n : 1);
  if (nt <= 1) {
    for (long i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[64];
  pf_arg args[64];
  if (nt > 64) nt = 64;
  for (int t = 0; t < nt; ++t) {
    args[t].fn = fn; args[t].ctx = ctx; args[t].n = n; args[t].t = t; args[t].nt = nt;
    pthread_create(&th[t], NULL, pf_run, &args[t]);
  }
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* fp32 sigmoid used for the selection key ([P5] 8.6: select on s_e + b_e)   */
/* ------------------------------------------------------------------------ */
/*
 * A top-K decision taken on sigma(s)+b flips if the two sides round sigma
 * differently, so the key is defined as one fixed sequence of IEEE binary32
 * operations (round-to-nearest-even, no contraction):
 *   exp32(z): clamp z to [-87, 87]; n = rint(z * log2(e)_f32);
 *             r = (z - n*L1) then r = fma(-n, L2, r), where L1 + L2 = ln 2 and
 *             L1 has 15 significant bits so that n*L1 is exact;
 *             p = Taylor series of e^r to degree 7, coefficients 1/k! rounded
 *             to binary32, evaluated by Horner's rule with fma;
 *             result = p * 2^n (2^n built from its exponent bits).
 *   sig32(z) = 1 / (1 + exp32(-z))   (correctly rounded division)
 * This file is compiled with -ffp-contract=off so no other fma is formed.
 */
static float exp32(float z) {
  const float LOG2E = 1.44269502162933349609375f;       /* log2(e) in binary32 */
  const float L1 = 0.693145751953125f;                  /* 0x3F317200 */
  const float L2 = 1.428606765330187045037746429443359375e-06f; /* ln2 - L1 */
  if (z > 87.0f) z = 87.0f;
  if (z < -87.0f) z = -87.0f;
  float t = z * LOG2E;
  float n = rintf(t);
  float nl1 = n * L1;
  float r = z - nl1;
  r = fmaf(-n, L2, r);
  const float c7 = (float)(1.0 / 5040.0), c6 = (float)(1.0 / 720.0), c5 = (float)(1.0 / 120.0);
  const float c4 = (float)(1.0 / 24.0), c3 = (float)(1.0 / 6.0);
  float p = c7;
  p = fmaf(p, r, c6);
  p = fmaf(p, r, c5);
  p = fmaf(p, r, c4);
  p = fmaf(p, r, c3);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  int ni = (int)n;
  uint32_t bits = (uint32_t)(ni + 127) << 23;
  float s;
  memcpy(&s, &bits, 4);
  return p * s;
}

float orc_exp32(float z) { return exp32(z); }
float orc_sig32(float z) {
  float e = exp32(-z);
  float d = 1.0f + e;
  return 1.0f / d;
}

/* ------------------------------------------------------------------------ */
/* O1: router logits  s[t,e] = sum_d x[t,d] W_r[e,d] (+ r_b[e])              */
/* [P3] Router/Gating Network (linear layer, then a score function);         */
/* [P5] 8.2 (s = x W_r).  Summed in double, rounded once to binary32.        */
/* ------------------------------------------------------------------------ */
typedef struct {
  const orc_cfg* c; const void* x; int xdt; const double* wr; const double* rb;
  float* out; double* out64; const int* tok;
} lg_ctx;

static void lg_body(void* p, long i) {
  lg_ctx* a = (lg_ctx*)p;
  const orc_cfg* c = a->c;
  long t = a->tok ? a->tok[i] : i;
  double* xr = (double*)malloc(sizeof(double) * c->D);
  for (int d = 0; d < c->D; ++d) xr[d] = ld(a->x, (size_t)t * c->D + d, a->xdt);
  for (int e = 0; e < c->E; ++e) {
    double s = 0.0;
    const double* w = a->wr + (size_t)e * c->D;
    for (int d = 0; d < c->D; ++d) s += xr[d] * w[d];
    if (a->rb) s += a->rb[e];
    if (a->out) a->out[(size_t)i * c->E + e] = (float)s;
    if (a->out64) a->out64[(size_t)i * c->E + e] = s;
  }
  free(xr);
}

/* logits for tokens tok[0..ntok) (all tokens when tok == NULL, ntok = T) */
void orc_logits(const orc_cfg* c, const void* x, int xdt, const double* wr, const double* rb,
                const int* tok, int ntok, float* out) {
  lg_ctx a = {c, x, xdt, wr, rb, out, NULL, tok};
  parallel_for(ntok, lg_body, &a);
}

/* the same sums left in double (used by finite-difference checks, where the
 * fp32 rounding of the logits would swamp the perturbation) */
void orc_logits64(const orc_cfg* c, const void* x, int xdt, const double* wr, const double* rb,
                  const int* tok, int ntok, double* out) {
  lg_ctx a = {c, x, xdt, wr, rb, NULL, out, tok};
  parallel_for(ntok, lg_body, &a);
}

/* ------------------------------------------------------------------------ */
/* O2-O4: selection key, top-K, gate weights, log-sum-exp                    */
/* ------------------------------------------------------------------------ */
/*
 * Selection ([P5] 8.2, [P3] KeepTopK): K rounds, each picking the not-yet-
 * picked expert with the largest key; equal keys go to the lower index.
 * softmax: the key is the logit itself (softmax is strictly increasing, so the
 *          chosen set equals the set chosen on probabilities).
 * sigmoid: key = sig32(s_e) + b_e in binary32 ([P5] 8.6: the bias only
 *          selects; aggregation uses the raw score).
 * Gate weights ([P5] 8.2):
 *   A: g_k = p_{i_k} with p the softmax over all E logits (sum < 1);
 *   B: g_k = exp(s_{i_k}) / sum_{j in top-K} exp(s_j)  (sum = 1), the same as
 *      renormalising the truncated p ([P3] KeepTopK gives the same weights).
 * sigmoid: A: g_k = sigma(s_{i_k});  B: g_k = sigma_{i_k} / sum_j sigma_{i_j}.
 * lse_t = log sum_e exp(s_e) (used by the router z-loss, [P3] ST-MoE).
 */
typedef struct {
  const orc_cfg* c; const double* lg; const float* selb;
  int* idx; double* w; double* lse; double* probs;
} rt_ctx;

static void rt_body(void* p, long t) {
  rt_ctx* a = (rt_ctx*)p;
  const orc_cfg* c = a->c;
  const int E = c->E, K = c->K;
  const double* s = a->lg + (size_t)t * E;
  double key[1024];
  char used[1024];
  for (int e = 0; e < E; ++e) {
    if (c->score == 0) key[e] = s[e];
    else {
      /* the logits handed to the selection are binary32 values */
      float sg = orc_sig32((float)s[e]);
      float b = a->selb ? a->selb[e] : 0.0f;
      key[e] = sg + b;
    }
    used[e] = 0;
  }
  int* idx = a->idx + (size_t)t * K;
  for (int k = 0; k < K; ++k) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (used[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e;  /* strict: ties keep lower e */
    }
    used[best] = 1;
    idx[k] = best;
  }
  /* softmax quantities in double */
  double m = -INFINITY;
  for (int e = 0; e < E; ++e) if ((double)s[e] > m) m = (double)s[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp((double)s[e] - m);
  if (a->lse) a->lse[t] = m + log(z);
  if (a->probs)
    for (int e = 0; e < E; ++e) a->probs[(size_t)t * E + e] = exp((double)s[e] - m) / z;
  double* w = a->w + (size_t)t * K;
  if (c->score == 0) {
    if (c->gating == 0) {
      for (int k = 0; k < K; ++k) w[k] = exp((double)s[idx[k]] - m) / z;
    } else {
      double zs = 0.0;
      for (int k = 0; k < K; ++k) zs += exp((double)s[idx[k]] - m);
      for (int k = 0; k < K; ++k) w[k] = exp((double)s[idx[k]] - m) / zs;
    }
  } else {
    double sg[1024];
    double tot = 0.0;
    for (int k = 0; k < K; ++k) {
      sg[k] = 1.0 / (1.0 + exp(-(double)s[idx[k]]));
      tot += sg[k];
    }
    for (int k = 0; k < K; ++k) w[k] = (c->gating == 0) ? sg[k] : sg[k] / tot;
  }
}

void orc_route(const orc_cfg* c, const double* logits, const float* selb, int* idx, double* w,
               double* lse, double* probs) {
  rt_ctx a = {c, logits, selb, idx, w, lse, probs};
  parallel_for(c->T, rt_body, &a);
}

/* ------------------------------------------------------------------------ */
/* O5: ownership, counts, capacity, expert-major row order                   */
/* ------------------------------------------------------------------------ */
/*
 * [P3] Expert Capacity / GShard pseudo-code (each expert buffer is filled in
 * token order, overflow is dropped), [P5] 8.5 (C ~ ceil(c*T*K/E)), [P1] cause
 * section (slots routed to experts not on this device are sentinels).
 *   counts_all[e] : slots choosing e, over all E, before capacity.
 *   pos           : rank of a local slot among the slots of its expert, in
 *                   token order (a token picks an expert at most once).
 *   kept          : pos < C.   Rows: expert-major (lo..hi-1), then by pos,
 *                   then the shared expert(s) with all T tokens in order.
 *   slot_row[t*K+k] = row, -1 (dropped) or -2 (sentinel).
 * offsets has G+1 entries, G = (hi-lo) + n_shared.  Returns C (or -1).
 */
long orc_capacity(const orc_cfg* c) {
  if (!(c->cap > 0.0)) return -1;
  return (long)ceil((c->cap * (double)c->T * (double)c->K) / (double)c->E);
}

void orc_dispatch(const orc_cfg* c, const int* idx, int* counts_all, int* offsets, int* slot_row,
                  int* row_token, int* row_slot, int* n_dropped) {
  const int T = c->T, K = c->K, E = c->E;
  const int EL = c->hi - c->lo;
  long C = orc_capacity(c);
  for (int e = 0; e < E; ++e) counts_all[e] = 0;
  for (long s = 0; s < (long)T * K; ++s) counts_all[idx[s]]++;
  int* kept = (int*)calloc((size_t)EL + 1, sizeof(int));
  int* fill = (int*)calloc((size_t)EL + 1, sizeof(int));
  int drop = 0;
  for (int j = 0; j < EL; ++j) {
    int n = counts_all[c->lo + j];
    kept[j] = (C >= 0 && n > C) ? (int)C : n;
    drop += n - kept[j];
  }
  offsets[0] = 0;
  for (int j = 0; j < EL; ++j) offsets[j + 1] = offsets[j] + kept[j];
  for (int sh = 0; sh < c->n_shared; ++sh) offsets[EL + sh + 1] = offsets[EL + sh] + T;
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      long s = (long)t * K + k;
      int e = idx[s];
      if (e < c->lo || e >= c->hi) { slot_row[s] = -2; continue; }
      int j = e - c->lo;
      int pos = fill[j]++;
      if (C >= 0 && pos >= C) { slot_row[s] = -1; continue; }
      int r = offsets[j] + pos;
      slot_row[s] = r;
      if (row_token) row_token[r] = t;
      if (row_slot) row_slot[r] = (int)s;
    }
  for (int sh = 0; sh < c->n_shared; ++sh)
    for (int t = 0; t < T; ++t) {
      int r = offsets[EL + sh] + t;
      if (row_token) row_token[r] = t;
      if (row_slot) row_slot[r] = -1;
    }
  *n_dropped = drop;
  free(kept);
  free(fill);
}

/* ------------------------------------------------------------------------ */
/* O6: SwiGLU expert ([P5] 8.1: ~3DF parameters per expert, no biases)       */
/*   a = x W_gate[g], b = x W_up[g] (length F), h = silu(a) * b,              */
/*   o = h W_down[g] (length D), silu(a) = a / (1 + e^-a).                    */
/* Weight layouts: W_gate, W_up [G][D][F]; W_down [G][F][D] (GShard's Wi and  */
/* Wo orientation, [P3] GShard pseudo-code).                                 */
/* ------------------------------------------------------------------------ */
typedef struct {
  const orc_cfg* c;
  const void* x; int xdt;
  const void* wg; const void* wu; const void* wd; int wdt;
} ffn_w;

static double silu(double a) { return a / (1.0 + exp(-a)); }
static double sigm(double a) { return 1.0 / (1.0 + exp(-a)); }

/* a, b, h: length F; o: length D (any may be NULL except a, b) */
static void ffn_row(const ffn_w* W, int g, long t, double* a, double* b, double* h, double* o) {
  const int D = W->c->D, F = W->c->F;
  const size_t gd = (size_t)g * D * F;
  for (int f = 0; f < F; ++f) { a[f] = 0.0; b[f] = 0.0; }
  for (int d = 0; d < D; ++d) {
    double xv = ld(W->x, (size_t)t * D + d, W->xdt);
    if (xv == 0.0) continue;
    for (int f = 0; f < F; ++f) {
      a[f] += xv * ld(W->wg, gd + (size_t)d * F + f, W->wdt);
      b[f] += xv * ld(W->wu, gd + (size_t)d * F + f, W->wdt);
    }
  }
  if (!h) return;
  for (int f = 0; f < F; ++f) h[f] = silu(a[f]) * b[f];
  if (!o) return;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int f = 0; f < F; ++f) {
    double hv = h[f];
    for (int d = 0; d < D; ++d) o[d] += hv * ld(W->wd, gd + (size_t)f * D + d, W->wdt);
  }
}

/* ------------------------------------------------------------------------ */
/* O7: forward combine                                                       */
/*   y_t = sum_{k kept, local} g_{t,k} o_{t,k} + sum_shared o_s(x_t)          */
/* [P5] 8.8 (weighted scatter-add back to token order; a token appears K      */
/* times so contributions accumulate), 8.7 (shared expert: unweighted, not   */
/* part of the top-K).  Sentinel and dropped slots contribute nothing.       */
/* ------------------------------------------------------------------------ */
typedef struct {
  ffn_w W; const int* idx; const double* w; const int* slot_row; const int* tok;
  double* y;
} fw_ctx;

static void fw_body(void* p, long i) {
  fw_ctx* a = (fw_ctx*)p;
  const orc_cfg* c = a->W.c;
  const int D = c->D, F = c->F, K = c->K, EL = c->hi - c->lo;
  long t = a->tok ? a->tok[i] : i;
  double* y = a->y + (size_t)i * D;
  double* A = (double*)malloc(sizeof(double) * (3 * (size_t)F + D));
  double *B = A + F, *H = B + F, *O = H + F;
  for (int d = 0; d < D; ++d) y[d] = 0.0;
  for (int k = 0; k < K; ++k) {
    long s = t * K + k;
    if (a->slot_row[s] < 0) continue;
    ffn_row(&a->W, a->idx[s] - c->lo, t, A, B, H, O);
    for (int d = 0; d < D; ++d) y[d] += a->w[s] * O[d];
  }
  for (int sh = 0; sh < c->n_shared; ++sh) {
    ffn_row(&a->W, EL + sh, t, A, B, H, O);
    for (int d = 0; d < D; ++d) y[d] += O[d];
  }
  free(A);
}

void orc_forward(const orc_cfg* c, const void* x, int xdt, const void* wg, const void* wu,
                 const void* wd, int wdt, const int* idx, const double* w, const int* slot_row,
                 const int* tok, int ntok, double* y) {
  fw_ctx a = {{c, x, xdt, wg, wu, wd, wdt}, idx, w, slot_row, tok, y};
  parallel_for(ntok, fw_body, &a);
}

/* per-row expert intermediates (a, b, h, o) for rows of selected tokens; used
 * by tests that compare saved activations */
void orc_expert_rows(const orc_cfg* c, const void* x, int xdt, const void* wg, const void* wu,
                     const void* wd, int wdt, const int* row_group, const int* row_tok, int nrows,
                     double* a_out, double* b_out, double* h_out, double* o_out) {
  ffn_w W = {c, x, xdt, wg, wu, wd, wdt};
  const int D = c->D, F = c->F;
  double* tmp = (double*)malloc(sizeof(double) * (3 * (size_t)F + D));
  for (int r = 0; r < nrows; ++r) {
    ffn_row(&W, row_group[r], row_tok[r], tmp, tmp + F, tmp + 2 * F, tmp + 3 * F);
    if (a_out) memcpy(a_out + (size_t)r * F, tmp, sizeof(double) * F);
    if (b_out) memcpy(b_out + (size_t)r * F, tmp + F, sizeof(double) * F);
    if (h_out) memcpy(h_out + (size_t)r * F, tmp + 2 * F, sizeof(double) * F);
    if (o_out) memcpy(o_out + (size_t)r * D, tmp + 3 * F, sizeof(double) * D);
  }
  free(tmp);
}

/* ------------------------------------------------------------------------ */
/* O8: Switch balance loss and router z-loss                                 */
/*   L_aux = alpha * E * sum_e f_e P_e, f_e = counts_all[e] / (T*K) (held     */
/*   constant), P_e = mean_t p[t,e]     ([P5] 8.5, [P4] load-balance section) */
/*   L_z = lambda * mean_t lse_t^2      ([P3] ST-MoE, [P5] 8.6)               */
/* and their logit gradients                                                 */
/*   d/ds_{t,i} L_aux = p_{t,i} (u_i - sum_e p_{t,e} u_e), u_e = aEf_e/T      */
/*   d/ds_{t,i} L_z   = lambda * (2/T) * lse_t * p_{t,i}                      */
/* losses[0] = L_aux, losses[1] = L_z, losses[2] = mean_t lse_t^2 (raw).      */
/* ------------------------------------------------------------------------ */
void orc_aux(const orc_cfg* c, const double* logits, const int* counts_all, double alpha,
             double zlam, double* losses, double* dlogits) {
  const int T = c->T, E = c->E, K = c->K;
  double* P = (double*)calloc((size_t)E, sizeof(double));
  double* p = (double*)malloc(sizeof(double) * E);
  double z2 = 0.0;
  for (int t = 0; t < T; ++t) {
    const double* s = logits + (size_t)t * E;
    double m = -INFINITY, z = 0.0;
    for (int e = 0; e < E; ++e) if ((double)s[e] > m) m = s[e];
    for (int e = 0; e < E; ++e) z += exp((double)s[e] - m);
    double lse = m + log(z);
    z2 += lse * lse;
    for (int e = 0; e < E; ++e) P[e] += exp((double)s[e] - m) / z;
  }
  double L = 0.0;
  for (int e = 0; e < E; ++e) {
    double f = (double)counts_all[e] / ((double)T * K);
    L += f * (P[e] / T);
  }
  losses[0] = alpha * E * L;
  losses[1] = zlam * z2 / T;
  losses[2] = z2 / T;
  if (dlogits) {
    for (int t = 0; t < T; ++t) {
      const double* s = logits + (size_t)t * E;
      double m = -INFINITY, z = 0.0;
      for (int e = 0; e < E; ++e) if ((double)s[e] > m) m = s[e];
      for (int e = 0; e < E; ++e) z += exp((double)s[e] - m);
      double lse = m + log(z);
      double pu = 0.0;
      for (int e = 0; e < E; ++e) {
        p[e] = exp((double)s[e] - m) / z;
        pu += p[e] * (alpha * E * ((double)counts_all[e] / ((double)T * K)) / T);
      }
      for (int e = 0; e < E; ++e) {
        double u = alpha * E * ((double)counts_all[e] / ((double)T * K)) / T;
        dlogits[(size_t)t * E + e] = p[e] * (u - pu) + zlam * (2.0 / T) * lse * p[e];
      }
    }
  }
  free(P);
  free(p);
}

/* ------------------------------------------------------------------------ */
/* Expert-choice routing ([P5] course notes 8.4: every expert takes a fixed  */
/* number of tokens from the batch; a token may be taken by several experts  */
/* or by none).  Reading: affinities p_{t,e} = softmax(s_t)_e; each local    */
/* expert e takes the C tokens with the largest p_{t,e}, C = ceil(c T K / E) */
/* (K: the average number of experts per token, c the capacity factor, 1 if  */
/* not given), at most T; equal keys go to the lower token.  The key is the  */
/* log-probability s_{t,e} - lse_t evaluated in double and rounded once to   */
/* binary32 (strictly increasing in p within a column).  The gate weight of  */
/* a taken pair is p_{t,e} (double).  Rows: expert-major, token order within */
/* an expert, then the shared expert.                                       */
/*   slot_row[t*E+e] = row, -1 (not taken), -2 (expert not local)            */
/*   w[t*E+e] = p_{t,e} for every pair (the gating backward needs them all)  */
/* ------------------------------------------------------------------------ */
long orc_ec_capacity(const orc_cfg* c) {
  const double cf = (c->cap > 0.0) ? c->cap : 1.0;
  long C = (long)ceil(cf * (double)c->T * (double)c->K / (double)c->E);
  return C < c->T ? C : c->T;
}

typedef struct { float key; int t; } ec_item;
static int ec_cmp(const void* a, const void* b) {
  const ec_item* x = (const ec_item*)a;
  const ec_item* y = (const ec_item*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->t < y->t) ? -1 : (x->t > y->t);
}

int orc_route_ec(const orc_cfg* c, const double* logits, int* slot_row, double* w, int* row_token,
                 int* offsets, double* lse_out) {
  const int T = c->T, E = c->E, EL = c->hi - c->lo, S = c->n_shared;
  if (c->score != 0) return -1;
  const long C = orc_ec_capacity(c);
  double* lse = (double*)malloc(sizeof(double) * (T > 0 ? T : 1));
  for (int t = 0; t < T; ++t) {
    const double* s = logits + (size_t)t * E;
    double m = -INFINITY, z = 0.0;
    for (int e = 0; e < E; ++e) if (s[e] > m) m = s[e];
    for (int e = 0; e < E; ++e) z += exp(s[e] - m);
    lse[t] = m + log(z);
    if (lse_out) lse_out[t] = lse[t];
    for (int e = 0; e < E; ++e) {
      w[(size_t)t * E + e] = exp(s[e] - lse[t]);
      slot_row[(size_t)t * E + e] = (e >= c->lo && e < c->hi) ? -1 : -2;
    }
  }
  ec_item* items = (ec_item*)malloc(sizeof(ec_item) * (T > 0 ? T : 1));
  int* taken = (int*)malloc(sizeof(int) * (T > 0 ? T : 1));
  for (int g = 0; g < EL; ++g) {
    const int e = c->lo + g;
    for (int t = 0; t < T; ++t) {
      items[t].key = (float)(logits[(size_t)t * E + e] - lse[t]);
      items[t].t = t;
    }
    qsort(items, (size_t)T, sizeof(ec_item), ec_cmp);
    for (int t = 0; t < T; ++t) taken[t] = 0;
    for (long i = 0; i < C; ++i) taken[items[i].t] = 1;
    long r = (long)g * C;
    for (int t = 0; t < T; ++t)
      if (taken[t]) {
        slot_row[(size_t)t * E + e] = (int)r;
        row_token[r] = t;
        ++r;
      }
  }
  for (int g = 0; g <= EL; ++g) offsets[g] = (int)((long)g * C);
  for (int s = 0; s < S; ++s) {
    offsets[EL + 1 + s] = (int)((long)EL * C + (long)(s + 1) * T);
    for (int t = 0; t < T; ++t) row_token[(long)EL * C + (long)s * T + t] = t;
  }
  free(items); free(taken); free(lse);
  return (int)C;
}

/* ------------------------------------------------------------------------ */
/* Load-driven selection-bias update ([P5] course notes 8.6; [P4] section on  */
/* the auxiliary-loss-free route): experts select on s_e + b_e; after a step  */
/* an overloaded expert lowers its b_e, an underloaded one raises it, by a    */
/* fixed step gamma.  Reading: overloaded means more slots than the mean load */
/* T*K/E (over all E, before capacity), underloaded fewer; an expert exactly  */
/* at the mean keeps b_e.  The comparison is exact in integers              */
/* (counts_e * E vs T * K); the update is one binary32 add or subtract.       */
/* ------------------------------------------------------------------------ */
void orc_bias_update(const orc_cfg* c, const int* counts_all, float gamma, float* selb) {
  const long long mean_num = (long long)c->T * c->K;
  for (int e = 0; e < c->E; ++e) {
    const long long load = (long long)counts_all[e] * c->E;
    if (load > mean_num) selb[e] = selb[e] - gamma;
    else if (load < mean_num) selb[e] = selb[e] + gamma;
  }
}

/* ------------------------------------------------------------------------ */
/* Sequence-wise balance loss ([P5] 8.6: a small complementary loss that is  */
/* kept beside the bias rule; 8.5: the balance loss L = alpha E sum_e f_e P_e */
/* with f the hard assignment fraction, held constant in the gradient, and P  */
/* the mean soft probability).  Reading: the same loss on each sequence of S  */
/* consecutive tokens, averaged over the T / S sequences:                     */
/*   f_{b,e} = n_{b,e} / (S K),   n = slots of sequence b that chose e       */
/*   P_{b,e} = (1/S) sum_{t in b} p_{t,e}                                     */
/*   L_seq   = alpha E (S / T) sum_b sum_e f_{b,e} P_{b,e}                    */
/* with p the scoring function's normalised probabilities: softmax(s) for     */
/* softmax scoring; sigma(s_e) / sum_j sigma(s_j) for sigmoid scoring.       */
/* Gradient (f constant), u_{b,e} = alpha E (S / T) f_{b,e} / S:              */
/*   d/ds_{t,i} = w_{t,i} (u_{b,i} - sum_e p_{t,e} u_{b,e}),                   */
/*   w = p_i (softmax) or sigma_i (1 - sigma_i) / sum_j sigma_j (sigmoid).    */
/* With S = T it is the batch loss above (f over all T).                     */
/* dlogits (optional) receives the gradient ([T][E]).                        */
/* ------------------------------------------------------------------------ */
static void seq_probs(const orc_cfg* c, const double* s, double* p, double* w) {
  const int E = c->E;
  if (c->score == 0) {
    double m = -INFINITY, z = 0.0;
    for (int e = 0; e < E; ++e) if (s[e] > m) m = s[e];
    for (int e = 0; e < E; ++e) z += exp(s[e] - m);
    for (int e = 0; e < E; ++e) { p[e] = exp(s[e] - m) / z; w[e] = p[e]; }
  } else {
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += sigm(s[e]);
    for (int e = 0; e < E; ++e) {
      const double sg = sigm(s[e]);
      p[e] = sg / z;
      w[e] = sg * (1.0 - sg) / z;
    }
  }
}

int orc_seq_aux(const orc_cfg* c, const double* logits, const int* idx, int S, double alpha,
                double* loss, double* dlogits) {
  const int T = c->T, E = c->E, K = c->K;
  if (S <= 0 || T % S) return -1;
  const int B = T / S;
  double* p = (double*)malloc(sizeof(double) * E);
  double* w = (double*)malloc(sizeof(double) * E);
  double* P = (double*)malloc(sizeof(double) * E);
  double* u = (double*)malloc(sizeof(double) * E);
  int* n = (int*)malloc(sizeof(int) * E);
  double L = 0.0;
  for (int b = 0; b < B; ++b) {
    for (int e = 0; e < E; ++e) { P[e] = 0.0; n[e] = 0; }
    for (int t = b * S; t < (b + 1) * S; ++t) {
      seq_probs(c, logits + (size_t)t * E, p, w);
      for (int e = 0; e < E; ++e) P[e] += p[e];
      for (int k = 0; k < K; ++k) n[idx[(size_t)t * K + k]] += 1;
    }
    double Lb = 0.0;
    for (int e = 0; e < E; ++e) {
      const double f = (double)n[e] / ((double)S * K);
      Lb += f * (P[e] / S);
      u[e] = alpha * E * ((double)S / T) * f / S;
    }
    L += Lb;
    if (dlogits) {
      for (int t = b * S; t < (b + 1) * S; ++t) {
        seq_probs(c, logits + (size_t)t * E, p, w);
        double pu = 0.0;
        for (int e = 0; e < E; ++e) pu += p[e] * u[e];
        for (int e = 0; e < E; ++e) dlogits[(size_t)t * E + e] = w[e] * (u[e] - pu);
      }
    }
  }
  *loss = alpha * E * ((double)S / T) * L;
  free(p); free(w); free(P); free(u); free(n);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O9-O12: backward                                                          */
/* ------------------------------------------------------------------------ */
/*
 * Combine backward ([P1] cause section: the gradient reaching a gate weight
 * is the expert output proj_out of that slot, so a slot that this device does
 * not serve must carry proj_out = 0):
 *   dg_{t,k} = dy_t . o_{t,k} for kept local slots; 0 for sentinel or dropped
 *   d_o      = g_{t,k} dy_t
 * Expert backward (chain rule through SwiGLU):
 *   dh = d_o W_down^T;  da = dh * b * sig(a)(1 + a(1 - sig(a)));  db = dh*silu(a)
 *   dW_down += h^T d_o;  dW_gate += x^T da;  dW_up += x^T db
 *   dx_t += da W_gate^T + db W_up^T
 * Gating backward (only through the continuous weights g; the top-K indices
 * are piecewise constant -- [P5] 8.3, [P2] section 2), with G = sum_k g_k dg_k:
 *   softmax A: dp_i = sum_k [i_k = i] dg_k; ds_i = p_i (dp_i - G)
 *   softmax B: ds_{i_k} = g_k (dg_k - G); unselected ds_i = 0
 *   sigmoid A: ds_{i_k} = dg_k sig(1 - sig)
 *   sigmoid B: ds_{i_k} = ((dg_k - G) / S) sig_{i_k}(1 - sig_{i_k}), S = sum sig
 *   (+ extra logit gradients from the auxiliary losses, passed in)
 * With K = 1 and B, g = 1 exactly so ds = 1 * (dg - dg) = 0 exactly
 * ([P2] section 2, [P5] 8.3).  The selection bias b_e gets no gradient.
 * Router backward: dx_t += ds_t W_r;  dW_r += ds_t^T x_t;  d r_b += ds_t.
 * With router-logit jitter s~ = s * u ([P3] ST-MoE), ds (taken w.r.t. s~)
 * is multiplied by u first; ds is then returned w.r.t. the raw logits.
 *
 * bug_mode (negative control for [P1]): a sentinel slot is computed by local
 * expert 0 and only its forward weight is zero; the backward takes
 * dg = dy . FFN_0(x_t) instead of 0.
 *
 * Sparse upstream gradient: the caller lists the tokens with non-zero dy
 * (tok[0..ntok)); dy holds their rows (ntok x D).  Every other token has
 * dy = 0 and (with no extra logit gradient) contributes nothing.  dx and ds
 * are returned for the listed tokens only.  Expert weight gradients are
 * returned for the F-columns fsel[0..nf) (all when fsel == NULL, nf = F):
 *   dwg, dwu: [G][D][nf];  dwd: [G][nf][D].
 */
/* O11 for one token: ds[0..E) from dg[0..K) (see the block comment above) */
static void gate_bwd(const orc_cfg* c, const double* s, const int* idx, const double* g,
                     const double* dg, double* ds) {
  const int E = c->E, K = c->K;
  for (int e = 0; e < E; ++e) ds[e] = 0.0;
  double G = 0.0;
  for (int k = 0; k < K; ++k) G += g[k] * dg[k];
  if (c->score == 0) {
    if (c->gating == 0) {
      double m = -INFINITY, z = 0.0;
      for (int e = 0; e < E; ++e) if (s[e] > m) m = s[e];
      for (int e = 0; e < E; ++e) z += exp(s[e] - m);
      for (int e = 0; e < E; ++e) {
        double dp = 0.0;
        for (int k = 0; k < K; ++k) if (idx[k] == e) dp += dg[k];
        ds[e] = exp(s[e] - m) / z * (dp - G);
      }
    } else {
      for (int k = 0; k < K; ++k) ds[idx[k]] = g[k] * (dg[k] - G);
    }
  } else {
    double S_ = 0.0;
    for (int k = 0; k < K; ++k) S_ += sigm(s[idx[k]]);
    for (int k = 0; k < K; ++k) {
      double sg = sigm(s[idx[k]]);
      double dsig = sg * (1.0 - sg);
      ds[idx[k]] = (c->gating == 0) ? dg[k] * dsig : ((dg[k] - G) / S_) * dsig;
    }
  }
}

/* O11 alone, for all T tokens: ds [T,E] from dg [T,K] */
void orc_gate_grad(const orc_cfg* c, const double* logits, const int* idx, const double* gw,
                   const double* dg, double* ds) {
  for (long t = 0; t < c->T; ++t)
    gate_bwd(c, logits + (size_t)t * c->E, idx + (size_t)t * c->K, gw + (size_t)t * c->K,
             dg + (size_t)t * c->K, ds + (size_t)t * c->E);
}

typedef struct {
  ffn_w W; const double* lg; const double* wr; const int* idx; const double* gw;
  const int* slot_row; const int* tok; int ntok; const double* dy; const double* dlx;
  const float* jit;   /* router-logit jitter u [T][E] (NULL: none) */
  double* dx; double* ds;
  /* per-(token,slot) intermediates for the weight-gradient pass */
  double* r_da; double* r_db; double* r_h; double* r_do;   /* [ntok*K(+S)][F or D] */
} bw_ctx;

static void bw_tok(void* p, long i) {
  bw_ctx* a = (bw_ctx*)p;
  const orc_cfg* c = a->W.c;
  const int D = c->D, F = c->F, K = c->K, E = c->E, EL = c->hi - c->lo, S = c->n_shared;
  long t = a->tok[i];
  const double* dy = a->dy + (size_t)i * D;
  double* dx = a->dx + (size_t)i * D;
  double* ds = a->ds + (size_t)i * E;
  double* A = (double*)malloc(sizeof(double) * (4 * (size_t)F + D));
  double *B = A + F, *H = B + F, *O = H + F, *DH = O + D;
  double dg[1024];
  for (int d = 0; d < D; ++d) dx[d] = 0.0;
  const int nslot = K + S;
  for (int q = 0; q < nslot; ++q) {
    size_t ri = (size_t)i * nslot + q;
    double* r_da = a->r_da + ri * F;
    double* r_db = a->r_db + ri * F;
    double* r_h = a->r_h + ri * F;
    double* r_do = a->r_do + ri * D;
    int grp;
    double gk;
    if (q < K) {
      long s = t * K + q;
      int row = a->slot_row[s];
      dg[q] = 0.0;
      if (row < 0) {
        if (c->bug_mode && row == -2) {
          /* unmasked sentinel: expert-0 output leaks into dg only */
          ffn_row(&a->W, 0, t, A, B, H, O);
          double acc = 0.0;
          for (int d = 0; d < D; ++d) acc += dy[d] * O[d];
          dg[q] = acc;
        }
        for (int f = 0; f < F; ++f) { r_da[f] = 0.0; r_db[f] = 0.0; r_h[f] = 0.0; }
        for (int d = 0; d < D; ++d) r_do[d] = 0.0;
        continue;
      }
      grp = a->idx[s] - c->lo;
      gk = a->gw[s];
    } else {
      grp = EL + (q - K);
      gk = 1.0;
    }
    ffn_row(&a->W, grp, t, A, B, H, O);
    if (q < K) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += dy[d] * O[d];
      dg[q] = acc;
    }
    for (int d = 0; d < D; ++d) r_do[d] = gk * dy[d];
    const size_t gd = (size_t)grp * D * F;
    for (int f = 0; f < F; ++f) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += r_do[d] * ld(a->W.wd, gd + (size_t)f * D + d, a->W.wdt);
      DH[f] = acc;
    }
    for (int f = 0; f < F; ++f) {
      double sg = sigm(A[f]);
      r_da[f] = DH[f] * B[f] * sg * (1.0 + A[f] * (1.0 - sg));
      r_db[f] = DH[f] * silu(A[f]);
      r_h[f] = H[f];
    }
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int f = 0; f < F; ++f)
        acc += r_da[f] * ld(a->W.wg, gd + (size_t)d * F + f, a->W.wdt) +
               r_db[f] * ld(a->W.wu, gd + (size_t)d * F + f, a->W.wdt);
      dx[d] += acc;
    }
  }
  /* gating backward */
  gate_bwd(c, a->lg + (size_t)t * E, a->idx + (size_t)t * K, a->gw + (size_t)t * K, dg, ds);
  if (a->dlx)
    for (int e = 0; e < E; ++e) ds[e] += a->dlx[(size_t)t * E + e];
  /* jittered logits s~ = s * u ([P3] ST-MoE): back to the raw logits */
  if (a->jit)
    for (int e = 0; e < E; ++e) ds[e] *= (double)a->jit[(size_t)t * E + e];
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e) acc += ds[e] * a->wr[(size_t)e * D + d];
    dx[d] += acc;
  }
  free(A);
}

typedef struct {
  bw_ctx* b; const int* fsel; int nf; double* dwg; double* dwu; double* dwd;
  double* dwr; double* drb;
} wg_ctx;

/* weight gradients of group g: fixed summation order (listed tokens, then k) */
static void wg_body(void* p, long gi) {
  wg_ctx* w = (wg_ctx*)p;
  bw_ctx* a = w->b;
  const orc_cfg* c = a->W.c;
  const int D = c->D, F = c->F, K = c->K, EL = c->hi - c->lo, S = c->n_shared;
  const int nslot = K + S, nf = w->nf;
  int g = (int)gi;
  double* dwg = w->dwg + (size_t)g * D * nf;
  double* dwu = w->dwu + (size_t)g * D * nf;
  double* dwd = w->dwd + (size_t)g * nf * D;
  memset(dwg, 0, sizeof(double) * D * nf);
  memset(dwu, 0, sizeof(double) * D * nf);
  memset(dwd, 0, sizeof(double) * D * nf);
  for (int i = 0; i < a->ntok; ++i) {
    long t = a->tok[i];
    for (int q = 0; q < nslot; ++q) {
      int grp;
      if (q < K) {
        long s = t * K + q;
        if (a->slot_row[s] < 0) continue;
        grp = a->idx[s] - c->lo;
      } else {
        grp = EL + (q - K);
      }
      if (grp != g) continue;
      size_t ri = (size_t)i * nslot + q;
      const double* da = a->r_da + ri * F;
      const double* db = a->r_db + ri * F;
      const double* h = a->r_h + ri * F;
      const double* dO = a->r_do + ri * D;
      for (int d = 0; d < D; ++d) {
        double xv = ld(a->W.x, (size_t)t * D + d, a->W.xdt);
        for (int j = 0; j < nf; ++j) {
          int f = w->fsel ? w->fsel[j] : j;
          dwg[(size_t)d * nf + j] += xv * da[f];
          dwu[(size_t)d * nf + j] += xv * db[f];
        }
      }
      for (int j = 0; j < nf; ++j) {
        int f = w->fsel ? w->fsel[j] : j;
        for (int d = 0; d < D; ++d) dwd[(size_t)j * D + d] += h[f] * dO[d];
      }
    }
  }
}

static void wr_body(void* p, long e) {
  wg_ctx* w = (wg_ctx*)p;
  bw_ctx* a = w->b;
  const orc_cfg* c = a->W.c;
  const int D = c->D, E = c->E;
  double* dwr = w->dwr + (size_t)e * D;
  double rb = 0.0;
  for (int d = 0; d < D; ++d) dwr[d] = 0.0;
  for (int i = 0; i < a->ntok; ++i) {
    long t = a->tok[i];
    double v = a->ds[(size_t)i * E + e];
    rb += v;
    if (v == 0.0) continue;
    for (int d = 0; d < D; ++d) dwr[d] += v * ld(a->W.x, (size_t)t * D + d, a->W.xdt);
  }
  w->drb[e] = rb;
}

void orc_backward(const orc_cfg* c, const void* x, int xdt, const double* wr, const void* wg,
                  const void* wu, const void* wd, int wdt, const double* logits, const int* idx,
                  const double* gw, const int* slot_row, const int* tok, int ntok, const double* dy,
                  const double* dlx, const int* fsel, int nf, double* dx, double* ds, double* dwr,
                  double* drb, double* dwg, double* dwu, double* dwd, const float* jit) {
  const int D = c->D, F = c->F, K = c->K, S = c->n_shared;
  const int G = (c->hi - c->lo) + S;
  const size_t nrow = (size_t)ntok * (K + S);
  bw_ctx b;
  memset(&b, 0, sizeof b);
  b.W.c = c; b.W.x = x; b.W.xdt = xdt; b.W.wg = wg; b.W.wu = wu; b.W.wd = wd; b.W.wdt = wdt;
  b.lg = logits; b.wr = wr; b.idx = idx; b.gw = gw; b.slot_row = slot_row; b.tok = tok;
  b.ntok = ntok; b.dy = dy; b.dlx = dlx; b.dx = dx; b.ds = ds; b.jit = jit;
  b.r_da = (double*)malloc(sizeof(double) * nrow * F);
  b.r_db = (double*)malloc(sizeof(double) * nrow * F);
  b.r_h = (double*)malloc(sizeof(double) * nrow * F);
  b.r_do = (double*)malloc(sizeof(double) * nrow * D);
  parallel_for(ntok, bw_tok, &b);
  wg_ctx w = {&b, fsel, fsel ? nf : F, dwg, dwu, dwd, dwr, drb};
  if (dwg && dwu && dwd) parallel_for(G, wg_body, &w);
  if (dwr && drb) parallel_for(c->E, wr_body, &w);
  free(b.r_da); free(b.r_db); free(b.r_h); free(b.r_do);
}

/* ------------------------------------------------------------------------ */
/* O10 restricted to F-columns, for one group, from every row of the group  */
/* with a dense upstream gradient dy [T][D].                                 */
/*   Column f of dW_gate / dW_up and row f of dW_down depend on a row only   */
/*   through a_f = x W_gate[:,f], b_f = x W_up[:,f], h_f = silu(a_f) b_f and  */
/*   dh_f = d_o . W_down[f,:] with d_o = g dy_t ([P5] 8.1 SwiGLU; 8.3 the    */
/*   gate weight multiplies the expert output).  So a full-size check of     */
/*   the weight gradients on sampled columns needs only these:               */
/*     dW_gate[d][f] = sum_rows x_d da_f,  dW_up[d][f] = sum_rows x_d db_f,   */
/*     dW_down[f][d] = sum_rows h_f (g dy_t)_d                               */
/*   with da_f = dh_f b_f s(a_f)(1 + a_f(1 - s(a_f))), db_f = dh_f silu(a_f).  */
/* Rows of routed group g (expert lo + g): the kept local slots t*K+k with    */
/* that expert, in token order, weight g_{t,k}; shared group (g >= hi - lo): */
/* every token, weight 1.  Outputs: dwg, dwu [D][nf], dwd [nf][D].           */
/* Each thread owns one column (fixed summation order: tokens ascending).    */
/* ------------------------------------------------------------------------ */
typedef struct {
  ffn_w W; const int* idx; const double* gw; const int* slot_row; const double* dy;
  int g; const int* fsel; int nf; double* dwg; double* dwu; double* dwd;
} gwc_ctx;

static void gwc_body(void* p, long j) {
  gwc_ctx* a = (gwc_ctx*)p;
  const orc_cfg* c = a->W.c;
  const int D = c->D, F = c->F, K = c->K, EL = c->hi - c->lo, nf = a->nf;
  const int f = a->fsel[j];
  const size_t gd = (size_t)a->g * D * F;
  for (int d = 0; d < D; ++d) {
    a->dwg[(size_t)d * nf + j] = 0.0;
    a->dwu[(size_t)d * nf + j] = 0.0;
    a->dwd[(size_t)j * D + d] = 0.0;
  }
  for (long t = 0; t < c->T; ++t) {
    /* weight of this token's row in group g, or skip */
    double gk;
    if (a->g >= EL) {
      gk = 1.0;
    } else {
      int k;
      for (k = 0; k < K; ++k) {
        long s = t * K + k;
        if (a->slot_row[s] >= 0 && a->idx[s] - c->lo == a->g) break;
      }
      if (k == K) continue;
      gk = a->gw[t * K + k];
    }
    const double* dy = a->dy + (size_t)t * D;
    double av = 0.0, bv = 0.0, dh = 0.0;
    for (int d = 0; d < D; ++d) {
      double xv = ld(a->W.x, (size_t)t * D + d, a->W.xdt);
      av += xv * ld(a->W.wg, gd + (size_t)d * F + f, a->W.wdt);
      bv += xv * ld(a->W.wu, gd + (size_t)d * F + f, a->W.wdt);
      dh += gk * dy[d] * ld(a->W.wd, gd + (size_t)f * D + d, a->W.wdt);
    }
    const double sg = sigm(av);
    const double h = silu(av) * bv;
    const double da = dh * bv * sg * (1.0 + av * (1.0 - sg));
    const double db = dh * silu(av);
    for (int d = 0; d < D; ++d) {
      double xv = ld(a->W.x, (size_t)t * D + d, a->W.xdt);
      a->dwg[(size_t)d * nf + j] += xv * da;
      a->dwu[(size_t)d * nf + j] += xv * db;
      a->dwd[(size_t)j * D + d] += h * (gk * dy[d]);
    }
  }
}

void orc_group_wgrad_cols(const orc_cfg* c, const void* x, int xdt, const void* wg,
                          const void* wu, const void* wd, int wdt, const int* idx,
                          const double* gw, const int* slot_row, const double* dy, int g,
                          const int* fsel, int nf, double* dwg, double* dwu, double* dwd) {
  gwc_ctx a;
  memset(&a, 0, sizeof a);
  a.W.c = c; a.W.x = x; a.W.xdt = xdt; a.W.wg = wg; a.W.wu = wu; a.W.wd = wd; a.W.wdt = wdt;
  a.idx = idx; a.gw = gw; a.slot_row = slot_row; a.dy = dy; a.g = g;
  a.fsel = fsel; a.nf = nf; a.dwg = dwg; a.dwu = dwu; a.dwd = dwd;
  parallel_for(nf, gwc_body, &a);
}
