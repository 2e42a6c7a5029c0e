// kernels.h -- host-side launchers of the HIP kernels (internal).
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>

#include "common.h"

namespace moe {

// workspace carve-up (all sub-buffers 256-byte aligned)
struct Workspace {
  size_t tile_counts, tile_base;   // int32 [ntiles][E]
  size_t aux_part;                 // float [aux_blocks][E + 1]
  size_t d_o, dact, dx_perm;       // dtype rows buffers
  size_t dg, ds;                   // float [T][W], [T][E]
  size_t dxr;                      // float [T][D] (router dgrad, large E)
  size_t dwr_part;                 // float [splits][E][D] (+ [splits][E] bias)
  size_t rb_part;                  // float [rb_splits][E rounded to 4] (large E)
  size_t seq_part;                 // float [T] per-sequence balance-loss partials
  size_t seq_blk_n, seq_blk_p;     // int32 / float [T][E] per-token-block partials
  size_t ec_keys;                  // uint32 [EL][T] expert-choice selection keys
  size_t fold_counts, fold_rank;   // int32 [ceil(T/16)][E], [T*K] (permute folded into the router)
  size_t total;
  int ntiles, aux_blocks, dwr_splits, rb_splits;
};
Workspace workspace_layout(const moe_config& c);

// slots per token in the slot tables: K (token choice) or E (expert choice,
// one slot per token-expert pair)
inline int slot_width(const moe_config& c) {
  return c.routing == MOE_EXPERT_CHOICE ? c.E : c.K;
}
// expert choice: tokens taken by every expert, min(ceil(c T K / E), T) in
// double, c = 1 when no capacity factor is given
inline int64_t ec_capacity(const moe_config& c) {
  const double cf = c.capacity_factor > 0.0 ? c.capacity_factor : 1.0;
  const double v = std::ceil(cf * (double)c.T * (double)c.K / (double)c.E);
  return v < (double)c.T ? (int64_t)v : (int64_t)c.T;
}
// bound on the routed rows (the shared expert's T rows come on top)
inline int64_t routed_rows_max(const moe_config& c) {
  if (c.routing == MOE_EXPERT_CHOICE) return (int64_t)(c.expert_hi - c.expert_lo) * ec_capacity(c);
  return (int64_t)c.T * c.K;
}

constexpr int kSlotTile = 256;  // slots per histogram / rank tile
// tokens per aux-loss workgroup: up to 64, with the [TB][E] probability tile
// plus four [TB] vectors kept within 64 KB of LDS
inline int aux_tokens_per_block(int E) { return std::max(1, std::min(64, (16384 - 256) / E)); }
// elements per lane of the few-expert router weight gradient: 8 bf16 (16-byte
// loads) when whole 512-wide d-blocks fit, else 4
inline int router_wgrad_width(const moe_config& c) {
  return (c.dtype == MOE_BF16 && c.D % 512 == 0) ? 8 : 4;
}

int launch_route(const moe_config& c, const void* x, const float* wr, const float* rb,
                 const float* selb, const float* jit, const float* wn, const float* eps,
                 float* nlg, float* logits, int32_t* idx, float* w, float* lse, bool logits_given,
                 hipStream_t st);

// moe_route followed by moe_permute, with the permute's counting, scan and
// row assignment folded into the few-expert router when it fits (route.hip)
int launch_route_permute(const moe_config& c, const void* x, const float* wr, const float* rb,
                         const float* selb, float* logits, int32_t* idx, float* w, float* lse,
                         int capacity, int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                         int32_t* row_token, int32_t* row_slot, int32_t* n_dropped,
                         void* x_perm, char* ws, const Workspace& L, hipStream_t st);

int launch_route_ec(const moe_config& c, const void* x, const float* wr, const float* rb,
                    float* logits, float* w, float* lse, int32_t* counts_all, int32_t* offsets,
                    int32_t* slot_row, int32_t* row_token, int32_t* row_slot, void* x_perm,
                    bool logits_given, char* ws, const Workspace& L, hipStream_t st);
// router logits out[T][E] = fl32(x W^T + b), fp64 accumulation (route.hip)
int router_logits(const moe_config& c, const void* x, const float* wr, const float* rb,
                  float* logits, hipStream_t st);
// shared-expert row maps and the x_perm gather of the routed rows (permute.hip)
int launch_shared_rows(const moe_config& c, const int32_t* offsets, int32_t* row_token,
                       int32_t* row_slot, hipStream_t st);
int launch_gather(const moe_config& c, const void* x, const int32_t* row_token,
                  const int32_t* offsets, void* x_perm, hipStream_t st);

int launch_permute(const moe_config& c, int capacity, const int32_t* idx, const void* x,
                   int32_t* counts_all, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                   int32_t* row_slot, int32_t* n_dropped, void* x_perm, char* ws,
                   const Workspace& L, hipStream_t st);

int launch_expert_ffn(const moe_config& c, const void* x, const void* x_perm,
                      const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                      void* act, void* h, void* o_perm, hipStream_t st);

int launch_combine(const moe_config& c, const void* o_perm, const int32_t* offsets,
                   const int32_t* slot_row, const float* topk_w, void* y, hipStream_t st);

int launch_aux(const moe_config& c, const float* logits, const int32_t* counts_all, float alpha,
               float zlam, float* losses, float* d_logits, char* ws, const Workspace& L,
               hipStream_t st);

int launch_bias_update(const moe_config& c, const int32_t* counts, float gamma, float* b,
                       hipStream_t st);
int launch_seq_aux(const moe_config& c, const float* logits, const int32_t* idx, int S,
                   float alpha, float* loss, float* dlog, bool accumulate, char* ws,
                   const Workspace& L, hipStream_t st);

int launch_backward(const moe_config& c, const void* x, const float* wr, const float* logits,
                    const int32_t* idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                    const void* o_perm, const void* wg, const void* wu, const void* wd,
                    const void* dy, const float* dlx, const float* jit, void* dx, float* dwr,
                    float* drb, void* dwg, void* dwu, void* dwd, float* d_logits_out, char* ws,
                    const Workspace& L, hipStream_t st);

// side streams (streams.hip): per-device side stream i (0 or 1), or null if
// they could not be created; fork_stream makes `to` wait for the work issued
// to `from` so far (join: the same, the other way)
hipStream_t side_stream(int i);
int fork_stream(hipStream_t from, hipStream_t to);

// grouped GEMM launchers (gemm.hip)
int gemm_swiglu_fwd(const moe_config& c, const void* x, const void* x_perm,
                    const int32_t* offsets, const void* wg, const void* wu, void* act, void* h,
                    hipStream_t st);
int gemm_down_fwd(const moe_config& c, const int32_t* offsets, const void* h, const void* wd,
                  void* o_perm, hipStream_t st);
int gemm_down_dgrad(const moe_config& c, const int32_t* offsets, const void* d_o, const void* dy,
                    const void* wd, const void* act, void* dact, hipStream_t st);
int gemm_down_wgrad(const moe_config& c, const int32_t* offsets, const void* h, const void* d_o,
                    const void* dy, void* dwd, hipStream_t st);
int gemm_up_dgrad(const moe_config& c, const int32_t* offsets, const void* dact, const void* wg,
                  const void* wu, void* dx_perm, hipStream_t st);
int gemm_up_wgrad(const moe_config& c, const int32_t* offsets, const void* x, const void* x_perm,
                  const void* dact, void* dwg, void* dwu, hipStream_t st);

// fp32 router GEMM for many experts on the matrix cores (gemm.hip):
//   C[z][m][n] = sum_{k in split z} A(m,k) B(k,n), A(m,k) = a_kc ? A[m*lda+k] :
//   A[k*lda+m], B(k,n) = B[k*ldb+n] (fp32, or bf16 when b_bf16), splits of kper
//   (a multiple of 32) k each.  router_gemm_fits says whether the shapes allow it.
bool router_gemm_fits(int64_t lda, int64_t ldb, int M, int N, int Kd, bool a_kc);
int router_gemm(const char* name, bool a_kc, bool b_bf16, const float* A, int64_t lda,
                const void* B, int64_t ldb, int M, int N, int Kd, int kper, int splits, float* C,
                int64_t ldc, int64_t split_stride, hipStream_t st);

}  // namespace moe
