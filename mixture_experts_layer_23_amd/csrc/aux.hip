// aux.hip -- Switch load-balance loss and router z-loss, with their logit
// gradients.
//
// [P5] course notes 8.5: L = alpha * E * sum_e f_e P_e where f_e is the hard
// fraction of assignments to expert e (held constant when differentiating)
// and P_e the mean routing probability; dL/dp_{t,e} = alpha E f_e / T.
// [P4] load-balance section: the same E sum_e f_e p_e form.  [P3] ST-MoE and
// [P5] 8.6: z-loss = lambda * mean_t (log sum_e exp s_te)^2.
//
// Two passes, deterministic: per block of kAuxTokens tokens, (1) per token
// max, normaliser, lse and sum_e p_e u_e (u_e = alpha E f_e / T), (2) per
// expert the block's sum of p_e in token order and, if asked, the logit
// gradient p (u - sum p u) + lambda (2/T) lse p.  A final single-workgroup
// kernel sums the block partials in block order.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ counts,
                                                          int T_, int E, int K, float alpha,
                                                          float zlam, float* __restrict__ part,
                                                          float* __restrict__ dlog) {
  __shared__ float sm[kAuxTokens], sz[kAuxTokens], slse[kAuxTokens], spu[kAuxTokens];
  const int t0 = blockIdx.x * kAuxTokens;
  const int nt = min(kAuxTokens, T_ - t0);
  const float inv_tk = 1.0f / ((float)T_ * (float)K);
  const float ucoef = alpha * (float)E * inv_tk / (float)T_;
  for (int i = threadIdx.x; i < nt; i += blockDim.x) {
    const float* s = logits + (size_t)(t0 + i) * E;
    float m = -INFINITY;
    for (int e = 0; e < E; ++e) m = fmaxf(m, s[e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(s[e] - m);
    float pu = 0.f;
    if (dlog)
      for (int e = 0; e < E; ++e) pu += (expf(s[e] - m) / z) * (ucoef * (float)counts[e]);
    sm[i] = m;
    sz[i] = z;
    slse[i] = m + logf(z);
    spu[i] = pu;
  }
  __syncthreads();
  float* pb = part + (size_t)blockIdx.x * (E + 1);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const float u = ucoef * (float)counts[e];
    float P = 0.f;
    for (int i = 0; i < nt; ++i) {
      const float p = expf(logits[(size_t)(t0 + i) * E + e] - sm[i]) / sz[i];
      P += p;
      if (dlog)
        dlog[(size_t)(t0 + i) * E + e] = p * (u - spu[i]) + zlam * (2.0f / (float)T_) * slse[i] * p;
    }
    pb[e] = P;
  }
  if (threadIdx.x == 0) {
    float z2 = 0.f;
    for (int i = 0; i < nt; ++i) z2 += slse[i] * slse[i];
    pb[E] = z2;
  }
}

__global__ __launch_bounds__(1024) void aux_final_kernel(const float* __restrict__ part,
                                                         int nblk, const int32_t* __restrict__ counts,
                                                         int T_, int E, int K, float alpha,
                                                         float zlam, float* __restrict__ losses) {
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  float v = 0.f;
  for (int e = tid; e < E; e += 1024) {
    float P = 0.f;
    for (int b = 0; b < nblk; ++b) P += part[(size_t)b * (E + 1) + e];
    const float f = (float)counts[e] / ((float)T_ * (float)K);
    v += f * (P / (float)T_);
  }
  red[tid] = v;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    float z2 = 0.f;
    for (int b = 0; b < nblk; ++b) z2 += part[(size_t)b * (E + 1) + E];
    losses[0] = alpha * (float)E * red[0];
    losses[1] = zlam * z2 / (float)T_;
    losses[2] = z2 / (float)T_;
  }
}

int launch_aux(const moe_config& c, const float* logits, const int32_t* counts_all, float alpha,
               float zlam, float* losses, float* d_logits, char* ws, const Workspace& L,
               hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws + L.aux_part);
  MOE_LAUNCH("aux_partial", aux_partial_kernel, dim3(L.aux_blocks), dim3(256), 0, st, logits,
             counts_all, c.T, c.E, c.K, alpha, zlam, part, d_logits);
  MOE_LAUNCH("aux_final", aux_final_kernel, dim3(1), dim3(1024), 0, st, part, L.aux_blocks,
             counts_all, c.T, c.E, c.K, alpha, zlam, losses);
  return MOE_OK;
}

}  // namespace moe
