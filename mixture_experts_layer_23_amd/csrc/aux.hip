// aux.hip -- Switch load-balance loss and router z-loss, with their logit
// gradients.
//
// [P5] course notes 8.5: L = alpha * E * sum_e f_e P_e where f_e is the hard
// fraction of assignments to expert e (held constant when differentiating)
// and P_e the mean routing probability; dL/dp_{t,e} = alpha E f_e / T.
// [P4] load-balance section: the same E sum_e f_e p_e form.  [P3] ST-MoE and
// [P5] 8.6: z-loss = lambda * mean_t (log sum_e exp s_te)^2.
//
// Deterministic two-level reduction: each workgroup takes TB tokens and
// computes per token the max, normaliser and lse, then every probability
// (kept in LDS), sum_e p_e u_e (u_e = alpha E f_e / T) and, if asked, the
// logit gradient p (u - sum p u) + lambda (2/T) lse p; then per expert the
// workgroup's sum of p_e in token order.  A final single-workgroup kernel
// sums the partials in workgroup order.
#include "common.h"
#include "kernels.h"

namespace moe {

// TB tokens per workgroup, four threads per token for the per-token
// reductions, all threads over (token, expert) pairs for the probabilities.
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ counts,
                                                          int T_, int E, int K, int TB,
                                                          float alpha, float zlam,
                                                          float* __restrict__ part,
                                                          float* __restrict__ dlog) {
  extern __shared__ float sh[];
  float* sp = sh;                  // [TB][E] probabilities
  float* sm = sh + (size_t)TB * E; // [TB] max
  float* sz = sm + TB;             // [TB] normaliser
  float* slse = sz + TB;           // [TB] log-sum-exp
  float* spu = slse + TB;          // [TB] sum_e p_e u_e
  const int t0 = blockIdx.x * TB;
  const int nt = min(TB, T_ - t0);
  const float ucoef = alpha * (float)E / ((float)T_ * (float)K) / (float)T_;
  const int tq = threadIdx.x >> 2, q = threadIdx.x & 3;  // token, quarter
  // per token max and normaliser (4 lanes per token, fixed combine order)
  if (tq < TB) {
    float m = -INFINITY, z = 0.f;
    if (tq < nt) {
      const float* s = logits + (size_t)(t0 + tq) * E;
      for (int e = q; e < E; e += 4) m = fmaxf(m, s[e]);
    }
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    if (tq < nt) {
      const float* s = logits + (size_t)(t0 + tq) * E;
      for (int e = q; e < E; e += 4) z += expf(s[e] - m);
    }
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    if (q == 0 && tq < nt) {
      sm[tq] = m;
      sz[tq] = z;
      slse[tq] = m + logf(z);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
    const int t = i / E, e = i - t * E;
    sp[i] = expf(logits[(size_t)(t0 + t) * E + e] - sm[t]) / sz[t];
  }
  __syncthreads();
  if (dlog) {
    if (tq < nt) {
      float pu = 0.f;
      for (int e = q; e < E; e += 4) pu += sp[tq * E + e] * (ucoef * (float)counts[e]);
      pu += __shfl_xor(pu, 1, 64);
      pu += __shfl_xor(pu, 2, 64);
      if (q == 0) spu[tq] = pu;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * E; i += blockDim.x) {
      const int t = i / E, e = i - t * E;
      const float p = sp[i];
      const float u = ucoef * (float)counts[e];
      dlog[(size_t)(t0 + t) * E + e] = p * (u - spu[t]) + zlam * (2.0f / (float)T_) * slse[t] * p;
    }
  }
  float* pb = part + (size_t)blockIdx.x * (E + 1);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float P = 0.f;
    for (int t = 0; t < nt; ++t) P += sp[t * E + e];
    pb[e] = P;
  }
  if (threadIdx.x == 0) {
    float z2 = 0.f;
    for (int t = 0; t < nt; ++t) z2 += slse[t] * slse[t];
    pb[E] = z2;
  }
}

// column sums of the partials (E mean-probability sums and the z-loss sum):
// wave w takes columns w, w+16, ..., its lanes take blocks lane, lane+64, ...,
// butterfly-added; then sum_e f_e P_e in a fixed tree.  No atomics.
__global__ __launch_bounds__(1024) void aux_final_kernel(const float* __restrict__ part,
                                                         int nblk, const int32_t* __restrict__ counts,
                                                         int T_, int E, int K, float alpha,
                                                         float zlam, float* __restrict__ losses) {
  __shared__ float col[1025];
  __shared__ float red[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int c = wave; c <= E; c += 16) {
    float s = 0.f;
    for (int b = lane; b < nblk; b += 64) s += part[(size_t)b * (E + 1) + c];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) col[c] = s;
  }
  __syncthreads();
  float v = 0.f;
  for (int e = tid; e < E; e += 1024) {
    const float f = (float)counts[e] / ((float)T_ * (float)K);
    v += f * (col[e] / (float)T_);
  }
  red[tid] = v;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    const float z2 = col[E];
    losses[0] = alpha * (float)E * red[0];
    losses[1] = zlam * z2 / (float)T_;
    losses[2] = z2 / (float)T_;
  }
}

int launch_aux(const moe_config& c, const float* logits, const int32_t* counts_all, float alpha,
               float zlam, float* losses, float* d_logits, char* ws, const Workspace& L,
               hipStream_t st) {
  float* part = reinterpret_cast<float*>(ws + L.aux_part);
  const int TB = aux_tokens_per_block(c.E);
  const size_t shm = ((size_t)TB * c.E + 4 * (size_t)TB) * sizeof(float);
  MOE_LAUNCH("aux_partial", aux_partial_kernel, dim3(L.aux_blocks), dim3(256), shm, st, logits,
             counts_all, c.T, c.E, c.K, TB, alpha, zlam, part, d_logits);
  MOE_LAUNCH("aux_final", aux_final_kernel, dim3(1), dim3(1024), 0, st, part, L.aux_blocks,
             counts_all, c.T, c.E, c.K, alpha, zlam, losses);
  return MOE_OK;
}

}  // namespace moe
