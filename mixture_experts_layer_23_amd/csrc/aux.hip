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
#include <algorithm>

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

// Few experts, few tokens: one workgroup of NT threads does both levels.
// Thread i takes tokens i, i + NT, ... (the E <= EM logits of a token in
// registers), keeps its own column sums, and the workgroup adds them in a
// fixed tree.  Each thread walks its tokens one dependent load after
// another, so the single workgroup pays off only for short batches: at
// T = 4096, E = 4 it takes 12.4 us against 13.5 us for the two-level
// kernels, at T = 16384, E = 8 it took 114 us against 15 us.
constexpr int kAuxSingleTokens = 8192;
template <int EM, int NT>
__global__ __launch_bounds__(NT) void aux_single_kernel(const float* __restrict__ logits,
                                                          const int32_t* __restrict__ counts,
                                                          int T_, int E, int K, float alpha,
                                                          float zlam, float* __restrict__ losses,
                                                          float* __restrict__ dlog) {
  __shared__ float red[NT / 64][EM + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float ucoef = alpha * (float)E / ((float)T_ * (float)K) / (float)T_;
  float u[EM], P[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    u[e] = (e < E) ? ucoef * (float)counts[e] : 0.f;
    P[e] = 0.f;
  }
  float z2 = 0.f;
  for (int t = tid; t < T_; t += NT) {
    const float* s = logits + (size_t)t * E;
    float sv[EM], m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      sv[e] = (e < E) ? s[e] : -INFINITY;
      m = fmaxf(m, sv[e]);
    }
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) z += expf(sv[e] - m);
    const float lse = m + logf(z);
    z2 += lse * lse;
    float pu = 0.f;
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      sv[e] = (e < E) ? expf(sv[e] - m) / z : 0.f;  // p
      P[e] += sv[e];
      pu += sv[e] * u[e];
    }
    if (dlog) {
#pragma unroll
      for (int e = 0; e < EM; ++e)
        if (e < E)
          dlog[(size_t)t * E + e] =
              sv[e] * (u[e] - pu) + zlam * (2.0f / (float)T_) * lse * sv[e];
    }
  }
#pragma unroll
  for (int e = 0; e <= EM; ++e) {
    float v = e < EM ? P[e] : z2;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][e] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float col[EM + 1];
#pragma unroll
    for (int e = 0; e <= EM; ++e) {
      col[e] = 0.f;
      for (int w = 0; w < NT / 64; ++w) col[e] += red[w][e];
    }
    float v = 0.f;
#pragma unroll
    for (int e = 0; e < EM; ++e)
      if (e < E) v += ((float)counts[e] / ((float)T_ * (float)K)) * (col[e] / (float)T_);
    losses[0] = alpha * (float)E * v;
    losses[1] = zlam * col[EM] / (float)T_;
    losses[2] = col[EM] / (float)T_;
  }
}

int launch_aux(const moe_config& c, const float* logits, const int32_t* counts_all, float alpha,
               float zlam, float* losses, float* d_logits, char* ws, const Workspace& L,
               hipStream_t st) {
  if (c.E <= 8 && c.T <= kAuxSingleTokens) {
#define AUX1(EMV, NTV)                                                                        \
  MOE_LAUNCH("aux_single", (aux_single_kernel<EMV, NTV>), dim3(1), dim3(NTV), 0, st, logits,  \
             counts_all, c.T, c.E, c.K, alpha, zlam, losses, d_logits)
    if (c.E <= 4) AUX1(4, 1024);
    else AUX1(8, 512);
#undef AUX1
    return MOE_OK;
  }
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

namespace moe {

// ---------------------------------------------------------------------------
// Load-driven selection-bias step ([P5] course notes 8.6): experts select on
// s_e + b_e; an expert with more slots than the mean load T*K/E lowers b_e by
// gamma, one with fewer raises it, one exactly at the mean keeps it.  The
// comparison is exact in integers (counts_e * E vs T * K).
// ---------------------------------------------------------------------------
__global__ void bias_update_kernel(const int32_t* __restrict__ counts, int E, int64_t tk,
                                   float gamma, float* __restrict__ b) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)counts[e] * E;
  if (load > tk) b[e] = b[e] - gamma;
  else if (load < tk) b[e] = b[e] + gamma;
}

int launch_bias_update(const moe_config& c, const int32_t* counts, float gamma, float* b,
                       hipStream_t st) {
  MOE_LAUNCH("bias_update", bias_update_kernel, dim3((unsigned)cdiv(c.E, 256)), dim3(256), 0,
             st, counts, c.E, (int64_t)c.T * c.K, gamma, b);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Sequence-wise balance loss ([P5] 8.5 balance loss applied per sequence of S
// consecutive tokens, averaged over the T/S sequences; 8.6 keeps such a term
// beside the bias rule):
//   f_{b,e} = n_{b,e} / (S K),  P_{b,e} = mean_{t in b} p_{t,e}
//   L = alpha E (S/T) sum_b sum_e f_{b,e} P_{b,e}
//   dL/ds_{t,i} = w_{t,i} (u_{b,i} - sum_e p_{t,e} u_{b,e}),
//   u_{b,e} = alpha E (S/T) f_{b,e} / S
// p = softmax(s) (w = p) or sigma(s_e) / sum_j sigma(s_j)
// (w = sigma_i (1 - sigma_i) / sum_j sigma_j).
// Three passes over blocks of tokens and sequences (below); no global
// atomics, every sum in a fixed order, so the result does not depend on
// scheduling.
// ---------------------------------------------------------------------------
struct TokProb {
  float m, z;  // softmax: max and normaliser; sigmoid: z = sum_j sigma_j
};

__device__ __forceinline__ TokProb tok_norm(const float* s, int E, int lane, int score) {
  TokProb r;
  if (score == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, s[e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += expf(s[e] - m);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
    r.m = m;
    r.z = z;
  } else {
    float z = 0.f;
    for (int e = lane; e < E; e += 64) z += 1.0f / (1.0f + expf(-s[e]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
    r.m = 0.f;
    r.z = z;
  }
  return r;
}

__device__ __forceinline__ void tok_prob(float s, const TokProb& n, int score, float& p, float& w) {
  if (score == MOE_SCORE_SOFTMAX) {
    p = expf(s - n.m) / n.z;
    w = p;
  } else {
    const float sg = 1.0f / (1.0f + expf(-s));
    p = sg / n.z;
    w = sg * (1.0f - sg) / n.z;
  }
}

// Pass 1, one workgroup per block of TB tokens (TB divides S, so a block
// never straddles two sequences): the block's expert histogram (integer LDS
// atomics, order-free) and its probability sums (each of the four waves takes
// every fourth token of the block, lanes own experts, the four wave rows are
// added in wave order) -> pN[blk][E], pP[blk][E].
__global__ __launch_bounds__(256) void seq_aux_blocks_kernel(const float* __restrict__ logits,
                                                             const int32_t* __restrict__ idx,
                                                             int E, int K, int TB, int score,
                                                             int32_t* __restrict__ pN,
                                                             float* __restrict__ pP) {
  extern __shared__ float sh[];
  int32_t* cnt = reinterpret_cast<int32_t*>(sh);  // [E]
  float* Pw = sh + E;                             // [4][E]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  for (int i = tid; i < 4 * E; i += 256) Pw[i] = 0.f;
  __syncthreads();
  for (int i = tid; i < TB * K; i += 256) atomicAdd(&cnt[idx[t0 * K + i]], 1);
  for (int t = wave; t < TB; t += 4) {
    const float* s = logits + (size_t)(t0 + t) * E;
    const TokProb n = tok_norm(s, E, lane, score);
    for (int e = lane; e < E; e += 64) {
      float p, w;
      tok_prob(s[e], n, score, p, w);
      Pw[wave * E + e] += p;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    pN[(size_t)blockIdx.x * E + e] = cnt[e];
    pP[(size_t)blockIdx.x * E + e] = ((Pw[e] + Pw[E + e]) + Pw[2 * E + e]) + Pw[3 * E + e];
  }
}

// Pass 2, one workgroup per sequence: sums its S/TB blocks in block order,
// writes u_{b,e} = alpha E / T * n_{b,e} / (S K) over the sequence's first
// block row of pP, and the sequence's sum_e f_e P_e.
__global__ __launch_bounds__(256) void seq_aux_seqs_kernel(const int32_t* __restrict__ pN,
                                                           float* __restrict__ pP, int T_, int E,
                                                           int K, int S, int TB, float alpha,
                                                           float* __restrict__ part) {
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = S / TB;
  const size_t r0 = (size_t)b * nb;
  const float inv_sk = 1.0f / ((float)S * (float)K);
  float acc = 0.f;
  for (int e = tid; e < E; e += 256) {
    int n = 0;
    float P = 0.f;
    for (int j = 0; j < nb; ++j) {
      n += pN[(r0 + j) * E + e];
      P += pP[(r0 + j) * E + e];
    }
    const float f = (float)n * inv_sk;
    acc += f * (P / (float)S);
    pP[r0 * E + e] = alpha * (float)E / (float)T_ * f;  // u (after every read of row r0)
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) part[b] = ((red[0] + red[1]) + red[2]) + red[3];
}

// Pass 3, one workgroup per block of TB tokens, one wave per token: the
// logit gradient w (u_b - sum_e p u_b), written or added.
__global__ __launch_bounds__(256) void seq_aux_grad_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ pP, int E,
                                                           int S, int TB, int score,
                                                           float* __restrict__ dlog,
                                                           int accumulate) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int64_t seq = t0 / S;
  const float* u = pP + (size_t)(seq * (S / TB)) * E;
  for (int t = wave; t < TB; t += 4) {
    const float* s = logits + (size_t)(t0 + t) * E;
    const TokProb n = tok_norm(s, E, lane, score);
    float pu = 0.f;
    for (int e = lane; e < E; e += 64) {
      float p, w;
      tok_prob(s[e], n, score, p, w);
      pu += p * u[e];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pu += __shfl_xor(pu, o, 64);
    float* d = dlog + (size_t)(t0 + t) * E;
    for (int e = lane; e < E; e += 64) {
      float p, w;
      tok_prob(s[e], n, score, p, w);
      const float g = w * (u[e] - pu);
      d[e] = accumulate ? d[e] + g : g;
    }
  }
}

// loss = alpha E (S/T) sum_b part[b]; 1024 threads, thread i sums b = i,
// i + 1024, ... then a fixed tree
__global__ __launch_bounds__(1024) void seq_aux_final_kernel(const float* __restrict__ part,
                                                             int nseq, float coef,
                                                             float* __restrict__ loss) {
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  float v = 0.f;
  for (int b = tid; b < nseq; b += 1024) v += part[b];
  red[tid] = v;
  __syncthreads();
  for (int o = 512; o >= 1; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) *loss = coef * red[0];
}

int launch_seq_aux(const moe_config& c, const float* logits, const int32_t* idx, int S,
                   float alpha, float* loss, float* dlog, bool accumulate, char* ws,
                   const Workspace& L, hipStream_t st) {
  // token blocks of TB | S tokens: the largest divisor of S up to 16
  int TB = 1;
  for (int d = std::min(S, 16); d >= 1; --d)
    if (S % d == 0) { TB = d; break; }
  const int nblk = c.T / TB, nseq = c.T / S;
  int32_t* pN = reinterpret_cast<int32_t*>(ws + L.seq_blk_n);
  float* pP = reinterpret_cast<float*>(ws + L.seq_blk_p);
  float* part = reinterpret_cast<float*>(ws + L.seq_part);
  const size_t shm = (size_t)5 * c.E * 4;
  MOE_LAUNCH("seq_aux", seq_aux_blocks_kernel, dim3(nblk), dim3(256), shm, st, logits, idx, c.E,
             c.K, TB, c.score_fn, pN, pP);
  MOE_LAUNCH("seq_aux_seqs", seq_aux_seqs_kernel, dim3(nseq), dim3(256), 0, st, pN, pP, c.T, c.E,
             c.K, S, TB, alpha, part);
  if (dlog)
    MOE_LAUNCH("seq_aux_grad", seq_aux_grad_kernel, dim3(nblk), dim3(256), 0, st, logits, pP,
               c.E, S, TB, c.score_fn, dlog, accumulate ? 1 : 0);
  const float coef = alpha * (float)c.E * ((float)S / (float)c.T);
  MOE_LAUNCH("seq_aux_final", seq_aux_final_kernel, dim3(1), dim3(1024), 0, st, part, nseq, coef,
             loss);
  return MOE_OK;
}

}  // namespace moe
