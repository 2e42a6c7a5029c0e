// backward.hip -- gating backward, router backward and the order of the
// backward kernels.
//
// [P5] course notes 8.3: the top-K indices are piecewise constant, so the
// router learns only through the continuous gate weights g; with gating B and
// K = 1 the single weight is identically 1 and the router gets no gradient
// from the layer output.  [P2] section 2 states the same for MiniMind's
// renormalised top-1.  [P1] cause section: sentinel slots must carry a zero
// expert output so that their gate weights receive no gradient.
//
// Gating backward in centred form (G = sum_k g_k dg_k):
//   softmax A: ds_i = p_i (sum_{k: i_k = i} dg_k - G)
//   softmax B: ds_{i_k} = g_k (dg_k - G); every other ds_i = 0
//   sigmoid A: ds_{i_k} = dg_k sig(1 - sig)
//   sigmoid B: ds_{i_k} = ((dg_k - G) / sum_j sig_{i_j}) sig(1 - sig)
// The centred form keeps the exact zeros: K = 1 with B gives 1*(dg - dg) = 0.
// Router backward: dx += ds W_r; dW_r = ds^T x; d r_b = sum_t ds_t.
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace moe {

int launch_combine_bwd(const moe_config& c, const void* o_perm, const void* dy,
                       const int32_t* slot_row, const float* topk_w, float* dg, void* d_o,
                       hipStream_t st);
int launch_unpermute(const moe_config& c, const void* dxp, const int32_t* slot_row,
                     const int32_t* offsets, const float* ds, const float* wr, const float* dxr,
                     void* dx, hipStream_t st);

// L lanes per token (L = min(64, pow2ceil(E))), EPL experts per lane.  With
// KM > 0 (token choice, K <= KM) a token's slot data (weights, gradients,
// indices, and the indexed logits) are loaded into registers up front, all
// loads in flight together (indices clamped to the last slot, extra entries
// never used); KM = 0 walks the slots in memory.  Same arithmetic and order.
template <int L, int EPL, int KM>
__global__ __launch_bounds__(256) void gating_bwd_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gw, const float* __restrict__ dg, const float* __restrict__ dlx,
    const float* __restrict__ jit, int T_, int E, int K, int score, int gating,
    float* __restrict__ ds, float* __restrict__ ds_copy) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = gid / L, sub = gid % L;
  if (t >= T_) return;
  const float* s = logits + (size_t)t * E;
  const float* g = gw + (size_t)t * K;
  const float* d = dg + (size_t)t * K;
  float out[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) out[j] = 0.f;
  if (!idx) {
    // expert choice: one slot per expert (K = E), g = p for every pair, so
    // ds_e = p_e (dg_e - G) with G = sum_e p_e dg_e (lane partials, then a
    // fixed shuffle tree)
    float G = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sub + L * j;
      if (e < E) G = fmaf(g[e], d[e], G);
    }
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) G += __shfl_xor(G, o, 64);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sub + L * j;
      if (e < E) out[j] = g[e] * (d[e] - G);
    }
  } else if constexpr (KM > 0) {
    const int32_t* it = idx + (size_t)t * K;
    float gk[KM], dk[KM], sk[KM];
    int ik[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      const int kk = k < K ? k : K - 1;
      gk[k] = g[kk];
      dk[k] = d[kk];
      ik[k] = it[kk];
    }
    float G = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (k < K) G = fmaf(gk[k], dk[k], G);
    if (score == 0 && gating == 0) {
      float sv[EPL], m = -INFINITY;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = sub + L * j;
        const float v = s[e < E ? e : 0];
        sv[j] = (e < E) ? v : -INFINITY;
        m = fmaxf(m, sv[j]);
      }
#pragma unroll
      for (int o = L / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (sub + L * j < E) z += expf(sv[j] - m);
#pragma unroll
      for (int o = L / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
      float dp[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) dp[j] = 0.f;
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        const int e = ik[k];
        if (k < K && (e % L) == sub) {
          const int jj = e / L;
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            if (j == jj) dp[j] += dk[k];
        }
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (sub + L * j < E) out[j] = (expf(sv[j] - m) / z) * (dp[j] - G);
    } else {
      if (score == 1) {
#pragma unroll
        for (int k = 0; k < KM; ++k) sk[k] = s[ik[k]];
      }
      float S = 0.f;
      if (score == 1 && gating == 1) {
#pragma unroll
        for (int k = 0; k < KM; ++k)
          if (k < K) S += 1.0f / (1.0f + expf(-sk[k]));
      }
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        const int e = ik[k];
        if (k >= K || (e % L) != sub) continue;
        float v;
        if (score == 0) {
          v = gk[k] * (dk[k] - G);
        } else {
          const float sg = 1.0f / (1.0f + expf(-sk[k]));
          const float dsig = sg * (1.0f - sg);
          v = (gating == 0) ? dk[k] * dsig : ((dk[k] - G) / S) * dsig;
        }
        const int jj = e / L;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (j == jj) out[j] = v;
      }
    }
  } else {
    const int32_t* it = idx + (size_t)t * K;
    float G = 0.f;
    for (int k = 0; k < K; ++k) G = fmaf(g[k], d[k], G);
    if (score == 0 && gating == 0) {
      float sv[EPL], m = -INFINITY;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = sub + L * j;
        sv[j] = (e < E) ? s[e] : -INFINITY;
        m = fmaxf(m, sv[j]);
      }
#pragma unroll
      for (int o = L / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (sub + L * j < E) z += expf(sv[j] - m);
#pragma unroll
      for (int o = L / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
      float dp[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) dp[j] = 0.f;
      for (int k = 0; k < K; ++k) {
        const int e = it[k];
        if ((e % L) == sub) {
          const int jj = e / L;
#pragma unroll
          for (int j = 0; j < EPL; ++j)
            if (j == jj) dp[j] += d[k];
        }
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (sub + L * j < E) out[j] = (expf(sv[j] - m) / z) * (dp[j] - G);
    } else {
      float S = 0.f;
      if (score == 1 && gating == 1)
        for (int k = 0; k < K; ++k) S += 1.0f / (1.0f + expf(-s[it[k]]));
      for (int k = 0; k < K; ++k) {
        const int e = it[k];
        if ((e % L) != sub) continue;
        float v;
        if (score == 0) {
          v = g[k] * (d[k] - G);
        } else {
          const float sg = 1.0f / (1.0f + expf(-s[e]));
          const float dsig = sg * (1.0f - sg);
          v = (gating == 0) ? d[k] * dsig : ((d[k] - G) / S) * dsig;
        }
        const int jj = e / L;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (j == jj) out[j] = v;
      }
    }
  }  // token choice
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + L * j;
    if (e >= E) continue;
    float v = out[j];
    if (dlx) v += dlx[(size_t)t * E + e];
    // jittered logits s~ = s u: the gradient w.r.t. the raw logits
    if (jit) v *= jit[(size_t)t * E + e];
    ds[(size_t)t * E + e] = v;
    if (ds_copy) ds_copy[(size_t)t * E + e] = v;
  }
}

template <int L, int EPL>
static int launch_gating_bwd_t(const moe_config& c, const float* lg, const int32_t* idx,
                               const float* gw, const float* dg, const float* dlx,
                               const float* jit, float* ds, float* ds_copy, hipStream_t st) {
  const int grid = (int)cdiv((int64_t)c.T * L, 256);
#define GBK(KMV)                                                                             \
  MOE_LAUNCH("gating_bwd", (gating_bwd_kernel<L, EPL, KMV>), dim3(grid), dim3(256), 0, st, lg, \
             idx, gw, dg, dlx, jit, c.T, c.E, slot_width(c), c.score_fn, c.gating, ds, ds_copy)
  if (idx && c.K <= 2) GBK(2);
  else if (idx && c.K <= 4) GBK(4);
  else if (idx && c.K <= 8) GBK(8);
#undef GBK
  else
    MOE_LAUNCH("gating_bwd", (gating_bwd_kernel<L, EPL, 0>), dim3(grid), dim3(256), 0, st, lg,
               idx, gw, dg, dlx, jit, c.T, c.E, slot_width(c), c.score_fn, c.gating, ds, ds_copy);
  return MOE_OK;
}

static int launch_gating_bwd(const moe_config& c, const float* lg, const int32_t* idx,
                             const float* gw, const float* dg, const float* dlx, const float* jit,
                             float* ds, float* ds_copy, hipStream_t st) {
  const int E = c.E;
#define GB(Lv, Ev) return launch_gating_bwd_t<Lv, Ev>(c, lg, idx, gw, dg, dlx, jit, ds, ds_copy, st)
  if (E <= 1) GB(1, 1);
  if (E <= 2) GB(2, 1);
  if (E <= 4) GB(4, 1);
  if (E <= 8) GB(8, 1);
  if (E <= 16) GB(16, 1);
  if (E <= 32) GB(32, 1);
  if (E <= 64) GB(64, 1);
  if (E <= 128) GB(64, 2);
  if (E <= 256) GB(64, 4);
  if (E <= 512) GB(64, 8);
  GB(64, 16);
#undef GB
}

// ---------------------------------------------------------------------------
// router weight gradient, few experts (E <= 16):
//   part[chunk][e][d] = sum_{t in chunk} ds[t,e] x[t,d],  part[chunk][E+e] = sum ds[t,e]
// A workgroup owns 64*W model dims (W consecutive per lane, one 8- or 16-byte
// load per token) and one token chunk; its four waves take every fourth token
// and are added in wave order at the end.  ds rows are wave-uniform scalar
// loads.  Workgroups with blockIdx.x == 0 also form the router-bias partial.
// The chunk partials are reduced in a fixed order afterwards.
// ---------------------------------------------------------------------------
template <typename T, int W> struct RowLoad;
template <> struct RowLoad<float, 4> {
  static MOE_DEV void f32(const float* p, float* o) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct RowLoad<bf16_t, 4> {
  static MOE_DEV void f32(const bf16_t* p, float* o) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
};
template <> struct RowLoad<bf16_t, 8> {
  static MOE_DEV void f32(const bf16_t* p, float* o) {
    Vec16<bf16_t> v;
    v.load(p);
    v.to_f32(o);
  }
};

template <typename T, int EM, int W>
__global__ __launch_bounds__(256) void router_wgrad_skinny_kernel(
    const float* __restrict__ ds, const T* __restrict__ x, int T_, int D, int E, int chunk_len,
    float* __restrict__ part) {
  __shared__ float red[3][64 * W];
  __shared__ float redb[4][EM];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.y;
  const int t0 = chunk * chunk_len;
  const int t1 = min(T_, t0 + chunk_len);
  const int d = blockIdx.x * 64 * W + lane * W;
  const bool dok = d < D;
  float acc[EM][W], accb[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    accb[e] = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) acc[e][i] = 0.f;
  }
  // four of the wave's tokens per step, every load issued before the
  // arithmetic: x unconditionally (lanes past D re-read column 0 and never
  // store), ds as wave-uniform scalar loads (tokens past the chunk and
  // experts past E get a zero weight); the sums run in token order
  const int dl = dok ? d : 0;
  for (int tb = t0 + wave; tb < t1; tb += 16) {
    float xv[4][W], sv[4][EM];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = __builtin_amdgcn_readfirstlane(min(tb + 4 * u, t1 - 1));
      RowLoad<T, W>::f32(x + (size_t)t * D + dl, xv[u]);
      const float* dsr = ds + (size_t)t * E;
#pragma unroll
      for (int e = 0; e < EM; ++e) sv[u][e] = dsr[e < E ? e : 0];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool tv = tb + 4 * u < t1;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const float s = (tv && e < E) ? sv[u][e] : 0.f;
        accb[e] += s;
#pragma unroll
        for (int i = 0; i < W; ++i) acc[e][i] = fmaf(s, xv[u][i], acc[e][i]);
      }
    }
  }
  // partial row stride rounded up to 4 floats (shared with the workspace layout)
  float* p = part + (size_t)chunk * (((size_t)E * D + E + 3) & ~(size_t)3);
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    if (e >= E) break;
    if (wave > 0)
#pragma unroll
      for (int i = 0; i < W; ++i) red[wave - 1][lane * W + i] = acc[e][i];
    __syncthreads();
    if (wave == 0 && dok) {
      float o[W];
#pragma unroll
      for (int i = 0; i < W; ++i)
        o[i] = ((acc[e][i] + red[0][lane * W + i]) + red[1][lane * W + i]) + red[2][lane * W + i];
#pragma unroll
      for (int i = 0; i < W; i += 4)
        *reinterpret_cast<float4*>(p + (size_t)e * D + d + i) =
            make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    }
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    if (lane == 0)
#pragma unroll
      for (int e = 0; e < EM; ++e) redb[wave][e] = accb[e];
    __syncthreads();
    if (threadIdx.x < E)
      p[(size_t)E * D + threadIdx.x] = ((redb[0][threadIdx.x] + redb[1][threadIdx.x]) +
                                        redb[2][threadIdx.x]) + redb[3][threadIdx.x];
  }
}

// fixed-order sum of the split partials: out[i] = sum_s part[s * stride + i].
// 64 columns (16 float4 lanes) x 16 split lanes per workgroup; lane ty sums
// splits ty, ty+16, ... and the 16 lane sums are added in lane order, so the
// result does not depend on scheduling.  stride and n_first are multiples of 4
// and part holds stride floats per split (columns n..stride-1 are padding).
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part,
                                                            int nsplit, int64_t n,
                                                            int64_t stride, float* __restrict__ out,
                                                            float* __restrict__ out2,
                                                            int64_t n_first) {
  __shared__ float4 red[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t i = ((int64_t)blockIdx.x * 16 + tx) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < n)
#pragma unroll 4
    for (int k = ty; k < nsplit; k += 16) {
      const float4 v = *reinterpret_cast<const float4*>(part + (size_t)k * stride + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && i < n) {
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float4 v = red[k][tx];
      t[0] += v.x; t[1] += v.y; t[2] += v.z; t[3] += v.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = i + j;
      if (c >= n) break;
      if (c < n_first) out[c] = t[j];
      else if (out2) out2[c - n_first] = t[j];
    }
  }
}

// ---------------------------------------------------------------------------
// router GEMMs for many experts when E is not a multiple of 4 (otherwise
// router_gemm_kernel, on the matrix cores): SIMT fp32 tiles of 64 x 64,
// k-slabs of 16 in LDS, 4 x 4 register micro-tile, optional split over k
// (partials).
//   C[split][m][n] = sum_{k in split} A(m,k) B(k,n)
//   A(m,k) = AKC ? A[m*lda + k] : A[k*lda + m];  B(k,n) = B[k*ldb + n]
// ---------------------------------------------------------------------------
template <typename TA, typename TB, bool AKC>
__global__ __launch_bounds__(256) void simt_gemm_kernel(const TA* __restrict__ A, int64_t lda,
                                                        const TB* __restrict__ B, int64_t ldb,
                                                        int M, int N, int Kd, int kper,
                                                        float* __restrict__ C, int64_t ldc,
                                                        int64_t split_stride) {
  __shared__ float sa[16][65];
  __shared__ float sb[16][65];
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64, split = blockIdx.z;
  const int kb = split * kper, ke = min(Kd, kb + kper);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
    float av[4], bv[4];
    if (AKC) {  // thread -> (m = tid/4, k = (tid%4)*4 + i)
      const int m = m0 + (threadIdx.x >> 2), kk = (threadIdx.x & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + kk + i;
        av[i] = (m < M && k < ke) ? Elem<TA>::to_f32(A[(int64_t)m * lda + k]) : 0.f;
      }
    } else {  // thread -> (k = tid/16, m = (tid%16)*4 + i)
      const int k = k0 + (threadIdx.x >> 4), mm = (threadIdx.x & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mm + i;
        av[i] = (m < M && k < ke) ? Elem<TA>::to_f32(A[(int64_t)k * lda + m]) : 0.f;
      }
    }
    {
      const int k = k0 + (threadIdx.x >> 4), nn = (threadIdx.x & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + nn + i;
        bv[i] = (n < N && k < ke) ? Elem<TB>::to_f32(B[(int64_t)k * ldb + n]) : 0.f;
      }
    }
    __syncthreads();
    if (AKC) {
      const int mm = threadIdx.x >> 2, kk = (threadIdx.x & 3) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[kk + i][mm] = av[i];
    } else {
      const int kk = threadIdx.x >> 4, mm = (threadIdx.x & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[kk][mm + i] = av[i];
    }
    {
      const int kk = threadIdx.x >> 4, nn = (threadIdx.x & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) sb[kk][nn + i] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sa[k][ty + 16 * i]; b[i] = sb[k][tx + 16 * i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
  float* Cs = C + (int64_t)split * split_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n < N) Cs[(int64_t)m * ldc + n] = acc[i][j];
    }
  }
}

// d r_b partials: part[chunk][e] = sum_{t in chunk} ds[t,e].  64 experts x 4
// token lanes per workgroup (lane ty takes every fourth token of the chunk),
// lanes added in order; the chunk partials are reduced in a fixed order after.
__global__ __launch_bounds__(256) void rbias_partial_kernel(const float* __restrict__ ds, int T_,
                                                            int E, int chunk_len, int64_t stride,
                                                            float* __restrict__ part) {
  __shared__ float red[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + tx;
  const int t0 = blockIdx.y * chunk_len, t1 = min(T_, t0 + chunk_len);
  float s = 0.f;
  if (e < E)
#pragma unroll 8
    for (int t = t0 + ty; t < t1; t += 4) s += ds[(size_t)t * E + e];
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && e < E)
    part[(size_t)blockIdx.y * stride + e] = ((red[0][tx] + red[1][tx]) + red[2][tx]) + red[3][tx];
}

template <typename T>
static int router_bwd_t(const moe_config& c, const void* x, const float* wr, const float* ds,
                        float* dxr, float* dwr, float* drb, char* ws, const Workspace& L,
                        hipStream_t st) {
  const int E = c.E, D = c.D, T_ = c.T;
  float* part = reinterpret_cast<float*>(ws + L.dwr_part);
  if (E <= 16) {
    const int nchunk = L.dwr_splits;
    const int chunk_len = (int)cdiv(T_, nchunk);
    const int W = router_wgrad_width(c);
    dim3 grid((unsigned)cdiv(D, 64 * W), (unsigned)nchunk);
#define RW(EMV, WV)                                                                        \
  MOE_LAUNCH("router_wgrad", (router_wgrad_skinny_kernel<T, EMV, WV>), grid, dim3(256), 0, st, \
             ds, (const T*)x, T_, D, E, chunk_len, part)
#define RWE(WV)                \
  if (E <= 4) RW(4, WV);       \
  else if (E <= 8) RW(8, WV);  \
  else RW(16, WV);
    if constexpr (sizeof(T) == 2) {
      if (W == 8) { RWE(8) } else { RWE(4) }
    } else {
      RWE(4)
    }
#undef RWE
#undef RW
    const int64_t n = (int64_t)E * D + E;
    const int64_t stride = (n + 3) & ~(int64_t)3;
    MOE_LAUNCH("router_wgrad_reduce", reduce_splits_kernel, dim3((unsigned)cdiv(n, 64)),
               dim3(256), 0, st, part, nchunk, n, stride, dwr, drb, (int64_t)E * D);
  } else {
    const bool mfma = router_gemm_fits(E, D, T_, D, E, true) &&
                      router_gemm_fits(E, D, E, D, T_, false);
    if (mfma) {
      // fp32 matrix cores: dxr[T,D] = ds[T,E] W_r[E,D]; dW_r[E,D] = ds^T x in
      // token splits of a multiple of 32
      int rc;
      if ((rc = router_gemm("router_dgrad", true, false, ds, E, wr, D, T_, D, E,
                            (int)cdiv(E, 32) * 32, 1, dxr, D, 0, st)))
        return rc;
      const int kper = (int)std::max<int64_t>(32, cdiv(cdiv(T_, L.dwr_splits), 32) * 32);
      const int splits = (int)std::max<int64_t>(1, cdiv(T_, kper));
      if ((rc = router_gemm("router_wgrad", false, sizeof(T) == 2, ds, E, x, D, E, D, T_, kper,
                            splits, part, D, (int64_t)E * D, st)))
        return rc;
      const int64_t n = (int64_t)E * D;
      MOE_LAUNCH("router_wgrad_reduce", reduce_splits_kernel, dim3((unsigned)cdiv(n, 64)),
                 dim3(256), 0, st, part, splits, n, n, dwr, (float*)nullptr, n);
    } else {
      // SIMT fallback (E not a multiple of 4)
      // dxr[T,D] = ds[T,E] W_r[E,D]
      dim3 g1((unsigned)cdiv(T_, 64), (unsigned)cdiv(D, 64), 1);
      MOE_LAUNCH("router_dgrad", (simt_gemm_kernel<float, float, true>), g1, dim3(256), 0, st, ds,
                 (int64_t)E, wr, (int64_t)D, T_, D, E, E, dxr, (int64_t)D, (int64_t)0);
      // dW_r[E,D] = ds^T x, split over tokens
      const int splits = L.dwr_splits;
      const int kper = (int)(cdiv(cdiv(T_, splits), 16) * 16);
      dim3 g2((unsigned)cdiv(E, 64), (unsigned)cdiv(D, 64), (unsigned)splits);
      MOE_LAUNCH("router_wgrad", (simt_gemm_kernel<float, T, false>), g2, dim3(256), 0, st, ds,
                 (int64_t)E, (const T*)x, (int64_t)D, E, D, T_, kper, part, (int64_t)D,
                 (int64_t)E * D);
      const int64_t n = (int64_t)E * D;
      MOE_LAUNCH("router_wgrad_reduce", reduce_splits_kernel, dim3((unsigned)cdiv(n, 64)),
                 dim3(256), 0, st, part, splits, n, n, dwr, (float*)nullptr, n);
    }
    if (drb) {
      float* rpart = reinterpret_cast<float*>(ws + L.rb_part);
      const int64_t rstride = ((int64_t)E + 3) & ~(int64_t)3;
      const int clen = (int)cdiv(T_, L.rb_splits);
      MOE_LAUNCH("router_bias_grad", rbias_partial_kernel,
                 dim3((unsigned)cdiv(E, 64), (unsigned)L.rb_splits), dim3(256), 0, st, ds, T_, E,
                 clen, rstride, rpart);
      MOE_LAUNCH("router_bias_reduce", reduce_splits_kernel, dim3((unsigned)cdiv(E, 64)),
                 dim3(256), 0, st, rpart, L.rb_splits, (int64_t)E, rstride, drb, (float*)nullptr,
                 (int64_t)E);
    }
  }
  return MOE_OK;
}

int launch_backward(const moe_config& c, const void* x, const float* wr, const float* logits,
                    const int32_t* idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* slot_row, const void* x_perm, const void* act, const void* h,
                    const void* o_perm, const void* wg, const void* wu, const void* wd,
                    const void* dy, const float* dlx, const float* jit, void* dx, float* dwr,
                    float* drb, void* dwg, void* dwu, void* dwd, float* d_logits_out, char* ws,
                    const Workspace& L, hipStream_t st) {
  void* d_o = ws + L.d_o;
  void* dact = ws + L.dact;
  void* dxp = ws + L.dx_perm;
  float* dg = reinterpret_cast<float*>(ws + L.dg);
  float* ds = reinterpret_cast<float*>(ws + L.ds);
  float* dxr = (c.E > 16) ? reinterpret_cast<float*>(ws + L.dxr) : nullptr;
  int rc;
  if ((rc = launch_combine_bwd(c, o_perm, dy, slot_row, topk_w, dg, d_o, st))) return rc;
  // Independent parts overlap on two side streams:
  //   main:   down dgrad -> up dgrad -> (router) -> un-permute
  //   side 0: down wgrad -> (after down dgrad) up wgrad
  //   side 1: gating backward, then the router weight / bias gradient (and
  //           dgrad for many experts); the un-permute waits for it
  // MOE_SERIAL_STREAMS set (measurement): everything on the caller's stream,
  // so that per-kernel timings are those of each kernel alone
  const bool serial = getenv("MOE_SERIAL_STREAMS") != nullptr;
  hipStream_t s0 = serial ? st : side_stream(0), s1 = serial ? st : side_stream(1);
  if (!serial && (!s0 || !s1)) {
    set_error("side streams", hipErrorInvalidResourceHandle);
    return MOE_ELAUNCH;
  }
  if ((rc = fork_stream(st, s0)) || (rc = fork_stream(st, s1))) return rc;
  if ((rc = launch_gating_bwd(c, logits, idx, topk_w, dg, dlx, jit, ds, d_logits_out, s1)))
    return rc;
  if (c.dtype == MOE_BF16) {
    if ((rc = router_bwd_t<bf16_t>(c, x, wr, ds, dxr, dwr, drb, ws, L, s1))) return rc;
  } else {
    if ((rc = router_bwd_t<float>(c, x, wr, ds, dxr, dwr, drb, ws, L, s1))) return rc;
  }
  if ((rc = gemm_down_wgrad(c, offsets, h, d_o, dy, dwd, s0))) return rc;
  if ((rc = gemm_down_dgrad(c, offsets, d_o, dy, wd, act, dact, st))) return rc;
  if ((rc = fork_stream(st, s0))) return rc;  // dact is ready
  if ((rc = gemm_up_wgrad(c, offsets, x, x_perm, dact, dwg, dwu, s0))) return rc;
  if ((rc = gemm_up_dgrad(c, offsets, dact, wg, wu, dxp, st))) return rc;
  if ((rc = fork_stream(s1, st))) return rc;  // join: router part of dx
  if ((rc = launch_unpermute(c, dxp, slot_row, offsets, ds, wr, dxr, dx, st))) return rc;
  return fork_stream(s0, st);                 // join: weight gradients
}

}  // namespace moe
