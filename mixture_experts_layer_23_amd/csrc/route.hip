// route.hip -- router logits, selection key, top-K and gate weights.
//
// [P3] "MoE" tutorial, Router/Gating Network: the router is a linear layer
// s = x W_g followed by a score function; KeepTopK keeps the K largest.
// [P5] course notes 8.2: token-choice top-K with gating A (truncated softmax)
// or B (softmax renormalised over the selected set); 8.6: sigmoid scores with a
// selection bias b_e that only selects, the weights use the raw scores.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// sig32: the fixed binary32 sigmoid of the selection key (no contraction; the
// only fma are the explicit ones).  exp32(z): clamp to [-87, 87];
// n = rint(z * log2e); r = (z - n*L1) then fma(-n, L2, r) with L1 + L2 = ln 2
// and n*L1 exact (L1 has 15 significant bits); Taylor degree 7 of e^r with
// coefficients 1/k! in binary32, Horner with fma; times 2^n from exponent
// bits.  sig32(z) = 1 / (1 + exp32(-z)) with IEEE division.
// ---------------------------------------------------------------------------
MOE_DEV float sig32(float z) {
#pragma clang fp contract(off)
  const float LOG2E = 1.44269502162933349609375f;
  const float L1 = 0.693145751953125f;
  const float L2 = 1.428606765330187045037746429443359375e-06f;
  float u = -z;
  u = u > 87.0f ? 87.0f : u;
  u = u < -87.0f ? -87.0f : u;
  const float t = u * LOG2E;
  const float n = __builtin_rintf(t);
  const float nl1 = n * L1;
  float r = u - nl1;
  r = __builtin_fmaf(-n, L2, r);
  float p = (float)(1.0 / 5040.0);
  p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const float s = __uint_as_float((uint32_t)((int)n + 127) << 23);
  const float e = p * s;
  const float d = 1.0f + e;
  return 1.0f / d;
}

MOE_DEV bool better(float ka, int ia, float kb, int ib) {
  return (ka > kb) || (ka == kb && ia < ib);
}

// Selection fused into the few-expert router: when idx is set, the lane that
// holds a token's logits also takes its top-K, gate weights and lse (the same
// keys, tie rule and weight definitions as route_select_kernel below).
struct FusedSelect {
  const float* selb;
  int32_t* idx;
  float* w;
  float* lse;
  int K, score, gating;
};

// ---------------------------------------------------------------------------
// Router logits.  Products of a bf16/fp32 activation and an fp32 weight are
// exact in double, the sum is accumulated in double and rounded once to
// binary32, so the result is (up to a ~1e-12 relative accumulation error) the
// correctly rounded dot product whatever the summation order.  A top-K taken
// on these logits is therefore reproducible by any other double-accumulating
// implementation.
// ---------------------------------------------------------------------------

// Skinny router (E <= 16): each wave takes two tokens at a time, lanes stride
// over D in 16-byte vectors (coalesced), four vectors per lane in flight at
// once; fp64 partials are reduced across the wave.  W_r (E*D fp32, at most
// 128 KB) is read straight from the caches when small (STAGE false) or staged
// in LDS once per workgroup.
template <typename T, int EM, bool STAGE>
__global__ __launch_bounds__(256) void router_skinny_kernel(const T* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ rb,
                                                            float* __restrict__ logits, int T_,
                                                            int D, int E, FusedSelect fs) {
  extern __shared__ float4 sw4[];
  const float* wsrc = wr;
  if constexpr (STAGE) {
    // staging in batches of eight 16-byte loads per thread, all in flight
    // before the first LDS store (whole batches unconditional, so that the
    // compiler does not sink each load into a guarded store); then the tail
    const float4* w4 = reinterpret_cast<const float4*>(wr);
    const int n4 = (E * D) >> 2, tid = (int)threadIdx.x;
    int i0 = 0;
    for (; i0 + 256 * 8 <= n4; i0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = w4[i0 + u * 256 + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) sw4[i0 + u * 256 + tid] = v[u];
    }
    for (int i = i0 + tid; i < n4; i += 256) sw4[i] = w4[i];
    __syncthreads();
    wsrc = reinterpret_cast<const float*>(sw4);
  }
  constexpr int VEC = Elem<T>::VEC, NV = 4;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nwave = gridDim.x * (blockDim.x >> 6);
  for (int t0 = wave * 2; t0 < T_; t0 += nwave * 2) {
    const bool two = (t0 + 1) < T_;
    double acc0[EM], acc1[EM];
#pragma unroll
    for (int e = 0; e < EM; ++e) { acc0[e] = 0.0; acc1[e] = 0.0; }
    // every load is issued (past-the-end lanes re-read column 0, a lone
    // last token re-reads itself; both are discarded below), so that no
    // branch makes the compiler wait for one load before issuing the next
    const T* xa_row = x + (size_t)t0 * D;
    const T* xb_row = x + (size_t)(two ? t0 + 1 : t0) * D;
    for (int dc = 0; dc < D; dc += 64 * VEC * NV) {
      Vec16<T> va[NV], vb[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int d0 = dc + (v * 64 + lane) * VEC;
        const int dl = d0 < D ? d0 : 0;
        va[v].load(xa_row + dl);
        vb[v].load(xb_row + dl);
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int d0 = dc + (v * 64 + lane) * VEC;
        if (d0 >= D) break;
        float xa[VEC], xb[VEC];
        va[v].to_f32(xa);
        if (two) {
          vb[v].to_f32(xb);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) xb[i] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < EM; ++e) {
          if (e < E) {
            const float* w = wsrc + e * D + d0;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
              acc0[e] = fma((double)xa[i], (double)w[i], acc0[e]);
              acc1[e] = fma((double)xb[i], (double)w[i], acc1[e]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EM; ++e) {
      if (e < E) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
          acc0[e] += shfl_xor_d(acc0[e], m);
          acc1[e] += shfl_xor_d(acc1[e], m);
        }
      }
    }
    if (lane < E) {
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int e = 0; e < EM; ++e)
        if (e == lane) { a0 = acc0[e]; a1 = acc1[e]; }
      const double b = rb ? (double)rb[lane] : 0.0;
      logits[(size_t)t0 * E + lane] = (float)(a0 + b);
      if (two) logits[(size_t)(t0 + 1) * E + lane] = (float)(a1 + b);
    }
    if (fs.idx && (lane == 0 || (lane == 1 && two))) {
      // lane 0 selects for token t0, lane 1 for t0 + 1; every lane holds
      // all E sums after the reduction
      const int t = t0 + lane;
      float sv[EM], key[EM];
      bool used[EM];
      float m = -INFINITY;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const bool ok = e < E;
        const double a = lane == 0 ? acc0[e] : acc1[e];
        sv[e] = ok ? (float)(a + (rb ? (double)rb[e] : 0.0)) : -INFINITY;
        key[e] = fs.score == 0 ? sv[e]
                               : (ok ? sig32(sv[e]) + (fs.selb ? fs.selb[e] : 0.0f) : -INFINITY);
        used[e] = !ok;
        m = fmaxf(m, sv[e]);
      }
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < EM; ++e)
        if (e < E) z += expf(sv[e] - m);
      if (fs.lse) fs.lse[t] = m + logf(z);
      // K <= E <= EM rounds; the weights stay in registers until the
      // normaliser is known
      float gsum = 0.f, gk[EM];
      int ik[EM];
#pragma unroll
      for (int k = 0; k < EM; ++k) {
        gk[k] = 0.f;
        ik[k] = 0;
        if (k >= fs.K) continue;
        float bk = -INFINITY, sc = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < EM; ++e)
          if (!used[e] && better(key[e], e, bk, bi)) { bk = key[e]; bi = e; sc = sv[e]; }
        bi = bi < E ? bi : 0;  // only reachable with non-finite logits (outside the contract)
#pragma unroll
        for (int e = 0; e < EM; ++e)
          if (e == bi) used[e] = true;
        const float g = fs.score == 0 ? expf(sc - m) : 1.0f / (1.0f + expf(-sc));
        gsum += g;
        gk[k] = g;
        ik[k] = bi;
      }
      float den = 1.f;
      if (fs.score == 0) den = (fs.gating == 0) ? z : gsum;
      else den = (fs.gating == 0) ? 1.f : gsum;
      const bool raw = fs.score == 1 && fs.gating == 0;
#pragma unroll
      for (int k = 0; k < EM; ++k) {
        if (k >= fs.K) break;
        fs.idx[(size_t)t * fs.K + k] = ik[k];
        fs.w[(size_t)t * fs.K + k] = raw ? gk[k] : gk[k] / den;
      }
    }
  }
}

// Tiled router (E > 16) on the fp64 matrix cores: 32 tokens x 64 experts per
// workgroup, each of KG k-groups of four waves (16 tokens x 32 experts each,
// two 16x16 blocks of v_mfma_f64_16x16x4f64) takes every KG-th k-slab of 32;
// the groups' fp64 sums are added in group order at the end, so short
// batches (few tiles) still bring several waves per SIMD.  Slabs are staged
// in LDS as binary32 (exact for both operands; rows padded by 4 floats) and
// widened to double when the fragments are read; each group fetches its next
// slab into registers while the current one is multiplied.
//   MFMA operands: lane l gives A[m = l%16][k = l/16] and B[k = l/16][n = l%16];
//   accumulator element r of lane l is C[m = l/16 + 4r][n = l%16] (the f64
//   form interleaves rows, unlike the f32 16x16 layout).
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kRtT = 32, kRtE = 64, kRtK = 32, kRtP = kRtK + 4;
// LDS bytes of one k-group's slab pair (x and W)
constexpr int kRtGroupBytes = (kRtT + kRtE) * kRtP * 4;

template <typename T> struct RtLoad;
template <> struct RtLoad<bf16_t> {
  // x slab: 32 rows x 32 k = 128 chunks of 8 bf16
  static MOE_DEV void load(const bf16_t* x, int T_, int D, int t0, int k0, int tid, float* v) {
    if (tid < 128) {
      const int r = tid >> 2, kc = (tid & 3) * 8;
      const int t = min(t0 + r, T_ - 1);
      Vec16<bf16_t> q;
      q.load(x + (size_t)t * D + k0 + kc);
      q.to_f32(v);
      if (t0 + r >= T_)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
  }
  static MOE_DEV void store(float (*sx)[kRtP], int tid, const float* v) {
    if (tid < 128) {
      const int r = tid >> 2, kc = (tid & 3) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) sx[r][kc + i] = v[i];
    }
  }
};
template <> struct RtLoad<float> {
  // x slab: 32 rows x 32 k = 256 chunks of 4 floats
  static MOE_DEV void load(const float* x, int T_, int D, int t0, int k0, int tid, float* v) {
    const int r = tid >> 3, kc = (tid & 7) * 4;
    const int t = min(t0 + r, T_ - 1);
    const float4 q = *reinterpret_cast<const float4*>(x + (size_t)t * D + k0 + kc);
    const bool ok = t0 + r < T_;
    v[0] = ok ? q.x : 0.f; v[1] = ok ? q.y : 0.f; v[2] = ok ? q.z : 0.f; v[3] = ok ? q.w : 0.f;
  }
  static MOE_DEV void store(float (*sx)[kRtP], int tid, const float* v) {
    const int r = tid >> 3, kc = (tid & 7) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) sx[r][kc + i] = v[i];
  }
};

template <typename T, int KG>
__global__ __launch_bounds__(256 * KG) void router_tiled_kernel(const T* __restrict__ x,
                                                                const float* __restrict__ wr,
                                                                const float* __restrict__ rb,
                                                                float* __restrict__ logits,
                                                                int T_, int D, int E) {
  // KG slab pairs; after the k loop the same bytes hold the sums of groups
  // 1..KG-1 (256 threads x 8 doubles each)
  static_assert((KG - 1) * 256 * 8 * 8 <= KG * kRtGroupBytes, "reduction does not fit");
  __shared__ __attribute__((aligned(16))) char smem[KG * kRtGroupBytes];
  const int tid = threadIdx.x & 255, grp = threadIdx.x >> 8;
  float(*sx)[kRtP] = reinterpret_cast<float(*)[kRtP]>(smem + grp * kRtGroupBytes);
  float(*sw)[kRtP] = reinterpret_cast<float(*)[kRtP]>(smem + grp * kRtGroupBytes +
                                                      kRtT * kRtP * 4);
  const int t0 = blockIdx.x * kRtT, e0 = blockIdx.y * kRtE;
  const int lane = tid & 63, wave = tid >> 6;
  const int wt = (wave & 1) * 16, we = (wave >> 1) * 32;
  // W slab: 64 rows x 32 k = 512 chunks of 4 floats, two per thread
  float xv[8], wv[2][4];
  auto load = [&](int k0) {
    RtLoad<T>::load(x, T_, D, t0, k0, tid, xv);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ch = tid + 256 * u, r = ch >> 3, kc = (ch & 7) * 4;
      const int e = min(e0 + r, E - 1);
      const float4 q = *reinterpret_cast<const float4*>(wr + (size_t)e * D + k0 + kc);
      const bool ok = e0 + r < E;
      wv[u][0] = ok ? q.x : 0.f; wv[u][1] = ok ? q.y : 0.f;
      wv[u][2] = ok ? q.z : 0.f; wv[u][3] = ok ? q.w : 0.f;
    }
  };
  f64x4_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] = 0.0;
  // group g takes slabs g, g + KG, ...; every group runs the same number of
  // rounds so that the block-wide barriers match
  const int nslab = D / kRtK, rounds = (nslab + KG - 1) / KG;
  if (grp < nslab) load(grp * kRtK);
  for (int rd = 0; rd < rounds; ++rd) {
    const int k0 = (rd * KG + grp) * kRtK;
    const bool have = k0 < D;
    __syncthreads();
    if (have) {
      RtLoad<T>::store(sx, tid, xv);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ch = tid + 256 * u, r = ch >> 3, kc = (ch & 7) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) sw[r][kc + i] = wv[u][i];
      }
    }
    __syncthreads();
    if (k0 + KG * kRtK < D) load(k0 + KG * kRtK);
    if (have) {
#pragma unroll
      for (int ks = 0; ks < kRtK; ks += 4) {
        const int kk = ks + (lane >> 4), i16 = lane & 15;
        const double a = (double)sx[wt + i16][kk];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const double b = (double)sw[we + 16 * j + i16][kk];
          acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[j], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (KG > 1) {
    __syncthreads();
    double* red = reinterpret_cast<double*>(smem);
    if (grp > 0) {
      double* mine = red + ((size_t)(grp - 1) * 256 + tid) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[j * 4 + r] = acc[j][r];
    }
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const double* o = red + ((size_t)(g - 1) * 256 + tid) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] += o[j * 4 + r];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + we + 16 * j + (lane & 15);
    if (e >= E) continue;
    const double bias = rb ? (double)rb[e] : 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + wt + (lane >> 4) + 4 * r;
      if (t < T_) logits[(size_t)t * E + e] = (float)(acc[j][r] + bias);
    }
  }
}

// ---------------------------------------------------------------------------
// Selection and gate weights: L lanes per token (L = min(64, pow2ceil(E))),
// EPL experts per lane (expert e = sub + L*j).  K rounds of a group-wide
// arg-max on (key, index) with equal keys going to the lower index.
// ---------------------------------------------------------------------------
// softplus in double, the overflow-free form log(1 + e^n) = max(n, 0) +
// log1p(e^-|n|)
MOE_DEV double softplus64(double n) { return fmax(n, 0.0) + log1p(exp(-fabs(n))); }

// Router-logit jitter and noisy selection ([P3] ST-MoE, KeepTopK; [P5] 8.6):
// with jit, s~ = s * u (one binary32 multiply) replaces the logits everywhere
// (written back to `logits`); with eps, the selection key is
// fl32(s~ + eps * softplus(n)) evaluated in double (n = the noise logits),
// while the weights and lse stay on s~ (the noise only selects).
template <int L, int EPL>
__global__ __launch_bounds__(256) void route_select_kernel(
    float* __restrict__ logits, const float* __restrict__ selb, const float* __restrict__ jit,
    const float* __restrict__ eps, const float* __restrict__ nlg, int T_, int E, int K,
    int score, int gating, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ lse_out) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = gid / L, sub = gid % L;
  const bool active = t < T_;  // whole L-groups are (in)active together
  if (!active) return;
  float* s = logits + (size_t)t * E;
  float sv[EPL], key[EPL];
  bool used[EPL];
  float m = -INFINITY;
  // all logit (and selection-bias) loads first, unconditional (index
  // clamped), so that they are in flight together
  float sl[EPL], bl[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + L * j;
    sl[j] = s[e < E ? e : 0];
    bl[j] = selb ? selb[e < E ? e : 0] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + L * j;
    const bool ok = e < E;
    sv[j] = ok ? sl[j] : -INFINITY;
    if (jit && ok) {
      sv[j] = sv[j] * jit[(size_t)t * E + e];
      s[e] = sv[j];
    }
    if (score == 0) {
      key[j] = sv[j];
      if (eps && ok)
        key[j] = (float)((double)sv[j] + (double)eps[(size_t)t * E + e] *
                                             softplus64((double)nlg[(size_t)t * E + e]));
    } else {
      key[j] = ok ? (sig32(sv[j]) + bl[j]) : -INFINITY;
    }
    used[j] = !ok;
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
  if (sub == 0 && lse_out) lse_out[t] = m + logf(z);

  // K rounds of arg-max (K <= L); lane sub == k keeps round k's expert and
  // weight in registers and writes them once the normaliser is known
  float gsum = 0.f, my_g = 0.f;
  int my_i = 0;
  for (int k = 0; k < K; ++k) {
    float bk = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = sub + L * j;
      if (!used[j] && better(key[j], e, bk, bi)) { bk = key[j]; bi = e; }
    }
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) {
      const float ok_ = __shfl_xor(bk, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ok_, oi, bk, bi)) { bk = ok_; bi = oi; }
    }
    bi = bi < E ? bi : 0;  // only reachable with non-finite logits (outside the contract)
    // the owner marks it used
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (sub + L * j == bi) used[j] = true;
    // the chosen expert's (jittered) logit, from the lane that holds it
    float sc = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (sub + L * j == bi) sc = sv[j];
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) sc = fmaxf(sc, __shfl_xor(sc, o, 64));
    float g;
    if (score == 0) g = expf(sc - m);                 // unnormalised softmax term
    else g = 1.0f / (1.0f + expf(-sc));               // raw sigmoid score
    gsum += g;
    if (sub == k) { my_i = bi; my_g = g; }
  }
  if (sub < K) {
    // normalise: softmax A divides by the full sum z; B by the selected sum;
    // sigmoid A keeps the raw score; sigmoid B divides by the selected sum.
    float den = 1.f;
    if (score == 0) den = (gating == 0) ? z : gsum;
    else den = (gating == 0) ? 1.f : gsum;
    topk_idx[(size_t)t * K + sub] = my_i;
    topk_w[(size_t)t * K + sub] = (score == 1 && gating == 0) ? my_g : my_g / den;
  }
}

struct SelectExtras {
  const float* jit;
  const float* eps;
  const float* nlg;
};

template <int L, int EPL>
static int launch_select(float* lg, const float* selb, const SelectExtras& x, int T_, int E, int K,
                         int score, int gating, int32_t* idx, float* w, float* lse,
                         hipStream_t st) {
  const int64_t threads = (int64_t)T_ * L;
  const int grid = (int)cdiv(threads, 256);
  MOE_LAUNCH("route_select", (route_select_kernel<L, EPL>), dim3(grid), dim3(256), 0, st, lg, selb,
             x.jit, x.eps, x.nlg, T_, E, K, score, gating, idx, w, lse);
  return MOE_OK;
}

// router logits out[T][E] = fl32(x W^T + b), fp64 accumulation
// the few-expert router can take the selection as well (fsp != nullptr);
// returns 1 (nothing launched) when it cannot, so the caller selects apart
static int router_logits_sel(const moe_config& c, const void* x, const float* wr,
                             const float* rb, float* logits, const FusedSelect* fsp,
                             hipStream_t st) {
  const int T_ = c.T, D = c.D, E = c.E;
  {
    if (E <= 16 && (size_t)E * D * 4 <= 128 * 1024) {
      const FusedSelect fs = fsp ? *fsp : FusedSelect{nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
      const char* name = fsp ? "route_fused" : "router_logits";
      // one token pair per wave, but no more workgroups than fit on the chip
      // at once (a staged W_r is loaded once per workgroup: with large tiles
      // the waves loop over several pairs).  W_r up to 32 KB is read through
      // the caches instead (no staging pass).
      const bool stage = (size_t)E * D * 4 > 32 * 1024;
      const size_t shm = stage ? (size_t)E * D * 4 : 0;
      const int waves_needed = (int)cdiv(T_, 2);
      const int64_t per_cu = stage ? std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / (int64_t)shm)) : 8;
      int grid = (int)std::min<int64_t>(cdiv(waves_needed, 4), 256 * per_cu);
      if (shm > 64 * 1024) {
        // W_r tiles above 64 KB need the kernels' dynamic-LDS limit raised:
        // once per process (outside any stream capture that comes later)
        static hipError_t lim = [] {
          const void* fns[] = {(const void*)router_skinny_kernel<bf16_t, 4, true>,
                               (const void*)router_skinny_kernel<bf16_t, 8, true>,
                               (const void*)router_skinny_kernel<bf16_t, 16, true>,
                               (const void*)router_skinny_kernel<float, 4, true>,
                               (const void*)router_skinny_kernel<float, 8, true>,
                               (const void*)router_skinny_kernel<float, 16, true>};
          for (const void* f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               128 * 1024);
            if (e != hipSuccess) return e;
          }
          return hipSuccess;
        }();
        if (lim != hipSuccess) { set_error("router_logits (LDS limit)", lim); return MOE_ELAUNCH; }
      }
#define SKINNY(TV, EMV, SV)                                                                 \
  MOE_LAUNCH(name, (router_skinny_kernel<TV, EMV, SV>), dim3(grid), dim3(256), shm, st,     \
             (const TV*)x, wr, rb, logits, T_, D, E, fs)
#define SKINNY_E(TV, SV)              \
  if (E <= 4) SKINNY(TV, 4, SV);      \
  else if (E <= 8) SKINNY(TV, 8, SV); \
  else SKINNY(TV, 16, SV);
      if (c.dtype == MOE_BF16) {
        if (stage) { SKINNY_E(bf16_t, true) } else { SKINNY_E(bf16_t, false) }
      } else {
        if (stage) { SKINNY_E(float, true) } else { SKINNY_E(float, false) }
      }
#undef SKINNY_E
#undef SKINNY
    } else {
      if (fsp) return 1;
      // k-groups per workgroup: about 1024 four-wave groups on the chip
      const int64_t tiles = cdiv(T_, kRtT) * cdiv(E, kRtE);
      const int kg = tiles >= 1024 ? 1 : (tiles >= 512 ? 2 : 4);
      dim3 grid((unsigned)cdiv(T_, kRtT), (unsigned)cdiv(E, kRtE));
#define RT(TV, KGV)                                                                        \
  MOE_LAUNCH("router_logits", (router_tiled_kernel<TV, KGV>), grid, dim3(256 * KGV), 0, st, \
             (const TV*)x, wr, rb, logits, T_, D, E)
      if (c.dtype == MOE_BF16) {
        if (kg == 1) RT(bf16_t, 1); else if (kg == 2) RT(bf16_t, 2); else RT(bf16_t, 4);
      } else {
        if (kg == 1) RT(float, 1); else if (kg == 2) RT(float, 2); else RT(float, 4);
      }
#undef RT
    }
  }
  return MOE_OK;
}

int router_logits(const moe_config& c, const void* x, const float* wr, const float* rb,
                  float* logits, hipStream_t st) {
  return router_logits_sel(c, x, wr, rb, logits, nullptr, st);
}

int launch_route(const moe_config& c, const void* x, const float* wr, const float* rb,
                 const float* selb, const float* jit, const float* wn, const float* eps,
                 float* nlg, float* logits, int32_t* idx, float* w, float* lse, bool logits_given,
                 hipStream_t st) {
  const int T_ = c.T, E = c.E;
  const int K = c.K, sc = c.score_fn, ga = c.gating;
  const float* sb = (sc == MOE_SCORE_SIGMOID) ? selb : nullptr;
  int rc;
  if (!logits_given && !jit && !wn) {
    // plain routing: the few-expert router selects in the same kernel
    const FusedSelect fs = {sb, idx, w, lse, K, sc, ga};
    rc = router_logits_sel(c, x, wr, rb, logits, &fs, st);
    if (rc <= 0) return rc;
  }
  if (!logits_given && (rc = router_logits(c, x, wr, rb, logits, st))) return rc;
  if (wn && (rc = router_logits(c, x, wn, nullptr, nlg, st))) return rc;
  const SelectExtras xs = {jit, wn ? eps : nullptr, wn ? nlg : nullptr};
#define SEL(Lv, Ev) return launch_select<Lv, Ev>(logits, sb, xs, T_, E, K, sc, ga, idx, w, lse, st)
  if (E <= 1) SEL(1, 1);
  if (E <= 2) SEL(2, 1);
  if (E <= 4) SEL(4, 1);
  if (E <= 8) SEL(8, 1);
  if (E <= 16) SEL(16, 1);
  if (E <= 32) SEL(32, 1);
  if (E <= 64) SEL(64, 1);
  if (E <= 128) SEL(64, 2);
  if (E <= 256) SEL(64, 4);
  if (E <= 512) SEL(64, 8);
  SEL(64, 16);
#undef SEL
}

}  // namespace moe
