// combine.hip -- weighted combine back to token order, its backward, and the
// un-permute reduction of the row gradients.
//
// [P5] course notes 8.8: after the expert matmuls the outputs are multiplied
// by their gate weights and scattered back with index_add -- a token appears
// once per selected expert, so its contributions accumulate; 8.7: the shared
// expert is added with weight 1.  [P1] cause section: the gradient of a gate
// weight is the expert output (proj_out) of that slot, which is zero for a
// slot this device does not serve (sentinel) -- and, by the same rule, for a
// dropped slot.
//
// All three kernels are HBM-bound row streams, one wave per token: 16-byte
// vector loads, fp32 accumulation in a fixed k order (no atomics,
// deterministic).
#include "common.h"
#include "kernels.h"

namespace moe {

// y[t] = sum_k [row>=0] g[t,k] * o[row] + o[shared row of t]; one wave per
// token, lanes stride over the row's 16-byte vectors.  The slots are taken in
// chunks of 64 (lane k holds slot k0+k's row and weight); a ballot of the
// taken slots skips the dropped, sentinel and (expert choice) untaken ones,
// and the kept slots are added in increasing k.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ o,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ offsets,
                                                      int EL, int n_shared, int T_, int K, int D,
                                                      T* __restrict__ y) {
  constexpr int VEC = Elem<T>::VEC;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  const int64_t srow = n_shared ? (int64_t)offsets[EL] + t : -1;
  // the first chunk (all slots when K <= 64) stays in registers over the
  // row.  The d loop runs on the whole wave (lanes past D only skip their
  // loads and stores) so that every ballot and shuffle sees all 64 slots.
  const int row0 = lane < K ? slot_row[(size_t)t * K + lane] : -1;
  const float g0 = lane < K ? topk_w[(size_t)t * K + lane] : 0.f;
  const uint64_t m0 = __ballot(row0 >= 0);
  for (int db = 0; db < D; db += 64 * VEC) {
    const int d0 = db + lane * VEC;
    const bool dok = d0 < D;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 64) {
      const int kk = k0 + lane;
      const int my_row = k0 == 0 ? row0 : (kk < K ? slot_row[(size_t)t * K + kk] : -1);
      const float my_g = k0 == 0 ? g0 : (kk < K ? topk_w[(size_t)t * K + kk] : 0.f);
      for (uint64_t m = k0 == 0 ? m0 : __ballot(my_row >= 0); m; m &= m - 1) {
        const int k = __builtin_ctzll(m);
        const int row = __shfl(my_row, k, 64);
        const float g = __shfl(my_g, k, 64);
        if (!dok) continue;
        Vec16<T> v;
        v.load(o + (size_t)row * D + d0);
        float f[VEC];
        v.to_f32(f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = fmaf(g, f[i], acc[i]);
      }
    }
    if (!dok) continue;
    if (srow >= 0) {
      Vec16<T> v;
      v.load(o + (size_t)srow * D + d0);
      float f[VEC];
      v.to_f32(f);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += f[i];
    }
    Vec16<T> out;
    out.from_f32(acc);
    out.store(y + (size_t)t * D + d0);
  }
}

// one wave per token: dg[t,k] = dy_t . o[row] (0 for sentinel / dropped /
// untaken slots), d_o[row] = g[t,k] * dy_t; slots in chunks of 64 as in the
// combine
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ o,
                                                          const T* __restrict__ dy,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ topk_w,
                                                          int T_, int K, int D,
                                                          float* __restrict__ dg,
                                                          T* __restrict__ d_o) {
  constexpr int VEC = Elem<T>::VEC;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int kk = k0 + lane;
    const int my_row = kk < K ? slot_row[(size_t)t * K + kk] : -1;
    const float my_g = kk < K ? topk_w[(size_t)t * K + kk] : 0.f;
    if (kk < K && my_row < 0) dg[(size_t)t * K + kk] = 0.f;
    for (uint64_t m = __ballot(my_row >= 0); m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const int row = __shfl(my_row, k, 64);
      const float g = __shfl(my_g, k, 64);
      float dot = 0.f;
      for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
        Vec16<T> vy, vo;
        vy.load(dy + (size_t)t * D + d0);
        vo.load(o + (size_t)row * D + d0);
        float fy[VEC], fo[VEC], fd[VEC];
        vy.to_f32(fy);
        vo.to_f32(fo);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          dot = fmaf(fy[i], fo[i], dot);
          fd[i] = g * fy[i];
        }
        Vec16<T> vd;
        vd.from_f32(fd);
        vd.store(d_o + (size_t)row * D + d0);
      }
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) dot += __shfl_xor(dot, mm, 64);
      if (lane == 0) dg[(size_t)t * K + k0 + k] = dot;
    }
  }
}

// Few slots per token (slot width <= KM <= 8): the same combine with the
// slot table read as wave-uniform scalars and, per 16-byte column chunk,
// every kept slot's row load issued before any is added (an unused slot
// re-reads row 0 and is not added); TPW consecutive tokens per wave.  Same
// terms in the same order as combine_kernel.
template <typename T, int KM, int TPW>
__global__ __launch_bounds__(256) void combine_few_kernel(const T* __restrict__ o,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ topk_w,
                                                          const int32_t* __restrict__ offsets,
                                                          int EL, int n_shared, int T_, int K,
                                                          int D, T* __restrict__ y) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int t0 = __builtin_amdgcn_readfirstlane((blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW);
  if (t0 >= T_) return;
  int rows[TPW][KM];
  float gk[TPW][KM];
  int64_t srow[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = t0 + j;
    const bool tv = t < T_;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      const bool ok = tv && k < K;
      rows[j][k] = ok ? slot_row[(size_t)t * K + k] : -1;
      gk[j][k] = ok ? topk_w[(size_t)t * K + k] : 0.f;
    }
    srow[j] = (tv && n_shared) ? (int64_t)offsets[EL] + t : -1;
  }
  for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
    Vec16<T> v[TPW][KM], vs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
#pragma unroll
      for (int k = 0; k < KM; ++k)
        v[j][k].load(o + (size_t)(rows[j][k] >= 0 ? rows[j][k] : 0) * D + d0);
      if (n_shared) vs[j].load(o + (size_t)(srow[j] >= 0 ? srow[j] : 0) * D + d0);
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if (t0 + j >= T_) continue;
      float acc[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (rows[j][k] >= 0) {
          float f[VEC];
          v[j][k].to_f32(f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] = fmaf(gk[j][k], f[i], acc[i]);
        }
      if (srow[j] >= 0) {
        float f[VEC];
        vs[j].to_f32(f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += f[i];
      }
      Vec16<T> out;
      out.from_f32(acc);
      out.store(y + (size_t)(t0 + j) * D + d0);
    }
  }
}

// Few slots per token: combine backward for all of a token's slots in one
// pass over the row (dy read once per chunk, every slot's row load in flight
// together), per-slot lane partials of the dot in the same order as
// combine_bwd_kernel, then the same shuffle tree.
template <typename T, int KM>
__global__ __launch_bounds__(256) void combine_bwd_few_kernel(const T* __restrict__ o,
                                                              const T* __restrict__ dy,
                                                              const int32_t* __restrict__ slot_row,
                                                              const float* __restrict__ topk_w,
                                                              int T_, int K, int D,
                                                              float* __restrict__ dg,
                                                              T* __restrict__ d_o) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T_) return;
  int rows[KM];
  float gk[KM], dot[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    rows[k] = k < K ? slot_row[(size_t)t * K + k] : -1;
    gk[k] = k < K ? topk_w[(size_t)t * K + k] : 0.f;
    dot[k] = 0.f;
  }
  for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
    Vec16<T> vy, vo[KM];
    vy.load(dy + (size_t)t * D + d0);
#pragma unroll
    for (int k = 0; k < KM; ++k) vo[k].load(o + (size_t)(rows[k] >= 0 ? rows[k] : 0) * D + d0);
    float fy[VEC];
    vy.to_f32(fy);
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (rows[k] < 0) continue;
      float fo[VEC], fd[VEC];
      vo[k].to_f32(fo);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        dot[k] = fmaf(fy[i], fo[i], dot[k]);
        fd[i] = gk[k] * fy[i];
      }
      Vec16<T> vd;
      vd.from_f32(fd);
      vd.store(d_o + (size_t)rows[k] * D + d0);
    }
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= K) break;
    float v = 0.f;
    if (rows[k] >= 0) {
      v = dot[k];
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) v += __shfl_xor(v, mm, 64);
    }
    if (lane == 0) dg[(size_t)t * K + k] = v;
  }
}

// dx[t] = sum_k [row>=0] dx_perm[row] + dx_perm[shared row of t]
//         + router part: sum_e ds[t,e] W_r[e,:] (inline for E <= EM) or dxr[t]
// one wave per token, lanes stride over 16-byte vectors of the row; slots in
// chunks of 64 as in the combine
template <typename T, int EM>
__global__ __launch_bounds__(256) void unpermute_kernel(
    const T* __restrict__ dxp, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ offsets, int EL, int n_shared, const float* __restrict__ ds,
    const float* __restrict__ wr, int E, const float* __restrict__ dxr, int T_, int K, int D,
    T* __restrict__ dx) {
  constexpr int VEC = Elem<T>::VEC;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  const int64_t srow = n_shared ? (int64_t)offsets[EL] + t : -1;
  const int row0 = lane < K ? slot_row[(size_t)t * K + lane] : -1;
  const uint64_t m0 = __ballot(row0 >= 0);
  float s_e[EM > 0 ? EM : 1];
  if constexpr (EM > 0) {
#pragma unroll
    for (int e = 0; e < EM; ++e) s_e[e] = (e < E) ? ds[(size_t)t * E + e] : 0.f;
  }
  for (int db = 0; db < D; db += 64 * VEC) {
    const int d0 = db + lane * VEC;
    const bool dok = d0 < D;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 64) {
      const int kk = k0 + lane;
      const int my_row = k0 == 0 ? row0 : (kk < K ? slot_row[(size_t)t * K + kk] : -1);
      for (uint64_t m = k0 == 0 ? m0 : __ballot(my_row >= 0); m; m &= m - 1) {
        const int row = __shfl(my_row, __builtin_ctzll(m), 64);
        if (!dok) continue;
        Vec16<T> v;
        v.load(dxp + (size_t)row * D + d0);
        float f[VEC];
        v.to_f32(f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += f[i];
      }
    }
    if (!dok) continue;
    if (srow >= 0) {
      Vec16<T> v;
      v.load(dxp + (size_t)srow * D + d0);
      float f[VEC];
      v.to_f32(f);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += f[i];
    }
    if constexpr (EM > 0) {
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        if (e < E) {
          const float* w = wr + (size_t)e * D + d0;
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] = fmaf(s_e[e], w[i], acc[i]);
        }
      }
    } else {
      const float* r = dxr + (size_t)t * D + d0;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += r[i];
    }
    Vec16<T> out;
    out.from_f32(acc);
    out.store(dx + (size_t)t * D + d0);
  }
}

// The same sums for few slots per token (slot width <= KM <= 8): each wave
// takes TPW consecutive tokens (1, or 8 / KM for long batches); per 16-byte
// column chunk it issues the row
// loads of every kept slot of its tokens before adding any (so they are in
// flight together) and reads each router-weight chunk once for its TPW
// tokens.  Terms are added in the order of unpermute_kernel (kept slots in
// increasing k, the shared row, then the router part), so the results are
// identical.
template <typename T, int EM, int KM, int TPW>
__global__ __launch_bounds__(256) void unpermute_few_kernel(
    const T* __restrict__ dxp, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ offsets, int EL, int n_shared, const float* __restrict__ ds,
    const float* __restrict__ wr, int E, const float* __restrict__ dxr, int T_, int K, int D,
    T* __restrict__ dx) {
  constexpr int VEC = Elem<T>::VEC;
  const int lane = threadIdx.x & 63;
  // wave-uniform token index (scalar loads of the slot table and ds)
  const int t0 = __builtin_amdgcn_readfirstlane((blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW);
  if (t0 >= T_) return;
  int rows[TPW][KM];
  int64_t srow[TPW];
  float s_e[TPW][EM > 0 ? EM : 1];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = t0 + j;
    const bool tv = t < T_;
#pragma unroll
    for (int k = 0; k < KM; ++k) rows[j][k] = (tv && k < K) ? slot_row[(size_t)t * K + k] : -1;
    srow[j] = (tv && n_shared) ? (int64_t)offsets[EL] + t : -1;
    if constexpr (EM > 0) {
#pragma unroll
      for (int e = 0; e < EM; ++e) s_e[j][e] = (tv && e < E) ? ds[(size_t)t * E + e] : 0.f;
    }
  }
  for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
    // every load is issued (an unused slot re-reads row 0 of the row buffer
    // and is not added), so that none waits for another; the router weights
    // come in groups of four experts (experts past E re-read expert 0 and are
    // not added), the first group together with the rows
    float w[4][VEC];
    auto load_w = [&](int e0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u;
        const float4* wp = reinterpret_cast<const float4*>(wr + (size_t)(e < E ? e : 0) * D + d0);
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
          const float4 f4 = wp[q];
          w[u][4 * q] = f4.x; w[u][4 * q + 1] = f4.y; w[u][4 * q + 2] = f4.z; w[u][4 * q + 3] = f4.w;
        }
      }
    };
    Vec16<T> v[TPW][KM], vs[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
#pragma unroll
      for (int k = 0; k < KM; ++k)
        v[j][k].load(dxp + (size_t)(rows[j][k] >= 0 ? rows[j][k] : 0) * D + d0);
      if (n_shared) vs[j].load(dxp + (size_t)(srow[j] >= 0 ? srow[j] : 0) * D + d0);
    }
    if constexpr (EM > 0) load_w(0);
    float acc[TPW][VEC];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[j][i] = 0.f;
#pragma unroll
      for (int k = 0; k < KM; ++k)
        if (rows[j][k] >= 0) {
          float f[VEC];
          v[j][k].to_f32(f);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[j][i] += f[i];
        }
      if (srow[j] >= 0) {
        float f[VEC];
        vs[j].to_f32(f);
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[j][i] += f[i];
      }
    }
    if constexpr (EM > 0) {
#pragma unroll
      for (int e0 = 0; e0 < EM; e0 += 4) {
        if (e0 > 0) load_w(e0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (e0 + u < E) {
#pragma unroll
            for (int j = 0; j < TPW; ++j)
#pragma unroll
              for (int i = 0; i < VEC; ++i) acc[j][i] = fmaf(s_e[j][e0 + u], w[u][i], acc[j][i]);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        if (t0 + j >= T_) continue;
        const float* r = dxr + (size_t)(t0 + j) * D + d0;
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[j][i] += r[i];
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if (t0 + j >= T_) continue;
      Vec16<T> out;
      out.from_f32(acc[j]);
      out.store(dx + (size_t)(t0 + j) * D + d0);
    }
  }
}

template <typename T>
static int combine_few(const moe_config& c, const void* o_perm, const int32_t* offsets,
                       const int32_t* slot_row, const float* topk_w, void* y, hipStream_t st) {
  const int EL = c.expert_hi - c.expert_lo, W = slot_width(c);
#define CF1(KMV, TPWV)                                                                     \
  MOE_LAUNCH("combine", (combine_few_kernel<T, KMV, TPWV>), dim3((unsigned)cdiv(c.T, 4 * TPWV)), \
             dim3(256), 0, st, (const T*)o_perm, slot_row, topk_w, offsets, EL, c.n_shared,    \
             c.T, W, c.D, (T*)y)
#define CF(KMV)                                                    \
  if (KMV < 8 && c.T >= 4096 * (8 / KMV)) CF1(KMV, 8 / KMV);         \
  else CF1(KMV, 1);
  if (W <= 2) { CF(2) } else if (W <= 4) { CF(4) } else { CF(8) }
#undef CF
#undef CF1
  return MOE_OK;
}

template <typename T>
static int combine_bwd_few(const moe_config& c, const void* o_perm, const void* dy,
                           const int32_t* slot_row, const float* topk_w, float* dg, void* d_o,
                           hipStream_t st) {
  const int W = slot_width(c);
  const dim3 grid((unsigned)cdiv(c.T, 4));
#define CB(KMV)                                                                               \
  MOE_LAUNCH("combine_bwd", (combine_bwd_few_kernel<T, KMV>), grid, dim3(256), 0, st,         \
             (const T*)o_perm, (const T*)dy, slot_row, topk_w, c.T, W, c.D, dg, (T*)d_o)
  if (W <= 2) CB(2); else if (W <= 4) CB(4); else CB(8);
#undef CB
  return MOE_OK;
}

int launch_combine(const moe_config& c, const void* o_perm, const int32_t* offsets,
                   const int32_t* slot_row, const float* topk_w, void* y, hipStream_t st) {
  if (slot_width(c) <= 8) {
    if (c.dtype == MOE_BF16)
      return combine_few<bf16_t>(c, o_perm, offsets, slot_row, topk_w, y, st);
    return combine_few<float>(c, o_perm, offsets, slot_row, topk_w, y, st);
  }
  const int EL = c.expert_hi - c.expert_lo;
  const int grid = (int)cdiv(c.T, 4);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH("combine", combine_kernel<bf16_t>, dim3(grid), dim3(256), 0, st,
               (const bf16_t*)o_perm, slot_row, topk_w, offsets, EL, c.n_shared, c.T, slot_width(c), c.D,
               (bf16_t*)y);
  else
    MOE_LAUNCH("combine", combine_kernel<float>, dim3(grid), dim3(256), 0, st,
               (const float*)o_perm, slot_row, topk_w, offsets, EL, c.n_shared, c.T, slot_width(c), c.D,
               (float*)y);
  return MOE_OK;
}

int launch_combine_bwd(const moe_config& c, const void* o_perm, const void* dy,
                       const int32_t* slot_row, const float* topk_w, float* dg, void* d_o,
                       hipStream_t st) {
  if (slot_width(c) <= 8) {
    if (c.dtype == MOE_BF16)
      return combine_bwd_few<bf16_t>(c, o_perm, dy, slot_row, topk_w, dg, d_o, st);
    return combine_bwd_few<float>(c, o_perm, dy, slot_row, topk_w, dg, d_o, st);
  }
  const int grid = (int)cdiv(c.T, 4);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH("combine_bwd", combine_bwd_kernel<bf16_t>, dim3(grid), dim3(256), 0, st,
               (const bf16_t*)o_perm, (const bf16_t*)dy, slot_row, topk_w, c.T, slot_width(c), c.D, dg,
               (bf16_t*)d_o);
  else
    MOE_LAUNCH("combine_bwd", combine_bwd_kernel<float>, dim3(grid), dim3(256), 0, st,
               (const float*)o_perm, (const float*)dy, slot_row, topk_w, c.T, slot_width(c), c.D, dg,
               (float*)d_o);
  return MOE_OK;
}

template <typename T>
static int unpermute_t(const moe_config& c, const void* dxp, const int32_t* slot_row,
                       const int32_t* offsets, const float* ds, const float* wr,
                       const float* dxr, void* dx, hipStream_t st) {
  const int EL = c.expert_hi - c.expert_lo;
  const int E = c.E, W = slot_width(c);
  if (W <= 8) {
    // few slots per token: KM slots; 8 / KM tokens per wave when that still
    // leaves at least 4096 waves, else one
#define UNPERM_FEW1(EMV, KMV, TPWV)                                                           \
  MOE_LAUNCH("unpermute_dx", (unpermute_few_kernel<T, EMV, KMV, TPWV>),                       \
             dim3((unsigned)cdiv(c.T, 4 * TPWV)), dim3(256), 0, st, (const T*)dxp, slot_row,  \
             offsets, EL, c.n_shared, ds, wr, E, dxr, c.T, W, c.D, (T*)dx)
#define UNPERM_FEW(EMV, KMV)                                            \
  if (KMV < 8 && c.T >= 4096 * (8 / KMV)) UNPERM_FEW1(EMV, KMV, 8 / KMV); \
  else UNPERM_FEW1(EMV, KMV, 1);
#define UNPERM_FEW_K(EMV)                   \
  if (W <= 2) { UNPERM_FEW(EMV, 2) }        \
  else if (W <= 4) { UNPERM_FEW(EMV, 4) }   \
  else { UNPERM_FEW(EMV, 8) }
    if (dxr) { UNPERM_FEW_K(0) }
    else if (E <= 4) { UNPERM_FEW_K(4) }
    else if (E <= 8) { UNPERM_FEW_K(8) }
    else { UNPERM_FEW_K(16) }
#undef UNPERM_FEW_K
#undef UNPERM_FEW
#undef UNPERM_FEW1
    return MOE_OK;
  }
  const int grid = (int)cdiv(c.T, 4);
#define UNPERM(EMV)                                                                          \
  MOE_LAUNCH("unpermute_dx", (unpermute_kernel<T, EMV>), dim3(grid), dim3(256), 0, st,        \
             (const T*)dxp, slot_row, offsets, EL, c.n_shared, ds, wr, E, dxr, c.T, W, c.D, \
             (T*)dx)
  if (dxr) UNPERM(0);
  else if (E <= 4) UNPERM(4);
  else if (E <= 8) UNPERM(8);
  else UNPERM(16);
#undef UNPERM
  return MOE_OK;
}

int launch_unpermute(const moe_config& c, const void* dxp, const int32_t* slot_row,
                     const int32_t* offsets, const float* ds, const float* wr, const float* dxr,
                     void* dx, hipStream_t st) {
  if (c.dtype == MOE_BF16)
    return unpermute_t<bf16_t>(c, dxp, slot_row, offsets, ds, wr, dxr, dx, st);
  return unpermute_t<float>(c, dxp, slot_row, offsets, ds, wr, dxr, dx, st);
}

}  // namespace moe
