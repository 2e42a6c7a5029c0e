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

// Few-expert router (E <= 16).  LPT lanes per token (8, or 16 for short
// batches): lane p of a token reads 16-byte vectors p, p + LPT, ... of each
// slab of the token's row (LPT lanes read 16 LPT contiguous bytes of a row
// per load instruction), so a lane's fp64 partial sums need only a
// reduction over its LPT lanes (DPP steps, no LDS traffic) instead of one
// over the whole wave.  Each lane works on TPL tokens (the same columns of
// TPL rows).  W_r goes through LDS in slabs of kFewSlab columns, widened to
// double once when staged and zero past E and D, so the products run over
// whole slabs and all EM experts without a branch (a branch per expert kept
// the compiler from issuing the next expert's LDS reads early: 81 -> 69 us
// on the Mixtral-like layer without it); double-buffered, one barrier per
// slab.  W_r is read from L2 once per workgroup, any D works, and the
// stripes of a wave read distinct 16-byte LDS words per instruction
// (few_swz spreads them over the banks).  The x vectors of slab s + 1 and
// the W_r values of slab s + 2 are loaded while slab s is multiplied, into
// registers that alternate between even and odd slabs, so no slab waits for
// a load it issued itself (with register copies at the end of each slab,
// every slab waited for them).  Workgroups start at different slabs.  Lane
// 0 of each token takes the top-K when fs.idx is set.
constexpr int kFewSlab = 256;  // columns per W_r slab

// sum over the eight lanes of a token (lanes 8j .. 8j + 7): pairs, quads,
// then the two quads of the half-row; every lane ends with the same bits
template <int CTRL>
MOE_DEV double dpp_d(double v) {
  const int2 u = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(0, u.x, CTRL, 0xF, 0xF, false);
  r.y = __builtin_amdgcn_update_dpp(0, u.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}
template <int LPT>
MOE_DEV double sum_lanes(double v) {
  v += dpp_d<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_d<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_d<0x141>(v);  // row_half_mirror
  if constexpr (LPT == 16) v += dpp_d<0x140>(v);  // row_mirror
  return v;
}
// LDS slot of double pair L of a staged slab: the stripes read pairs 4 apart
// (bf16 rows), so stripes p, p + 4, p + 8, p + 12 would share banks;
// permuting the four pairs of a stripe by (L >> 4) & 3 separates them
MOE_DEV int few_swz(int L) { return L ^ ((L >> 4) & 3); }

// logits, then (fs.idx set, lane 0 of the token) top-K, weights and lse of
// token t from its fp64 sums
template <int EM, int LPT>
MOE_DEV void few_finish(const double* acc, int t, int p, int E, const float* __restrict__ rb,
                        float* __restrict__ logits, const FusedSelect& fs, int32_t* s_pick) {
  // logits: lane p stores experts p, p + LPT, ...
#pragma unroll
  for (int h = 0; h < EM; h += LPT) {
    const int e = h + p;
    if (e < E) {
      double a = 0.0;
#pragma unroll
      for (int f = 0; f < EM; ++f)
        if (f == e) a = acc[f];
      logits[(size_t)t * E + e] = (float)(a + (rb ? (double)rb[e] : 0.0));
    }
  }
  if (!fs.idx || p != 0) return;
  float sv[EM], key[EM];
  bool used[EM];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const bool ok = e < E;
    sv[e] = ok ? (float)(acc[e] + (rb ? (double)rb[e] : 0.0)) : -INFINITY;
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
  // K <= E <= EM rounds; the weights stay in registers until the normaliser
  // is known
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
    if (s_pick) s_pick[k] = ik[k];
  }
}

// The permute of the same slots folded into the few-expert router (fewer
// launches; [P3] efficient inference: group the tokens by expert; [P5] 8.5
// capacity).  Every router workgroup ranks its own slots per expert in slot
// order (ballots per 64-slot group, then the groups before it) and stores
// its per-expert counts; scatter_slots_kernel, the next launch, adds the
// counts of the router workgroups before a slot's own to its rank, forms
// the capacity-limited group offsets from all counts, gives every slot its
// row and moves its token's row of x.  The positions are the stable
// in-expert ranks of moe_permute, so every output is identical.  (Letting
// the router's last workgroup -- found by an atomic counter -- do the scan
// put a device-scope fence in every workgroup and a serial tail on the
// router: MiniMind 26 us against 17 us without it.)
struct FusedPermute {
  int32_t* wg_counts;   // [router workgroups][E] slots per expert
  int32_t* local_rank;  // [T K] rank of a slot among its workgroup's slots of its expert
  int K, nbits;
};
constexpr int kFoldWgs = 1024;  // router workgroups the folded permute takes

// the router workgroup's slots: tokens blockIdx.x TPW ..., K each, their
// experts in s_pick
MOE_DEV void fold_permute(const FusedPermute& fp, const int32_t* s_pick, int TPW, int T_,
                          int E) {
  __shared__ int32_t gcnt[4][16];  // slots per expert of each 64-slot group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, K = fp.K;
  if (tid < 64) gcnt[tid >> 4][tid & 15] = 0;
  __syncthreads();
  const int tb = blockIdx.x * TPW;
  const int nslots = min(TPW, T_ - tb) * K;  // <= 256
  const bool v = tid < nslots;
  const int e = v ? s_pick[tid] : 0;
  const uint64_t peers = same_expert_peers(v, e, fp.nbits);
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  if (v && (63 - __clzll(peers)) == lane) gcnt[wave][e] = __popcll(peers);
  __syncthreads();
  if (v) {
    int r = __popcll(peers & lt);
    for (int w = 0; w < wave; ++w) r += gcnt[w][e];
    fp.local_rank[(size_t)tb * K + tid] = r;
  }
  if (tid < E) fp.wg_counts[(size_t)blockIdx.x * E + tid] =
      gcnt[0][tid] + gcnt[1][tid] + gcnt[2][tid] + gcnt[3][tid];
}

// The rows of the folded permute.  A workgroup takes kScatterSlots
// consecutive slots (all of one router workgroup g): it sums the counts of
// the router workgroups before g (the slots' bases) and of all of them (the
// totals, hence the group offsets) per expert, then every wave takes a slot
// at a time: slot_row -2 for an expert outside [lo, hi), -1 past its
// expert's capacity, else row = offset + base + rank, with the token's row
// of x moved to x_perm.  Workgroup 0 also writes counts_all, offsets and
// n_dropped.  tpw: tokens per router workgroup.
constexpr int kScatterSlots = 16;
template <typename T>
__global__ __launch_bounds__(256) void scatter_slots_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ wg_counts, const int32_t* __restrict__ local_rank, int nwg,
    int tpw, int TK, int K, int E, int lo, int hi, int capacity, int n_shared, int T_, int D,
    int32_t* __restrict__ counts_all, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot, T* __restrict__ x_perm) {
  constexpr int VEC = Elem<T>::VEC;
  __shared__ int32_t part[4][2][16];
  __shared__ int32_t base[16], off[17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = blockIdx.x * kScatterSlots;
  const int g = (s0 / K) / tpw;
  // per expert: counts of the router workgroups before g, and of all
  int pre[16], tot[16];
#pragma unroll
  for (int x2 = 0; x2 < 16; ++x2) { pre[x2] = 0; tot[x2] = 0; }
  for (int h = tid; h < nwg; h += 256) {
#pragma unroll
    for (int x2 = 0; x2 < 16; ++x2) {
      if (x2 < E) {
        const int c = wg_counts[(size_t)h * E + x2];
        tot[x2] += c;
        pre[x2] += h < g ? c : 0;
      }
    }
  }
#pragma unroll
  for (int x2 = 0; x2 < 16; ++x2) {
    if (x2 < E) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        pre[x2] += __shfl_xor(pre[x2], o, 64);
        tot[x2] += __shfl_xor(tot[x2], o, 64);
      }
      if (lane == 0) { part[wave][0][x2] = pre[x2]; part[wave][1][x2] = tot[x2]; }
    }
  }
  __syncthreads();
  if (tid < E) base[tid] = part[0][0][tid] + part[1][0][tid] + part[2][0][tid] + part[3][0][tid];
  if (tid == 0) {
    const int EL = hi - lo;
    int r = 0, drop = 0;
    for (int x2 = 0; x2 < E; ++x2) {
      const int n = part[0][1][x2] + part[1][1][x2] + part[2][1][x2] + part[3][1][x2];
      if (blockIdx.x == 0) counts_all[x2] = n;
      if (x2 >= lo && x2 < hi) {
        const int k = (capacity >= 0 && n > capacity) ? capacity : n;
        off[x2 - lo] = r;
        r += k;
        drop += n - k;
      }
    }
    off[EL] = r;
    if (blockIdx.x == 0) {
      for (int x2 = 0; x2 <= EL; ++x2) offsets[x2] = off[x2];
      for (int sh = 0; sh < n_shared; ++sh) offsets[EL + 1 + sh] = r + (sh + 1) * T_;
      *n_dropped = drop;
    }
  }
  __syncthreads();
  for (int i = wave; i < kScatterSlots; i += 4) {
    const int s = s0 + i;
    if (s >= TK) break;
    const int e = idx[s];
    const int tok = s / K;
    const int pos = base[e] + local_rank[s];
    int row = -1;
    if (e < lo || e >= hi) {
      if (lane == 0) slot_row[s] = -2;
    } else if (capacity >= 0 && pos >= capacity) {
      if (lane == 0) slot_row[s] = -1;
    } else {
      row = off[e - lo] + pos;
      if (lane == 0) {
        slot_row[s] = row;
        row_token[row] = tok;
        row_slot[row] = s;
      }
    }
    if (row < 0) continue;
    const T* src = x + (size_t)tok * D;
    T* dst = x_perm + (size_t)row * D;
    for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
      Vec16<T> v;
      v.load(src + d0);
      v.store(dst + d0);
    }
  }
}

template <typename T, int EM, int TPL, int LPT>
__global__ __launch_bounds__(256) void router_few_kernel(const T* __restrict__ x,
                                                         const float* __restrict__ wr,
                                                         const float* __restrict__ rb,
                                                         float* __restrict__ logits, int T_,
                                                         int D, int E, FusedSelect fs,
                                                         FusedPermute fp) {
  static_assert(TPL == 1, "the folded permute takes one token per lane");
  constexpr int VEC = Elem<T>::VEC;            // elements per 16-byte vector
  constexpr int NJ = kFewSlab / (LPT * VEC);   // vectors per lane and row per full slab
  constexpr int TPW = 256 / LPT;               // tokens per workgroup and TPL step
  constexpr int WQ = EM * kFewSlab / 4 / 256;  // float4 of a W_r slab per thread
  constexpr int QR = kFewSlab / 4;             // float4 per expert row of a slab
  __shared__ double2 sw[2][EM * kFewSlab / 2];  // [e][column pair], few_swz order
  __shared__ int32_t s_pick[256];                 // folded permute: the slots' experts
  const int tid = threadIdx.x, lane = tid & 63;
  const int p = lane & (LPT - 1);
  // token i of this lane: block base + TPW i + tid / LPT
  const int t0 = blockIdx.x * (TPW * TPL) + tid / LPT;
  const T* xrow[TPL];
#pragma unroll
  for (int i = 0; i < TPL; ++i) {
    const int t = t0 + TPW * i;
    // rows past the end re-read the last row (discarded): no load is guarded
    xrow[i] = x + (size_t)(t < T_ ? t : T_ - 1) * D;
  }
  const int nslab = (D + kFewSlab - 1) / kFewSlab;
  // workgroups start at different slabs (pass k covers slab (k + rot) mod
  // nslab), so the column ranges read at one time differ across the chip
  const int rot = blockIdx.x % nslab;
  auto phys = [&](int k) __attribute__((always_inline)) {
    const int q = k + rot;
    return q >= nslab ? q - nslab : q;
  };

  // W_r slab s -> registers: float4 q of the slab is expert q / QR, columns
  // 4 (q % QR) .. +3; experts past E and columns past D are zero (the load
  // reads row 0 and is discarded), so the products run over all EM experts
  // and whole slabs without a branch: a zero W_r times a finite x adds
  // nothing, and the unused sums are never read
  auto load_w = [&](int k, float4* wv) __attribute__((always_inline)) {
    const int s = phys(k);
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      const int q = u * 256 + tid, e = q / QR, c = s * kFewSlab + 4 * (q % QR);
      const bool ok = e < E && c < D;
      const float4 v = *reinterpret_cast<const float4*>(wr + (ok ? (size_t)e * D + c : 0));
      wv[u] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_w = [&](int buf, const float4* wv) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < WQ; ++u) {
      const int q = u * 256 + tid;
      sw[buf][few_swz(2 * q)] = make_double2((double)wv[u].x, (double)wv[u].y);
      sw[buf][few_swz(2 * q + 1)] = make_double2((double)wv[u].z, (double)wv[u].w);
    }
  };
  // x vectors of slab s (columns past D re-read column 0: their W_r is zero)
  auto load_x = [&](int k, Vec16<T> (*xv)[NJ]) __attribute__((always_inline)) {
    const int s = phys(k);
#pragma unroll
    for (int i = 0; i < TPL; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = s * kFewSlab + (j * LPT + p) * VEC;
        xv[i][j].load(xrow[i] + (c < D ? c : 0));
      }
  };

  double acc[TPL][EM];
#pragma unroll
  for (int i = 0; i < TPL; ++i)
#pragma unroll
    for (int e = 0; e < EM; ++e) acc[i][e] = 0.0;
  // Register buffers alternate between even and odd slabs (the loop runs
  // two slabs per pass), so no register copy waits for a load in flight.
  float4 w0[WQ], w1[WQ];
  Vec16<T> x0[TPL][NJ], x1[TPL][NJ];
  load_w(0, w0);
  load_x(0, x0);
  if (nslab > 1) load_w(1, w1);
  store_w(0, w0);
  // slab s: its x vectors in xc (loaded one slab earlier), W_r slab s + 1 in
  // wst (loaded two slabs earlier); x of slab s + 1 goes into xn and W_r of
  // slab s + 2 into wld
  auto slab = [&](int s, Vec16<T> (*xc)[NJ], Vec16<T> (*xn)[NJ], const float4* wst, float4* wld)
                  __attribute__((always_inline)) {
    // W_r slab s is in sw[s & 1]; every wave is done with slab s - 1
    __syncthreads();
    if (s + 1 < nslab) load_x(s + 1, xn);
    if (s + 2 < nslab) load_w(s + 2, wld);
    const double2* w2 = sw[s & 1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      double xd[TPL][VEC];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        float xf[VEC];
        xc[i][j].to_f32(xf);
#pragma unroll
        for (int v = 0; v < VEC; ++v) xd[i][v] = (double)xf[v];
      }
      const int c = (j * LPT + p) * VEC;  // column within the slab
#pragma unroll
      for (int e = 0; e < EM; ++e) {
#pragma unroll
        for (int h = 0; h < VEC / 2; ++h) {
          const double2 w = w2[few_swz((e * kFewSlab + c) / 2 + h)];
#pragma unroll
          for (int i = 0; i < TPL; ++i) {
            acc[i][e] = fma(xd[i][2 * h], w.x, acc[i][e]);
            acc[i][e] = fma(xd[i][2 * h + 1], w.y, acc[i][e]);
          }
        }
      }
    }
    // slab s + 1 into the slot of slab s - 1
    if (s + 1 < nslab) store_w((s + 1) & 1, wst);
  };
  for (int s = 0; s < nslab; s += 2) {
    slab(s, x0, x1, w1, w0);
    if (s + 1 < nslab) slab(s + 1, x1, x0, w0, w1);
  }
#pragma unroll
  for (int i = 0; i < TPL; ++i) {
#pragma unroll
    for (int e = 0; e < EM; ++e) acc[i][e] = sum_lanes<LPT>(acc[i][e]);
    const int t = t0 + TPW * i;
    if (t < T_)
      few_finish<EM, LPT>(acc[i], t, p, E, rb, logits, fs,
                          fp.wg_counts ? s_pick + (tid / LPT) * fp.K : nullptr);
  }
  if (fp.wg_counts) {
    __syncthreads();
    fold_permute(fp, s_pick, TPW, T_, E);
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
// tokens per workgroup of the few-expert router (8 or 16 lanes per token)
static int few_tokens_per_wg(int T_) { return cdiv(T_, 32) < 512 ? 16 : 32; }

static int router_logits_sel(const moe_config& c, const void* x, const float* wr,
                             const float* rb, float* logits, const FusedSelect* fsp,
                             const FusedPermute* fpp, hipStream_t st) {
  const int T_ = c.T, D = c.D, E = c.E;
  {
    if (E <= 16) {
      const FusedSelect fs = fsp ? *fsp : FusedSelect{nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
      FusedPermute fp = {};
      if (fpp) fp = *fpp;
      const char* name = fsp ? "route_fused" : "router_logits";
      // One token per lane (two halved the workgroups and measured slower on
      // the Mixtral-like layer and MiniMind); eight lanes per token, or
      // sixteen (16 tokens per workgroup) when eight would leave fewer than
      // two workgroups per CU: MiniMind 14.6 -> 11.1 us, while the
      // Mixtral-like layer is faster with eight (72 against 86 us).
      const bool wide = few_tokens_per_wg(T_) == 16;
#define FEW(TV, EMV, LPTV)                                                                  \
  MOE_LAUNCH(name, (router_few_kernel<TV, EMV, 1, LPTV>), dim3((unsigned)cdiv(T_, 256 / LPTV)), \
             dim3(256), 0, st, (const TV*)x, wr, rb, logits, T_, D, E, fs, fp)
#define FEW_L(TV, EMV)            \
  if (wide) FEW(TV, EMV, 16);     \
  else FEW(TV, EMV, 8);
#define FEW_E(TV)                 \
  if (E <= 4) { FEW_L(TV, 4) }    \
  else if (E <= 8) { FEW_L(TV, 8) } \
  else { FEW_L(TV, 16) }
      if (c.dtype == MOE_BF16) { FEW_E(bf16_t) } else { FEW_E(float) }
#undef FEW_E
#undef FEW_L
#undef FEW
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
  return router_logits_sel(c, x, wr, rb, logits, nullptr, nullptr, st);
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
    rc = router_logits_sel(c, x, wr, rb, logits, &fs, nullptr, st);
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

int launch_route_permute(const moe_config& c, const void* x, const float* wr, const float* rb,
                         const float* selb, float* logits, int32_t* idx, float* w, float* lse,
                         int capacity, int32_t* counts_all, int32_t* offsets, int32_t* slot_row,
                         int32_t* row_token, int32_t* row_slot, int32_t* n_dropped,
                         void* x_perm, char* ws, const Workspace& L, hipStream_t st) {
  const int E = c.E, K = c.K;
  const int64_t TK = (int64_t)c.T * K;
  // the fold needs the few-expert router (its last workgroup does the
  // scan), at most 256 slots per workgroup, and a batch whose slots one
  // workgroup assigns quickly (the one-workgroup permute's range)
  const int tpw = few_tokens_per_wg(c.T);
  const bool fold = E <= 16 && tpw * K <= 256 && TK <= 32768 && cdiv(c.T, tpw) <= kFoldWgs;
  if (!fold) {
    int rc = launch_route(c, x, wr, rb, selb, nullptr, nullptr, nullptr, nullptr, logits, idx,
                          w, lse, false, st);
    if (rc) return rc;
    return launch_permute(c, capacity, idx, x, counts_all, offsets, slot_row, row_token,
                          row_slot, n_dropped, x_perm, ws, L, st);
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const float* sb = (c.score_fn == MOE_SCORE_SIGMOID) ? selb : nullptr;
  const FusedSelect fs = {sb, idx, w, lse, K, c.score_fn, c.gating};
  int32_t* wg_counts = reinterpret_cast<int32_t*>(ws + L.fold_counts);
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws + L.fold_rank);
  const FusedPermute fp = {wg_counts, local_rank, K, nbits};
  int rc = router_logits_sel(c, x, wr, rb, logits, &fs, &fp, st);
  if (rc) return rc;
  const int nwg = (int)cdiv(c.T, tpw);
  const dim3 grid((unsigned)cdiv(TK, kScatterSlots));
#define SCATTER(TV)                                                                           \
  MOE_LAUNCH("permute_scatter", scatter_slots_kernel<TV>, grid, dim3(256), 0, st, (const TV*)x, \
             idx, wg_counts, local_rank, nwg, tpw, (int)TK, K, E, c.expert_lo, c.expert_hi,   \
             capacity, c.n_shared, c.T, c.D, counts_all, offsets, n_dropped, slot_row,         \
             row_token, row_slot, (TV*)x_perm)
  if (c.dtype == MOE_BF16) SCATTER(bf16_t);
  else SCATTER(float);
#undef SCATTER
  return launch_shared_rows(c, offsets, row_token, row_slot, st);
}

}  // namespace moe
