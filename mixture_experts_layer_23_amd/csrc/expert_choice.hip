// expert_choice.hip -- expert-choice routing: every expert takes its C best
// tokens of the batch.
//
// [P5] course notes 8.4: instead of each token choosing experts, each expert
// chooses a fixed number of tokens; the load of every expert is then exactly
// that number, while a token can be served by several experts or by none.
// The affinity of a pair is the softmax probability p_{t,e}, which is also
// the pair's gate weight; C = min(ceil(c T K / E), T) with K the average
// number of experts per token and c the capacity factor (1 when not given).
//
// Selection key of a pair: fl32(s_{t,e} - lse_t), the log-probability
// evaluated in double from the binary32 logits and rounded once, so the
// decision does not depend on a summation order of probabilities; within one
// expert's column it orders the tokens as p does.  Equal keys go to the lower
// token.  The rows of a local expert are its C taken tokens in token order.
//
// Kernels: ec_token (one L-lane group per token: lse, p, keys, and the fixed
// offsets / counts), ec_select (one 1024-thread workgroup per local expert:
// an exact radix select of the C-th largest key over three digit passes,
// then an ordered compaction of the taken tokens with ballots and scans),
// then the shared-row maps and the x_perm gather of the token-choice path.
#include "common.h"
#include "kernels.h"

namespace moe {

// binary32 -> uint32 with the same order (larger float, larger code)
MOE_DEV uint32_t ordered_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// L lanes per token (L = min(64, pow2ceil(E))), EPL experts per lane
// (expert e = sub + L*j)
template <int L, int EPL>
__global__ __launch_bounds__(256) void ec_token_kernel(
    const float* __restrict__ logits, int T_, int E, int lo, int hi, int n_shared, int C,
    float* __restrict__ w, float* __restrict__ lse_out, uint32_t* __restrict__ keys,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ counts_all,
    int32_t* __restrict__ offsets) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int EL = hi - lo;
  if (blockIdx.x == 0) {
    // every expert takes exactly C tokens: counts and group offsets are fixed
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts_all[e] = C;
    for (int g = threadIdx.x; g <= EL; g += blockDim.x) offsets[g] = g * C;
    for (int s = threadIdx.x; s < n_shared; s += blockDim.x)
      offsets[EL + 1 + s] = EL * C + (s + 1) * T_;
  }
  const int t = gid / L, sub = gid % L;
  if (t >= T_) return;
  const float* s = logits + (size_t)t * E;
  double sv[EPL];
  double m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + L * j;
    sv[j] = (e < E) ? (double)s[e] : -INFINITY;
    m = fmax(m, sv[j]);
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  double z = 0.0;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (sub + L * j < E) z += exp(sv[j] - m);
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
  const double lse = m + log(z);
  if (sub == 0 && lse_out) lse_out[t] = (float)lse;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = sub + L * j;
    if (e >= E) continue;
    const double lp = sv[j] - lse;
    w[(size_t)t * E + e] = (float)exp(lp);
    if (e >= lo && e < hi) keys[(size_t)(e - lo) * T_ + t] = ordered_bits((float)lp);
    else slot_row[(size_t)t * E + e] = -2;
  }
}

constexpr int kEcThreads = 1024;
constexpr int kEcWaves = kEcThreads / 64;

// One workgroup per local expert g = blockIdx.x.  Radix select over the
// ordered key codes, most significant digit first (bits [21,32), [10,21),
// [0,10)): each pass histograms the keys that match the digits fixed so far
// and picks the digit whose bin holds the need-th largest of them.  After
// three passes v* is the C-th largest code, `need` the number of tokens with
// code == v* that are taken (the lowest tokens first) and every code > v* is
// taken.  The compaction then walks the tokens in order, 1024 at a time.
// Keys are read as ordered codes; with R > 0 they stay in registers.
// R > 0: the expert's keys (R * 1024 >= T) are loaded once into registers;
// R == 0: every pass reads them from memory.
template <int R>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(
    const uint32_t* __restrict__ keys, int T_, int E, int lo, int C,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot) {
  __shared__ uint32_t hist[2048];
  __shared__ int wsum[kEcWaves], wsum2[kEcWaves];
  __shared__ int sel_digit, sel_above;
  const int g = blockIdx.x, e = lo + g;
  const uint32_t* kp = keys + (size_t)g * T_;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int nr = R ? R : (T_ + kEcThreads - 1) / kEcThreads;
  uint32_t kr[R ? R : 1];
  if constexpr (R > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = r * kEcThreads + tid;
      kr[r] = t < T_ ? kp[t] : 0u;
    }
  }
  auto key = [&](int r, int t) __attribute__((always_inline)) {
    if constexpr (R > 0) return kr[r];
    else return t < T_ ? kp[t] : 0u;
  };
  uint32_t prefix = 0, pmask = 0;
  int need = C;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const uint32_t dmask = (uint32_t)nb - 1;
    for (int i = tid; i < 2048; i += kEcThreads) hist[i] = 0;
    if (tid == 0) {
      sel_digit = 0;
      sel_above = 0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < nr; ++r) {
      const int t = r * kEcThreads + tid;
      if (r * kEcThreads >= T_) break;  // uniform
      const uint32_t u = key(r, t);
      const bool in = t < T_ && (u & pmask) == prefix;
      const uint32_t dg = (u >> shift) & dmask;
      const uint64_t act = __ballot(in);
      if (!act) continue;  // wave-uniform
      // one atomic for the lanes that share the first active lane's digit
      // (nearby keys share their leading digits), one per lane otherwise
      const int leader = __builtin_ctzll(act);
      const uint32_t dl = __shfl(dg, leader, 64);
      const uint64_t same = __ballot(in && dg == dl);
      if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
      if (in && dg != dl) atomicAdd(&hist[dg], 1u);
    }
    __syncthreads();
    // thread j owns bins nb-1-2j and nb-2-2j: an inclusive scan in
    // descending bin order gives the count of keys above each bin
    const int b1 = nb - 1 - 2 * tid, b0 = b1 - 1;
    const int c1 = b0 >= 0 ? (int)hist[b1] : 0;
    const int c0 = b0 >= 0 ? (int)hist[b0] : 0;
    const int v = c1 + c0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int above = incl - v;
    for (int w = 0; w < wave; ++w) above += wsum[w];
    if (b0 >= 0) {
      if (above < need && need <= above + c1) {
        sel_digit = b1;
        sel_above = above;
      } else if (above + c1 < need && need <= above + v) {
        sel_digit = b0;
        sel_above = above + c1;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel_digit << shift;
    pmask |= dmask << shift;
    need -= sel_above;
    __syncthreads();  // hist, wsum and the selection are rewritten next pass
  }
  const uint32_t vstar = prefix;
  int carry_eq = 0, carry_tk = 0;
#pragma unroll
  for (int r = 0; r < nr; ++r) {
    const int t = r * kEcThreads + tid;
    if (r * kEcThreads >= T_) break;  // uniform
    const bool valid = t < T_;
    const uint32_t u = valid ? key(r, t) : 0u;
    const bool eq = valid && u == vstar;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wsum[wave] = __popcll(beq);
    __syncthreads();
    int eq_before = carry_eq + __popcll(beq & lt), eq_tot = 0;
    for (int w = 0; w < kEcWaves; ++w) {
      const int n = wsum[w];
      if (w < wave) eq_before += n;
      eq_tot += n;
    }
    const bool taken = valid && (u > vstar || (eq && eq_before < need));
    const uint64_t btk = __ballot(taken);
    if (lane == 0) wsum2[wave] = __popcll(btk);
    __syncthreads();
    int tk_before = carry_tk + __popcll(btk & lt), tk_tot = 0;
    for (int w = 0; w < kEcWaves; ++w) {
      const int n = wsum2[w];
      if (w < wave) tk_before += n;
      tk_tot += n;
    }
    if (valid) {
      const int64_t slot = (int64_t)t * E + e;
      if (taken && tk_before < C) {  // exactly C are taken; the bound guards the rows
        const int row = g * C + tk_before;
        slot_row[slot] = row;
        row_token[row] = t;
        row_slot[row] = (int32_t)slot;
      } else {
        slot_row[slot] = -1;
      }
    }
    carry_eq += eq_tot;
    carry_tk += tk_tot;
    __syncthreads();  // wsum / wsum2 are rewritten by the next chunk
  }
}

template <int L, int EPL>
static int launch_ec_token(const moe_config& c, int C, const float* logits, float* w, float* lse,
                           uint32_t* keys, int32_t* slot_row, int32_t* counts_all,
                           int32_t* offsets, hipStream_t st) {
  const int grid = (int)std::max<int64_t>(1, cdiv((int64_t)c.T * L, 256));
  MOE_LAUNCH("ec_token", (ec_token_kernel<L, EPL>), dim3(grid), dim3(256), 0, st, logits, c.T,
             c.E, c.expert_lo, c.expert_hi, c.n_shared, C, w, lse, keys, slot_row, counts_all,
             offsets);
  return MOE_OK;
}

int launch_route_ec(const moe_config& c, const void* x, const float* wr, const float* rb,
                    float* logits, float* w, float* lse, int32_t* counts_all, int32_t* offsets,
                    int32_t* slot_row, int32_t* row_token, int32_t* row_slot, void* x_perm,
                    bool logits_given, char* ws, const Workspace& L, hipStream_t st) {
  int rc;
  if (!logits_given && (rc = router_logits(c, x, wr, rb, logits, st))) return rc;
  const int C = (int)ec_capacity(c);
  const int E = c.E, EL = c.expert_hi - c.expert_lo;
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws + L.ec_keys);
#define TOK(Lv, Ev) \
  rc = launch_ec_token<Lv, Ev>(c, C, logits, w, lse, keys, slot_row, counts_all, offsets, st)
  if (E <= 1) TOK(1, 1);
  else if (E <= 2) TOK(2, 1);
  else if (E <= 4) TOK(4, 1);
  else if (E <= 8) TOK(8, 1);
  else if (E <= 16) TOK(16, 1);
  else if (E <= 32) TOK(32, 1);
  else if (E <= 64) TOK(64, 1);
  else if (E <= 128) TOK(64, 2);
  else if (E <= 256) TOK(64, 4);
  else if (E <= 512) TOK(64, 8);
  else TOK(64, 16);
#undef TOK
  if (rc) return rc;
  if (EL > 0 && C > 0) {
#define SEL(Rv)                                                                                \
  MOE_LAUNCH("ec_select", ec_select_kernel<Rv>, dim3(EL), dim3(kEcThreads), 0, st, keys, c.T, E, \
             c.expert_lo, C, slot_row, row_token, row_slot)
    if (c.T <= 4 * kEcThreads) SEL(4);
    else if (c.T <= 16 * kEcThreads) SEL(16);
    else SEL(0);
#undef SEL
  }
  if ((rc = launch_shared_rows(c, offsets, row_token, row_slot, st))) return rc;
  return launch_gather(c, x, row_token, offsets, x_perm, st);
}

}  // namespace moe
