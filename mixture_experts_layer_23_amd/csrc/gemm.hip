// gemm.hip -- grouped GEMMs of the expert FFNs (forward and backward) on
// CDNA4 matrix cores.
//
// [P5] course notes 8.1 (SwiGLU expert: a = x W_gate, b = x W_up,
// h = silu(a) * b, o = h W_down), 8.8 (the production form is a grouped GEMM
// over the per-expert row blocks instead of a Python loop); [P3] efficient
// inference (after grouping, each expert sees one dense batch).
//
// One kernel template covers the six GEMMs of the layer:
//   forward  GEMM1: [a|b] = X_g W_{gate|up}[g]    + SwiGLU epilogue (h, a, b)
//            GEMM2: o = h W_down[g]
//   backward dgrad2: dh = d_o W_down[g]^T          + SwiGLU-backward epilogue
//            wgrad2: dW_down[g] = h^T d_o           (reduction over the rows)
//            dgrad1: dx_perm = da W_gate^T + db W_up^T
//            wgrad1: dW_gate|up[g] = X^T [da|db]
// Groups are the local experts (row ranges from the permutation offsets,
// read on the device: no host synchronisation) plus the shared expert, whose
// rows are the tokens themselves (it reads x / dy directly).
//
// Tile: 128 x 128 outputs, 256 threads = 4 waves (2 x 2), each wave 64 x 64
// as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 (fp32: 4 x v_mfma_f32_32x32x2f32
// per 16-byte fragment).  K-slabs of 128 bytes per row (64 bf16 / 32 fp32)
// are double-buffered in LDS; the k-chunks of 16 bytes are XOR-swizzled by
// row so that both the transposing stores and the fragment reads are free of
// bank conflicts.  Operands stored with K contiguous are copied as 16-byte
// vectors; operands stored with M/N contiguous are loaded as coalesced
// 16-byte row vectors and transposed in registers (4 k x VEC) before the LDS
// store.  Workgroup ids are remapped so that consecutive tiles (same rows,
// same expert weights) land on the same XCD and share its L2.
#include <cstdlib>
#include <string>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kThreads = 256;

enum OpMode { KC = 0, MC = 1 };  // K contiguous / M (or N) contiguous in memory
enum Grouping { GROUP_M = 0, GROUP_K = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };
enum BSplit { BS_NONE = 0, BS_N = 1, BS_K = 2 };

struct GemmParams {
  int G;              // groups (local experts + shared)
  int EL_A, EL_B;     // groups >= EL_A (EL_B) read A (B) from the shared pointer
  const int32_t* offsets;
  int N;              // output columns (for BS_N: 2 * width of each half)
  int Kdim;           // reduction length for GROUP_M
  int Mfix;           // output rows for GROUP_K
  int ntn, ntm;       // tiles along N (and M for GROUP_K)
  int mt_total;       // m-tiles in the tile space (GROUP_M: an upper bound)
  int64_t nblocks;
  int64_t routed_rows_max;  // routed-row bound when local experts exist, else 0
  int64_t shared_rows;      // n_shared*T
  int n_routed;             // local routed groups
  // A operand: routed pointer (rows at offsets[g]) and shared pointer (row 0)
  const void* A;
  const void* A_sh;
  int64_t lda;
  // B operand: group g at B + g * strideB (two halves for BS_N / BS_K)
  const void* B0;
  const void* B1;
  int64_t ldb, strideB;
  int bsplit;         // BS_N: columns per half; BS_K: k where B1 starts
  // outputs
  void* C0;
  void* C1;           // second half (wgrad1 dW_up) or SwiGLU h
  int64_t ldc;
  int csplit;         // columns of C0 before C1 (wgrad1)
  int64_t strideC;    // per-group stride of C (GROUP_K)
  const void* act;    // SwiGLU-backward input [rows][2F]
  void* act_out;      // SwiGLU forward a|b output [rows][2F]
  int F;
  int xcd_xn;         // > 0: 2-D tile blocks per XCD (xcd_xn column groups)
  int a_cap, b_cap;   // rows of lda / ldb bf16 elements in 2^31 - 1 bytes
  int xcd_m;          // GROUP_M: each XCD takes a block of the real m-tiles
  // weight-gradient loop kernel: multipliers for n / per and n / (2 ntm)
  // (ceil(2^32 / d), UINT32_MAX for d = 1; see udiv_magic)
  uint32_t per_magic, span_magic;
};

// n / d for n < 2^31 from m = ceil(2^32 / d) (UINT32_MAX for d = 1): the
// multiply-high estimate is floor(n / d) or one above (one below for d = 1),
// and one correction each way makes it exact.  Uniform operands compile to
// scalar multiplies, where a division would keep a reciprocal in vector
// registers for the whole kernel.
MOE_DEV uint32_t udiv_magic(uint32_t n, uint32_t d, uint32_t m) {
  uint32_t q = __umulhi(n, m);
  if (q * d > n) --q;
  if ((q + 1) * d <= n) ++q;
  return q;
}

MOE_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }

// XCD-aware remap: hardware places workgroup b on XCD b % 8; give each XCD a
// contiguous range of logical tiles.
MOE_DEV int64_t remap_xcd(int64_t b, int64_t n) {
  const int64_t q = n / 8, r = n % 8;
  const int64_t x = b % 8, i = b / 8;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Weight-gradient (GROUP_K) tile order for launch index b of n tiles: the
// shared expert's tiles -- each a reduction over all T rows, much longer
// than a routed expert's -- come first, so they are spread over the CUs and
// finish early instead of forming the tail; the routed experts' tiles
// follow in group order (the shared expert is the last group).  Launch
// order is tile order, so the hardware's
// round-robin placement (workgroup b on XCD b % 8) hands every XCD every
// eighth tile of each group: the XCDs carry equal shares of every group's
// slabs however skewed the expert loads are, and all of them stream the
// same group's operands at about the same time.  Contiguous per-XCD tile
// ranges (better L2 reuse in principle) left the XCD with the heaviest
// experts 1.8 ms behind the lightest on the DeepSeek-V3-like gate/up
// gradient (60 k against 99 k slabs per XCD); the round-robin order
// measured gate/up 7.73 -> 6.78 ms, down 4.32 -> 3.47 ms there and 7.44 ->
// 4.82, 3.70 -> 2.36 ms on the Mixtral-like layer (chunks of 4 or 16
// consecutive tiles per XCD were no better).  g: group, tl: tile within it.
MOE_DEV void groupk_tile(int64_t b, int64_t per, bool shared, int G, int& g, int64_t& tl) {
  const int64_t sh = shared ? per : 0;
  if (b < sh) {
    g = G - 1;
    tl = b;
  } else {
    g = (int)((b - sh) / per);
    tl = (b - sh) - (int64_t)g * per;
  }
}

// wave-parallel search of the group holding global m-tile mt (GROUP_M) for
// tiles of bm rows
MOE_DEV bool find_group(const int32_t* offsets, int G, int mt, int& g_out, int& mt_local,
                        int bm = kBM) {
  const int lane = threadIdx.x & 63;
  const int gpl = (G + 63) / 64;
  int mine = 0;
  for (int j = 0; j < gpl; ++j) {
    const int g = lane * gpl + j;
    if (g < G) mine += (offsets[g + 1] - offsets[g] + bm - 1) / bm;
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int excl = incl - mine;
  const uint64_t hit = __ballot(mt >= excl && mt < incl);
  if (hit == 0) return false;
  const int owner = __ffsll((unsigned long long)hit) - 1;
  int gsel = 0, base = 0;
  if (lane == owner) {
    int run = excl;
    for (int j = 0; j < gpl; ++j) {
      const int g = lane * gpl + j;
      if (g >= G) break;
      const int n = (offsets[g + 1] - offsets[g] + bm - 1) / bm;
      if (mt < run + n) { gsel = g; base = run; break; }
      run += n;
    }
  }
  g_out = __shfl(gsel, owner, 64);
  mt_local = mt - __shfl(base, owner, 64);
  return true;
}

// Cost-balanced XCD ranges of the weight-gradient tiles (persistent kernel).
// Expert loads are skewed, so equal tile counts per XCD give some XCDs far
// more slabs than others (per-tile timestamps: 0.78 of the chip busy, the
// last XCD 2.7 ms behind on the DeepSeek-V3-like gate/up gradient).  Each
// XCD x takes an eighth of the shared expert's tiles (its reductions run over
// all T rows: on one XCD they made that XCD the straggler) and the routed
// tiles, in group order, whose cumulative cost starts in [x C / 8,
// (x + 1) C / 8): a tile of group g costs its padded slab count plus
// kTileOverhead slab-times (epilogue and hand-over), C is the routed total.
// Wave-uniform; every wave computes the same ranges.
constexpr int kTileOverhead = 2;
MOE_DEV int groupk_slabs(const int32_t* offsets, int g) {
  const int n = offsets[g + 1] - offsets[g];
  int nk = max(2, (n + 63) / 64);
  return nk + (nk & 1);
}
// routed tiles [begin, end) of XCD x (tile r = group r / per, tile r % per)
MOE_DEV void groupk_xcd_range(const int32_t* offsets, int Gr, int64_t per, int x,
                              int64_t& begin, int64_t& end) {
  const int lane = threadIdx.x & 63;
  const int L = (Gr + 63) / 64;  // groups per lane
  int64_t sum = 0;
  for (int i = 0; i < L; ++i) {
    const int q = lane * L + i;
    if (q < Gr) sum += per * (groupk_slabs(offsets, q) + kTileOverhead);
  }
  int64_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  const int64_t total = __shfl(incl, 63, 64);
  const int64_t excl = incl - sum;
  // first tile whose cumulative cost start is >= B (B = k C / 8)
  auto tile_at = [&](int k) -> int64_t {
    const int64_t B = total * k / 8;
    const uint64_t who = __ballot(B >= excl && B < incl);
    if (k >= 8 || who == 0) return (int64_t)Gr * per;
    const int owner = __ffsll((long long)who) - 1;
    int64_t t = 0;
    if (lane == owner) {
      int64_t c = excl;
      for (int i = 0; i < L; ++i) {
        const int q = lane * L + i;
        if (q >= Gr) break;
        const int64_t ct = groupk_slabs(offsets, q) + kTileOverhead;
        if (B < c + per * ct) {
          t = (int64_t)q * per + (B - c + ct - 1) / ct;
          break;
        }
        c += per * ct;
      }
    }
    return __shfl(t, owner, 64);
  };
  begin = tile_at(x);
  end = tile_at(x + 1);
}

// Total m-tiles of bm rows over all groups (uniform).
MOE_DEV int total_mtiles(const int32_t* offsets, int G, int bm) {
  const int lane = threadIdx.x & 63;
  const int gpl = (G + 63) / 64;
  int mine = 0;
  for (int j = 0; j < gpl; ++j) {
    const int g = lane * gpl + j;
    if (g < G) mine += (offsets[g + 1] - offsets[g] + bm - 1) / bm;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
  return __builtin_amdgcn_readfirstlane(mine);
}

// Row-GEMM tile order for layers with many small groups: XCD x (workgroup b
// runs on XCD b % 8) takes the real m-tiles [x mh, (x + 1) mh), mh =
// ceil(mt_real / 8), with all their column tiles.  A row panel is then
// fetched by one XCD, and a group's weights by the one or two XCDs holding
// its few m-tiles, where giving each XCD a column band makes every XCD fetch
// every row panel.  Inside the block, each group's share runs column by
// column with the group's m-tiles innermost, so the workgroups that read
// one weight panel run side by side on the XCD and share it through its L2
// (with the column fastest, a group's second m-tile came a full round of
// column tiles later and fetched the weights again: DeepSeek-V3-like gate/up
// input gradient 5.71 -> 5.12 ms).  The grid holds 8 ceil(mt_total / 8) ntn
// blocks (mt_total bounds mt_real); blocks past an XCD's share return
// false.  Out: the tile (mt, nt), its group g and m-tile mtl within it.
MOE_DEV bool xcd_mblock_tile(int64_t b, const int32_t* offsets, int G, int bm, int ntn, int& mt,
                             int& nt, int& g, int& mtl) {
  const int mt_real = total_mtiles(offsets, G, bm);
  const int x = (int)(b % 8);
  const int64_t i = b / 8;
  const int mh = (mt_real + 7) / 8;
  const int hi = min((x + 1) * mh, mt_real);
  const int row = x * mh + (int)(i / ntn);  // the m-tile in column-fastest order
  if (row >= hi) return false;
  // the group segment holding that m-tile, clipped to the XCD's block: the
  // same segment holds this block index in the group-column order
  int ml;
  if (!find_group(offsets, G, row, g, ml, bm)) return false;
  g = __builtin_amdgcn_readfirstlane(g);
  ml = __builtin_amdgcn_readfirstlane(ml);
  const int sg = row - ml;
  const int eg = sg + (offsets[g + 1] - offsets[g] + bm - 1) / bm;
  const int a = max(sg, x * mh), len = min(eg, hi) - a;
  const int64_t j = i - (int64_t)(a - x * mh) * ntn;
  nt = (int)(j / len);
  mt = a + (int)(j % len);
  mtl = mt - sg;
  return true;
}

template <typename T>
struct Frag;
template <>
struct Frag<bf16_t> {
  static constexpr int BK = 64, KSTEP = 16, VEC = 8;
};
template <>
struct Frag<float> {
  static constexpr int BK = 32, KSTEP = 8, VEC = 4;
};

// One operand tile (128 rows x BK) : global -> registers -> LDS.
// Element (r, k) of the tile (r = output row for A / output column for B).
template <typename T, int MODE>
struct TileLoader {
  static constexpr int VEC = Frag<T>::VEC, BK = Frag<T>::BK;
  uint4 reg[4];
  uint32_t ok;  // bit i: vector i is in range (out-of-range vectors store as zeros)
  // KC: element (r,k) at p[r*ld + k]; thread loads vectors v = tid + 256*i:
  //     row v / 8, chunk v % 8.
  // MC: element (r,k) at p[k*ld + r]; thread loads rows k = kg*4 + j of the
  //     VEC columns mg*VEC.., kg = tid / MG, mg = tid % MG, MG = 128 / VEC.
  // Every load is issued (out-of-range lanes read element (0, k0) of the
  // slab, which is always in bounds) so that no branch forces an early wait on
  // the loads in flight; the mask is applied when the registers go to LDS.
  MOE_DEV void load(const T* p, int64_t ld, int r_valid, int k0, int k_valid) {
    const int tid = threadIdx.x;
    ok = 0;
    if constexpr (MODE == KC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = tid + 256 * i, r = v >> 3, ch = v & 7;
        const int k = k0 + ch * VEC;
        const bool in = (r < r_valid) && (k < k_valid);
        const T* q = in ? p + (int64_t)r * ld + k : p + k0;
        reg[i] = *reinterpret_cast<const uint4*>(q);
        ok |= (uint32_t)in << i;
      }
    } else {
      constexpr int MG = 128 / VEC;
      const int kg = tid / MG, mg = tid % MG;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + kg * 4 + j, r = mg * VEC;
        const bool in = (k < k_valid) && (r < r_valid);
        const T* q = in ? p + (int64_t)k * ld + r : p + (int64_t)k0 * ld;
        reg[j] = *reinterpret_cast<const uint4*>(q);
        ok |= (uint32_t)in << j;
      }
    }
  }
  // for BS_N (SwiGLU forward): rows [0,64) from p0, rows [64,128) from p1
  MOE_DEV void load_split_n(const T* p0, const T* p1, int64_t ld, int col0, int k0) {
    static_assert(MODE == MC, "split-N operand is N-contiguous");
    constexpr int MG = 128 / VEC;
    const int tid = threadIdx.x;
    const int kg = tid / MG, mg = tid % MG;
    const int r = mg * VEC;
    const T* p = (r < 64) ? p0 + col0 + r : p1 + col0 + (r - 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + kg * 4 + j;
      reg[j] = *reinterpret_cast<const uint4*>(p + (int64_t)k * ld);
    }
    ok = 0xF;
  }
  MOE_DEV void store(char* lds) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!((ok >> i) & 1)) reg[i] = make_uint4(0, 0, 0, 0);
    if constexpr (MODE == KC) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = tid + 256 * i, r = v >> 3, ch = v & 7;
        *reinterpret_cast<uint4*>(lds + r * 128 + ((ch ^ swz(r)) << 4)) = reg[i];
      }
    } else {
      constexpr int MG = 128 / VEC;
      const int kg = tid / MG, mg = tid % MG;
      if constexpr (sizeof(T) == 2) {
        // 4 rows (k) x 8 bf16 columns -> 8 rows of 4 consecutive k (8 bytes)
        const uint32_t w0[4] = {reg[0].x, reg[0].y, reg[0].z, reg[0].w};
        const uint32_t w1[4] = {reg[1].x, reg[1].y, reg[1].z, reg[1].w};
        const uint32_t w2[4] = {reg[2].x, reg[2].y, reg[2].z, reg[2].w};
        const uint32_t w3[4] = {reg[3].x, reg[3].y, reg[3].z, reg[3].w};
        const int ch = kg >> 1, half = kg & 1;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int wi = c >> 1;
          uint32_t lo, hi;
          if (c & 1) {
            lo = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
            hi = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
          } else {
            lo = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
            hi = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
          }
          const int r = mg * 8 + c;
          *reinterpret_cast<uint2*>(lds + r * 128 + ((ch ^ swz(r)) << 4) + (half << 3)) =
              make_uint2(lo, hi);
        }
      } else {
        // 4 rows (k) x 4 fp32 columns -> 4 rows of 4 consecutive k (a chunk)
        const float* f0 = reinterpret_cast<const float*>(&reg[0]);
        const float* f1 = reinterpret_cast<const float*>(&reg[1]);
        const float* f2 = reinterpret_cast<const float*>(&reg[2]);
        const float* f3 = reinterpret_cast<const float*>(&reg[3]);
        const int ch = kg;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = mg * 4 + c;
          *reinterpret_cast<float4*>(lds + r * 128 + ((ch ^ swz(r)) << 4)) =
              make_float4(f0[c], f1[c], f2[c], f3[c]);
        }
      }
    }
  }
};

// MFMA on one LDS slab: acc[i][j] += A[rows ra_i..] * B[rows rb_j..]^T
template <typename T>
MOE_DEV void mma_slab(const char* la, const char* lb, const int ra[2], const int rb[2],
                      f32x16_t acc[2][2]) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  constexpr int NSTEP = Frag<T>::BK / Frag<T>::KSTEP;  // 4
#pragma unroll
  for (int ks = 0; ks < NSTEP; ++ks) {
    const int ch = ks * 2 + hi;
    uint4 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ra[i] + l32;
      fa[i] = *reinterpret_cast<const uint4*>(la + r * 128 + ((ch ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = rb[j] + l32;
      fb[j] = *reinterpret_cast<const uint4*>(lb + r * 128 + ((ch ^ swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(T) == 2) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, fa[i]), __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j],
              0, 0, 0);
        } else {
          const float* a = reinterpret_cast<const float*>(&fa[i]);
          const float* b = reinterpret_cast<const float*>(&fb[j]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc[i][j], 0, 0, 0);
        }
      }
  }
}

// SwiGLU's logistic function in the GEMM epilogues from the hardware base-2
// exponential (v_exp_f32) and reciprocal (v_rcp_f32), each within about one
// ulp: a few instructions instead of the library exp and an IEEE division,
// far below the bf16 rounding of a, b, h and the gradients that follows
// (measured: gate/up forward -6 %, SwiGLU-backward GEMM -9 % on MiniMind).
// Large |a| saturates correctly (exp2 -> inf or 0, rcp(inf) = 0).
MOE_DEV float sigmoid_hw(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}
MOE_DEV float silu_f(float a) { return a * sigmoid_hw(a); }

// Epilogue shared by both GEMM kernels: each wave's 64 x 64 fp32 tile goes
// through its own 16 KB region of LDS (chunks of 4 floats
// XOR-swizzled by row) and is read back as rows of 8 consecutive columns, so
// global loads and stores are 16-byte vectors.
template <typename T, int GROUPING, int EPI>
MOE_DEV void gemm_epilogue(const GemmParams& P, f32x16_t (&acc)[2][2], char* region, int m0,
                           int n0, int rows_valid, int cols_valid, int64_t arow0, int g) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi4 = (lane >> 5) * 4;
  const int row_base = wm * 64;  // tile-relative first row of this wave
  // SwiGLU backward: the activation chunks of this lane's eight items are
  // loaded before the tile is staged, all in flight at once (items outside
  // the valid rows / columns read the tile's first row and column and are not
  // used), so one memory latency overlaps the staging; they are read once,
  // non-temporally
  constexpr int NVV = sizeof(T) == 2 ? 1 : 2;  // 16-byte vectors per 8 values
  constexpr int NPF = EPI == EPI_SWIGLU_BWD ? 8 : 1;
  Vec16<T> pa[NPF][NVV], pb[NPF][NVV];
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    const T* act = reinterpret_cast<const T*>(P.act);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int item = lane + 64 * it;
      const int row = item >> 3, col = wn * 64 + (item & 7) * 8;
      const bool ok = row_base + row < rows_valid && col < cols_valid;
      const T* src = act + (arow0 + m0 + (ok ? row_base + row : 0)) * 2 * P.F + n0 + (ok ? col : 0);
#pragma unroll
      for (int q = 0; q < NVV; ++q) {
        pa[it][q].load_nt(src + q * 4);
        pb[it][q].load_nt(src + P.F + q * 4);
      }
    }
  }
  float* ep = reinterpret_cast<float*>(region);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + (r >> 2) * 8 + hi4 + (r & 3);
        const int col = j * 32 + l32;
        ep[row * 64 + (((col >> 2) ^ (row & 15)) << 2) + (col & 3)] = acc[i][j][r];
      }
  __syncthreads();
  auto read8 = [&](int row, int col0, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(ep + row * 64 + (((col0 >> 2) ^ (row & 15)) << 2));
    const float4 b = *reinterpret_cast<const float4*>(ep + row * 64 + ((((col0 >> 2) + 1) ^ (row & 15)) << 2));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  };
  // NT: a non-temporal store (the SwiGLU activations and h, written once
  // and read by a later kernel: measured 4-6 % faster for the gate/up
  // forward than stores that allocate in the cache)
  auto store8 = [&](T* dst, const float* v, bool nt = false) {
    if constexpr (sizeof(T) == 2) {
      Vec16<T> o;
      o.from_f32(v);
      if (nt) o.store_nt(dst);
      else o.store(dst);
    } else {
      Vec16<T> o0, o1;
      o0.from_f32(v);
      o1.from_f32(v + 4);
      if (nt) {
        o0.store_nt(dst);
        o1.store_nt(dst + 4);
      } else {
        o0.store(dst);
        o1.store(dst + 4);
      }
    }
  };
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    // LDS columns [0,32) hold a (gate), [32,64) hold b (up) of the same f's
    T* hout = reinterpret_cast<T*>(P.C1);
    T* aout = reinterpret_cast<T*>(P.act_out);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = lane + 64 * it;
      const int row = item >> 2, fg = (item & 3) * 8;
      if (row_base + row >= rows_valid) continue;
      float a[8], b[8], h[8];
      read8(row, fg, a);
      read8(row, 32 + fg, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = silu_f(a[q]) * b[q];
      const int64_t grow = arow0 + m0 + row_base + row;
      const int f = n0 / 2 + wn * 32 + fg;
      store8(aout + grow * 2 * P.F + f, a, true);
      store8(aout + grow * 2 * P.F + P.F + f, b, true);
      store8(hout + grow * P.F + f, h, true);
    }
  } else {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int item = lane + 64 * it;
      const int row = item >> 3, cg = (item & 7) * 8;
      const int col = wn * 64 + cg;  // tile-relative column
      if (row_base + row >= rows_valid || col >= cols_valid) continue;
      float v[8];
      read8(row, cg, v);
      if constexpr (EPI == EPI_SWIGLU_BWD) {
        T* dact = reinterpret_cast<T*>(P.C0);
        const int64_t grow = arow0 + m0 + row_base + row;
        const int f = n0 + col;
        float a[8], b[8], da[8], db[8];
#pragma unroll
        for (int q = 0; q < NVV; ++q) {
          pa[it][q].to_f32(a + q * 4);
          pb[it][q].to_f32(b + q * 4);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float sg = sigmoid_hw(a[q]);
          da[q] = v[q] * b[q] * sg * (1.0f + a[q] * (1.0f - sg));
          db[q] = v[q] * a[q] * sg;
        }
        store8(dact + grow * 2 * P.F + f, da);
        store8(dact + grow * 2 * P.F + P.F + f, db);
      } else if constexpr (GROUPING == GROUP_M) {
        T* C = reinterpret_cast<T*>(P.C0);
        store8(C + (arow0 + m0 + row_base + row) * P.ldc + n0 + col, v);
      } else {
        const int n = n0 + col;
        const int64_t mrow = m0 + row_base + row;
        if (n < P.csplit)
          store8(reinterpret_cast<T*>(P.C0) + (int64_t)g * P.strideC + mrow * P.ldc + n, v);
        else
          store8(reinterpret_cast<T*>(P.C1) + (int64_t)g * P.strideC + mrow * P.ldc +
                     (n - P.csplit), v);
      }
    }
  }
}

template <typename T, int AMODE, int BMODE, int GROUPING, int EPI, int BSPL>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams P) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][kBM * 128];  // [buf][A/B]
  constexpr int BK = Frag<T>::BK;
  const int64_t lin = remap_xcd(blockIdx.x, P.nblocks);
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int g, m0, n0, rows_valid, kdim;
  int64_t arow0;  // first row of this group's rows in the output/row buffers
  const T* Ap;
  const T* Bp0;
  const T* Bp1 = nullptr;
  if constexpr (GROUPING == GROUP_M) {
    const int mt = (int)(lin / P.ntn), nt = (int)(lin % P.ntn);
    int mtl;
    if (!find_group(P.offsets, P.G, mt, g, mtl)) return;
    const int nrows = P.offsets[g + 1] - P.offsets[g];
    m0 = mtl * kBM;
    n0 = nt * kBN;
    rows_valid = min(kBM, nrows - m0);
    kdim = P.Kdim;
    arow0 = P.offsets[g];
    if (g < P.EL_A)
      Ap = reinterpret_cast<const T*>(P.A) + (arow0 + m0) * P.lda;
    else
      Ap = reinterpret_cast<const T*>(P.A_sh) + (int64_t)m0 * P.lda;
  } else {
    const int per = P.ntm * P.ntn;
    g = (int)(lin / per);
    const int rem = (int)(lin % per);
    m0 = (rem / P.ntn) * kBM;
    n0 = (rem % P.ntn) * kBN;
    rows_valid = min(kBM, P.Mfix - m0);
    kdim = P.offsets[g + 1] - P.offsets[g];
    arow0 = P.offsets[g];
    if (g < P.EL_A)
      Ap = reinterpret_cast<const T*>(P.A) + arow0 * P.lda + m0;
    else
      Ap = reinterpret_cast<const T*>(P.A_sh) + m0;
  }
  Bp0 = reinterpret_cast<const T*>(P.B0) + (int64_t)g * P.strideB;
  if constexpr (BSPL != BS_NONE) Bp1 = reinterpret_cast<const T*>(P.B1) + (int64_t)g * P.strideB;
  // B row/col origin of this tile
  int cols_valid;
  const T* Bt;  // tile origin for the unsplit cases
  if constexpr (GROUPING == GROUP_M) {
    cols_valid = min(kBN, P.N - n0);
    if constexpr (BMODE == KC) Bt = Bp0 + (int64_t)n0 * P.ldb;
    else Bt = Bp0 + n0;
  } else {
    cols_valid = min(kBN, P.N - n0);
    // B(k = row r, n) at (g < EL ? B0 + arow0*ldb : B1 (shared)) + r*ldb + n
    if (g < P.EL_B) Bt = reinterpret_cast<const T*>(P.B0) + arow0 * P.ldb + n0;
    else Bt = reinterpret_cast<const T*>(P.B1) + n0;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Two register sets, prefetch distance two: while slab kt is multiplied
  // from LDS, slab kt+1 is in registers (or arriving) and slab kt+2 is being
  // loaded.  The loop is unrolled by two so that the sets are static.
  TileLoader<T, AMODE> la0, la1;
  TileLoader<T, BMODE> lb0, lb1;
  const int nk = (kdim + BK - 1) / BK;

  auto load_k = [&](TileLoader<T, AMODE>& la, TileLoader<T, BMODE>& lb, int kt) {
    const int k0 = kt * BK;
    if constexpr (GROUPING == GROUP_M) {
      la.load(Ap, P.lda, rows_valid, k0, kdim);
      if constexpr (BSPL == BS_N) {
        lb.load_split_n(Bp0, Bp1, P.ldb, n0 / 2, k0);
      } else if constexpr (BSPL == BS_K) {
        if (k0 < P.bsplit) lb.load(Bp0 + (int64_t)n0 * P.ldb, P.ldb, cols_valid, k0, P.bsplit);
        else lb.load(Bp1 + (int64_t)n0 * P.ldb - P.bsplit, P.ldb, cols_valid, k0, kdim);
      } else {
        lb.load(Bt, P.ldb, cols_valid, k0, kdim);
      }
    } else {
      la.load(Ap, P.lda, rows_valid, k0, kdim);
      lb.load(Bt, P.ldb, cols_valid, k0, kdim);
    }
  };

  int ra[2], rb[2];
  ra[0] = wm * 64;
  ra[1] = wm * 64 + 32;
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    rb[0] = wn * 32;        // gate columns
    rb[1] = 64 + wn * 32;   // matching up columns
  } else {
    rb[0] = wn * 64;
    rb[1] = wn * 64 + 32;
  }

  if (nk > 0) {
    load_k(la0, lb0, 0);
    if (nk > 1) load_k(la1, lb1, 1);
    la0.store(smem[0][0]);
    lb0.store(smem[0][1]);
    __syncthreads();
    // pairs of slabs: buffer 0 holds the even slab, buffer 1 the odd one
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      if (kt + 2 < nk) load_k(la0, lb0, kt + 2);
      mma_slab<T>(smem[0][0], smem[0][1], ra, rb, acc);
      la1.store(smem[1][0]);
      lb1.store(smem[1][1]);
      __syncthreads();
      if (kt + 3 < nk) load_k(la1, lb1, kt + 3);
      mma_slab<T>(smem[1][0], smem[1][1], ra, rb, acc);
      if (kt + 2 < nk) {
        la0.store(smem[0][0]);
        lb0.store(smem[0][1]);
      }
      __syncthreads();
    }
    if (kt < nk) {  // odd slab count: the last slab is in buffer 0
      mma_slab<T>(smem[0][0], smem[0][1], ra, rb, acc);
      __syncthreads();
    }
  }

  gemm_epilogue<T, GROUPING, EPI>(P, acc, &smem[0][0][0] + (threadIdx.x >> 6) * 16384, m0, n0,
                                   rows_valid, cols_valid, arow0, g);
}


// ===========================================================================
// CDNA4 path (bf16, full 128-column tiles): operand slabs are copied global ->
// LDS by the LDS-DMA loads (no register staging), through a ring of S stages.
//  * K-contiguous operand: LDS tile [128 rows][64 k] (128-byte rows, 16-byte
//    chunks XOR-swizzled by swz(row)); MFMA fragments by ds_read_b128.
//  * M/N-contiguous operand: LDS tile [64 k][128 m|n] as stored in memory
//    (256-byte rows, chunk swizzle mcswz(k)); MFMA fragments by
//    ds_read_b64_tr_b16, which hands lane l of each 16-lane group element l%4
//    of the 8-byte chunk addressed by lane 4j + l/4 (j = 0..3): with lane
//    4j + q pointing at (k0 + j, n0 + 4q), lane l receives column n0 + l for
//    k0..k0+3 -- the transposed fragment.
// Activation rows are read with buffer loads whose range ends at the group's
// last row, so rows past a ragged group end (or past a group's k extent in
// the weight-gradient GEMMs) arrive as zeros; full weight tiles use per-lane
// global addresses.
// ===========================================================================
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBufDword3 = 0x00020000;  // raw buffer descriptor word 3 (CDNA)

// A raw buffer descriptor (base, stride 0, num_records, word 3) in four
// scalar registers: every dword goes through readfirstlane, so the DMA
// instructions take it from SGPRs (the values are wave-uniform by
// construction).
typedef int rsrc_t __attribute__((ext_vector_type(4)));
MOE_DEV rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nb = bytes > 0x7fffffffLL ? 0x7fffffff : bytes < 0 ? 0 : (int)bytes;
  const uint64_t b = (uint64_t)(uintptr_t)base;
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(nb);
  r.w = kBufDword3;
  return r;
}

// Descriptor over rows [r0, rows) of a row-major bf16 operand with rows of ld
// elements, based at row r0.  Every DMA of a tile (rows r0 .. r0 + 255, row
// operand) or of a k-slab (rows r0 .. r0 + 63, k-major operand) then has an
// offset below 256 * ld * 2 bytes, which the host keeps under 2^31 (D and F
// at most 2^20), however large the whole tensor is; rows at or past `rows`
// read zeros.  The range is capped at cap = floor((2^31 - 1) / (2 ld)) rows
// (from the host), which always covers the rows one tile or slab reads, so an
// offset of 2^31 is always out of range (the padding slabs use that).  All
// 32-bit scalar arithmetic: this runs once per slab.
MOE_DEV rsrc_t rows_rsrc(const bf16_t* base, int r0, int rows, int ld, int cap) {
  const int rem = min(max(rows - r0, 0), cap);
  const uint64_t b = (uint64_t)(uintptr_t)(base + (int64_t)r0 * ld);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane(rem * ld * 2);
  r.w = kBufDword3;
  return r;
}

MOE_DEV lds_void_t* to_lds(char* p) {
  return (lds_void_t*)(__attribute__((address_space(3))) char*)(p);
}

// 16-byte LDS-DMA loads (global_load_lds_dwordx4 / buffer_load_dwordx4 ...
// lds, LDS destination in M0), issued as inline assembly.  The kernels order
// every slab themselves -- an explicit vmcnt wait for their own DMA, then a
// workgroup barrier, before any wave reads the slab or overwrites a stage --
// so the compiler's own tracking of LDS-DMA is not needed; left to it, the
// tracking loses the destination object of some fragment reads and then
// waits for the DMA just issued (for the slab after next) before reading the
// current slab, which serialises the pipeline (measured on the DeepSeek-V3-
// like weight gradients: 8.7 -> 10.3 ms after an unrelated change moved such
// a wait into the main loop).  The instructions write no register (data goes
// to LDS) and read their operands at issue; "memory" keeps every LDS access
// on its side.  M0 is written here and read by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
MOE_DEV void dma16_global(const void* src, lds_void_t* dst) {
  const uint32_t m = (uint32_t)(uintptr_t)dst;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m), "v"(src) : "memory", "m0");
}
// The descriptor operand must sit in SGPRs: a descriptor kept across a
// loop of tiles can end up in VGPRs (as the compiler sees fit for a value it
// knows is uniform), which the assembler rejects, so each dword goes through
// readfirstlane here (a plain move when it already is scalar).
MOE_DEV rsrc_t sgpr_rsrc(rsrc_t r) {
  rsrc_t o;
  o.x = __builtin_amdgcn_readfirstlane(r.x);
  o.y = __builtin_amdgcn_readfirstlane(r.y);
  o.z = __builtin_amdgcn_readfirstlane(r.z);
  o.w = __builtin_amdgcn_readfirstlane(r.w);
  return o;
}
MOE_DEV void dma16_buffer(rsrc_t rs, lds_void_t* dst, uint32_t voff) {
  const uint32_t m = (uint32_t)(uintptr_t)dst;
  rs = sgpr_rsrc(rs);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m), "v"(voff), "s"(rs) : "memory", "m0");
}
// as dma16_buffer, with a wave-uniform byte offset in soffset (added to the
// address; the layouts here keep it inside one row of the range, so the
// row-validity of the range check is decided by voff either way)
MOE_DEV void dma16_buffer_so(rsrc_t rs, lds_void_t* dst, uint32_t voff, uint32_t soff) {
  const uint32_t m = (uint32_t)(uintptr_t)dst;
  rs = sgpr_rsrc(rs);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt wait with expcnt / lgkmcnt left open (gfx9 s_waitcnt encoding)
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wave-uniform read of a group offset through the constant address space,
// so it compiles to a scalar load (waited for on lgkmcnt): a vector load
// would be waited for on vmcnt, and with LDS-DMA in flight that wait would
// also wait for every DMA issued before it.  The offsets are written by an
// earlier kernel and only read here.
MOE_DEV int group_offset(const int32_t* offsets, int g) {
  typedef const __attribute__((address_space(4))) int32_t* cptr_t;
  return ((cptr_t)offsets)[g];
}

// Workgroup barrier for LDS hand-overs without a memory fence: this wave's
// LDS reads and writes are complete (lgkmcnt 0), then s_barrier.  The fence
// of __syncthreads() would also wait for every global store in flight (on
// CDNA one counter covers vector loads and stores), which a pipeline that
// stores one tile while loading the next must not do.  The "memory" clobber
// keeps the compiler from moving memory accesses across it.
MOE_DEV void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inside a k-step, spread the next k-step's fragment reads between the M
// MFMAs (one MFMA, then up to Q LDS reads, M times) instead of letting the
// scheduler issue every read ahead of the first MFMA, so that the reads of
// the waves sharing the LDS do not all queue at the start of a k-step
// (DeepSeek-V3-like SwiGLU forward 5.10 -> 4.95 ms, step -1 %; Mixtral-like
// SwiGLU forward 5.39 -> 5.16 ms, step -1 %).
template <int M, int Q>
MOE_DEV void interleave_reads() {
#pragma unroll
  for (int i = 0; i < M; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, Q, 0);  // Q LDS reads
  }
}

// per-lane source of one DMA instruction (u = 0..3) of this wave
// KC tile: chunk P = 64*t + lane, row = P/8, logical chunk = (P%8) ^ swz(row)
MOE_DEV void kc_slot(int t, int lane, int& row, int& lc) {
  const int P = 64 * t + lane;
  row = P >> 3;
  lc = (P & 7) ^ swz(row);
}
// Chunk swizzle of the M/N-contiguous tiles: 16-byte chunk c of k-row k is
// stored at c ^ mcswz(k).  A transposing fragment read has each 16-lane group
// read 32 bytes from each of four consecutive k-rows (two such groups 32
// bytes apart in the same rows per 32 lanes); rows one tile pitch apart fall
// on the same banks, so the four rows are spread over the banks.
MOE_DEV int mcswz(int k) { return (k & 3) << 2; }
// MC tile: chunk P = 64*t + lane, k row = P/16, logical chunk = (P%16) ^ mcswz(k)
MOE_DEV void mc_slot(int t, int lane, int& krow, int& lc) {
  const int P = 64 * t + lane;
  krow = P >> 4;
  lc = (P & 15) ^ mcswz(krow);
}

// fragment reads: 8 bf16 of one 32x32x16 MFMA operand for block rows rbase
// Chunk ch = 2 ks + (lane >> 5) sits at (ch ^ swz(r)) << 4 in its 128-byte
// row; since 2 ks has no low bit, that is ((((lane >> 5) ^ swz(r)) << 4) ^
// (32 ks)): one per-lane offset for all four k-steps, XORed with a uniform
// constant, instead of a separate address register per k-step and stage.
MOE_DEV uint4 frag_kc(const char* tile, int rbase, int ks, int lane) {
  const int r = rbase + (lane & 31);
  const int off = (r * 128 + (((lane >> 5) ^ swz(r)) << 4)) ^ (ks << 5);
  return *reinterpret_cast<const uint4*>(tile + off);
}
MOE_DEV uint4 frag_mc(char* tile, int rbase, int ks, int lane, int pitch) {
  const int gi = lane >> 4, a = lane & 15, j = a >> 2, q = a & 3;
  const int col = rbase + (gi & 1) * 16 + 4 * q;
  const int lc = col >> 3, half = (col >> 2) & 1;
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int krow = ks * 16 + (gi >> 1) * 8 + 4 * h + j;
    char* p = tile + krow * pitch + ((lc ^ mcswz(krow)) << 4) + (half << 3);
    const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(__attribute__((address_space(3))) char*)p);
    w[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    w[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Tile order: super-columns of kSuperColsM / kSuperColsK n-tiles; inside one, all m-tiles,
// n fastest.  Together with the XCD remap, the workgroups that run together on
// one XCD share one or two weight panels and stream the row panels past them
// (measured against widths 1, 4, 8 and 16: width 2 is 3-8 % faster per step
// on all five layer shapes).
constexpr int kSuperColsM = 2;  // row GEMMs (forward, data gradients)
constexpr int kSuperColsK = 2;  // weight gradients
// 2-D blocks of tiles per XCD (workgroup b runs on XCD b % 8): XCD
// (xm, xn) takes m-tiles [xm mh, (xm + 1) mh) x n-tiles [xn ng, (xn + 1) ng)
// row by row, so each row panel is fetched by xn_n XCDs and each weight
// panel by 8 / xn_n, where contiguous super-columns per XCD make every XCD
// stream all rows.  Needs mt_total % (8 / xn_n) == 0 and ntn % xn_n == 0.
MOE_DEV void xcd_block_tile(int64_t b, int mt_total, int ntn, int xn_n, int& mt, int& nt) {
  const int xm_n = 8 / xn_n;
  const int x = (int)(b % 8), i = (int)(b / 8);
  const int xn = x % xn_n, xm = x / xn_n;
  const int ng = ntn / xn_n, mh = mt_total / xm_n;
  mt = xm * mh + i / ng;
  nt = xn * ng + i % ng;
}
template <int SC>
MOE_DEV void supercol_tile(int64_t lin, int mt_total, int ntn, int& mt, int& nt) {
  const int full = ntn / SC, rem = ntn % SC;
  const int64_t span = (int64_t)mt_total * SC;
  const int64_t sc = lin / span;
  if (sc < full) {
    const int64_t w = lin - sc * span;
    mt = (int)(w / SC);
    nt = (int)(sc * SC + w % SC);
  } else {
    const int64_t w = lin - (int64_t)full * span;
    mt = (int)(w / rem);
    nt = full * SC + (int)(w % rem);
  }
}

// BMT x 128 tiles, NW = BMT / 32 waves (a (BMT/64) x 2 grid of 64 x 64 wave
// tiles), S LDS stages.
template <int AMODE, int BMODE, int GROUPING, int EPI, int BSPL, int BMT, int S>
__global__ __launch_bounds__(BMT * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_dma_kernel(GemmParams P) {
  typedef bf16_t T;
  constexpr int BK = 64;
  constexpr int NW = BMT / 32;
  constexpr int ATILE = BMT * 128;   // bytes of the A slab
  constexpr int BTILE = 16384;       // bytes of the B slab (128 x 64 bf16)
  constexpr int A_PER_WAVE = ATILE / 1024 / NW;  // DMA instructions per wave
  constexpr int B_PER_WAVE = BTILE / 1024 / NW;
  static_assert(A_PER_WAVE * NW * 1024 == ATILE && B_PER_WAVE * NW * 1024 == BTILE, "split");
  static_assert(S == 2 || S == 3, "two or three stages");
  static_assert(S * (ATILE + BTILE) >= NW * 16384, "the epilogue needs 16 KB per wave");
  // one LDS array per stage and operand: distinct objects let the compiler
  // see that the DMA into one stage does not alias the reads of another, so
  // it inserts no blanket wait for the loads in flight
  __shared__ __attribute__((aligned(1024))) char sA0[ATILE];
  __shared__ __attribute__((aligned(1024))) char sB0[BTILE];
  __shared__ __attribute__((aligned(1024))) char sA1[ATILE];
  __shared__ __attribute__((aligned(1024))) char sB1[BTILE];
  __shared__ __attribute__((aligned(1024))) char sA2[S == 3 ? ATILE : 16];
  __shared__ __attribute__((aligned(1024))) char sB2[S == 3 ? BTILE : 16];
  const int64_t lin = remap_xcd(blockIdx.x, P.nblocks);
  // the wave index as a scalar: DMA destinations must be wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;

  int g, m0, n0, rows_valid, kdim;
  int64_t arow0;
  int nrows_g = 0;
  if constexpr (GROUPING == GROUP_M) {
    int mt, nt, mtl;
    if (P.xcd_xn > 0) xcd_block_tile(blockIdx.x, P.mt_total, P.ntn, P.xcd_xn, mt, nt);
    else supercol_tile<kSuperColsM>(lin, P.mt_total, P.ntn, mt, nt);
    if (!find_group(P.offsets, P.G, mt, g, mtl, BMT)) return;
    g = __builtin_amdgcn_readfirstlane(g);
    mtl = __builtin_amdgcn_readfirstlane(mtl);
    nrows_g = P.offsets[g + 1] - P.offsets[g];
    m0 = mtl * BMT;
    n0 = nt * kBN;
    rows_valid = min(BMT, nrows_g - m0);
    kdim = P.Kdim;
    arow0 = P.offsets[g];
  } else {
    const int64_t per = (int64_t)P.ntm * P.ntn;
    int64_t tl;
    groupk_tile(blockIdx.x, per, P.shared_rows > 0, P.G, g, tl);
    int mt, nt;
    supercol_tile<kSuperColsK>(tl, P.ntm, P.ntn, mt, nt);
    m0 = mt * BMT;
    n0 = nt * kBN;
    rows_valid = BMT;
    kdim = P.offsets[g + 1] - P.offsets[g];
    arow0 = P.offsets[g];
  }
  const int cols_valid = kBN;

  // ---- A source: the group's rows.  Row-major A (the row GEMMs): one
  // descriptor based at the tile's first row.  k-major A (the weight
  // gradients, k = the group's rows): a descriptor per k-slab, based at the
  // slab's first row.
  static_assert((GROUPING == GROUP_M) == (AMODE == KC), "A is row-major exactly for GROUP_M");
  const T* a_base = (g < P.EL_A) ? reinterpret_cast<const T*>(P.A) + arow0 * P.lda
                                 : reinterpret_cast<const T*>(P.A_sh);
  const int64_t a_rows = (GROUPING == GROUP_M) ? nrows_g : kdim;
  const rsrc_t a_rs_tile = rows_rsrc(a_base, (AMODE == KC) ? m0 : 0, a_rows, P.lda, P.a_cap);
  uint32_t a_off[A_PER_WAVE];
#pragma unroll
  for (int u = 0; u < A_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * A_PER_WAVE + u) + lane;  // 16-byte chunk of the slab
    if constexpr (AMODE == KC) {
      const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
      a_off[u] = (uint32_t)(((int64_t)r * P.lda + 8 * lc) * 2);
    } else {
      constexpr int CPR = BMT / 8;  // chunks per k-row
      const int kr = P_ / CPR, lc = (P_ % CPR) ^ mcswz(kr);
      a_off[u] = (uint32_t)(((int64_t)kr * P.lda + m0 + 8 * lc) * 2);
    }
  }
  // ---- B source.  GROUP_M: weights, full tiles, per-lane global addresses.
  // GROUP_K: activations (k = rows of the group), buffer over the group rows.
  const T* b_ptr[B_PER_WAVE];
  uint32_t b_off[B_PER_WAVE];
  const T* b_base = nullptr;  // GROUP_K: the group's activation rows (k-major)
  const T* Bw0 = reinterpret_cast<const T*>(P.B0) + (int64_t)g * P.strideB;
  const T* Bw1 = (BSPL != BS_NONE) ? reinterpret_cast<const T*>(P.B1) + (int64_t)g * P.strideB
                                   : nullptr;
  if constexpr (GROUPING == GROUP_M) {
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
      if constexpr (BMODE == KC) {
        const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
        b_ptr[u] = Bw0 + (int64_t)(n0 + r) * P.ldb + 8 * lc;  // + k0 per slab
      } else {
        const int kr = P_ >> 4, lc = (P_ & 15) ^ mcswz(kr);
        if constexpr (BSPL == BS_N) {
          const int col0 = n0 / 2;
          b_ptr[u] = (lc < 8) ? Bw0 + (int64_t)kr * P.ldb + col0 + 8 * lc
                              : Bw1 + (int64_t)kr * P.ldb + col0 + 8 * (lc - 8);
        } else {
          b_ptr[u] = Bw0 + (int64_t)kr * P.ldb + n0 + 8 * lc;
        }
      }
    }
  } else {
    b_base = (g < P.EL_B) ? reinterpret_cast<const T*>(P.B0) + arow0 * P.ldb
                          : reinterpret_cast<const T*>(P.B1);
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
      const int kr = P_ >> 4, lc = (P_ & 15) ^ mcswz(kr);
      b_off[u] = (uint32_t)(((int64_t)kr * P.ldb + n0 + 8 * lc) * 2);
    }
  }

  // issue this wave's DMA instructions for slab kt into (la, lb)
  auto issue = [&](int kt, char* la, char* lb) {
    const int k0 = kt * BK;
    // row-major A: the k offset inside the tile's rows; k-major A: a
    // descriptor based at the slab's first row
    const rsrc_t a_rs =
        (AMODE == KC) ? a_rs_tile : rows_rsrc(a_base, k0, a_rows, P.lda, P.a_cap);
    const uint32_t kadd = (AMODE == KC) ? (uint32_t)(k0 * 2) : 0u;
#pragma unroll
    for (int u = 0; u < A_PER_WAVE; ++u)
      dma16_buffer(a_rs, to_lds(la + (wave * A_PER_WAVE + u) * 1024), a_off[u] + kadd);
    rsrc_t b_rs = {0, 0, 0, 0};  // GROUP_K only: the slab's activation rows
    if constexpr (GROUPING == GROUP_K) b_rs = rows_rsrc(b_base, k0, kdim, P.ldb, P.b_cap);
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      char* dst = lb + (wave * B_PER_WAVE + u) * 1024;
      if constexpr (GROUPING == GROUP_M) {
        const T* src;
        if constexpr (BMODE == KC) {
          if constexpr (BSPL == BS_K) {
            // k < bsplit from W_gate, above from W_up (the same row layout)
            src = (k0 < P.bsplit) ? b_ptr[u] + k0 : (b_ptr[u] - Bw0) + Bw1 + (k0 - P.bsplit);
          } else {
            src = b_ptr[u] + k0;
          }
        } else {
          src = b_ptr[u] + (int64_t)k0 * P.ldb;
        }
        dma16_global(src, to_lds(dst));
      } else {
        dma16_buffer(b_rs, to_lds(dst), b_off[u]);
      }
    }
  };

  int ra[2], rb[2];
  ra[0] = wm * 64;
  ra[1] = wm * 64 + 32;
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    rb[0] = wn * 32;
    rb[1] = 64 + wn * 32;
  } else {
    rb[0] = wn * 64;
    rb[1] = wn * 64 + 32;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (kdim + BK - 1) / BK;
  constexpr int PER_SLAB = A_PER_WAVE + B_PER_WAVE;  // DMA instructions per slab
  // The pipeline for NB active 32-row blocks of this wave's 64 rows: a
  // ragged group's last tile multiplies (and reads A fragments for) only the
  // blocks that hold rows of the group; every wave still issues its DMA share
  // and joins every barrier.
  auto pipeline = [&](auto nb_c) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb_c)::value;
    // fragments of k-step ks + 1 are read while the MFMAs of k-step ks run
    auto mma = [&](char* la, char* lb) {
      uint4 fa[2][2], fb[2][2];
      auto frags = [&](int ks, uint4* a, uint4* b) {
#pragma unroll
        for (int i = 0; i < NB; ++i)
          a[i] = (AMODE == KC) ? frag_kc(la, ra[i], ks, lane) : frag_mc(la, ra[i], ks, lane, BMT * 2);
        if constexpr (NB > 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
            b[j] = (BMODE == KC) ? frag_kc(lb, rb[j], ks, lane) : frag_mc(lb, rb[j], ks, lane, 256);
        }
      };
      frags(0, fa[0], fb[0]);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < BK / 16) frags(ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, fa[cur][i]), __builtin_bit_cast(bf16x8_t, fb[cur][j]),
                acc[i][j], 0, 0, 0);
      }
    };
    // one pipeline step: slab kt is in (la, lb); slab kt + S - 1 goes to (na, nb)
    auto step = [&](int kt, char* la, char* lb, char* na, char* nb) {
      // slab kt has landed once at most the next slab's loads are outstanding
      if (S == 3 && kt + 1 < nk) wait_vmcnt<PER_SLAB>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (kt + S - 1 < nk) issue(kt + S - 1, na, nb);
      // keep the DMA at the head of this slab's MFMAs (the compiler would
      // otherwise sink it towards the next wait)
      __builtin_amdgcn_sched_barrier(0);
      mma(la, lb);
    };
    if (nk > 0) issue(0, sA0, sB0);
    if (S == 3 && nk > 1) issue(1, sA1, sB1);
    if constexpr (S == 2) {
      int kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(kt, sA0, sB0, sA1, sB1);
        step(kt + 1, sA1, sB1, sA0, sB0);
      }
      if (kt < nk) step(kt, sA0, sB0, sA1, sB1);
    } else {
      int kt = 0;
      for (; kt + 2 < nk; kt += 3) {
        step(kt, sA0, sB0, sA2, sB2);
        step(kt + 1, sA1, sB1, sA0, sB0);
        step(kt + 2, sA2, sB2, sA1, sB1);
      }
      if (kt < nk) step(kt, sA0, sB0, sA2, sB2);
      if (kt + 1 < nk) step(kt + 1, sA1, sB1, sA0, sB0);
    }
  };
  if constexpr (GROUPING == GROUP_M) {
    // 32-row blocks of this wave's 64 rows that hold group rows (uniform)
    const int nb = __builtin_amdgcn_readfirstlane(max(0, min(2, (rows_valid - wm * 64 + 31) / 32)));
    if (nb == 2) pipeline(std::integral_constant<int, 2>{});
    else if (nb == 1) pipeline(std::integral_constant<int, 1>{});
    else pipeline(std::integral_constant<int, 0>{});
  } else {
    pipeline(std::integral_constant<int, 2>{});
  }
  __syncthreads();
  // 16 KB of LDS per wave for the epilogue, carved from the stage arrays
  char* region;
  if constexpr (BMT == 128) {
    region = wave == 0 ? sA0 : wave == 1 ? sB0 : wave == 2 ? sA1 : sB1;
  } else {
    region = wave < 2 ? sA0 + wave * 16384 : wave == 2 ? sB0 : wave < 5 ? sA1 + (wave - 3) * 16384
           : wave == 5 ? sB1 : sA2 + (wave - 6) * 16384;
  }
  gemm_epilogue<T, GROUPING, EPI>(P, acc, region, m0, n0, rows_valid, cols_valid, arow0, g);
}

// ---------------------------------------------------------------------------
// Large tiles: 256 x BN outputs (BN = 256 or 128) per workgroup of NW = 4 or
// 8 waves.  Wave grid and wave tile:
//   BN 256, 4 waves: 2 x 2 of 128 x 128     BN 256, 8 waves: 2 x 4 of 128 x 64
//   BN 128, 4 waves: 2 x 2 of 128 x 64      BN 128, 8 waves: 4 x 2 of 64 x 64
// Wave tiles of 128 rows let each 16-byte fragment read from LDS feed several
// MFMAs; eight waves give each SIMD a second wave to issue from while the
// other waits on LDS or on the DMA queue.  K-slabs of 64 arrive by LDS-DMA,
// double-buffered; the MFMA operands are swapped (B first) so that lane l
// holds output row l % 32 of each block in 4-column runs.  The epilogue
// stages each 32-row block of a wave through LDS and writes whole 16-byte
// row segments.
// ---------------------------------------------------------------------------
MOE_DEV uint2 pack_bf16x4(const float* v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

template <int BN, int NW>
struct BigShape {
  static constexpr int WMW = (NW == 8 && BN == 128) ? 4 : 2;  // waves along M
  static constexpr int WNW = NW / WMW;                          // waves along N
  static constexpr int WTM = 256 / WMW, WTN = BN / WNW;        // wave tile
  static constexpr int NI = WTM / 32, NJ = WTN / 32;           // 32 x 32 blocks
};

// BK: reduction depth of one LDS slab.  64 everywhere except the weight-
// gradient variant on 256 x 128 tiles with 4 waves, which takes 32-deep slabs
// (48 KB of LDS for two stages) so that two workgroups share a CU: the
// reductions of a weight gradient run only over one group's rows, so each
// tile is short and its prologue and epilogue stores are a large part of it;
// with two workgroups per CU they overlap the other workgroup's main loop.
template <int AMODE, int BMODE, int GROUPING, int EPI, int BSPL, int BN, int NW, int BK = 64>
__global__ __launch_bounds__(NW * 64) void grouped_gemm_big_kernel(GemmParams P) {
  typedef bf16_t T;
  typedef BigShape<BN, NW> S;
  constexpr int BM = 256;
  static_assert(BK == 64 || (BK == 32 && GROUPING == GROUP_K && AMODE == MC && BMODE == MC),
                "32-deep slabs only for the weight gradients (both operands k-major)");
  constexpr int KS = BK / 16;        // 16-deep MFMA k-steps per slab
  constexpr int NI = S::NI, NJ = S::NJ, WTM = S::WTM, WTN = S::WTN;
  constexpr int ATILE = BM * BK * 2;  // bytes of the A slab
  constexpr int BTILE = BN * BK * 2;  // bytes of the B slab
  constexpr int A_PER_WAVE = ATILE / 1024 / NW;
  constexpr int B_PER_WAVE = BTILE / 1024 / NW;
  constexpr int CPRB = BN / 8;       // 16-byte chunks per k-row of an MC B slab
  static_assert(A_PER_WAVE * NW * 1024 == ATILE && B_PER_WAVE * NW * 1024 == BTILE, "split");
  // epilogue staging: 32 rows x WTN fp32 per wave, half the waves in each A slab
  static_assert((NW / 2) * 32 * WTN * 4 <= ATILE, "epilogue staging");
  __shared__ __attribute__((aligned(1024))) char sA0[ATILE];
  __shared__ __attribute__((aligned(1024))) char sB0[BTILE];
  __shared__ __attribute__((aligned(1024))) char sA1[ATILE];
  __shared__ __attribute__((aligned(1024))) char sB1[BTILE];
  const int64_t lin = remap_xcd(blockIdx.x, P.nblocks);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave / S::WNW, wn = wave % S::WNW;

  int g, m0, n0, rows_valid, kdim;
  int64_t arow0;
  int nrows_g = 0;
  if constexpr (GROUPING == GROUP_M) {
    int mt, nt, mtl;
    if (P.xcd_m) {
      if (!xcd_mblock_tile(blockIdx.x, P.offsets, P.G, BM, P.ntn, mt, nt, g, mtl)) return;
    } else {
      supercol_tile<kSuperColsM>(lin, P.mt_total, P.ntn, mt, nt);
      if (!find_group(P.offsets, P.G, mt, g, mtl, BM)) return;
    }
    g = __builtin_amdgcn_readfirstlane(g);
    mtl = __builtin_amdgcn_readfirstlane(mtl);
    nrows_g = P.offsets[g + 1] - P.offsets[g];
    m0 = mtl * BM;
    n0 = nt * BN;
    rows_valid = min(BM, nrows_g - m0);
    kdim = P.Kdim;
    arow0 = P.offsets[g];
  } else {
    const int64_t per = (int64_t)P.ntm * P.ntn;
    int64_t tl;
    groupk_tile(blockIdx.x, per, P.shared_rows > 0, P.G, g, tl);
    int mt, nt;
    supercol_tile<kSuperColsK>(tl, P.ntm, P.ntn, mt, nt);
    m0 = mt * BM;
    n0 = nt * BN;
    rows_valid = BM;
    kdim = P.offsets[g + 1] - P.offsets[g];
    arow0 = P.offsets[g];
  }

  // ---- A source: the group's rows (rows past the end read 0); descriptor
  // based at the tile's first row (row-major A) or per k-slab (k-major A)
  static_assert((GROUPING == GROUP_M) == (AMODE == KC), "A is row-major exactly for GROUP_M");
  const T* a_base = (g < P.EL_A) ? reinterpret_cast<const T*>(P.A) + arow0 * P.lda
                                 : reinterpret_cast<const T*>(P.A_sh);
  const int64_t a_rows = (GROUPING == GROUP_M) ? nrows_g : kdim;
  const rsrc_t a_rs_tile = rows_rsrc(a_base, (AMODE == KC) ? m0 : 0, a_rows, P.lda, P.a_cap);
  uint32_t a_off[A_PER_WAVE];
#pragma unroll
  for (int u = 0; u < A_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * A_PER_WAVE + u) + lane;
    if constexpr (AMODE == KC) {
      const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
      a_off[u] = (uint32_t)(((int64_t)r * P.lda + 8 * lc) * 2);
    } else {
      const int kr = P_ / 32, lc = (P_ % 32) ^ mcswz(kr);
      a_off[u] = (uint32_t)(((int64_t)kr * P.lda + m0 + 8 * lc) * 2);
    }
  }
  // ---- B source (GROUP_M: weights, per-lane global addresses; GROUP_K:
  // activation rows of the group through a buffer)
  const T* b_ptr[B_PER_WAVE];
  uint32_t b_off[B_PER_WAVE];
  const T* b_base = nullptr;  // GROUP_K: the group's activation rows (k-major)
  const T* Bw0 = reinterpret_cast<const T*>(P.B0) + (int64_t)g * P.strideB;
  const T* Bw1 = (BSPL != BS_NONE) ? reinterpret_cast<const T*>(P.B1) + (int64_t)g * P.strideB
                                   : nullptr;
  if constexpr (GROUPING == GROUP_M) {
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
      if constexpr (BMODE == KC) {
        const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
        b_ptr[u] = Bw0 + (int64_t)(n0 + r) * P.ldb + 8 * lc;
      } else {
        const int kr = P_ / CPRB, lc = (P_ % CPRB) ^ mcswz(kr);
        if constexpr (BSPL == BS_N) {
          const int col0 = n0 / 2;
          b_ptr[u] = (lc < CPRB / 2) ? Bw0 + (int64_t)kr * P.ldb + col0 + 8 * lc
                                     : Bw1 + (int64_t)kr * P.ldb + col0 + 8 * (lc - CPRB / 2);
        } else {
          b_ptr[u] = Bw0 + (int64_t)kr * P.ldb + n0 + 8 * lc;
        }
      }
    }
  } else {
    b_base = (g < P.EL_B) ? reinterpret_cast<const T*>(P.B0) + arow0 * P.ldb
                          : reinterpret_cast<const T*>(P.B1);
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
      const int kr = P_ / CPRB, lc = (P_ % CPRB) ^ mcswz(kr);
      b_off[u] = (uint32_t)(((int64_t)kr * P.ldb + n0 + 8 * lc) * 2);
    }
  }

  // DMA of slab kt.  Slabs at or past nk (the even padding and the two the
  // pipeline runs ahead at the end) load zeros for A -- an offset past the
  // buffer range reads 0 without touching memory (GROUP_K: B too, its rows
  // run out the same way) -- and, for GROUP_M, re-read the last weight slab:
  // any finite B times a zero A adds nothing.
  const int nk = (kdim + BK - 1) / BK;
  // (q_lo, q_hi: only the DMA instructions of that index range, A's first;
  // q_hi < 0: all of them)
  auto issue = [&](int kt, char* la, char* lb, int q_lo = 0, int q_hi = -1)
                   __attribute__((always_inline)) {
    if (q_hi < 0) q_hi = A_PER_WAVE + B_PER_WAVE;
    const bool pad = kt >= nk;
    const int k0 = (GROUPING == GROUP_M && pad) ? (nk - 1) * BK : kt * BK;
    // k-major operands: descriptors based at the slab's first row (a slab
    // past the group's rows gets an empty range and reads zeros)
    const rsrc_t a_rs =
        (AMODE == KC) ? a_rs_tile : rows_rsrc(a_base, k0, a_rows, P.lda, P.a_cap);
    rsrc_t b_rs = {0, 0, 0, 0};  // GROUP_K only: the slab's activation rows
    if constexpr (GROUPING == GROUP_K) b_rs = rows_rsrc(b_base, k0, kdim, P.ldb, P.b_cap);
    const uint32_t kadd = (AMODE == KC) ? (uint32_t)(k0 * 2) : 0u;
#pragma unroll
    for (int u = 0; u < A_PER_WAVE; ++u)
      if (u >= q_lo && u < q_hi)
        dma16_buffer(a_rs, to_lds(la + (wave * A_PER_WAVE + u) * 1024),
                     (GROUPING == GROUP_M && pad) ? 0x80000000u : a_off[u] + kadd);
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      if (A_PER_WAVE + u < q_lo || A_PER_WAVE + u >= q_hi) continue;
      char* dst = lb + (wave * B_PER_WAVE + u) * 1024;
      if constexpr (GROUPING == GROUP_M) {
        const T* src;
        if constexpr (BMODE == KC) {
          if constexpr (BSPL == BS_K) {
            src = (k0 < P.bsplit) ? b_ptr[u] + k0 : (b_ptr[u] - Bw0) + Bw1 + (k0 - P.bsplit);
          } else {
            src = b_ptr[u] + k0;
          }
        } else {
          src = b_ptr[u] + (int64_t)k0 * P.ldb;
        }
        dma16_global(src, to_lds(dst));
      } else {
        dma16_buffer(b_rs, to_lds(dst), b_off[u]);
      }
    }
  };

  // B-slab columns of this wave's blocks.  SwiGLU forward: the slab holds
  // [gate | up] halves; block j < NJ/2 is gate, j + NJ/2 the up block of the
  // same f's.
  int rb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      rb[j] = (j < NJ / 2) ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - NJ / 2) * 32;
    else
      rb[j] = wn * WTN + j * 32;
  }

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Software pipeline.  Fragments of k-step ks + 1 are read into the other
  // register slot while the MFMAs of k-step ks run.  The slab hand-over sits
  // inside the last k-step: wait for the next slab's DMA, barrier (every wave
  // has its last fragments of this slab in registers by then), start the DMA
  // two slabs ahead into the buffer just released, read the first fragments
  // of the next slab -- all while the MFMAs already issued keep the matrix
  // cores busy.  Scheduling barriers keep the compiler from moving the
  // reads and the DMA behind the MFMAs.
  uint4 fa[2][NI], fb[2][NJ];
  constexpr int PER_SLAB = A_PER_WAVE + B_PER_WAVE;  // DMA instructions per slab
  const int nkp = nk + (nk & 1);
  // The main loop for NB active 32-row blocks of the wave tile: a ragged
  // group's last tile computes (and reads A fragments for) only the blocks
  // that hold rows of the group; a wave with none still issues its DMA share
  // and joins every barrier.
  auto main_loop = [&](auto nb_c) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb_c)::value;
    auto frags = [&](const char* la, const char* lb, int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
        fa[slot][i] = (AMODE == KC) ? frag_kc(la, wm * WTM + i * 32, ks, lane)
                                    : frag_mc(const_cast<char*>(la), wm * WTM + i * 32, ks, lane, BM * 2);
      if constexpr (NB > 0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          fb[slot][j] = (BMODE == KC) ? frag_kc(lb, rb[j], ks, lane)
                                      : frag_mc(const_cast<char*>(lb), rb[j], ks, lane, BN * 2);
      }
    };
    auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, fb[slot][j]), __builtin_bit_cast(bf16x8_t, fa[slot][i]),
              acc[i][j], 0, 0, 0);
    };
    // Slab kt is in (la, lb) with its k-step 0 fragments in register slot 0;
    // slab kt + 1 is landing in (na, nb).  The body is branch-free: the slab
    // count is padded to even and the DMA runs on past the end (see issue).
    auto step = [&](int kt, char* la, char* lb, char* na, char* nb) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 1; ks < KS; ++ks) {
        frags(la, lb, ks, ks & 1);
        // (not for the K-split gate/up input gradient: 5.07 -> 5.32 ms on the
        // DeepSeek-V3-like layer with the reads interleaved)
        if constexpr (NB > 0 && BSPL != BS_K) {
          constexpr int RD = NB * (AMODE == KC ? 1 : 2) + NJ * (BMODE == KC ? 1 : 2);
          interleave_reads<NB * NJ, (RD + NB * NJ - 1) / (NB * NJ)>();
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas((ks - 1) & 1);
      }
      wait_vmcnt<0>();
      __syncthreads();
      // hand-over: the last k-step's MFMAs start right after the barrier,
      // with half the DMA ahead of the first, the rest ahead of the second,
      // and one fragment read of the next slab ahead of each later MFMA
      // (B fragments first: the next slab's first MFMA needs fb[0], fa[0]).
      // Against the DMA, the reads and then the MFMAs: down dgrad alone
      // 2.70 -> 2.65 ms (DeepSeek-V3-like), 3.06 -> 2.99 ms (Mixtral-like),
      // 0.321 -> 0.310 ms (OLMoE-like); the other GEMMs 0-1 % faster
      {
        constexpr int PS = A_PER_WAVE + B_PER_WAVE, D0 = (PS + 1) / 2;
        constexpr int M = NB * NJ, F = (NB > 0) ? NB + NJ : 0, sl = (KS - 1) & 1;
        auto mf = [&](int q) __attribute__((always_inline)) {
          if (q < M) {
            __builtin_amdgcn_sched_barrier(0);
            acc[q / NJ][q % NJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, fb[sl][q % NJ]),
                __builtin_bit_cast(bf16x8_t, fa[sl][q / NJ]), acc[q / NJ][q % NJ], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        issue(kt + 2, la, lb, 0, D0);
        mf(0);
        issue(kt + 2, la, lb, D0, PS);
        mf(1);
#pragma unroll
        for (int f = 0; f < F; ++f) {
          if (f < NJ)
            fb[0][f] = (BMODE == KC) ? frag_kc(nb, rb[f], 0, lane) : frag_mc(nb, rb[f], 0, lane, BN * 2);
          else
            fa[0][f - NJ] = (AMODE == KC) ? frag_kc(na, wm * WTM + (f - NJ) * 32, 0, lane)
                                          : frag_mc(na, wm * WTM + (f - NJ) * 32, 0, lane, BM * 2);
          mf(2 + f);
        }
#pragma unroll
        for (int q = 2 + F; q < M; ++q) mf(q);
      }
    };
    if (nkp > 0) {
      issue(0, sA0, sB0);
      issue(1, sA1, sB1);
      wait_vmcnt<PER_SLAB>();
      __syncthreads();
      frags(sA0, sB0, 0, 0);
    }
    for (int kt = 0; kt < nkp; kt += 2) {
      step(kt, sA0, sB0, sA1, sB1);
      step(kt + 1, sA1, sB1, sA0, sB0);
    }
  };
  if constexpr (GROUPING == GROUP_M) {
    // 32-row blocks of this wave's rows that hold group rows (uniform)
    const int nb = __builtin_amdgcn_readfirstlane(
        max(0, min(NI, (rows_valid - wm * WTM + 31) / 32)));
    if (nb >= NI) main_loop(std::integral_constant<int, NI>{});
    else if (nb == 0) main_loop(std::integral_constant<int, 0>{});
    else if (nb == 1) main_loop(std::integral_constant<int, 1>{});
    else if constexpr (NI > 2) {
      if (nb == 2) main_loop(std::integral_constant<int, 2>{});
      else main_loop(std::integral_constant<int, (NI > 3 ? 3 : NI)>{});
    }
  } else {
    main_loop(std::integral_constant<int, NI>{});
  }
  // the run-ahead DMA must land, and every wave be done with the slabs,
  // before the stage buffers are reused for the epilogue
  wait_vmcnt<0>();
  __syncthreads();

  // ---- epilogue.  Element r of block (i, j) is row l % 32 of block i and
  // column (r / 4) * 8 + (l / 32) * 4 + r % 4 of block j.  Each 32-row block
  // of the wave is staged in the wave's own LDS region (16-byte chunks
  // XOR-swizzled by row) and written back as row segments.
  char* reg = (wave < NW / 2 ? sA0 : sA1) + (wave % (NW / 2)) * (32 * WTN * 4);
  const int lrow = lane & 31, lcol = (lane >> 5) * 4;
  // bf16 staging of a [32][W] array at base: 4 values at (lrow, col); the
  // chunk swizzle stays inside the row (W / 8 chunks, at most 8 permuted)
  auto put4 = [&](char* base, int W, int col, const float* v) __attribute__((always_inline)) {
    const int ch = col >> 3, half = (col >> 2) & 1, msk = min(W / 8, 8) - 1;
    *reinterpret_cast<uint2*>(base + lrow * W * 2 + ((ch ^ (lrow & msk)) << 4) + (half << 3)) =
        pack_bf16x4(v);
  };
  auto get16 = [&](const char* base, int W, int row, int ch) __attribute__((always_inline)) {
    const int msk = min(W / 8, 8) - 1;
    return *reinterpret_cast<const uint4*>(base + row * W * 2 + ((ch ^ (row & msk)) << 4));
  };
  // SwiGLU backward: activation rows of 32-row block ib, 8 columns per lane
  constexpr int ACT_IT = (EPI == EPI_SWIGLU_BWD) ? 32 / (64 / (WTN / 8)) : 1;
  uint4 av[2][ACT_IT], bv[2][ACT_IT];
  auto load_act = [&](int ib, uint4* a, uint4* b) __attribute__((always_inline)) {
    constexpr int CPR = WTN / 8, RPI = 64 / CPR;
    const int f = n0 + wn * WTN + (lane % CPR) * 8;
#pragma unroll
    for (int it = 0; it < ACT_IT; ++it) {
      const int row_t = wm * WTM + ib * 32 + it * RPI + lane / CPR;
      if (row_t < rows_valid) {
        const T* act = reinterpret_cast<const T*>(P.act) + (arow0 + m0 + row_t) * 2 * P.F;
        a[it] = *reinterpret_cast<const uint4*>(act + f);
        b[it] = *reinterpret_cast<const uint4*>(act + P.F + f);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row_t0 = wm * WTM + i * 32;  // tile-relative first row of the block
    if (row_t0 >= rows_valid) break;       // uniform
    const int64_t grow0 = arow0 + m0 + row_t0;
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      constexpr int W = WTN / 2;            // f columns of the wave
      char* sa = reg;
      char* sb = reg + 32 * W * 2;
      char* sh = reg + 64 * W * 2;
#pragma unroll
      for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a[4], b[4], h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = acc[i][j][4 * q + e];
            b[e] = acc[i][j + NJ / 2][4 * q + e];
            h[e] = silu_f(a[e]) * b[e];
          }
          const int col = j * 32 + q * 8 + lcol;
          put4(sa, W, col, a);
          put4(sb, W, col, b);
          put4(sh, W, col, h);
        }
      constexpr int CPR = W / 8, RPI = 64 / CPR;
      const int ch = lane % CPR;
      const int f = n0 / 2 + wn * W + ch * 8;
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + lane / CPR;
        if (row_t0 + row >= rows_valid) continue;
        const int64_t grow = grow0 + row;
        T* aout = reinterpret_cast<T*>(P.act_out) + grow * 2 * P.F;
        *reinterpret_cast<uint4*>(aout + f) = get16(sa, W, row, ch);
        *reinterpret_cast<uint4*>(aout + P.F + f) = get16(sb, W, row, ch);
        *reinterpret_cast<uint4*>(reinterpret_cast<T*>(P.C1) + grow * P.F + f) = get16(sh, W, row, ch);
      }
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      // dh stays fp32: 16-byte chunks of 4 floats, swizzled by row.  The
      // activations of block i + 1 are loaded while block i is processed
      // (those of block 0 before the loop), so their latency overlaps.
      constexpr int CPR = WTN / 8, RPI = 64 / CPR;   // lanes per row: 8 columns each
      const int ch = lane % CPR;
      const int f = n0 + wn * WTN + ch * 8;
      if (i == 0) load_act(0, av[0], bv[0]);
      if (i + 1 < NI) load_act(i + 1, av[(i + 1) & 1], bv[(i + 1) & 1]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c4 = (j * 32 + q * 8 + lcol) >> 2;
          *reinterpret_cast<float4*>(reg + lrow * WTN * 4 + ((c4 ^ (lrow & 15)) << 4)) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]);
        }
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + lane / CPR;
        if (row_t0 + row >= rows_valid) continue;
        float v[8], a[8], b[8], da[8], db[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int c4 = 2 * ch + hh;
          const float4 d = *reinterpret_cast<const float4*>(reg + row * WTN * 4 + ((c4 ^ (row & 15)) << 4));
          v[4 * hh] = d.x; v[4 * hh + 1] = d.y; v[4 * hh + 2] = d.z; v[4 * hh + 3] = d.w;
        }
        Vec16<T> va, vb;
        va.v = av[i & 1][it];
        vb.v = bv[i & 1][it];
        va.to_f32(a);
        vb.to_f32(b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = sigmoid_hw(a[e]);
          da[e] = v[e] * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
          db[e] = v[e] * a[e] * sg;
        }
        T* dact = reinterpret_cast<T*>(P.C0) + (grow0 + row) * 2 * P.F;
        Vec16<T> oa, ob;
        oa.from_f32(da);
        ob.from_f32(db);
        oa.store(dact + f);
        ob.store(dact + P.F + f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          put4(reg, WTN, j * 32 + q * 8 + lcol, v);
        }
      constexpr int CPR = WTN / 8, RPI = 64 / CPR;
      const int ch = lane % CPR;
      const int col = n0 + wn * WTN + ch * 8;  // output column of the chunk
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + lane / CPR;
        if (row_t0 + row >= rows_valid) continue;
        const uint4 v = get16(reg, WTN, row, ch);
        if constexpr (GROUPING == GROUP_M) {
          *reinterpret_cast<uint4*>(reinterpret_cast<T*>(P.C0) + (grow0 + row) * P.ldc + col) = v;
        } else {
          // weight gradients: streaming stores.  dW is written once and not
          // read again by this layer; cached stores displaced the operand
          // slabs the other tiles of the group re-read from L2 (DeepSeek-V3-
          // like layer: operand fetches 5.9 GB per launch without the dW
          // stores, 8.1 GB with them; gate/up weight gradient 6.81 -> 6.60
          // ms, down 3.45 -> 3.31 ms)
          const int64_t mrow = m0 + row_t0 + row;
          T* C = (col < P.csplit)
                     ? reinterpret_cast<T*>(P.C0) + (int64_t)g * P.strideC + mrow * P.ldc + col
                     : reinterpret_cast<T*>(P.C1) + (int64_t)g * P.strideC + mrow * P.ldc +
                           (col - P.csplit);
          Vec16<T> o;
          o.v = v;
          o.store_nt(C);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent large tiles: the same 256 x BN tile and 8-wave main loop as
// grouped_gemm_big_kernel, but each workgroup walks a strided list of tiles
// and the DMA pipeline runs straight across tile boundaries: the two slabs
// the loop fetches ahead at the end of a tile are the first two slabs of the
// workgroup's next tile, so they land while the epilogue of the current tile
// runs.  The epilogue therefore stages through an LDS region of its own (4 KB
// per wave; the SwiGLU epilogues in two 16-row passes), not the stage
// buffers.  Tile state is uniform (scalars); per-lane DMA offsets are fixed
// for the whole kernel.  Every tile runs at least two slabs (padding), which
// keeps the hand-over identical for empty weight-gradient groups.
// ---------------------------------------------------------------------------
template <int AMODE, int BMODE, int GROUPING, int EPI, int BSPL, int BN>
__global__ __launch_bounds__(512) void grouped_gemm_persist_kernel(GemmParams P) {
  typedef bf16_t T;
  constexpr int NW = 8;
  typedef BigShape<BN, NW> S;
  constexpr int BM = 256, BK = 64;
  constexpr int NI = S::NI, NJ = S::NJ, WTM = S::WTM, WTN = S::WTN;
  constexpr int ATILE = BM * 128, BTILE = BN * 128;
  constexpr int A_PER_WAVE = ATILE / 1024 / NW, B_PER_WAVE = BTILE / 1024 / NW;
  constexpr int CPRB = BN / 8;
  constexpr int EREG = 4096;  // epilogue staging bytes per wave
  static_assert(WTN == 64, "epilogue staging sized for 64-column wave tiles");
  // one LDS object: the two A stages side by side, then the two B stages, so
  // a stage-1 fragment address is the stage-0 one plus an offset that fits
  // the ds_read immediate (no second address register per fragment)
  __shared__ __attribute__((aligned(1024))) char smem[2 * ATILE + 2 * BTILE + NW * EREG];
  char* const sA0 = smem;
  char* const sA1 = smem + ATILE;
  char* const sB0 = smem + 2 * ATILE;
  char* const sB1 = smem + 2 * ATILE + BTILE;
  char* const sE = smem + 2 * ATILE + 2 * BTILE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave / S::WNW, wn = wave % S::WNW;

  // ---- number of real tiles (GROUP_M: from the group sizes)
  int64_t n_tiles;
  int mt_real = 0;
  if constexpr (GROUPING == GROUP_M) {
    const int gpl = (P.G + 63) / 64;
    int mine = 0;
    for (int j = 0; j < gpl; ++j) {
      const int g = lane * gpl + j;
      if (g < P.G) mine += (P.offsets[g + 1] - P.offsets[g] + BM - 1) / BM;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
    mt_real = __builtin_amdgcn_readfirstlane(mine);
    n_tiles = (int64_t)mt_real * P.ntn;
  } else {
    n_tiles = (int64_t)P.G * P.ntm * P.ntn;
  }
  // GROUP_M: tiles blockIdx.x, + gridDim.x, ... (XCD-remapped).  GROUP_K:
  // the cost-balanced range of this workgroup's XCD, tiles w, w + nw, ... of
  // it (w = blockIdx.x / 8 of the nw = gridDim.x / 8 workgroups on the XCD)
  // GROUP_K: virtual tiles 0 .. nsh + (rt1 - rt0) of this workgroup's XCD --
  // its share [sh0, sh0 + nsh) of the shared expert's tiles, then its
  // routed range [rt0, rt1) -- tiles w, w + nw, ... of them (w =
  // blockIdx.x / 8 of the nw = gridDim.x / 8 workgroups on the XCD)
  int64_t nwg = gridDim.x, j_end = n_tiles;
  int64_t j = blockIdx.x;
  int64_t sh0 = 0, nsh = 0, rt0 = 0;
  if constexpr (GROUPING == GROUP_K) {
    const int64_t per = (int64_t)P.ntm * P.ntn;
    const int x = (int)(blockIdx.x % 8);
    const bool shared = P.shared_rows > 0;
    if (shared) {
      sh0 = per * x / 8;
      nsh = per * (x + 1) / 8 - sh0;
    }
    int64_t rt1;
    groupk_xcd_range(P.offsets, P.G - (shared ? 1 : 0), per, x, rt0, rt1);
    nwg = gridDim.x / 8;
    j = blockIdx.x / 8;
    j_end = nsh + (rt1 - rt0);
  }
  if (j >= j_end) return;

  // ---- per-lane DMA offsets, fixed for the kernel
  uint32_t a_lane[A_PER_WAVE];
#pragma unroll
  for (int u = 0; u < A_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * A_PER_WAVE + u) + lane;
    if constexpr (AMODE == KC) {
      const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
      a_lane[u] = (uint32_t)(((int64_t)r * P.lda + 8 * lc) * 2);
    } else {
      const int kr = P_ / 32, lc = (P_ % 32) ^ mcswz(kr);
      a_lane[u] = (uint32_t)(((int64_t)kr * P.lda + 8 * lc) * 2);
    }
  }
  int32_t b_lane[B_PER_WAVE];  // elements (GROUP_M) or bytes (GROUP_K)
  bool b_hi[B_PER_WAVE];       // BS_N: chunk from the second (up) matrix
#pragma unroll
  for (int u = 0; u < B_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
    b_hi[u] = false;
    if constexpr (GROUPING == GROUP_M) {
      if constexpr (BMODE == KC) {
        const int r = P_ >> 3, lc = (P_ & 7) ^ swz(r);
        b_lane[u] = r * P.ldb + 8 * lc;
      } else {
        const int kr = P_ / CPRB, lc = (P_ % CPRB) ^ mcswz(kr);
        if constexpr (BSPL == BS_N) {
          b_hi[u] = lc >= CPRB / 2;
          b_lane[u] = kr * P.ldb + 8 * (lc % (CPRB / 2));
        } else {
          b_lane[u] = kr * P.ldb + 8 * lc;
        }
      }
    } else {
      const int kr = P_ / CPRB, lc = (P_ % CPRB) ^ mcswz(kr);
      b_lane[u] = (kr * P.ldb + 8 * lc) * 2;
    }
  }

  // ---- tile state (uniform)
  struct Tile {
    int g, m0, n0, rows_valid, nk, kdim;
    int64_t arow0, a_rows;
    bool real;
    const T* a_base;               // the group's A rows
    const T* b_base;               // GROUP_K: the group's B rows
    rsrc_t a_rs;   // row-major A: based at the tile's first row
  };
  auto decode = [&](int64_t j, bool real) __attribute__((always_inline)) {
    Tile t;
    t.real = real;
    const int64_t lin = (GROUPING == GROUP_M) ? remap_xcd(j, n_tiles) : j;
    int kdim, nrows_g = 0;
    if constexpr (GROUPING == GROUP_M) {
      int mt, nt, mtl, g;
      supercol_tile<kSuperColsM>(lin, mt_real, P.ntn, mt, nt);
      find_group(P.offsets, P.G, mt, g, mtl, BM);
      t.g = __builtin_amdgcn_readfirstlane(g);
      mtl = __builtin_amdgcn_readfirstlane(mtl);
      nrows_g = group_offset(P.offsets, t.g + 1) - group_offset(P.offsets, t.g);
      t.m0 = mtl * BM;
      t.n0 = nt * BN;
      t.rows_valid = min(BM, nrows_g - t.m0);
      kdim = P.Kdim;
    } else {
      const int64_t per = (int64_t)P.ntm * P.ntn;
      int64_t tl;
      if (j < nsh) {
        t.g = P.G - 1;
        tl = sh0 + j;
      } else {
        const int64_t r = rt0 + (j - nsh);
        t.g = (int)(r / per);
        tl = r - (int64_t)t.g * per;
      }
      int mt, nt;
      supercol_tile<kSuperColsK>(tl, P.ntm, P.ntn, mt, nt);
      t.m0 = mt * BM;
      t.n0 = nt * BN;
      t.rows_valid = BM;
      kdim = group_offset(P.offsets, t.g + 1) - group_offset(P.offsets, t.g);
    }
    t.arow0 = group_offset(P.offsets, t.g);
    t.kdim = kdim;
    t.nk = max(2, (kdim + BK - 1) / BK);
    t.nk += t.nk & 1;  // even: the next tile's slab 0 always lands in stage 0
    t.a_base = (t.g < P.EL_A) ? reinterpret_cast<const T*>(P.A) + t.arow0 * P.lda
                              : reinterpret_cast<const T*>(P.A_sh);
    t.a_rows = (GROUPING == GROUP_M) ? nrows_g : kdim;
    t.a_rs = rows_rsrc(t.a_base, (AMODE == KC) ? t.m0 : 0, t.a_rows, P.lda, P.a_cap);
    t.b_base = nullptr;
    if constexpr (GROUPING == GROUP_K)
      t.b_base = (t.g < P.EL_B) ? reinterpret_cast<const T*>(P.B0) + t.arow0 * P.ldb
                                : reinterpret_cast<const T*>(P.B1);
    // slabs holding real data: the rest of the (padded) slab count reads 0
    t.rows_valid = real ? t.rows_valid : 0;
    return t;
  };
  // real k-slabs of a tile (for GROUP_M: Kdim / BK; GROUP_K: the group rows)
  auto real_slabs = [&](const Tile& t) __attribute__((always_inline)) {
    if constexpr (GROUPING == GROUP_M) return (P.Kdim + BK - 1) / BK;
    else return (t.kdim + BK - 1) / BK;
  };

  // DMA of slab s of tile t into (la, lb); slabs past the real ones read
  // zeros for A (offset past the buffer range; GROUP_K: B too) and, for
  // GROUP_M, re-read the tile's last weight slab (times a zero A: nothing)
  auto issue = [&](const Tile& t, int nreal, int s, char* la, char* lb) __attribute__((always_inline)) {
    if constexpr (GROUPING == GROUP_K) {
      // both operands k-major: descriptors based at the slab's first row, the
      // tile's column offset in soffset, the per-lane offsets fixed for the
      // kernel; a slab past the group's rows, and every slab of the padding
      // tile, gets an empty range and reads zeros
      const int rows = t.real ? t.kdim : 0;
      const rsrc_t a_rs = rows_rsrc(t.a_base, s * BK, rows, P.lda, P.a_cap);
      const rsrc_t b_rs = rows_rsrc(t.b_base, s * BK, rows, P.ldb, P.b_cap);
      const uint32_t a_so = __builtin_amdgcn_readfirstlane(t.m0 * 2);
      const uint32_t b_so = __builtin_amdgcn_readfirstlane(t.n0 * 2);
#pragma unroll
      for (int u = 0; u < A_PER_WAVE; ++u)
        dma16_buffer_so(a_rs, to_lds(la + (wave * A_PER_WAVE + u) * 1024), a_lane[u], a_so);
#pragma unroll
      for (int u = 0; u < B_PER_WAVE; ++u)
        dma16_buffer_so(b_rs, to_lds(lb + (wave * B_PER_WAVE + u) * 1024), (uint32_t)b_lane[u], b_so);
      return;
    }
    const bool pad = !t.real || s >= nreal;
    const int k0 = (GROUPING == GROUP_M && pad) ? max(nreal - 1, 0) * BK : s * BK;
    // row-major A: tile-based descriptor plus the k offset; k-major A: a
    // descriptor based at the slab's first row plus the tile's m offset
    const rsrc_t a_rs =
        (AMODE == KC) ? t.a_rs : rows_rsrc(t.a_base, k0, t.a_rows, P.lda, P.a_cap);
    const uint32_t tbase = (AMODE == KC) ? 0u : (uint32_t)(t.m0 * 2);
    const uint32_t kadd = (AMODE == KC) ? (uint32_t)(k0 * 2) : 0u;
    rsrc_t b_rs = {0, 0, 0, 0};  // GROUP_K only: the slab's activation rows
    if constexpr (GROUPING == GROUP_K) b_rs = rows_rsrc(t.b_base, k0, t.kdim, P.ldb, P.b_cap);
#pragma unroll
    for (int u = 0; u < A_PER_WAVE; ++u)
      dma16_buffer(a_rs, to_lds(la + (wave * A_PER_WAVE + u) * 1024),
                   pad ? 0x80000000u : tbase + a_lane[u] + kadd);
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u) {
      char* dst = lb + (wave * B_PER_WAVE + u) * 1024;
      if constexpr (GROUPING == GROUP_M) {
        const T* Bw0 = reinterpret_cast<const T*>(P.B0) + (int64_t)t.g * P.strideB;
        const T* src;
        if constexpr (BMODE == KC) {
          const T* row = Bw0 + (int64_t)t.n0 * P.ldb + b_lane[u];
          if constexpr (BSPL == BS_K) {
            const T* Bw1 = reinterpret_cast<const T*>(P.B1) + (int64_t)t.g * P.strideB;
            src = (k0 < P.bsplit) ? row + k0 : (row - Bw0) + Bw1 + (k0 - P.bsplit);
          } else {
            src = row + k0;
          }
        } else {
          if constexpr (BSPL == BS_N) {
            const T* Bw1 = reinterpret_cast<const T*>(P.B1) + (int64_t)t.g * P.strideB;
            src = (b_hi[u] ? Bw1 : Bw0) + t.n0 / 2 + b_lane[u] + (int64_t)k0 * P.ldb;
          } else {
            src = Bw0 + t.n0 + b_lane[u] + (int64_t)k0 * P.ldb;
          }
        }
        dma16_global(src, to_lds(dst));
      } else {
        dma16_buffer(b_rs, to_lds(dst), pad ? 0x80000000u : (uint32_t)(t.n0 * 2 + b_lane[u]));
      }
    }
  };

  int rb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      rb[j] = (j < NJ / 2) ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - NJ / 2) * 32;
    else
      rb[j] = wn * WTN + j * 32;
  }
  f32x16_t acc[NI][NJ];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  uint4 fa[2][NI], fb[2][NJ];
  auto frags = [&](const char* la, const char* lb, int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      fa[slot][i] = (AMODE == KC) ? frag_kc(la, wm * WTM + i * 32, ks, lane)
                                  : frag_mc(const_cast<char*>(la), wm * WTM + i * 32, ks, lane, BM * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[slot][j] = (BMODE == KC) ? frag_kc(lb, rb[j], ks, lane)
                                  : frag_mc(const_cast<char*>(lb), rb[j], ks, lane, BN * 2);
  };
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, fb[slot][j]), __builtin_bit_cast(bf16x8_t, fa[slot][i]),
            acc[i][j], 0, 0, 0);
  };
  constexpr int PER_SLAB = A_PER_WAVE + B_PER_WAVE;
  // vector-memory instructions each wave issues in a tile's epilogue (a
  // lower bound): the weight gradients store every row of the tile, four
  // 16-byte chunks per lane and 32-row block; the row GEMMs skip rows past
  // the group's end, so nothing is counted for them
  constexpr int EPI_VM = (GROUPING == GROUP_K && EPI == EPI_STORE) ? NI * 4 : 0;

  Tile cur = decode(j, true);
  int cur_real = real_slabs(cur);
  Tile nxt;
  int nxt_real = 0;
  issue(cur, cur_real, 0, sA0, sB0);
  issue(cur, cur_real, 1, sA1, sB1);
  wait_vmcnt<PER_SLAB>();
  lds_barrier();
  frags(sA0, sB0, 0, 0);
  zero_acc();
  bool after_epi = false;  // this tile follows an epilogue of the workgroup

  // k-steps 1..3 of the slab in (la, lb), the fragments one k-step ahead of
  // the MFMAs (see grouped_gemm_big_kernel)
  auto body = [&](char* la, char* lb) __attribute__((always_inline)) {
    frags(la, lb, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
    frags(la, lb, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    frags(la, lb, 3, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0);
  };
  // hand-over from slab kt (in la, lb) to slab kt + 1 (in na, nb): wait for
  // slab kt + 1 -- at the first hand-over after an epilogue, the epilogue's
  // stores were issued after it and may stay in flight -- then barrier, DMA
  // slab kt + 2 (the next tile's slab 0 once the current one runs out) into
  // the stage just released, first fragments of slab kt + 1
  auto hand = [&](int kt, bool first, char* la, char* lb, char* na, char* nb)
                  __attribute__((always_inline)) {
    if (first) wait_vmcnt<EPI_VM>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (kt + 2 < cur.nk) issue(cur, cur_real, kt + 2, la, lb);
    else issue(nxt, nxt_real, kt + 2 - cur.nk, la, lb);
    frags(na, nb, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
  };

  const int lrow = lane & 31, lcol = (lane >> 5) * 4;
  char* reg = sE + wave * EREG;
  // bf16 staging of a [rows][W] array at base (chunk swizzle inside the row)
  auto put4 = [&](char* base, int W, int row, int col, const float* v) __attribute__((always_inline)) {
    const int ch = col >> 3, half = (col >> 2) & 1, msk = min(W / 8, 8) - 1;
    *reinterpret_cast<uint2*>(base + row * W * 2 + ((ch ^ (row & msk)) << 4) + (half << 3)) =
        pack_bf16x4(v);
  };
  auto get16 = [&](const char* base, int W, int row, int ch) __attribute__((always_inline)) {
    const int msk = min(W / 8, 8) - 1;
    return *reinterpret_cast<const uint4*>(base + row * W * 2 + ((ch ^ (row & msk)) << 4));
  };

  for (;;) {
    // slab pairs of cur (nk is even); the last pair is peeled
    int kt = 0;
    for (; kt + 2 < cur.nk; kt += 2) {
      body(sA0, sB0);
      hand(kt, after_epi && kt == 0, sA0, sB0, sA1, sB1);
      body(sA1, sB1);
      hand(kt + 1, false, sA1, sB1, sA0, sB0);
    }
    // last pair: the next tile (or, past the list, a padding tile that
    // reads zeros) is decoded; its slab 0 goes into stage 0 at the first
    // hand-over, its slab 1 into stage 1 as soon as every wave has read the
    // last slab -- no wait for it: the epilogue comes first
    const bool more = j + nwg < j_end;
    nxt = more ? decode(j + nwg, true) : decode(j, false);
    nxt_real = real_slabs(nxt);
    body(sA0, sB0);
    hand(kt, after_epi && kt == 0, sA0, sB0, sA1, sB1);
    body(sA1, sB1);
    lds_barrier();
    issue(nxt, nxt_real, 1, sA1, sB1);
    mfmas(1);
  // ---- epilogue of cur (its own LDS region; the next tile's first slabs
    // are landing meanwhile)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row_t0 = wm * WTM + i * 32;
      // (a weight-gradient tile stores all its rows: its stores are counted)
      if (GROUPING == GROUP_M && row_t0 >= cur.rows_valid) break;
      const int64_t grow0 = cur.arow0 + cur.m0 + row_t0;
      if constexpr (EPI == EPI_SWIGLU_FWD) {
        constexpr int W = WTN / 2;  // 32 f columns
        char* sa = reg;
        char* sb = reg + 16 * W * 2;
        char* sh = reg + 32 * W * 2;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          if ((lrow >> 4) == pass) {
#pragma unroll
            for (int jj = 0; jj < NJ / 2; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float a[4], b[4], h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  a[e] = acc[i][jj][4 * q + e];
                  b[e] = acc[i][jj + NJ / 2][4 * q + e];
                  h[e] = silu_f(a[e]) * b[e];
                }
                const int col = jj * 32 + q * 8 + lcol;
                put4(sa, W, lrow & 15, col, a);
                put4(sb, W, lrow & 15, col, b);
                put4(sh, W, lrow & 15, col, h);
              }
          }
          // 16 rows x 4 chunks: one row per 4 lanes
          const int row = lane >> 2, ch = lane & 3;
          const int rt = row_t0 + pass * 16 + row;
          if (rt < cur.rows_valid) {
            const int64_t grow = cur.arow0 + cur.m0 + rt;
            const int f = cur.n0 / 2 + wn * W + ch * 8;
            T* aout = reinterpret_cast<T*>(P.act_out) + grow * 2 * P.F;
            *reinterpret_cast<uint4*>(aout + f) = get16(sa, W, row, ch);
            *reinterpret_cast<uint4*>(aout + P.F + f) = get16(sb, W, row, ch);
            *reinterpret_cast<uint4*>(reinterpret_cast<T*>(P.C1) + grow * P.F + f) =
                get16(sh, W, row, ch);
          }
        }
      } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        // dh in fp32, 16 rows per pass: 8 lanes per row (8 columns each)
        const int ch = lane & 7, rsub = lane >> 3;  // rows rsub and rsub + 8 of the pass
        const int f = cur.n0 + wn * WTN + ch * 8;
        uint4 av[2][2], bv[2][2];
        auto load_pass = [&](int pass, uint4* a, uint4* b) __attribute__((always_inline)) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int rt = row_t0 + pass * 16 + h2 * 8 + rsub;
            if (rt < cur.rows_valid) {
              const T* act = reinterpret_cast<const T*>(P.act) + (cur.arow0 + cur.m0 + rt) * 2 * P.F;
              a[h2] = *reinterpret_cast<const uint4*>(act + f);
              b[h2] = *reinterpret_cast<const uint4*>(act + P.F + f);
            }
          }
        };
        load_pass(0, av[0], bv[0]);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          if (pass == 0) load_pass(1, av[1], bv[1]);
          if ((lrow >> 4) == pass) {
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int c4 = (jj * 32 + q * 8 + lcol) >> 2;
                const int r16 = lrow & 15;
                *reinterpret_cast<float4*>(reg + r16 * WTN * 4 + ((c4 ^ r16) << 4)) =
                    make_float4(acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2],
                                acc[i][jj][4 * q + 3]);
              }
          }
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int r16 = h2 * 8 + rsub;
            const int rt = row_t0 + pass * 16 + r16;
            if (rt >= cur.rows_valid) continue;
            float v[8], a[8], b[8], da[8], db[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int c4 = 2 * ch + hh;
              const float4 d = *reinterpret_cast<const float4*>(reg + r16 * WTN * 4 + ((c4 ^ r16) << 4));
              v[4 * hh] = d.x; v[4 * hh + 1] = d.y; v[4 * hh + 2] = d.z; v[4 * hh + 3] = d.w;
            }
            Vec16<T> va, vb;
            va.v = av[pass][h2];
            vb.v = bv[pass][h2];
            va.to_f32(a);
            vb.to_f32(b);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float sg = sigmoid_hw(a[e]);
              da[e] = v[e] * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
              db[e] = v[e] * a[e] * sg;
            }
            T* dact = reinterpret_cast<T*>(P.C0) + (cur.arow0 + cur.m0 + rt) * 2 * P.F;
            Vec16<T> oa, ob;
            oa.from_f32(da);
            ob.from_f32(db);
            oa.store(dact + f);
            ob.store(dact + P.F + f);
          }
        }
      } else {
        // 32 rows x 64 columns of bf16 in one pass
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][jj][4 * q + e];
            put4(reg, WTN, lrow, jj * 32 + q * 8 + lcol, v);
          }
        const int ch = lane & 7;
        const int col = cur.n0 + wn * WTN + ch * 8;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int row = it * 8 + (lane >> 3);
          if (GROUPING == GROUP_M && row_t0 + row >= cur.rows_valid) continue;
          const uint4 v = get16(reg, WTN, row, ch);
          if constexpr (GROUPING == GROUP_M) {
            *reinterpret_cast<uint4*>(reinterpret_cast<T*>(P.C0) + (grow0 + row) * P.ldc + col) = v;
          } else {
            const int64_t mrow = cur.m0 + row_t0 + row;
            T* Cp = (col < P.csplit)
                        ? reinterpret_cast<T*>(P.C0) + (int64_t)cur.g * P.strideC + mrow * P.ldc + col
                        : reinterpret_cast<T*>(P.C1) + (int64_t)cur.g * P.strideC + mrow * P.ldc +
                              (col - P.csplit);
            *reinterpret_cast<uint4*>(Cp) = v;
          }
        }
      }
    }
    if (!more) break;
    j += nwg;
    cur = nxt;
    cur_real = nxt_real;
    // the next tile's slab 0 has landed once at most its slab 1 and the
    // epilogue's stores (issued after it) are outstanding
    wait_vmcnt<PER_SLAB + EPI_VM>();
    lds_barrier();
    frags(sA0, sB0, 0, 0);
    zero_acc();
    after_epi = true;
  }
  // the run-ahead DMA (padding) must land before the LDS is released
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Weight gradients (both operands k-major) on 256 x 256 tiles with the next
// tile's first slabs fetched during the current tile's epilogue.  One
// workgroup per CU takes tiles w, w + W, w + 2 W, ... of the round-robin
// weight-gradient order (W = gridDim.x = 256 whenever there are that many
// tiles, a multiple of 8, so tile t still runs on XCD t mod 8 and every XCD
// keeps an equal share of every group; placement only, not correctness).
// The main loop is grouped_gemm_big_kernel's; its run-ahead DMA (the two
// slabs past a tile's end) loads slabs 0 and 1 of the workgroup's next
// tile, so the next tile starts with slab 0 in LDS instead of paying a full
// DMA round trip (each tile of a routed expert runs only four or five
// slabs).  The epilogue stages through a 32 KB LDS region of its own (4 KB of
// bf16 per wave), not the stage buffers.  Per-lane DMA offsets are fixed for
// the kernel and a tile's column offsets go in soffset, so the hand-over
// needs no vector registers: the tile state is scalar.  A tile of an empty
// group runs no main loop: it stores its zero accumulators through the same
// epilogue and then issues the next tile's first slabs.  Ordering: vector
// loads and stores retire in issue order on one counter; a tile that waits
// for its own slab 0 issued it after the previous epilogue's stores, so that
// wait also covers them.
// ---------------------------------------------------------------------------
struct WgTile {
  int g, m0, n0, kdim, nkp;
  const bf16_t* a;  // the group's k-major A rows
  const bf16_t* b;  // the group's k-major B rows
};

// BK-deep slabs through NS stages (64 x 2 or 32 x 4: 128 KB either way).
template <int BK, int NS>
__global__ __launch_bounds__(512) void grouped_gemm_wgrad_loop_kernel(GemmParams P) {
  typedef bf16_t T;
  typedef BigShape<256, 8> S;
  constexpr int BM = 256, BN = 256, NW = 8, KS = BK / 16;
  static_assert((BK == 64 && NS == 2) || (BK == 32 && NS == 4), "stages");
  constexpr int NI = S::NI, NJ = S::NJ, WTM = S::WTM, WTN = S::WTN;
  constexpr int ATILE = BM * BK * 2, BTILE = BN * BK * 2;
  constexpr int A_PER_WAVE = ATILE / 1024 / NW, B_PER_WAVE = BTILE / 1024 / NW;
  constexpr int PER_SLAB = A_PER_WAVE + B_PER_WAVE;  // DMA instructions per slab and wave
  constexpr int CPRB = BN / 8;
  constexpr int EWAVE = 32 * WTN * 2;  // epilogue staging bytes per wave
  constexpr int NSTORE = NI * 4;       // epilogue store instructions per wave
  static_assert(NS * (ATILE + BTILE) + NW * EWAVE <= 160 * 1024, "LDS");
  static_assert((NS - 2) * PER_SLAB + NSTORE < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char sA[NS][ATILE];
  __shared__ __attribute__((aligned(1024))) char sB[NS][BTILE];
  __shared__ __attribute__((aligned(1024))) char sE[NW * EWAVE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave / S::WNW, wn = wave % S::WNW;
  const int64_t per = (int64_t)P.ntm * P.ntn;
  const int64_t n_tiles = (int64_t)P.G * per;
  const bool shared = P.shared_rows > 0;
  int64_t t = blockIdx.x;
  if (t >= n_tiles) return;

  // per-lane DMA offsets (bytes) within a slab, tile-independent
  uint32_t a_lane[A_PER_WAVE], b_lane[B_PER_WAVE];
#pragma unroll
  for (int u = 0; u < A_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * A_PER_WAVE + u) + lane;
    const int kr = P_ / 32, lc = (P_ % 32) ^ mcswz(kr);
    a_lane[u] = (uint32_t)(((int64_t)kr * P.lda + 8 * lc) * 2);
  }
#pragma unroll
  for (int u = 0; u < B_PER_WAVE; ++u) {
    const int P_ = 64 * (wave * B_PER_WAVE + u) + lane;
    const int kr = P_ / CPRB, lc = (P_ % CPRB) ^ mcswz(kr);
    b_lane[u] = (uint32_t)(((int64_t)kr * P.ldb + 8 * lc) * 2);
  }
  // tile tt of the order of groupk_tile + supercol_tile<2>, in 32-bit
  // scalar arithmetic (the host keeps n_tiles below 2^31)
  static_assert(kSuperColsK == 2, "two-column super-columns");
  const uint32_t uper = (uint32_t)per, span = 2u * (uint32_t)P.ntm;
  const uint32_t full = (uint32_t)P.ntn / 2;
  auto tile_of = [&](int64_t tt, WgTile& w) __attribute__((always_inline)) {
    const uint32_t b = (uint32_t)tt, sh = shared ? uper : 0u;
    uint32_t g, tl;
    if (b < sh) {
      g = (uint32_t)P.G - 1;
      tl = b;
    } else {
      g = udiv_magic(b - sh, uper, P.per_magic);
      tl = b - sh - g * uper;
    }
    const uint32_t sc = udiv_magic(tl, span, P.span_magic);
    uint32_t mt, nt;
    if (sc < full) {
      const uint32_t q = tl - sc * span;
      mt = q >> 1;
      nt = sc * 2 + (q & 1);
    } else {  // the last, single column (odd ntn)
      mt = tl - full * span;
      nt = full * 2;
    }
    w.g = __builtin_amdgcn_readfirstlane((int)g);
    w.m0 = __builtin_amdgcn_readfirstlane((int)mt * BM);
    w.n0 = __builtin_amdgcn_readfirstlane((int)nt * BN);
    const int r0 = group_offset(P.offsets, w.g), r1 = group_offset(P.offsets, w.g + 1);
    w.kdim = r1 - r0;
    const int nk = (w.kdim + BK - 1) / BK;
    w.nkp = (nk + NS - 1) / NS * NS;
    w.a = (w.g < P.EL_A) ? reinterpret_cast<const T*>(P.A) + (int64_t)r0 * P.lda
                         : reinterpret_cast<const T*>(P.A_sh);
    w.b = (w.g < P.EL_B) ? reinterpret_cast<const T*>(P.B0) + (int64_t)r0 * P.ldb
                         : reinterpret_cast<const T*>(P.B1);
  };
  // slab kt of tile w (rows at or past its k extent read zeros)
  auto issue = [&](int kt, const WgTile& w, char* la, char* lb) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const rsrc_t a_rs = rows_rsrc(w.a, k0, w.kdim, P.lda, P.a_cap);
    const rsrc_t b_rs = rows_rsrc(w.b, k0, w.kdim, P.ldb, P.b_cap);
#pragma unroll
    for (int u = 0; u < A_PER_WAVE; ++u)
      dma16_buffer_so(a_rs, to_lds(la + (wave * A_PER_WAVE + u) * 1024), a_lane[u],
                      (uint32_t)(w.m0 * 2));
#pragma unroll
    for (int u = 0; u < B_PER_WAVE; ++u)
      dma16_buffer_so(b_rs, to_lds(lb + (wave * B_PER_WAVE + u) * 1024), b_lane[u],
                      (uint32_t)(w.n0 * 2));
  };
  auto out_ptr = [&](const WgTile& w, int64_t mrow, int col) __attribute__((always_inline)) {
    return (col < P.csplit)
               ? reinterpret_cast<T*>(P.C0) + (int64_t)w.g * P.strideC + mrow * P.ldc + col
               : reinterpret_cast<T*>(P.C1) + (int64_t)w.g * P.strideC + mrow * P.ldc +
                     (col - P.csplit);
  };

  int rb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) rb[j] = wn * WTN + j * 32;
  uint4 fa[2][NI], fb[2][NJ];
  f32x16_t acc[NI][NJ];
  auto frags = [&](const char* la, const char* lb, int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      fa[slot][i] = frag_mc(const_cast<char*>(la), wm * WTM + i * 32, ks, lane, BM * 2);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[slot][j] = frag_mc(const_cast<char*>(lb), rb[j], ks, lane, BN * 2);
  };
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, fb[slot][j]), __builtin_bit_cast(bf16x8_t, fa[slot][i]),
            acc[i][j], 0, 0, 0);
  };

  WgTile cur, nxt;
  tile_of(t, cur);
#pragma unroll
  for (int q = 0; q < NS; ++q) issue(q, cur, sA[q], sB[q]);
  // ready: slab 0 of cur has landed and every wave has passed a barrier
  // since; its slabs 1 .. NS-1 were issued before the previous tile's
  // epilogue stores (the run-ahead), so those stores are younger than them
  bool ready = false;
  const int lrow = lane & 31, lcol = (lane >> 5) * 4;
  char* reg = sE + wave * EWAVE;
  for (;;) {
    const int64_t tn = t + gridDim.x;
    const bool has_next = tn < n_tiles;
    if (has_next) tile_of(tn, nxt);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if (cur.nkp > 0) {
      const bool after_stores = ready;
      if (!ready) {
        // slabs 1 .. NS-1 (issued after slab 0) may still be in flight
        wait_vmcnt<(NS - 1) * PER_SLAB>();
        lds_barrier();
      }
      frags(sA[0], sB[0], 0, 0);
      const int nkp = cur.nkp;
      // slab kt + NS of this tile, or slab kt + NS - nkp of the next one
      auto run_ahead = [&](int kt, char* la, char* lb) __attribute__((always_inline)) {
        const int q = kt + NS;
        if (q < nkp || !has_next) issue(q, cur, la, lb);
        else issue(q - nkp, nxt, la, lb);
      };
      // Slab kt (stage s = kt mod NS) is computed while slabs kt + 1 ..
      // kt + NS - 1 are in flight; at its end the wait is for slab kt + 1
      // only: the NS - 2 slabs issued after it may stay in flight, and in
      // the first NS - 1 slabs of a tile that follows a computed tile so may
      // that tile's NSTORE epilogue stores (issued after slab kt + 1).
      auto step = [&](int kt, auto sc, bool first) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value, sn = (s + 1) % NS;
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) {
          frags(sA[s], sB[s], ks, ks & 1);
          interleave_reads<NI * NJ, (2 * (NI + NJ) + NI * NJ - 1) / (NI * NJ)>();
          __builtin_amdgcn_sched_barrier(0);
          mfmas((ks - 1) & 1);
        }
        if (s <= NS - 2 && first && after_stores) wait_vmcnt<(NS - 2) * PER_SLAB + NSTORE>();
        else wait_vmcnt<(NS - 2) * PER_SLAB>();
        lds_barrier();
        run_ahead(kt, sA[s], sB[s]);
        frags(sA[sn], sB[sn], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas((KS - 1) & 1);
      };
      for (int kt = 0; kt < nkp; kt += NS) {
        const bool first = kt == 0;
        step(kt, std::integral_constant<int, 0>{}, first);
        step(kt + 1, std::integral_constant<int, 1>{}, first);
        if constexpr (NS == 4) {
          step(kt + 2, std::integral_constant<int, NS == 4 ? 2 : 0>{}, first);
          step(kt + 3, std::integral_constant<int, NS == 4 ? 3 : 0>{}, first);
        }
      }
    }
    // (an empty group's tile, nkp = 0, stores the zeros)
    {
      // epilogue: each 32-row block of the wave through its LDS region
      // (bf16, 16-byte chunks XOR-swizzled within the row), 16-byte row
      // segments out, streaming (dW is not read again by this layer)
      constexpr int CPR = WTN / 8, RPI = 64 / CPR, MSK = (CPR < 8 ? CPR : 8) - 1;
      const int ch = lane % CPR;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
            const int col = j * 32 + q * 8 + lcol;
            const int c8 = col >> 3, half = (col >> 2) & 1;
            *reinterpret_cast<uint2*>(reg + lrow * WTN * 2 + ((c8 ^ (lrow & MSK)) << 4) + (half << 3)) =
                pack_bf16x4(v);
          }
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int row = it * RPI + lane / CPR;
          Vec16<T> o;
          o.v = *reinterpret_cast<const uint4*>(reg + row * WTN * 2 + ((ch ^ (row & MSK)) << 4));
          o.store_nt(out_ptr(cur, cur.m0 + wm * WTM + i * 32 + row, cur.n0 + wn * WTN + ch * 8));
        }
      }
    }
    if (cur.nkp > 0) {
      // the last step waited for the next tile's slab 0 (issued by the
      // run-ahead) and every wave has passed its barrier since; slab 1 is
      // in flight
      ready = has_next;
    } else {
      // the next tile's first slabs, issued after this tile's stores so that
      // its wait for slab 0 also covers them
      if (has_next) {
#pragma unroll
        for (int q = 0; q < NS; ++q) issue(q, nxt, sA[q], sB[q]);
      }
      ready = false;
    }
    if (!has_next) break;
    t = tn;
    cur = nxt;
  }
  // the run-ahead DMA (zeros past the last tile) must land before the LDS is
  // released
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int groups_of(const moe_config& c) { return (c.expert_hi - c.expert_lo) + c.n_shared; }

// tile-space sizes for tiles of bm rows
static void tile_space(GemmParams& P, int grouping, int bm) {
  if (grouping == GROUP_M) {
    // sum over groups of ceil(n_g / bm) <= ceil(rows / bm) + groups
    int64_t b = (P.routed_rows_max > 0) ? cdiv(P.routed_rows_max, bm) + P.n_routed : 0;
    if (P.shared_rows > 0) b += cdiv(P.shared_rows, bm);
    P.mt_total = (int)b;
    P.nblocks = b * P.ntn;
  } else {
    P.ntm = (int)cdiv(P.Mfix, bm);
    P.nblocks = (int64_t)P.G * P.ntm * P.ntn;
  }
}

// GEMM configuration of the LDS-DMA kernels: 0 = register-staged kernel,
// 1 = 128-row tiles / 2 stages, 2 = 256-row tiles / 3 stages, 3 / 4 = 256 x
// 256 / 256 x 128 large tiles on 4 waves, 5 / 6 = the same on 8 waves,
// 7 / 8 = persistent 256 x 256 / 256 x 128 on 8 waves, 9 = 256 x 128 on 4
// waves with 32-deep slabs, two workgroups per CU, 10 / 11 = 256 x 256 tile
// loop with the next tile's first slabs fetched during the epilogue, two
// 64-deep / four 32-deep stages (9-11: weight gradients; the row GEMMs then
// take 1).
// MOE_GEMM_CFG overrides the choice (measurement, and tests that run every
// kernel variant): a number for every GEMM, or "name=cfg" pairs separated by
// commas (e.g. "gemm_down_dgrad=1,gemm_gate_up_fwd=5").  Read at every
// launch, so a process can change it between calls.
static int cfg_override(const char* name) {
  const char* env = getenv("MOE_GEMM_CFG");
  const std::string spec(env ? env : "");
  if (spec.empty()) return -1;
  if (spec.find('=') == std::string::npos) return atoi(spec.c_str());
  const std::string key = std::string(name) + "=";
  const size_t at = spec.find(key);
  if (at == std::string::npos || (at > 0 && spec[at - 1] != ',')) return -1;
  return atoi(spec.c_str() + at + key.size());
}

template <int AM, int BM_, int GR, int EPI, int BS, int BMT, int S>
static int launch_dma(const char* name, GemmParams P, hipStream_t st) {
  tile_space(P, GR, BMT);
  if (P.nblocks <= 0) return MOE_OK;
  if (GR == GROUP_M && BMT == 128 && EPI == EPI_SWIGLU_FWD && P.Kdim <= 1024 &&
      (int64_t)P.n_routed * 16 <= P.mt_total) {
    // the gate/up forward with short reductions takes 2-D tile blocks per
    // XCD (measured on MiniMind: -4 to -7 % for this GEMM; with 2048-deep
    // reductions, and for the other row GEMMs, slower); the extra m-tiles
    // that round mt_total up find no group and exit.  The m-tile bound
    // exceeds the real m-tiles by up to one per routed group, and those
    // surplus tiles all fall to the XCDs of the last row block: with few
    // groups next to the m-tiles that imbalance stays small
    P.xcd_xn = (P.ntn % 4 == 0) ? 4 : (P.ntn % 2 == 0) ? 2 : 0;
    if (P.xcd_xn) {
      const int xm = 8 / P.xcd_xn;
      P.mt_total = (P.mt_total + xm - 1) / xm * xm;
      P.nblocks = (int64_t)P.mt_total * P.ntn;
    }
  }
  MOE_LAUNCH(name, (grouped_gemm_dma_kernel<AM, BM_, GR, EPI, BS, BMT, S>),
             dim3((unsigned)P.nblocks), dim3(BMT * 2), 0, st, P);
  return MOE_OK;
}

// bf16 with whole 128-column (and, for the weight gradients, whole-tile-row)
// tiles runs on the LDS-DMA kernel -- 256-row tiles when that still gives at
// least two workgroups per CU, else 128-row tiles; fp32 and ragged shapes
// run on the register-staged kernel.
template <int AM, int BM_, int GR, int EPI, int BS, int BN, int NW, int BK = 64>
static int launch_big(const char* name, GemmParams P, hipStream_t st) {
  P.ntn = P.N / BN;
  tile_space(P, GR, 256);
  if (P.nblocks <= 0) return MOE_OK;
  if (GR == GROUP_M && P.n_routed >= 64) {
    // many small groups: XCD blocks of the real m-tiles (rounded grid).
    // Measured on the DeepSeek-V3-like layer: down projection 3.08 -> 2.83
    // ms, gate/up input gradient 5.79 -> 5.67 ms (5.12 with the group-column
    // order inside the blocks), SwiGLU-backward GEMM 3.33 -> 2.76 ms (against
    // 2.94 ms on the 128 x 128 tiles, whose column bands per XCD made every
    // XCD stream all of d_o: 19.3 GB fetched per launch).  The SwiGLU
    // forward takes the same time either way (5.11 / 5.16 against 5.16 /
    // 5.17 ms, alternating runs on one box: its main loop bounds it) but
    // fetches 19.9 instead of 27.6 GB per launch
    P.xcd_m = 1;
    P.nblocks = (int64_t)cdiv(P.mt_total, 8) * 8 * P.ntn;
  }
  MOE_LAUNCH(name, (grouped_gemm_big_kernel<AM, BM_, GR, EPI, BS, BN, NW, BK>),
             dim3((unsigned)P.nblocks), dim3(NW * 64), 0, st, P);
  return MOE_OK;
}

// one persistent workgroup per CU (at most one tile each when there are fewer)
template <int AM, int BM_, int GR, int EPI, int BS, int BN>
static int launch_persist(const char* name, GemmParams P, hipStream_t st) {
  P.ntn = P.N / BN;
  tile_space(P, GR, 256);
  if (P.nblocks <= 0) return MOE_OK;
  // GROUP_K: 32 workgroups per XCD, each XCD its cost-balanced tile range
  const int64_t grid = (GR == GROUP_K) ? 256 : std::min<int64_t>(P.nblocks, 256);
  MOE_LAUNCH(name, (grouped_gemm_persist_kernel<AM, BM_, GR, EPI, BS, BN>), dim3((unsigned)grid),
             dim3(512), 0, st, P);
  return MOE_OK;
}

// weight gradients on 256 x 256 tiles, one workgroup per CU walking its tiles
// with the next tile's first slabs fetched during the epilogue
template <int BK, int NS>
static int launch_wgrad_loop(const char* name, GemmParams P, hipStream_t st) {
  P.ntn = P.N / 256;
  tile_space(P, GROUP_K, 256);
  if (P.nblocks <= 0) return MOE_OK;
  const uint64_t per = (uint64_t)P.ntm * P.ntn, span = 2ull * (uint64_t)P.ntm;
  P.per_magic = (per == 1) ? UINT32_MAX : (uint32_t)(((1ull << 32) + per - 1) / per);
  P.span_magic = (uint32_t)(((1ull << 32) + span - 1) / span);
  MOE_LAUNCH(name, (grouped_gemm_wgrad_loop_kernel<BK, NS>),
             dim3((unsigned)std::min<int64_t>(P.nblocks, 256)), dim3(512), 0, st, P);
  return MOE_OK;
}

template <typename T, int AM, int BM_, int GR, int EPI, int BS>
static int run_gemm(const char* name, GemmParams& P, hipStream_t st) {
  P.a_cap = (int)(INT32_MAX / (std::max<int64_t>(P.lda, 1) * 2));
  P.b_cap = (int)(INT32_MAX / (std::max<int64_t>(P.ldb, 1) * 2));
  if constexpr (sizeof(T) == 2) {
    const bool full128 = (P.N % kBN == 0) && (GR == GROUP_M ? P.Kdim % 64 == 0 : P.Mfix % 128 == 0);
    const bool full256 = full128 && (GR == GROUP_M || P.Mfix % 256 == 0);
    const bool wide = full256 && P.N % 256 == 0;
    int cfg = cfg_override(name);
    // 256 x 256 tiles of a row GEMM: the m-tile bound times the column tiles
    int64_t tiles256 = 0;
    if (GR == GROUP_M && EPI == EPI_STORE && wide) {
      GemmParams Q = P;
      Q.ntn = P.N / 256;
      tile_space(Q, GR, 256);
      tiles256 = Q.nblocks;
    }
    // the SwiGLU-backward GEMM with long reductions takes the 256 x 256
    // tiles below on large groups (Mixtral-like 3.43 -> 3.10 ms, OLMoE-like
    // 0.371 -> 0.356 ms) and on many small groups, where each XCD then takes
    // a block of the real m-tiles (DeepSeek-V3-like, ~256 rows per expert:
    // 2.94 -> 2.76 ms; 3.33 ms in the column-band order); on a few small
    // groups or short reductions (MiniMind, K = 768: 58 against 77 us) the
    // 128 x 128 tiles stay
    const bool bwd_big = EPI == EPI_SWIGLU_BWD && wide && P.Kdim >= 2048 && P.n_routed > 0 &&
                         (P.routed_rows_max / P.n_routed >= 1024 || P.n_routed >= 64);
    if (cfg < 0 && ((EPI == EPI_SWIGLU_BWD && !bwd_big) ||
                    (GR == GROUP_M && EPI != EPI_SWIGLU_BWD &&
                     (P.Kdim < 2048 ||
                      (P.Kdim == 2048 && !(EPI == EPI_STORE && P.n_routed >= 64 &&
                                           tiles256 >= 1024)))))) {
      // 128 x 128 tiles run two workgroups per CU, so one's epilogue and
      // first-slab wait overlap the other's main loop.  That wins for the
      // row GEMMs with short reductions (K <= 2048: a tile's main loop is
      // then not much longer than its prologue and epilogue) and for the
      // SwiGLU-backward epilogue (activations read, two gradients written)
      // on small groups or short reductions; long reductions, and the
      // plain-store row GEMM at K = 2048 on many small groups with many
      // tiles (DeepSeek-V3-like down projection: 3.04 vs 3.33 ms, with the
      // XCD m-tile blocks of launch_big), favour the 256-wide tiles.  Not
      // the SwiGLU forward at OLMoE-like K = 2048 (0.53 vs 0.38 ms), nor the
      // gate/up input gradient there (32 local experts of ~1000 rows: 0.506
      // vs 0.348 ms).
      cfg = 1;
    }
    if (cfg < 0 && GR == GROUP_K && wide && P.n_routed > 0 &&
        P.routed_rows_max / P.n_routed <= 512 && (int64_t)(P.Mfix / 256) * (P.N / 256) >= 256) {
      // weight gradients with short reductions (a few hundred rows per
      // expert: each tile runs four or five slabs and its first-slab wait is
      // a large part of it) and at least one tile per CU in every group: the
      // tile loop that fetches the next tile's first slabs during the
      // epilogue, on four 32-deep stages (three slabs in flight).  Measured
      // alone against the 256 x 256 kernel (cfg 5), DeepSeek-V3-like gate/up
      // weight gradient: cfg 11 5.64 / 5.65 ms, cfg 10 (two 64-deep stages)
      // 5.92 / 5.94, cfg 5 6.36 (step 27.6 -> 26.7 ms).  Its down weight
      // gradient (224 tiles per group) and the long-reduction layers tie
      // alone (Mixtral-like gate/up 4.77 both) but lose in the overlapped
      // step (Mixtral-like 23.9 -> 24.4 ms): one workgroup holding a CU's
      // whole LDS leaves no room for the data-gradient GEMM beside it
      cfg = 11;
    }
    if (cfg < 0) {
      // 256 x 256 tiles on 8 waves when they give enough tiles (a weight
      // gradient, with its long reduction over the group rows, needs fewer);
      // else 256 x 128 or 128 x 128 tiles on the 8- / 4-wave DMA kernel.
      GemmParams Q = P;
      if (wide) {
        Q.ntn = P.N / 256;
        tile_space(Q, GR, 256);
      }
      if (wide && Q.nblocks >= (GR == GROUP_K ? 192 : 384)) {
        // 256 x 256 tiles on 8 waves.  The persistent variant was measured
        // no faster: Mixtral-like down projection 2.79 vs 2.83 ms; weight
        // gradients with cost-balanced XCD ranges, Mixtral-like gate/up 5.51
        // against 4.82 ms, DeepSeek-V3-like 8.55 against 6.78 ms.
        cfg = 5;
      } else {
        Q = P;
        tile_space(Q, GR, 256);
        cfg = (full256 && Q.nblocks >= 512) ? 2 : 1;
      }
    }
    if (cfg == 3 && wide) return launch_big<AM, BM_, GR, EPI, BS, 256, 4>(name, P, st);
    if (cfg == 4 && full256) return launch_big<AM, BM_, GR, EPI, BS, 128, 4>(name, P, st);
    if (cfg == 5 && wide) return launch_big<AM, BM_, GR, EPI, BS, 256, 8>(name, P, st);
    if (cfg == 7 && wide) return launch_persist<AM, BM_, GR, EPI, BS, 256>(name, P, st);
    if (cfg == 8 && full256) return launch_persist<AM, BM_, GR, EPI, BS, 128>(name, P, st);
    if (cfg == 6 && full256) return launch_big<AM, BM_, GR, EPI, BS, 128, 8>(name, P, st);
    if constexpr (GR == GROUP_K && AM == MC && BM_ == MC) {
      if (cfg == 9 && full256) return launch_big<AM, BM_, GR, EPI, BS, 128, 4, 32>(name, P, st);
      if constexpr (EPI == EPI_STORE && BS == BS_NONE) {
        // (tile indices in 32 bits)
        const bool fits = wide && (int64_t)P.G * (P.Mfix / 256) * (P.N / 256) < INT32_MAX;
        if (cfg == 10 && fits) return launch_wgrad_loop<64, 2>(name, P, st);
        if (cfg == 11 && fits) return launch_wgrad_loop<32, 4>(name, P, st);
      }
    }
    if (cfg == 2 && full256) return launch_dma<AM, BM_, GR, EPI, BS, 256, 3>(name, P, st);
    if (cfg >= 1 && full128) return launch_dma<AM, BM_, GR, EPI, BS, 128, 2>(name, P, st);
  }
  tile_space(P, GR, kBM);
  if (P.nblocks <= 0) return MOE_OK;
  MOE_LAUNCH(name, (grouped_gemm_kernel<T, AM, BM_, GR, EPI, BS>), dim3((unsigned)P.nblocks),
             dim3(kThreads), 0, st, P);
  return MOE_OK;
}

static GemmParams base_params(const moe_config& c, const int32_t* offsets) {
  GemmParams P = {};
  P.G = groups_of(c);
  P.EL_A = P.EL_B = c.expert_hi - c.expert_lo;
  P.n_routed = c.expert_hi - c.expert_lo;
  P.routed_rows_max = (P.n_routed > 0) ? routed_rows_max(c) : 0;
  P.shared_rows = (int64_t)c.n_shared * c.T;
  P.offsets = offsets;
  P.F = c.F;
  P.csplit = 1 << 30;
  return P;
}

int gemm_swiglu_fwd(const moe_config& c, const void* x, const void* x_perm,
                    const int32_t* offsets, const void* wg, const void* wu, void* act, void* h,
                    hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.N = 2 * c.F;
  P.Kdim = c.D;
  P.ntn = (int)cdiv(P.N, kBN);
  P.A = x_perm; P.A_sh = x; P.lda = c.D;
  P.B0 = wg; P.B1 = wu; P.ldb = c.F; P.strideB = (int64_t)c.D * c.F;
  P.C1 = h; P.act_out = act;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, KC, MC, GROUP_M, EPI_SWIGLU_FWD, BS_N>("gemm_gate_up_fwd", P, st);
  return run_gemm<float, KC, MC, GROUP_M, EPI_SWIGLU_FWD, BS_N>("gemm_gate_up_fwd", P, st);
}

int gemm_down_fwd(const moe_config& c, const int32_t* offsets, const void* h, const void* wd,
                  void* o_perm, hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.N = c.D;
  P.Kdim = c.F;
  P.ntn = (int)cdiv(P.N, kBN);
  // shared rows of h live in the same row buffer: every group reads its rows
  P.EL_A = P.G;
  P.A = h; P.A_sh = h; P.lda = c.F;
  P.B0 = wd; P.ldb = c.D; P.strideB = (int64_t)c.F * c.D;
  P.C0 = o_perm; P.ldc = c.D;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, KC, MC, GROUP_M, EPI_STORE, BS_NONE>("gemm_down_fwd", P, st);
  return run_gemm<float, KC, MC, GROUP_M, EPI_STORE, BS_NONE>("gemm_down_fwd", P, st);
}

int gemm_down_dgrad(const moe_config& c, const int32_t* offsets, const void* d_o, const void* dy,
                    const void* wd, const void* act, void* dact, hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.N = c.F;
  P.Kdim = c.D;
  P.ntn = (int)cdiv(P.N, kBN);
  P.A = d_o; P.A_sh = dy; P.lda = c.D;
  // B(k = d, n = f) = W_down[f][d]: row n, K contiguous
  P.B0 = wd; P.ldb = c.D; P.strideB = (int64_t)c.F * c.D;
  P.C0 = dact; P.act = act;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, KC, KC, GROUP_M, EPI_SWIGLU_BWD, BS_NONE>("gemm_down_dgrad", P, st);
  return run_gemm<float, KC, KC, GROUP_M, EPI_SWIGLU_BWD, BS_NONE>("gemm_down_dgrad", P, st);
}

int gemm_up_dgrad(const moe_config& c, const int32_t* offsets, const void* dact, const void* wg,
                  const void* wu, void* dx_perm, hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.N = c.D;
  P.Kdim = 2 * c.F;
  P.ntn = (int)cdiv(P.N, kBN);
  P.EL_A = P.G;  // dact holds the shared rows too
  P.A = dact; P.A_sh = dact; P.lda = 2 * c.F;
  // B(k = f, n = d) = W_gate[d][f] for f < F, W_up[d][f - F] above
  P.B0 = wg; P.B1 = wu; P.ldb = c.F; P.strideB = (int64_t)c.D * c.F; P.bsplit = c.F;
  P.C0 = dx_perm; P.ldc = c.D;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, KC, KC, GROUP_M, EPI_STORE, BS_K>("gemm_gate_up_dgrad", P, st);
  return run_gemm<float, KC, KC, GROUP_M, EPI_STORE, BS_K>("gemm_gate_up_dgrad", P, st);
}

int gemm_down_wgrad(const moe_config& c, const int32_t* offsets, const void* h, const void* d_o,
                    const void* dy, void* dwd, hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.Mfix = c.F;
  P.N = c.D;
  P.ntn = (int)cdiv(P.N, kBN);
  // A(m = f, k = row) = h[row][f]: every group (shared too) reads its h rows;
  // B(k = row, n = d) = d_o[row][d] for routed groups, dy[token][d] for shared
  P.EL_A = P.G;
  P.A = h; P.A_sh = h; P.lda = c.F;
  P.B0 = d_o; P.B1 = dy; P.ldb = c.D;
  P.C0 = dwd; P.ldc = c.D; P.strideC = (int64_t)c.F * c.D;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, MC, MC, GROUP_K, EPI_STORE, BS_NONE>("gemm_down_wgrad", P, st);
  return run_gemm<float, MC, MC, GROUP_K, EPI_STORE, BS_NONE>("gemm_down_wgrad", P, st);
}

int gemm_up_wgrad(const moe_config& c, const int32_t* offsets, const void* x, const void* x_perm,
                  const void* dact, void* dwg, void* dwu, hipStream_t st) {
  GemmParams P = base_params(c, offsets);
  P.Mfix = c.D;
  P.N = 2 * c.F;
  P.ntn = (int)cdiv(P.N, kBN);
  P.A = x_perm; P.A_sh = x; P.lda = c.D;
  // B(k = row, n) = dact[row][n], n in [0, 2F): every group reads dact rows
  P.EL_B = P.G;
  P.B0 = dact; P.B1 = dact; P.ldb = 2 * c.F;
  P.C0 = dwg; P.C1 = dwu; P.ldc = c.F; P.csplit = c.F; P.strideC = (int64_t)c.D * c.F;
  if (c.dtype == MOE_BF16) return run_gemm<bf16_t, MC, MC, GROUP_K, EPI_STORE, BS_NONE>("gemm_gate_up_wgrad", P, st);
  return run_gemm<float, MC, MC, GROUP_K, EPI_STORE, BS_NONE>("gemm_gate_up_wgrad", P, st);
}

// ---------------------------------------------------------------------------
// Router GEMMs for many experts, fp32 end to end on the fp32 matrix cores:
//   C[z][m][n] = sum over k in [z*kper, min(Kd, (z+1)*kper)) of A(m,k) B(k,n)
//   A(m,k) = AMODE == KC ? A[m*lda + k] : A[k*lda + m]   (fp32)
//   B(k,n) = B[k*ldb + n]   (fp32, or bf16 widened exactly on its way to LDS)
// 128 x 128 tiles, k-slabs of 32, the register-staged two-slab pipeline and
// v_mfma_f32_32x32x2f32 fragments of grouped_gemm_kernel (products exact,
// fp32 sums).  The accumulators go straight to C: each half-wave stores 32
// consecutive columns of one row.  Shapes: lda, ldb, N and (MC) M multiples
// of 4, (KC) Kd a multiple of 4, kper a multiple of 32; A, C and fp32 B
// 16-byte aligned, bf16 B 8-byte aligned.
// ---------------------------------------------------------------------------
template <typename TB>
struct RouterBLoader;
template <>
struct RouterBLoader<float> : TileLoader<float, MC> {};
template <>
struct RouterBLoader<bf16_t> {
  TileLoader<float, MC> t;
  uint2 raw[4];
  // same element map as TileLoader<float, MC>: rows k = kg*4 + j of the four
  // columns mg*4.., kg = tid / 32, mg = tid % 32
  MOE_DEV void load(const bf16_t* p, int64_t ld, int r_valid, int k0, int k_valid) {
    const int kg = threadIdx.x >> 5, mg = threadIdx.x & 31;
    t.ok = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + kg * 4 + j, r = mg * 4;
      const bool in = (k < k_valid) && (r < r_valid);
      const bf16_t* q = in ? p + (int64_t)k * ld + r : p + (int64_t)k0 * ld;
      raw[j] = *reinterpret_cast<const uint2*>(q);
      t.ok |= (uint32_t)in << j;
    }
  }
  MOE_DEV void store(char* lds) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.reg[j] = make_uint4(raw[j].x << 16, raw[j].x & 0xFFFF0000u, raw[j].y << 16,
                            raw[j].y & 0xFFFF0000u);
    t.store(lds);
  }
};

template <int AMODE, typename TB>
__global__ __launch_bounds__(256) void router_gemm_kernel(const float* __restrict__ A,
                                                          int64_t lda, const TB* __restrict__ B,
                                                          int64_t ldb, int M, int N, int Kd,
                                                          int kper, float* __restrict__ C,
                                                          int64_t ldc, int64_t split_stride) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][128 * 128];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
  const int kb = blockIdx.z * kper, ke = min(Kd, kb + kper);
  const int rows_valid = min(128, M - m0), cols_valid = min(128, N - n0);
  const float* At = (AMODE == KC) ? A + (int64_t)m0 * lda : A + m0;
  const TB* Bt = B + n0;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileLoader<float, AMODE> la0, la1;
  RouterBLoader<TB> lb0, lb1;
  const int nk = (ke - kb + 31) / 32;
  auto load_k = [&](TileLoader<float, AMODE>& la, RouterBLoader<TB>& lb, int kt) {
    const int k0 = kb + kt * 32;
    la.load(At, lda, rows_valid, k0, ke);
    lb.load(Bt, ldb, cols_valid, k0, ke);
  };
  const int ra[2] = {wm * 64, wm * 64 + 32};
  const int rb[2] = {wn * 64, wn * 64 + 32};
  if (nk > 0) {
    load_k(la0, lb0, 0);
    if (nk > 1) load_k(la1, lb1, 1);
    la0.store(smem[0][0]);
    lb0.store(smem[0][1]);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      if (kt + 2 < nk) load_k(la0, lb0, kt + 2);
      mma_slab<float>(smem[0][0], smem[0][1], ra, rb, acc);
      la1.store(smem[1][0]);
      lb1.store(smem[1][1]);
      __syncthreads();
      if (kt + 3 < nk) load_k(la1, lb1, kt + 3);
      mma_slab<float>(smem[1][0], smem[1][1], ra, rb, acc);
      if (kt + 2 < nk) {
        la0.store(smem[0][0]);
        lb0.store(smem[0][1]);
      }
      __syncthreads();
    }
    if (kt < nk) mma_slab<float>(smem[0][0], smem[0][1], ra, rb, acc);
  }

  float* Cs = C + (int64_t)blockIdx.z * split_stride;
  const int l32 = lane & 31, hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + (r >> 2) * 8 + hi4 + (r & 3);
      if (row >= rows_valid) continue;
      float* crow = Cs + (int64_t)(m0 + row) * ldc + n0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + l32;
        if (col < cols_valid) crow[col] = acc[i][j][r];
      }
    }
}

bool router_gemm_fits(int64_t lda, int64_t ldb, int M, int N, int Kd, bool a_kc) {
  if (lda % 4 || ldb % 4 || N % 4) return false;
  return a_kc ? (Kd % 4 == 0) : (M % 4 == 0);
}

int router_gemm(const char* name, bool a_kc, bool b_bf16, const float* A, int64_t lda,
                const void* B, int64_t ldb, int M, int N, int Kd, int kper, int splits, float* C,
                int64_t ldc, int64_t split_stride, hipStream_t st) {
  if (M <= 0 || N <= 0) return MOE_OK;
  dim3 grid((unsigned)cdiv(N, 128), (unsigned)cdiv(M, 128), (unsigned)splits);
#define RG(AM, TBV)                                                                          \
  MOE_LAUNCH(name, (router_gemm_kernel<AM, TBV>), grid, dim3(256), 0, st, A, lda,           \
             reinterpret_cast<const TBV*>(B), ldb, M, N, Kd, kper, C, ldc, split_stride)
  if (a_kc) {
    if (b_bf16) RG(KC, bf16_t); else RG(KC, float);
  } else {
    if (b_bf16) RG(MC, bf16_t); else RG(MC, float);
  }
#undef RG
  return MOE_OK;
}

}  // namespace moe
