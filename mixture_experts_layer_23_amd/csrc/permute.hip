// permute.hip -- expert histogram, scan, stable in-expert rank, capacity
// drops, row maps and the row gather.
//
// [P3] "MoE" tutorial, efficient inference: tokens are grouped by expert so
// that the sparse, irregular expert access becomes dense batches (sort, then
// gather); GShard pseudo-code: each expert buffer is filled in token order and
// overflow beyond the capacity is dropped.  [P5] course notes 8.5: capacity
// ~ ceil(c*T*K/E); 8.8: group tokens by expert, a token may appear K times.
// [P1] cause section: slots routed to experts that this device does not hold
// are sentinels and must not contribute.
//
// Determinism: the position of a slot inside its expert is computed from
// per-tile counts, an exclusive scan over tiles and a stable in-tile rank
// (wave ballots), never from atomic slot grabbing, so every run produces the
// same rows.
#include "common.h"
#include "kernels.h"

namespace moe {

// K1: per-tile expert histogram (LDS atomics only count; order-free)
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int64_t TK,
                                                   int E, int32_t* __restrict__ tile_counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * kSlotTile + threadIdx.x;
  if (s < TK) atomicAdd(&hist[idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    tile_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// K2: exclusive scan over the tiles of one expert (one workgroup per expert):
// tile_base[t][e] = sum_{t' < t} tile_counts[t'][e], counts_all[e] = total.
__global__ __launch_bounds__(256) void scan_tiles_kernel(const int32_t* __restrict__ tile_counts,
                                                         int ntiles, int E,
                                                         int32_t* __restrict__ tile_base,
                                                         int32_t* __restrict__ counts_all) {
  __shared__ int32_t wsum[4];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int t0 = 0; t0 < ntiles; t0 += 256) {
    const int t = t0 + tid;
    const int v = t < ntiles ? tile_counts[(size_t)t * E + e] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (t < ntiles) tile_base[(size_t)t * E + e] = before + incl - v;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) counts_all[e] = carry;
}

// K3: stable rank inside each tile (one wave per tile, 64 slots per round,
// running per-expert counters in LDS), then the slot and row maps.  Every
// workgroup first derives the group offsets from the expert counts (capacity
// applied, exclusive scan over the local experts); workgroup 0 also publishes
// them, with the shared-expert blocks after the routed rows, and the number
// of dropped slots.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int64_t TK,
                                                  int K, int E, int lo, int hi, int capacity,
                                                  int nbits, int n_shared, int T_,
                                                  const int32_t* __restrict__ tile_base,
                                                  const int32_t* __restrict__ counts_all,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ n_dropped,
                                                  int32_t* __restrict__ slot_row,
                                                  int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ row_slot) {
  extern __shared__ int32_t lds[];
  int32_t* cnt = lds;       // [E] running per-expert counts of this tile
  int32_t* off = lds + E;   // [EL + 1] group offsets
  const int lane = threadIdx.x;
  const int EL = hi - lo;
  // this lane's slot experts of every round, loaded up front (unconditional,
  // index clamped; slots past TK are marked invalid below)
  constexpr int R = kSlotTile / 64;
  int ev[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = (int64_t)blockIdx.x * kSlotTile + r * 64 + lane;
    ev[r] = idx[s < TK ? s : 0];
  }
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  {
    // lane j owns local experts [j*per, (j+1)*per)
    const int per = (EL + 63) / 64;  // <= 16 (E <= 1024)
    int nk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane * per + i;
      nk[i] = (i < per && e < EL) ? counts_all[lo + e] : 0;
    }
    int kept = 0, drop = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = nk[i];
      const int k = (capacity >= 0 && n > capacity) ? capacity : n;
      kept += k;
      drop += n - k;
    }
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int run = incl - kept;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane * per + i;
      if (i < per && e < EL) {
        off[e] = run;
        const int n = nk[i];
        run += (capacity >= 0 && n > capacity) ? capacity : n;
      }
    }
    if (lane == 63) off[EL] = incl;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) drop += __shfl_xor(drop, o, 64);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int e = lane; e <= EL; e += 64) offsets[e] = off[e];
      for (int s = lane; s < n_shared; s += 64) offsets[EL + 1 + s] = off[EL] + (s + 1) * T_;
      if (lane == 0) *n_dropped = drop;
    }
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // this tile's base position of each slot's expert, all loaded together
  int tb[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = (int64_t)blockIdx.x * kSlotTile + r * 64 + lane;
    tb[r] = tile_base[(size_t)blockIdx.x * E + (s < TK ? ev[r] : 0)];
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t s = (int64_t)blockIdx.x * kSlotTile + r * 64 + lane;
    const bool valid = s < TK;
    const int e = valid ? ev[r] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const int rank = __popcll(peers & lt);
    const int base = valid ? cnt[e] : 0;
    __syncthreads();
    if (valid && (63 - __clzll(peers)) == lane) cnt[e] = base + __popcll(peers);
    __syncthreads();
    if (!valid) continue;
    const int pos = tb[r] + base + rank;
    if (e < lo || e >= hi) {
      slot_row[s] = -2;
    } else if (capacity >= 0 && pos >= capacity) {
      slot_row[s] = -1;
    } else {
      const int row = off[e - lo] + pos;
      slot_row[s] = row;
      row_token[row] = (int32_t)(s / K);
      row_slot[row] = (int32_t)s;
    }
  }
}

// One-workgroup permute for small slot counts (hist + scan + rank in one
// launch).  Wave w owns the contiguous slot chunk [w*CH, (w+1)*CH), CH a
// multiple of 64, and walks it 64 slots at a time with its own per-expert
// counters (wave-private LDS, updated by the lane that closes each group of
// equal experts).  Pass 1 counts; the workgroup then forms the expert totals,
// the capacity-limited offsets (as rank_kernel does) and every wave's base
// per expert (the counts of the waves before it); pass 2 walks the chunk
// again and assigns positions.  Chunks are in slot order, so the positions
// are the stable in-expert ranks of the tiled path.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int64_t kSmallSlots = 32768;  // up to 32 groups of 64 slots per wave
constexpr int kSmallExperts = 256;      // LDS: (17 E + EL + 1) int32

template <int R>  // groups of 64 slots per wave, held in registers (16 * 64 * R >= TK)
__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(
    const int32_t* __restrict__ idx, int TK, int K, int E, int lo, int hi, int capacity,
    int nbits, int n_shared, int T_, int32_t* __restrict__ counts_all,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot) {
  extern __shared__ int32_t lds[];
  const int EL = hi - lo;
  int32_t* cnt = lds;                       // [E] slots per expert
  int32_t* off = cnt + E;                   // [EL + 1] group offsets
  int32_t* wc = off + EL + 1;               // [16][E] wave counts, then wave bases
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t* mine = wc + wave * E;            // this wave's counters
  const int s_begin = wave * R * 64;
  int ev[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = s_begin + r * 64 + lane;
    ev[r] = s < TK ? idx[s] : -1;
  }
  for (int e = lane; e < E; e += 64) mine[e] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool valid = ev[r] >= 0;
    const int e = valid ? ev[r] : 0;
    const uint64_t peers = same_expert_peers(valid, e, nbits);
    if (valid && (63 - __clzll(peers)) == lane) mine[e] += __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // expert totals and per-wave bases (exclusive scan over the 16 waves)
  for (int x = tid; x < E; x += kSmallThreads) {
    int r = 0;
    for (int w = 0; w < kSmallWaves; ++w) {
      const int c = wc[w * E + x];
      wc[w * E + x] = r;
      r += c;
    }
    cnt[x] = r;
    counts_all[x] = r;
  }
  __syncthreads();
  if (wave == 0) {
    const int per = (EL + 63) / 64;
    int kept = 0, drop = 0;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < EL) {
        const int n = cnt[lo + e];
        const int k = (capacity >= 0 && n > capacity) ? capacity : n;
        kept += k;
        drop += n - k;
      }
    }
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    int r = incl - kept;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < EL) {
        off[e] = r;
        offsets[e] = r;
        const int n = cnt[lo + e];
        r += (capacity >= 0 && n > capacity) ? capacity : n;
      }
    }
    const int total = __shfl(incl, 63, 64);
    if (lane == 0) {
      off[EL] = total;
      offsets[EL] = total;
    }
    for (int sh = lane; sh < n_shared; sh += 64) offsets[EL + 1 + sh] = total + (sh + 1) * T_;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) drop += __shfl_xor(drop, o, 64);
    if (lane == 0) *n_dropped = drop;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int s = s_begin + r * 64 + lane;
    const bool valid = ev[r] >= 0;
    const int e = valid ? ev[r] : 0;
    const uint64_t peers = same_expert_peers(valid, e, nbits);
    const int pos = valid ? mine[e] + __popcll(peers & lt) : 0;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid && (63 - __clzll(peers)) == lane) mine[e] += __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      if (e < lo || e >= hi) {
        slot_row[s] = -2;
      } else if (capacity >= 0 && pos >= capacity) {
        slot_row[s] = -1;
      } else {
        const int row = off[e - lo] + pos;
        slot_row[s] = row;
        row_token[row] = s / K;
        row_slot[row] = s;
      }
    }
  }
}

// shared-expert rows: one per token, after the routed rows
__global__ void shared_rows_kernel(const int32_t* __restrict__ offsets, int EL, int T_,
                                   int n_shared, int32_t* __restrict__ row_token,
                                   int32_t* __restrict__ row_slot) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_shared * T_) return;
  const int64_t r = offsets[EL] + i;
  row_token[r] = (int32_t)(i % T_);
  row_slot[r] = -1;
}

// K4: x_perm[r] = x[row_token[r]] for the routed rows; one wave per row,
// lanes stride over 16-byte vectors; rows beyond offsets[EL] exit.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets, int EL,
                                                     int D, T* __restrict__ x_perm) {
  constexpr int VEC = Elem<T>::VEC;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= offsets[EL]) return;
  const T* src = x + (size_t)row_token[r] * D;
  T* dst = x_perm + (size_t)r * D;
  for (int d0 = lane * VEC; d0 < D; d0 += 64 * VEC) {
    Vec16<T> v;
    v.load(src + d0);
    v.store(dst + d0);
  }
}

int launch_permute(const moe_config& c, int capacity, const int32_t* idx, const void* x,
                   int32_t* counts_all, int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                   int32_t* row_slot, int32_t* n_dropped, void* x_perm, char* ws,
                   const Workspace& L, hipStream_t st) {
  const int64_t TK = (int64_t)c.T * c.K;
  const int E = c.E, EL = c.expert_hi - c.expert_lo;
  int32_t* tile_counts = reinterpret_cast<int32_t*>(ws + L.tile_counts);
  int32_t* tile_base = reinterpret_cast<int32_t*>(ws + L.tile_base);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int rc;
  if (TK <= kSmallSlots && E <= kSmallExperts) {
    const size_t shm = (size_t)(E + EL + 1 + kSmallWaves * E) * sizeof(int32_t);
#define SMALL(Rv)                                                                              \
  MOE_LAUNCH("permute_small", permute_small_kernel<Rv>, dim3(1), dim3(kSmallThreads), shm, st, \
             idx, (int)TK, c.K, E, c.expert_lo, c.expert_hi, capacity, nbits, c.n_shared, c.T,  \
             counts_all, offsets, n_dropped, slot_row, row_token, row_slot)
    if (TK <= 4 * kSmallThreads) SMALL(4);
    else if (TK <= 8 * kSmallThreads) SMALL(8);
    else if (TK <= 16 * kSmallThreads) SMALL(16);
    else SMALL(32);
#undef SMALL
    if ((rc = launch_shared_rows(c, offsets, row_token, row_slot, st))) return rc;
    return launch_gather(c, x, row_token, offsets, x_perm, st);
  }
  MOE_LAUNCH("permute_hist", hist_kernel, dim3(L.ntiles), dim3(256), E * sizeof(int32_t), st, idx,
             TK, E, tile_counts);
  MOE_LAUNCH("permute_scan", scan_tiles_kernel, dim3(E), dim3(256), 0, st, tile_counts,
             L.ntiles, E, tile_base, counts_all);
  MOE_LAUNCH("permute_rank", rank_kernel, dim3(L.ntiles), dim3(64),
             (size_t)(E + EL + 1) * sizeof(int32_t), st, idx, TK, c.K, E, c.expert_lo,
             c.expert_hi, capacity, nbits, c.n_shared, c.T, tile_base, counts_all, offsets,
             n_dropped, slot_row, row_token, row_slot);
  if ((rc = launch_shared_rows(c, offsets, row_token, row_slot, st))) return rc;
  return launch_gather(c, x, row_token, offsets, x_perm, st);
}

int launch_shared_rows(const moe_config& c, const int32_t* offsets, int32_t* row_token,
                       int32_t* row_slot, hipStream_t st) {
  if (c.n_shared > 0) {
    const int64_t n = (int64_t)c.n_shared * c.T;
    MOE_LAUNCH("permute_shared_rows", shared_rows_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256),
               0, st, offsets, c.expert_hi - c.expert_lo, c.T, c.n_shared, row_token, row_slot);
  }
  return MOE_OK;
}

// grid from the routed-row bound; rows at or beyond offsets[EL] exit
int launch_gather(const moe_config& c, const void* x, const int32_t* row_token,
                  const int32_t* offsets, void* x_perm, hipStream_t st) {
  const int EL = c.expert_hi - c.expert_lo;
  const int64_t rows = routed_rows_max(c);
  if (EL > 0 && rows > 0) {
    const int grid = (int)cdiv(rows, 4);
    if (c.dtype == MOE_BF16)
      MOE_LAUNCH("permute_gather", gather_kernel<bf16_t>, dim3(grid), dim3(256), 0, st,
                 (const bf16_t*)x, row_token, offsets, EL, c.D, (bf16_t*)x_perm);
    else
      MOE_LAUNCH("permute_gather", gather_kernel<float>, dim3(grid), dim3(256), 0, st,
                 (const float*)x, row_token, offsets, EL, c.D, (float*)x_perm);
  }
  return MOE_OK;
}

}  // namespace moe
