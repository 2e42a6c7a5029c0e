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

// K2: exclusive scan over tiles per expert, global counts, capacity, group
// offsets and the dropped count.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ tile_counts,
                                                    int ntiles, int E, int lo, int hi,
                                                    int n_shared, int T_, int capacity,
                                                    int32_t* __restrict__ tile_base,
                                                    int32_t* __restrict__ counts_all,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ n_dropped) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t sd[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int t = 0; t < ntiles; ++t) {
      const int v = tile_counts[(size_t)t * E + e];
      tile_base[(size_t)t * E + e] = run;
      run += v;
    }
    counts_all[e] = run;
    sc[e] = run;  // E <= 1024
  }
  __syncthreads();
  const int EL = hi - lo;
  int kept = 0, drop = 0;
  if (tid < EL) {
    const int n = sc[lo + tid];
    kept = (capacity >= 0 && n > capacity) ? capacity : n;
    drop = n - kept;
  }
  __syncthreads();
  sc[tid] = kept;
  sd[tid] = drop;
  __syncthreads();
  // inclusive Hillis-Steele scan of kept, tree sum of drop
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = (tid >= o) ? sc[tid - o] : 0;
    const int b = (tid + o < 1024 && (tid % (2 * o)) == 0) ? sd[tid + o] : 0;
    __syncthreads();
    sc[tid] += a;
    sd[tid] += b;
    __syncthreads();
  }
  if (tid < EL) offsets[tid + 1] = sc[tid];
  if (tid == 0) {
    offsets[0] = 0;
    const int tot = EL > 0 ? sc[EL - 1] : 0;
    for (int s = 0; s < n_shared; ++s) offsets[EL + 1 + s] = tot + (s + 1) * T_;
    *n_dropped = sd[0];
  }
}

// K3: stable rank inside each tile (one wave per tile, 64 slots per round,
// running per-expert counters in LDS), then the slot and row maps.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int64_t TK,
                                                  int K, int E, int lo, int hi, int capacity,
                                                  int nbits, const int32_t* __restrict__ tile_base,
                                                  const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ slot_row,
                                                  int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ row_slot) {
  extern __shared__ int32_t cnt[];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kSlotTile / 64; ++r) {
    const int64_t s = (int64_t)blockIdx.x * kSlotTile + r * 64 + lane;
    const bool valid = s < TK;
    const int e = valid ? idx[s] : 0;
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
    const int pos = tile_base[(size_t)blockIdx.x * E + e] + base + rank;
    if (e < lo || e >= hi) {
      slot_row[s] = -2;
    } else if (capacity >= 0 && pos >= capacity) {
      slot_row[s] = -1;
    } else {
      const int row = offsets[e - lo] + pos;
      slot_row[s] = row;
      row_token[row] = (int32_t)(s / K);
      row_slot[row] = (int32_t)s;
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

// K4: x_perm[r] = x[row_token[r]] for the routed rows; 16-byte vectors,
// four in flight per thread; surplus threads (rows beyond offsets[EL]) exit.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets, int EL,
                                                     int nv, int D, T* __restrict__ x_perm) {
  const int64_t nrows = offsets[EL];
  const int64_t total = nrows * nv;
  const int64_t b0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  Vec16<T> v[4];
  int64_t dst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t it = b0 + u * 256;
    dst[u] = -1;
    if (it < total) {
      const int64_t r = it / nv;
      const int c = (int)(it - r * nv);
      const int src = row_token[r];
      v[u].load(x + (size_t)src * D + (size_t)c * Elem<T>::VEC);
      dst[u] = r * D + (int64_t)c * Elem<T>::VEC;
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (dst[u] >= 0) v[u].store(x_perm + dst[u]);
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
  MOE_LAUNCH("permute_hist", hist_kernel, dim3(L.ntiles), dim3(256), E * sizeof(int32_t), st, idx,
             TK, E, tile_counts);
  MOE_LAUNCH("permute_scan", scan_kernel, dim3(1), dim3(1024), 0, st, tile_counts, L.ntiles, E,
             c.expert_lo, c.expert_hi, c.n_shared, c.T, capacity, tile_base, counts_all, offsets,
             n_dropped);
  MOE_LAUNCH("permute_rank", rank_kernel, dim3(L.ntiles), dim3(64), E * sizeof(int32_t), st, idx,
             TK, c.K, E, c.expert_lo, c.expert_hi, capacity, nbits, tile_base, offsets, slot_row,
             row_token, row_slot);
  if (c.n_shared > 0) {
    const int64_t n = (int64_t)c.n_shared * c.T;
    MOE_LAUNCH("permute_shared_rows", shared_rows_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256),
               0, st, offsets, EL, c.T, c.n_shared, row_token, row_slot);
  }
  if (EL > 0) {
    if (c.dtype == MOE_BF16) {
      const int nv = c.D / 8;
      const int grid = (int)cdiv(TK * nv, 1024);
      MOE_LAUNCH("permute_gather", gather_kernel<bf16_t>, dim3(grid), dim3(256), 0, st,
                 (const bf16_t*)x, row_token, offsets, EL, nv, c.D, (bf16_t*)x_perm);
    } else {
      const int nv = c.D / 4;
      const int grid = (int)cdiv(TK * nv, 1024);
      MOE_LAUNCH("permute_gather", gather_kernel<float>, dim3(grid), dim3(256), 0, st,
                 (const float*)x, row_token, offsets, EL, nv, c.D, (float*)x_perm);
    }
  }
  return MOE_OK;
}

}  // namespace moe
