// common.h -- internal helpers of the MI355X MoE library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // bf16 storage: the upper 16 bits of an IEEE binary32

// largest D and F: a grouped-GEMM tile addresses its 256 rows of up to 2F
// bf16 elements with 32-bit byte offsets inside a descriptor based at the tile
constexpr int kMaxDim = 1 << 20;

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------
MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// round to nearest even (inputs are finite)
// fp32 -> bf16, round to nearest even, two values per instruction
// (v_cvt_pk_bf16_f32: the same bits as rounding the fp32 pattern by hand
// for every finite value, in one instruction instead of about eight)
MOE_DEV uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2));
}
MOE_DEV bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static MOE_DEV float load(const float* p) { return *p; }
  static MOE_DEV float to_f32(float v) { return v; }
  static MOE_DEV float from_f32(float v) { return v; }
  static constexpr int VEC = 4;  // elements per 16 bytes
};
template <> struct Elem<bf16_t> {
  static MOE_DEV float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static MOE_DEV bf16_t from_f32(float v) { return f32_to_bf16(v); }
  static constexpr int VEC = 8;
};

// 16-byte vector of elements, widened/narrowed through fp32
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  float4 v;
  MOE_DEV void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  MOE_DEV void store(float* p) const { *reinterpret_cast<float4*>(p) = v; }
  MOE_DEV void store_nt(float* p) const { store(p); }
  MOE_DEV void load_nt(const float* p) { load(p); }
  MOE_DEV float get(int i) const { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
  MOE_DEV void to_f32(float* o) const { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
  MOE_DEV void from_f32(const float* o) { v = make_float4(o[0], o[1], o[2], o[3]); }
};
template <> struct Vec16<bf16_t> {
  uint4 v;
  MOE_DEV void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  MOE_DEV void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = v; }
  // non-temporal (streaming) forms, for data read once much later or read
  // once here: they do not displace the cached GEMM operand panels
  MOE_DEV void store_nt(bf16_t* p) const {
    typedef unsigned int nv4 __attribute__((ext_vector_type(4)));
    const nv4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<nv4*>(p));
  }
  MOE_DEV void load_nt(const bf16_t* p) {
    typedef unsigned int nv4 __attribute__((ext_vector_type(4)));
    const nv4 x = __builtin_nontemporal_load(reinterpret_cast<const nv4*>(p));
    v = make_uint4(x.x, x.y, x.z, x.w);
  }
  MOE_DEV void to_f32(float* o) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  MOE_DEV void from_f32(const float* o) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
MOE_DEV int lane_id() { return __lane_id(); }

template <typename V> MOE_DEV V shfl_xor(V v, int m) { return __shfl_xor(v, m, 64); }

MOE_DEV double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }

// lanes of the wave whose (valid) expert index equals this lane's, from one
// ballot per index bit (nbits bits cover the expert indices); 0 for an
// invalid lane
MOE_DEV uint64_t same_expert_peers(bool valid, int e, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    peers &= bit ? bb : ~bb;
  }
  return valid ? peers : 0ull;
}

// ---------------------------------------------------------------------------
// host side: launch bookkeeping (errors, optional per-kernel timing)
// ---------------------------------------------------------------------------
namespace moe {

void set_error(const char* where, hipError_t e);
bool timing_on();
void timing_before(const char* name, hipStream_t s);
void timing_after(hipStream_t s);

// launch a kernel and check the launch status
#define MOE_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                       \
  do {                                                                                 \
    if (moe::timing_on()) moe::timing_before(name, stream);                            \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);               \
    hipError_t e_ = hipGetLastError();                                                 \
    if (moe::timing_on()) moe::timing_after(stream);                                   \
    if (e_ != hipSuccess) {                                                            \
      moe::set_error(name, e_);                                                        \
      return MOE_ELAUNCH;                                                              \
    }                                                                                  \
  } while (0)

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
