// Device-side helpers shared by the DCOCO kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcoco {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// bf16 values are stored as their 16-bit patterns.
struct bf16 {
  uint16_t bits;
};

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to the nearest bf16, ties to even (NaN -> canonical quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<bf16> {
  static constexpr int kPer16B = 8;
  __device__ static float to_f32(bf16 v) { return bf16_to_f32(v.bits); }
  __device__ static bf16 from_f32(float f) { return bf16{f32_to_bf16(f)}; }
};
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float f) { return f; }
};

template <typename T>
__device__ __forceinline__ float load_f32(const T* p) {
  return Elem<T>::to_f32(*p);
}

// ------------------------------------------------------------ ordering keys
// A total order on logit values used for top-K and for argmax: larger values
// map to larger unsigned keys, -0 and +0 share a key, and every NaN maps to 0,
// below -inf (whose key is the smallest a number can get).
__device__ __forceinline__ uint32_t order_key(bf16 v) {
  const uint32_t b = v.bits;
  const uint32_t a = b & 0x7fffu;
  if (a > 0x7f80u) return 0u;
  return (b & 0x8000u) ? (0x8000u - a) : (0x8000u + a);
}
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return 0u;
  return (b & 0x80000000u) ? (0x80000000u - a) : (0x80000000u + a);
}

// --------------------------------------------------------- wave utilities
__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, kWave);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// inclusive prefix sum over the wave
__device__ __forceinline__ int wave_prefix_incl(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int w = __shfl_up(v, o, kWave);
    if (l >= o) v += w;
  }
  return v;
}

}  // namespace dcoco
