// LayerNorm of projection rows straight into a bf16 MFMA operand tile in LDS
// (non-affine: (x - mean) / sqrt(var + eps), two-pass statistics in fp32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "wave.h"

namespace dcoco {

// One wave normalises RPW rows m = mfirst .. mfirst + RPW - 1 of the sum of
// SPLIT fp32 partial blocks x[s][M][ldx] over columns col0 .. col0 + r - 1
// (r <= 256, r % 4 == 0) and writes them as bf16 to tile rows 0 .. RPW - 1
// (kStr bytes apart).  Lane l covers columns 4l .. 4l + 3; rows past M are
// written as zeros.  Every load is issued before the first wait: lanes past r
// and rows past M re-read a valid element and are masked afterwards.  The
// partial blocks are added in order 0 .. SPLIT - 1.
template <int RPW, int SPLIT>
__device__ __forceinline__ void ln_rows_tile(const float* __restrict__ x, int M, int ldx, int col0, int r,
                                             float eps, int mfirst, char* tile_rows, int kStr, int l) {
  const int c4 = 4 * l;
  const bool on = c4 < r;
  const int cc = on ? c4 : 0;
  const float inv_r = 1.0f / static_cast<float>(r);
  float4 v[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const long long m = min(mfirst + q, M - 1);
    v[q] = *reinterpret_cast<const float4*>(x + m * ldx + col0 + cc);
  }
#pragma unroll
  for (int s2 = 1; s2 < SPLIT; ++s2)
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const long long m = min(mfirst + q, M - 1);
      const float4 b = *reinterpret_cast<const float4*>(x + (s2 * static_cast<long long>(M) + m) * ldx + col0 + cc);
      v[q].x += b.x; v[q].y += b.y; v[q].z += b.z; v[q].w += b.w;
    }
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    if (!on) v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    const float mean = wave_sum_dpp((v[q].x + v[q].y) + (v[q].z + v[q].w)) * inv_r;
    float4 d = make_float4(v[q].x - mean, v[q].y - mean, v[q].z - mean, v[q].w - mean);
    if (!on) d = make_float4(0.f, 0.f, 0.f, 0.f);
    const float sq = (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
    const float inv = rsqrtf(wave_sum_dpp(sq) * inv_r + eps);
    const bool live = mfirst + q < M;
    if (on) {
      uint2 pk;
      pk.x = live ? (static_cast<uint32_t>(f32_to_bf16(d.x * inv)) |
                     (static_cast<uint32_t>(f32_to_bf16(d.y * inv)) << 16)) : 0u;
      pk.y = live ? (static_cast<uint32_t>(f32_to_bf16(d.z * inv)) |
                     (static_cast<uint32_t>(f32_to_bf16(d.w * inv)) << 16)) : 0u;
      *reinterpret_cast<uint2*>(tile_rows + q * kStr + c4 * 2) = pk;
    }
  }
}

}  // namespace dcoco
