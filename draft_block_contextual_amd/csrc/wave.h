// Wave64 reductions on DPP lane moves (gfx9 family): no LDS round trips.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcoco {

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over all 64 lanes, returned to every lane: within each 16-lane row by
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror and row_mirror
// (each step adds the partner lane's partial sum), then the four row sums
// read out of lanes 0, 16, 32 and 48.  The order of additions is fixed.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t read_lane_u32(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Maximum over all 64 lanes, same lane moves as wave_sum_dpp.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, dpp_move_u32<0xB1>(v));
  v = max(v, dpp_move_u32<0x4E>(v));
  v = max(v, dpp_move_u32<0x141>(v));
  v = max(v, dpp_move_u32<0x140>(v));
  return max(max(read_lane_u32(v, 0), read_lane_u32(v, 16)), max(read_lane_u32(v, 32), read_lane_u32(v, 48)));
}

}  // namespace dcoco
