// Wavefront-wide selection in the routing order (value descending, id ascending), shared by the
// routing, substitution and remapping kernels.  A 64-bit key packs the order-preserving image of
// an fp32 value (-0.0 folded onto +0.0, so the two tie and the lower id wins) above the
// complemented id, so one unsigned maximum picks the largest value with the lowest id.  Every
// finite value gives a key above 0, which therefore stands for "no candidate".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeapq {

__device__ __forceinline__ uint64_t order_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

// Lane `lane`'s value of v, uniform (a scalar read, not an LDS permute).
__device__ __forceinline__ int lane_int(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}
__device__ __forceinline__ float lane_float(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}


__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xf, 0xf, false);
  return o > v ? o : v;
}

// Wavefront maximum of a 32-bit value, returned uniform: DPP butterflies inside each 16-lane row
// (quad swaps, then half-row and row mirrors), then the four row maxima through scalar registers.
// Every lane of the wavefront must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp32<0xB1>(v);   // quad_perm [1,0,3,2]
  v = max_dpp32<0x4E>(v);   // quad_perm [2,3,0,1]
  v = max_dpp32<0x141>(v);  // row_half_mirror
  v = max_dpp32<0x140>(v);  // row_mirror
  const uint32_t a = lane_u32(v, 0), b = lane_u32(v, 16), c = lane_u32(v, 32), d = lane_u32(v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Inclusive prefix sum over the 64 lanes of a wavefront by DPP: shifts by 1, 2, 4 and 8 inside
// each 16-lane row (lanes without a source add 0), then the total of row 0 broadcast into row 1
// and of row 2 into row 3, then the total of rows 0-1 into rows 2-3.  Every lane must be active.
__device__ __forceinline__ int wave_inclusive_add(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Wavefront sum of an fp32 value, returned uniform: DPP butterflies inside each 16-lane row, then
// the four row sums through scalar registers, in the fixed order (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
  return (lane_float(v, 0) + lane_float(v, 16)) + (lane_float(v, 32) + lane_float(v, 48));
}

// Wavefront maximum of a 64-bit key, returned uniform: the maximum high word, then the maximum
// low word among the lanes that hold it (the lexicographic order of the two words is the order of
// the key), as two 32-bit reductions.  Every lane of the wavefront must be active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = static_cast<uint32_t>(v >> 32), lo = static_cast<uint32_t>(v);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
  return (static_cast<uint64_t>(mh) << 32) | ml;
}


}  // namespace moeapq
