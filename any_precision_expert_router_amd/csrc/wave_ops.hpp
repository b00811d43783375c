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
