// Streaming-read probe: the access pattern that reaches the highest HBM read rate on this device
// (each wavefront reads one contiguous run of 1-KiB units, 16 non-temporal loads in flight, one
// 256-thread workgroup per compute unit), timed by callers to report the achievable read ceiling.
// The refill of each ring slot is unconditional (past the end of its run a wave re-reads its
// last unit) so the loads stay in flight across the loop; the XOR folded into the sink counts
// each unit exactly once, so a caller can check that the whole buffer was read.
#include "internal.hpp"

namespace moeapq {
namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeDepth = 16;

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const u32x4* __restrict__ p, uint32_t units,
                                                              uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t waves = gridDim.x * 4u;
  const uint32_t w = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t per = units / waves, extra = units % waves;
  const uint32_t begin = w * per + (w < extra ? w : extra);
  const uint32_t n = per + (w < extra ? 1u : 0u);
  if (n == 0) return;  // uniform per wavefront
  const u32x4* base = p + static_cast<size_t>(begin) * 64 + lane;
  uint32_t acc = 0;
  u32x4 buf[kProbeDepth];
#pragma unroll
  for (int s = 0; s < kProbeDepth; ++s)
    buf[s] = __builtin_nontemporal_load(base + static_cast<size_t>(s < static_cast<int>(n) ? s : n - 1) * 64);
  for (uint32_t i0 = 0; i0 < n; i0 += kProbeDepth) {
#pragma unroll
    for (int s = 0; s < kProbeDepth; ++s) {
      const uint32_t i = i0 + s;
      const uint32_t x = buf[s].x ^ buf[s].y ^ buf[s].z ^ buf[s].w;
      acc ^= i < n ? x : 0u;
      const uint32_t nx = i + kProbeDepth < n ? i + kProbeDepth : n - 1;
      buf[s] = __builtin_nontemporal_load(base + static_cast<size_t>(nx) * 64);
    }
  }
  // fold the wavefront's lanes, then one vector atomic per wavefront
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) atomicXor(sink, acc);
}
}  // namespace

int launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  ProfileScope prof("hbm_read_probe", stream);
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(device_cu_count()), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), static_cast<uint32_t>(bytes / 1024), sink);
  return check_launch("hbm_read_probe");
}
}  // namespace moeapq
