// down stage of the fused Any-Precision expert FFN, and the deterministic gate-weighted combine.
#include "apq_engine.hpp"

namespace moeapq {
namespace apq {
namespace {
// y[t][r] = fp16( sum_s sum_j part[s][t*k + j][r] + sum_s part_shared[s][t][r] ), in this fixed
// order, so the result does not depend on which workgroup finished first.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                      const float* __restrict__ part_shared, int T,
                                                      int H, int k, int segs, int segs_shared,
                                                      uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ err,
                                                      int32_t* __restrict__ status) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  // the FFN launches of this call ran before: their error word is final
  if (status && i == 0) *status = err[0];
  const size_t TH = static_cast<size_t>(T) * H;
  if (i >= TH) return;
  const size_t t = i / H, r = i - t * H;
  const size_t seg_stride = TH * k;
  float s = 0.0f;
  for (int g = 0; g < segs; ++g)
    for (int j = 0; j < k; ++j) s += part[g * seg_stride + (t * k + j) * H + r];
  if (part_shared)
    for (int g = 0; g < segs_shared; ++g) s += part_shared[g * TH + i];
  y[i] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s));
}

}  // namespace

int launch_down(const KArgs& k, int max_items, hipStream_t stream) {
  ProfileScope prof("apq_down", stream);
  hipLaunchKernelGGL(apq_tile_kernel<kDown>, dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                     stream, k);
  return check_launch("apq_down");
}

int launch_combine(const float* part, const float* part_shared, int T, int H, int k, int segs,
                   int segs_shared, uint16_t* y, const int32_t* err, int32_t* status,
                   hipStream_t stream) {
  const size_t n = static_cast<size_t>(T) * H;
  ProfileScope prof("combine", stream);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, part, part_shared, T, H, k, segs, segs_shared, y, err, status);
  return check_launch("combine");
}
}  // namespace apq
}  // namespace moeapq
