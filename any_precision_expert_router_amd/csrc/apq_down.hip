// down stage of the fused Any-Precision expert FFN, and the deterministic gate-weighted combine.
#include "apq_engine.hpp"

namespace moeapq {
namespace apq {
namespace {
// y[t][r] = fp16( sum_s sum_j part[s][t*k + j][r] + sum_s part_shared[s][t][r] ), in this fixed
// order, so the result does not depend on which workgroup finished first.
// Four consecutive columns of one token per thread (H is a multiple of 64): 16-byte partial-sum
// loads and one 8-byte store (four 2-byte stores when y is not 8-byte aligned), the sums in the
// fixed order segment, then slot j, then the shared expert's segments.
template <bool Y_ALIGNED>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                      const float* __restrict__ part_shared, int T,
                                                      int H, int k, int segs, int segs_shared,
                                                      uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ err,
                                                      int32_t* __restrict__ status) {
  const uint32_t q = blockIdx.x * 256u + threadIdx.x;   // quad of columns
  // the FFN launches of this call ran before: their error word is final
  if (status && q == 0) *status = err[0];
  const uint32_t hq = static_cast<uint32_t>(H) / 4;
  if (q >= static_cast<uint32_t>(T) * hq) return;
  const uint32_t t = q / hq, r = (q - t * hq) * 4;
  const size_t TH = static_cast<size_t>(T) * H;
  const size_t seg_stride = TH * k;
  float4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = 0; g < segs; ++g)
    for (int j = 0; j < k; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(part + g * seg_stride + (static_cast<size_t>(t) * k + j) * H + r);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  const size_t i = static_cast<size_t>(t) * H + r;
  if (part_shared)
    for (int g = 0; g < segs_shared; ++g) {
      const float4 v = *reinterpret_cast<const float4*>(part_shared + g * TH + i);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
  const uint16_t h0 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s.x));
  const uint16_t h1 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s.y));
  const uint16_t h2 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s.z));
  const uint16_t h3 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s.w));
  if constexpr (Y_ALIGNED) {
    *reinterpret_cast<uint2*>(y + i) = make_uint2(h0 | (static_cast<uint32_t>(h1) << 16),
                                                  h2 | (static_cast<uint32_t>(h3) << 16));
  } else {
    y[i] = h0;
    y[i + 1] = h1;
    y[i + 2] = h2;
    y[i + 3] = h3;
  }
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
  const size_t n = static_cast<size_t>(T) * H / 4;   // column quads (H % 64 == 0)
  ProfileScope prof("combine", stream);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if ((reinterpret_cast<uintptr_t>(y) & 7) == 0)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, stream, part, part_shared, T, H, k, segs,
                       segs_shared, y, err, status);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, stream, part, part_shared, T, H, k, segs,
                       segs_shared, y, err, status);
  return check_launch("combine");
}
}  // namespace apq
}  // namespace moeapq
