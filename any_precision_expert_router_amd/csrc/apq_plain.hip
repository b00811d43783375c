// Single-block decode GEMV (the FFN's tile engine in plain mode) and the index decoder, both for
// parity checks of the decode path.
#include "apq_engine.hpp"

namespace moeapq {
namespace apq {
namespace {
// Debug / parity: every q-bit index of a block, row-major uint8.
template <int Q>
MOE_INLINE void decode_unit(const AS_GLOBAL u32x4* pbase, size_t plane_u4, uint8_t* dst) {
  u32x4 u[Q];
#pragma unroll
  for (int p = 0; p < Q; ++p) u[p] = pbase[p * plane_u4];
#pragma unroll
  for (int jw = 0; jw < 4; ++jw) {
    uint32_t w[Q];
#pragma unroll
    for (int p = 0; p < Q; ++p) w[p] = word_of(u[p], jw);
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      const uint32_t s = single_word<Q>(w, o);
#pragma unroll
      for (int b = 0; b < 4; ++b) dst[jw * 32 + 8 * b + 2 * (o & 3) + (o >> 2)] = (s >> (8 * b)) & 0xff;
    }
  }
}

__global__ __launch_bounds__(64) void decode_indices_kernel(const uint32_t* __restrict__ planes,
                                                            int rows, int cols, int q,
                                                            uint8_t* __restrict__ out) {
  const int nc4 = cols / kColChunk;
  const int panel = blockIdx.x / nc4, c4 = blockIdx.x - panel * nc4;
  const int lane = threadIdx.x;
  const int row = panel * kRowPanel + lane;
  const AS_GLOBAL u32x4* pbase = gview<u32x4>(planes) + (static_cast<size_t>(panel) * nc4 + c4) * 64 + lane;
  const size_t plane_u4 = static_cast<size_t>(rows) * cols / 128;
  uint8_t* dst = out + static_cast<size_t>(row) * cols + c4 * kColChunk;
  switch (q) {
    case 1: decode_unit<1>(pbase, plane_u4, dst); break;
    case 2: decode_unit<2>(pbase, plane_u4, dst); break;
    case 3: decode_unit<3>(pbase, plane_u4, dst); break;
    case 4: decode_unit<4>(pbase, plane_u4, dst); break;
    case 5: decode_unit<5>(pbase, plane_u4, dst); break;
    case 6: decode_unit<6>(pbase, plane_u4, dst); break;
    case 7: decode_unit<7>(pbase, plane_u4, dst); break;
    default: decode_unit<8>(pbase, plane_u4, dst); break;
  }
}

}  // namespace

int launch_plain(const KArgs& k, int max_items, hipStream_t stream) {
  ProfileScope prof("apq_gemv", stream);
  hipLaunchKernelGGL(apq_tile_kernel<kPlain>, dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                     stream, k);
  return check_launch("apq_gemv");
}

int launch_decode(const moe_apq_block& blk, uint8_t* idx_out, hipStream_t stream) {
  const int units = (blk.rows / kRowPanel) * (blk.cols / kColChunk);
  ProfileScope prof("apq_decode_indices", stream);
  hipLaunchKernelGGL(decode_indices_kernel, dim3(units), dim3(64), 0, stream, blk.planes, blk.rows,
                     blk.cols, static_cast<int>(blk.q), idx_out);
  return check_launch("apq_decode_indices");
}
}  // namespace apq
}  // namespace moeapq
