// gate_up + SiLU(gate) * up stage of the fused Any-Precision expert FFN.
#include "apq_engine.hpp"

namespace moeapq {
namespace apq {
int launch_gate_up(const KArgs& k, int max_items, hipStream_t stream) {
  ProfileScope prof("apq_gate_up_silu", stream);
  hipLaunchKernelGGL(apq_tile_kernel<kGateUp>, dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                     stream, k);
  return check_launch("apq_gate_up_silu");
}
}  // namespace apq
}  // namespace moeapq
