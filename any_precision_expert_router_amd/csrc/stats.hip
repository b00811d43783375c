// Online routing statistics of a call (PagedWeight, Key Components 2: the routing mass of an
// expert is its selection frequency and weight) and the gate mass on non-resident experts
// ("Which Expert Misses Are Worth Waiting For?", Methodology: substituted gate mass).
//
// One workgroup.  Thread e walks expert e's pairs in the grouping's order (ascending pair id)
// and sums their gates in double; it alone updates the expert's accumulators, so no atomics are
// needed and the result does not depend on timing.  The per-thread totals are reduced in LDS
// in a fixed tree order.
#include "internal.hpp"

namespace moeapq {
namespace {
constexpr int kStatsThreads = 1024;

__global__ __launch_bounds__(kStatsThreads) void routing_stats_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    const float* __restrict__ gates, int E, const uint8_t* __restrict__ resident,
    unsigned long long* __restrict__ count, double* __restrict__ mass, double* __restrict__ sums) {
  __shared__ double red[2][kStatsThreads];
  double sub = 0.0, tot = 0.0;
  for (int e = threadIdx.x; e < E; e += kStatsThreads) {
    const int b = offsets[e], n = offsets[e + 1] - b;
    double m = 0.0;
    for (int i = 0; i < n; ++i) m += static_cast<double>(gates[pairs[b + i]]);
    count[e] += static_cast<unsigned long long>(n);
    mass[e] += m;
    tot += m;
    if (resident && resident[e] == 0) sub += m;
  }
  red[0][threadIdx.x] = sub;
  red[1][threadIdx.x] = tot;
  __syncthreads();
  for (int w = kStatsThreads / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    sums[0] += red[0][0];
    sums[1] += red[1][0];
  }
}
}  // namespace

int launch_routing_stats(const int32_t* offsets, const int32_t* pairs, const float* gates, int E,
                         const uint8_t* resident, unsigned long long* count, double* mass,
                         double* sums, hipStream_t stream) {
  ProfileScope prof("routing_stats", stream);
  hipLaunchKernelGGL(routing_stats_kernel, dim3(1), dim3(kStatsThreads), 0, stream, offsets, pairs,
                     gates, E, resident, count, mass, sums);
  return check_launch("routing_stats");
}
}  // namespace moeapq
