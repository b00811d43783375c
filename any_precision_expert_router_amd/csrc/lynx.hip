// Batch-aware expert remapping (LYNX, 2.2 System Components): a confidence analyser cuts each
// token's router confidence, taken from the gap between its best logits, into bins whose width
// and count follow from the sparsity ratio k/N alone (AffinityBinning), and an expert remapper
// redirects the low-affinity token-expert assignments to the surviving critical set of experts,
// so that every token still activates exactly k experts while the batch activates fewer
// distinct ones.
//
// Readings: confidence c = l(slot 0) - l(slot 1), one fp32 subtraction on the routed slots;
// bins of width w = k/N (passed in, fp32) and ceil(N/k) of them, b = min(floor(c / w), last), at
// least 0, with the quotient rounded once (IEEE fp32 division); a token in bin b keeps its first min(k, b + 1)
// slots as critical assignments; the critical set is the union of those slots' experts.  Every
// other slot whose expert is outside the critical set takes the token's highest-logit critical
// expert not already among its experts (ties: lower id, as in routing), slots in order
// j = 0..k-1, and keeps its gate weight; with no such expert left it keeps its own.
//
// One workgroup: pass 1, a wavefront per token, sets the critical bits in an LDS bitmap; after
// a barrier, pass 2 remaps with the token's logits and critical bits spread over the lanes
// (E/64 per lane) so the slot loop runs on shuffles and a wavefront arg-max.
#include <cfloat>
#include <climits>

#include "internal.hpp"

namespace moeapq {
namespace {
constexpr int kLynxThreads = 1024;

__device__ __forceinline__ bool lynx_before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// Critical slots of a token: min(k, bin + 1) (all k for k = 1).  Uniform across the wavefront.
__device__ __forceinline__ int lynx_keep(const float* __restrict__ row, int e0, int e1, int E, int k,
                                         float bin_width) {
  if (k < 2) return k;
  const float c = row[e0] - row[e1];
  const float q = __fdiv_rn(c, bin_width);
  const int last = (E + k - 1) / k - 1;
  const float f = floorf(q);
  // bins 0 .. last; a negative gap (slots not in routing order) counts as bin 0
  const int b = f >= static_cast<float>(last) ? last : (f <= 0.0f ? 0 : static_cast<int>(f));
  return min(k, b + 1);
}

template <int PER_LANE>
__global__ __launch_bounds__(kLynxThreads) void lynx_kernel(
    const float* __restrict__ logits, int T, int E, int k, float bin_width, int32_t* __restrict__ ids,
    int32_t* __restrict__ remapped, uint8_t* __restrict__ critical) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ uint32_t s_crit[(MOE_MAX_EXPERTS + 31) / 32];
  for (int w = tid; w < (E + 31) / 32; w += kLynxThreads) s_crit[w] = 0u;
  __syncthreads();
  // pass 1: critical assignments
  for (int t = wave; t < T; t += kLynxThreads / 64) {
    const size_t base = static_cast<size_t>(t) * k;
    const int slot_id = lane < k ? ids[base + lane] : 0;
    const float* row = logits + static_cast<size_t>(t) * E;
    const int keep = lynx_keep(row, __shfl(slot_id, 0, 64), __shfl(slot_id, k > 1 ? 1 : 0, 64), E, k,
                               bin_width);
    if (lane < keep) atomicOr(&s_crit[slot_id >> 5], 1u << (slot_id & 31));
  }
  __syncthreads();
  // pass 2: remap the other slots onto the critical set
  for (int t = wave; t < T; t += kLynxThreads / 64) {
    const size_t base = static_cast<size_t>(t) * k;
    const int slot_id = lane < k ? ids[base + lane] : 0;
    const float* row = logits + static_cast<size_t>(t) * E;
    float lg[PER_LANE];
    uint32_t crit = 0;  // bit i: expert lane + 64 i is critical
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      lg[i] = e < E ? row[e] : -FLT_MAX;
      if (e < E && ((s_crit[e >> 5] >> (e & 31)) & 1u)) crit |= 1u << i;
    }
    const int keep = lynx_keep(row, __shfl(slot_id, 0, 64), __shfl(slot_id, k > 1 ? 1 : 0, 64), E, k,
                               bin_width);
    uint32_t taken = 0;  // bit i: expert lane + 64 i is among the token's experts
    for (int j = 0; j < k; ++j) {
      const int e = __shfl(slot_id, j, 64);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
    }
    int out_id = slot_id, out_r = -1;
    for (int j = keep; j < k; ++j) {
      const int e = __shfl(slot_id, j, 64);
      if ((s_crit[e >> 5] >> (e & 31)) & 1u) continue;
      float bv = -FLT_MAX;
      int best = INT_MAX;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int c = lane + 64 * i;
        if (((crit & ~taken) >> i) & 1u && (best == INT_MAX || lynx_before(lg[i], c, bv, best))) {
          bv = lg[i];
          best = c;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(best, off, 64);
        if (oi != INT_MAX && (best == INT_MAX || lynx_before(ov, oi, bv, best))) {
          bv = ov;
          best = oi;
        }
      }
      if (best == INT_MAX) continue;  // no free critical expert: the slot keeps its own
      if (lane == j) {
        out_id = best;
        out_r = e;
      }
      if ((best & 63) == lane) taken |= 1u << (best >> 6);
    }
    if (lane < k) {
      ids[base + lane] = out_id;
      remapped[base + lane] = out_r;
    }
  }
  for (int e = tid; e < E; e += kLynxThreads) critical[e] = (s_crit[e >> 5] >> (e & 31)) & 1u;
}
}  // namespace

int launch_lynx_remap(const float* logits, int T, int E, int k, float bin_width, int32_t* ids,
                      int32_t* remapped, uint8_t* critical, hipStream_t stream) {
  ProfileScope prof("lynx_remap", stream);
#define MOE_LYNX_CASE(PL)                                                                          \
  hipLaunchKernelGGL(lynx_kernel<PL>, dim3(1), dim3(kLynxThreads), 0, stream, logits, T, E, k,      \
                     bin_width, ids, remapped, critical)
  if (E <= 64) MOE_LYNX_CASE(1);
  else if (E <= 128) MOE_LYNX_CASE(2);
  else if (E <= 256) MOE_LYNX_CASE(4);
  else if (E <= 512) MOE_LYNX_CASE(8);
  else MOE_LYNX_CASE(16);
#undef MOE_LYNX_CASE
  return check_launch("lynx_remap");
}
}  // namespace moeapq
