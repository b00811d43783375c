// Residency-aware substitution and background admission ("Which Expert Misses Are Worth Waiting
// For?", Methodology): a routed expert that is not GPU-resident is either fetched or replaced by
// a resident one, by policy -- fetch every miss; fetch a miss only if it is the router's first
// choice or its gate weight reaches a threshold (the 0.15 rule); fetch only a missed first
// choice -- and an expert whose substituted gate weight accumulates to a threshold (0.5) is
// admitted to the cache.
//
// Readings: slots are taken in order j = 0..k-1; a substituted slot gets the token's
// highest-logit resident expert that is not already among its experts (ties: the lower id, as
// in routing), keeps its gate weight, and the token keeps exactly k distinct experts; with no
// such expert left the miss is fetched.  Admission adds, per expert, the gates of this call's
// slots substituted away from it in pair order (fp32), admits at the threshold and restarts the
// accumulator at 0.
//
// One workgroup: a wavefront per token (lane j holds slot j; each lane E/64 of the token's
// logits and their residency bits, so the slot loop runs on shuffles), then one thread per
// expert for the admission.
#include <cfloat>
#include <climits>

#include "internal.hpp"

namespace moeapq {
namespace {
constexpr int kSubThreads = 1024;
constexpr int kSubStage = 4096;   // slots staged in LDS for the admission pass (32 KiB)

// (value desc, id asc) order of routing: true if (v, i) comes before (w, j)
__device__ __forceinline__ bool before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

template <int PER_LANE>
__global__ __launch_bounds__(kSubThreads) void substitute_kernel(
    const float* __restrict__ logits, int T, int E, int k, const uint8_t* __restrict__ resident,
    int policy, float gate_threshold, int32_t* __restrict__ ids, const float* __restrict__ gates,
    int32_t* __restrict__ missed, uint8_t* __restrict__ fetch, float* __restrict__ admit_mass,
    float admit_threshold, uint8_t* __restrict__ admit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int TK = T * k;
  const bool staged = TK <= kSubStage;
  __shared__ uint32_t s_fetch[(MOE_MAX_EXPERTS + 31) / 32];  // experts that must be fetched
  __shared__ int32_t s_missed[kSubStage];
  __shared__ float s_gates[kSubStage];
  for (int w = tid; w < (E + 31) / 32; w += kSubThreads) s_fetch[w] = 0u;
  // this thread's admission accumulators, loaded early (expert tid + i * kSubThreads)
  float acc0 = admit_mass && tid < E ? admit_mass[tid] : 0.0f;
  __syncthreads();
  for (int t = wave; t < T; t += kSubThreads / 64) {
    // every load of the token is issued up front: lane j < k holds slot j, each lane the
    // logits and residency of experts lane + 64 i
    const size_t base = static_cast<size_t>(t) * k;
    const int slot_id = lane < k ? ids[base + lane] : 0;
    const float slot_g = lane < k ? gates[base + lane] : 0.0f;
    float lg[PER_LANE];
    uint32_t resmask = 0;  // bit i: expert lane + 64 i is resident
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      lg[i] = e < E ? logits[static_cast<size_t>(t) * E + e] : -FLT_MAX;
      if (e < E && resident[e] != 0) resmask |= 1u << i;
    }
    uint32_t taken = 0;  // bit i: expert lane + 64 i is among the token's experts
    for (int j = 0; j < k; ++j) {
      const int e = __shfl(slot_id, j, 64);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
    }
    int out_id = slot_id, out_m = -1;
    for (int j = 0; j < k; ++j) {
      const int e = __shfl(slot_id, j, 64);
      if ((__shfl(resmask, e & 63, 64) >> (e >> 6)) & 1u) continue;
      const float g = __shfl(slot_g, j, 64);
      const bool keep = policy == MOE_POLICY_FETCH_ALL ||
                        (policy == MOE_POLICY_GATE_RULE && (j == 0 || g >= gate_threshold)) ||
                        (policy == MOE_POLICY_FIRST_CHOICE && j == 0);
      int best = INT_MAX;
      if (!keep) {
        float bv = -FLT_MAX;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
          const int c = lane + 64 * i;
          if (((resmask & ~taken) >> i) & 1u && (best == INT_MAX || before(lg[i], c, bv, best))) {
            bv = lg[i];
            best = c;
          }
        }
        for (int off = 32; off > 0; off >>= 1) {
          const float ov = __shfl_xor(bv, off, 64);
          const int oi = __shfl_xor(best, off, 64);
          if (oi != INT_MAX && (best == INT_MAX || before(ov, oi, bv, best))) {
            bv = ov;
            best = oi;
          }
        }
      }
      if (best != INT_MAX) {
        if (lane == j) {
          out_id = best;
          out_m = e;
        }
        if ((best & 63) == lane) taken |= 1u << (best >> 6);
      } else if (lane == 0) {
        atomicOr(&s_fetch[e >> 5], 1u << (e & 31));
      }
    }
    if (lane < k) {
      ids[base + lane] = out_id;
      missed[base + lane] = out_m;
      if (staged) {
        s_missed[base + lane] = out_m;
        s_gates[base + lane] = slot_g;
      }
    }
  }
  __syncthreads();  // every slot is decided: the LDS bitmap and copies are complete
  for (int e = tid; e < E; e += kSubThreads) {
    fetch[e] = (s_fetch[e >> 5] >> (e & 31)) & 1u;
    if (!admit_mass) continue;
    float acc = e == tid ? acc0 : admit_mass[e];
    // two loops, so that each reads one address space (a pointer to either compiles to flat
    // loads); a call too large to stage reads the slots back from global memory
    if (staged) {
      for (int p = 0; p < TK; ++p)
        if (s_missed[p] == e) acc += s_gates[p];
    } else {
      for (int p = 0; p < TK; ++p)
        if (missed[p] == e) acc += gates[p];
    }
    const bool a = acc >= admit_threshold;
    admit[e] = a ? 1 : 0;
    admit_mass[e] = a ? 0.0f : acc;
  }
}
}  // namespace

int launch_substitute(const float* logits, int T, int E, int k, const uint8_t* resident, int policy,
                      float gate_threshold, int32_t* ids, const float* gates, int32_t* missed,
                      uint8_t* fetch, float* admit_mass, float admit_threshold, uint8_t* admit,
                      hipStream_t stream) {
  ProfileScope prof("substitute", stream);
#define MOE_SUB_CASE(PL)                                                                          \
  hipLaunchKernelGGL(substitute_kernel<PL>, dim3(1), dim3(kSubThreads), 0, stream, logits, T, E, k, \
                     resident, policy, gate_threshold, ids, gates, missed, fetch, admit_mass,       \
                     admit_threshold, admit)
  if (E <= 64) MOE_SUB_CASE(1);
  else if (E <= 128) MOE_SUB_CASE(2);
  else if (E <= 256) MOE_SUB_CASE(4);
  else if (E <= 512) MOE_SUB_CASE(8);
  else MOE_SUB_CASE(16);
#undef MOE_SUB_CASE
  return check_launch("substitute");
}
}  // namespace moeapq
