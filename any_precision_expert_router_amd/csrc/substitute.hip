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
// A wavefront per token (lane j holds slot j; each lane E/64 of the token's logits and their
// residency bits; the slot loop reads slots with scalar lane reads and picks a substitute with a
// DPP key maximum), then one thread per expert for the fetch flags and the admission, which scans
// the staged slots four at a time in pair order.  Calls of up to 16 tokens run in one workgroup;
// larger ones spread the tokens over many workgroups and run the per-expert step after them.
#include "internal.hpp"
#include "wave_ops.hpp"

namespace moeapq {
namespace {
constexpr int kSubThreads = 1024;
constexpr int kSubStage = 4096;        // slots staged in LDS for the admission pass (32 KiB)
constexpr int kSubFusedTokens = 16;    // calls up to this many tokens run in one workgroup
constexpr int kSubTokenThreads = 256;  // larger calls: four tokens per workgroup

// A token's inputs: lane j < k holds slot j's expert and gate, every lane the logits of experts
// lane + 64 i.
template <int PER_LANE>
struct SubToken {
  int slot_id;
  float slot_g;
  float lg[PER_LANE];
};

template <int PER_LANE>
__device__ __forceinline__ void load_token(const float* __restrict__ logits, const int32_t* __restrict__ ids,
                                           const float* __restrict__ gates, int t, int E, int k, int lane,
                                           SubToken<PER_LANE>& x) {
  const size_t base = static_cast<size_t>(t) * k;
  x.slot_id = lane < k ? ids[base + lane] : 0;
  x.slot_g = lane < k ? gates[base + lane] : 0.0f;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    x.lg[i] = e < E ? logits[static_cast<size_t>(t) * E + e] : 0.0f;
  }
}

// Decides one token's slots (one wavefront, every lane active): lane j < k gets its slot's final
// expert and, for a substituted slot, the original one (else -1).  Slot values come from scalar
// lane reads and the substitute from the routing's DPP key maximum, so the loop waits on no LDS
// permute.  A kept miss is marked in s_fetch when given.
template <int PER_LANE>
__device__ __forceinline__ void decide_token(const SubToken<PER_LANE>& cur, uint32_t resmask, int k, int policy,
                                             float gate_threshold, int lane, int& out_id, int& out_m,
                                             uint32_t* s_fetch) {
  uint64_t cand[PER_LANE];  // keys of the lane's resident experts (0: not a candidate)
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i)
    cand[i] = (resmask >> i) & 1u ? order_key(cur.lg[i], lane + 64 * i) : 0ull;
  uint32_t taken = 0;  // bit i: expert lane + 64 i is among the token's experts
  for (int j = 0; j < k; ++j) {
    const int e = lane_int(cur.slot_id, j);
    if ((e & 63) == lane) taken |= 1u << (e >> 6);
  }
  out_id = cur.slot_id;
  out_m = -1;
  for (int j = 0; j < k; ++j) {
    const int e = lane_int(cur.slot_id, j);
    if ((lane_u32(resmask, e & 63) >> (e >> 6)) & 1u) continue;
    const float g = lane_float(cur.slot_g, j);
    const bool keep = policy == MOE_POLICY_FETCH_ALL ||
                      (policy == MOE_POLICY_GATE_RULE && (j == 0 || g >= gate_threshold)) ||
                      (policy == MOE_POLICY_FIRST_CHOICE && j == 0);
    uint64_t win = 0;
    if (!keep) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const uint64_t c = (taken >> i) & 1u ? 0ull : cand[i];
        best = c > best ? c : best;
      }
      win = wave_max_u64(best);
    }
    if (win != 0) {
      const int b = key_id(win);
      if (lane == j) {
        out_id = b;
        out_m = e;
      }
      if ((b & 63) == lane) taken |= 1u << (b >> 6);
    } else if (s_fetch && lane == 0) {
      atomicOr(&s_fetch[e >> 5], 1u << (e & 31));
    }
  }
}

// Bit i: expert lane + 64 i is resident.
template <int PER_LANE>
__device__ __forceinline__ uint32_t lane_residency(const uint8_t* __restrict__ resident, int E, int lane) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    if (e < E && resident[e] != 0) m |= 1u << i;
  }
  return m;
}

// Background admission of expert e: its accumulator plus the gates of the slots substituted away
// from it, in pair order (fp32), admitted at the threshold (then restarted at 0).
__device__ __forceinline__ void admit_expert(int e, float acc, bool staged, const int32_t* s_missed,
                                             const float* s_gates, const int32_t* __restrict__ missed,
                                             const float* __restrict__ gates, int TK, float admit_threshold,
                                             float* __restrict__ admit_mass, uint8_t* __restrict__ admit) {
  // two loops, so that each reads one address space (a pointer to either compiles to flat
  // loads); a call too large to stage reads the slots back from global memory
  if (staged) {
    int p = 0;
#pragma unroll 4
    for (; p + 4 <= TK; p += 4) {
      const int4 m = *reinterpret_cast<const int4*>(s_missed + p);
      const float4 gv = *reinterpret_cast<const float4*>(s_gates + p);
      acc = m.x == e ? acc + gv.x : acc;
      acc = m.y == e ? acc + gv.y : acc;
      acc = m.z == e ? acc + gv.z : acc;
      acc = m.w == e ? acc + gv.w : acc;
    }
    for (; p < TK; ++p)
      if (s_missed[p] == e) acc += s_gates[p];
  } else {
    for (int p = 0; p < TK; ++p)
      if (missed[p] == e) acc += gates[p];
  }
  const bool a = acc >= admit_threshold;
  admit[e] = a ? 1 : 0;
  admit_mass[e] = a ? 0.0f : acc;
}

// Calls of at most kSubFusedTokens tokens: one workgroup decides every token (a wavefront per
// token, the next token's loads issued before the current one is decided), marks kept misses in
// an LDS bitmap and stages the slots in LDS, then one thread per expert writes the fetch flags
// and runs the admission.
template <int PER_LANE>
__global__ __launch_bounds__(kSubThreads) void substitute_kernel(
    const float* __restrict__ logits, int T, int E, int k, const uint8_t* __restrict__ resident,
    int policy, float gate_threshold, int32_t* __restrict__ ids, const float* __restrict__ gates,
    int32_t* __restrict__ missed, uint8_t* __restrict__ fetch, float* __restrict__ admit_mass,
    float admit_threshold, uint8_t* __restrict__ admit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kSubThreads / 64;
  const int TK = T * k;
  const bool staged = TK <= kSubStage;
  __shared__ uint32_t s_fetch[(MOE_MAX_EXPERTS + 31) / 32];  // experts that must be fetched
  __shared__ __align__(16) int32_t s_missed[kSubStage];
  __shared__ __align__(16) float s_gates[kSubStage];
  for (int w = tid; w < (E + 31) / 32; w += kSubThreads) s_fetch[w] = 0u;
  // this thread's admission accumulators, loaded early (expert tid + i * kSubThreads)
  float acc0 = admit_mass && tid < E ? admit_mass[tid] : 0.0f;
  const uint32_t resmask = lane_residency<PER_LANE>(resident, E, lane);
  __syncthreads();
  SubToken<PER_LANE> cur{}, nxt{};
  if (wave < T) load_token<PER_LANE>(logits, ids, gates, wave, E, k, lane, cur);
  for (int t = wave; t < T; t += kWaves) {
    if (t + kWaves < T) load_token<PER_LANE>(logits, ids, gates, t + kWaves, E, k, lane, nxt);
    int out_id, out_m;
    decide_token<PER_LANE>(cur, resmask, k, policy, gate_threshold, lane, out_id, out_m, s_fetch);
    if (lane < k) {
      const size_t base = static_cast<size_t>(t) * k;
      ids[base + lane] = out_id;
      missed[base + lane] = out_m;
      if (staged) {
        s_missed[base + lane] = out_m;
        s_gates[base + lane] = cur.slot_g;
      }
    }
    cur = nxt;
  }
  __syncthreads();  // every slot is decided: the LDS bitmap and copies are complete
  for (int e = tid; e < E; e += kSubThreads) {
    fetch[e] = (s_fetch[e >> 5] >> (e & 31)) & 1u;
    if (admit_mass)
      admit_expert(e, e == tid ? acc0 : admit_mass[e], staged, s_missed, s_gates, missed, gates, TK,
                   admit_threshold, admit_mass, admit);
  }
}

// Larger calls, step 1: the tokens spread over many workgroups, a wavefront per token.
template <int PER_LANE>
__global__ __launch_bounds__(kSubTokenThreads) void substitute_tokens_kernel(
    const float* __restrict__ logits, int T, int E, int k, const uint8_t* __restrict__ resident,
    int policy, float gate_threshold, int32_t* __restrict__ ids, const float* __restrict__ gates,
    int32_t* __restrict__ missed) {
  const int lane = threadIdx.x & 63;
  const int t = static_cast<int>(blockIdx.x) * (kSubTokenThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // a whole wavefront; the kernel has no barrier
  const uint32_t resmask = lane_residency<PER_LANE>(resident, E, lane);
  SubToken<PER_LANE> cur{};
  load_token<PER_LANE>(logits, ids, gates, t, E, k, lane, cur);
  int out_id, out_m;
  decide_token<PER_LANE>(cur, resmask, k, policy, gate_threshold, lane, out_id, out_m, nullptr);
  if (lane < k) {
    const size_t base = static_cast<size_t>(t) * k;
    ids[base + lane] = out_id;
    missed[base + lane] = out_m;
  }
}

// Larger calls, step 2 (one workgroup): a non-resident expert that is still routed after step 1
// is exactly a kept miss, so the fetch flags come from the final ids; then the admission.
__global__ __launch_bounds__(kSubThreads) void substitute_admit_kernel(
    int T, int E, int k, const uint8_t* __restrict__ resident, const int32_t* __restrict__ ids,
    const float* __restrict__ gates, const int32_t* __restrict__ missed, uint8_t* __restrict__ fetch,
    float* __restrict__ admit_mass, float admit_threshold, uint8_t* __restrict__ admit) {
  const int tid = threadIdx.x;
  const int TK = T * k;
  const bool staged = TK <= kSubStage;
  __shared__ uint32_t s_fetch[(MOE_MAX_EXPERTS + 31) / 32];
  __shared__ __align__(16) int32_t s_missed[kSubStage];
  __shared__ __align__(16) float s_gates[kSubStage];
  for (int w = tid; w < (E + 31) / 32; w += kSubThreads) s_fetch[w] = 0u;
  float acc0 = admit_mass && tid < E ? admit_mass[tid] : 0.0f;
  __syncthreads();
  for (int p = tid; p < TK; p += kSubThreads) {
    const int e = ids[p];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E) && resident[e] == 0)
      atomicOr(&s_fetch[e >> 5], 1u << (e & 31));
    if (staged) {
      s_missed[p] = missed[p];
      s_gates[p] = gates[p];
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSubThreads) {
    fetch[e] = (s_fetch[e >> 5] >> (e & 31)) & 1u;
    if (admit_mass)
      admit_expert(e, e == tid ? acc0 : admit_mass[e], staged, s_missed, s_gates, missed, gates, TK,
                   admit_threshold, admit_mass, admit);
  }
}
}  // namespace

int launch_substitute(const float* logits, int T, int E, int k, const uint8_t* resident, int policy,
                      float gate_threshold, int32_t* ids, const float* gates, int32_t* missed,
                      uint8_t* fetch, float* admit_mass, float admit_threshold, uint8_t* admit,
                      hipStream_t stream) {
  ProfileScope prof("substitute", stream);
  if (T <= kSubFusedTokens) {
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
  const dim3 grid((T + kSubTokenThreads / 64 - 1) / (kSubTokenThreads / 64));
#define MOE_SUB_CASE(PL)                                                                           \
  hipLaunchKernelGGL(substitute_tokens_kernel<PL>, grid, dim3(kSubTokenThreads), 0, stream, logits, T, \
                     E, k, resident, policy, gate_threshold, ids, gates, missed)
  if (E <= 64) MOE_SUB_CASE(1);
  else if (E <= 128) MOE_SUB_CASE(2);
  else if (E <= 256) MOE_SUB_CASE(4);
  else if (E <= 512) MOE_SUB_CASE(8);
  else MOE_SUB_CASE(16);
#undef MOE_SUB_CASE
  if (int rc = check_launch("substitute_tokens")) return rc;
  hipLaunchKernelGGL(substitute_admit_kernel, dim3(1), dim3(kSubThreads), 0, stream, T, E, k, resident,
                     ids, gates, missed, fetch, admit_mass, admit_threshold, admit);
  return check_launch("substitute_admit");
}
}  // namespace moeapq
