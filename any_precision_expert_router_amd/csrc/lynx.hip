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
// (E/64 per lane), the slot loop on scalar lane reads and a wavefront DPP key maximum.  Both
// passes read a token's ids and logit row together, one token ahead.
#include "internal.hpp"
#include "wave_ops.hpp"

namespace moeapq {
namespace {
constexpr int kLynxThreads = 1024;

// Critical slots of a token with confidence gap c (k >= 2): min(k, bin + 1).
__device__ __forceinline__ int lynx_keep_gap(float c, int E, int k, float bin_width) {
  const float q = __fdiv_rn(c, bin_width);
  const int last = (E + k - 1) / k - 1;
  const float f = floorf(q);
  // bins 0 .. last; a negative gap (slots not in routing order) counts as bin 0
  const int b = f >= static_cast<float>(last) ? last : (f <= 0.0f ? 0 : static_cast<int>(f));
  return min(k, b + 1);
}


// A token's inputs, one wavefront: lane j < k holds slot j's expert, every lane the logits of
// experts lane + 64 i.
template <int PER_LANE>
struct LynxToken {
  int slot_id;
  float lg[PER_LANE];
};

template <int PER_LANE>
__device__ __forceinline__ void load_lynx_token(const float* __restrict__ logits, const int32_t* __restrict__ ids,
                                                int t, int E, int k, int lane, LynxToken<PER_LANE>& x) {
  x.slot_id = lane < k ? ids[static_cast<size_t>(t) * k + lane] : 0;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    x.lg[i] = e < E ? logits[static_cast<size_t>(t) * E + e] : 0.0f;
  }
}

// Expert e's logit, uniform (it sits in lane e % 64, register e / 64).
template <int PER_LANE>
__device__ __forceinline__ float token_logit(const LynxToken<PER_LANE>& x, int e) {
  float v = lane_float(x.lg[0], e & 63);
#pragma unroll
  for (int i = 1; i < PER_LANE; ++i)
    if ((e >> 6) == i) v = lane_float(x.lg[i], e & 63);
  return v;
}

// Critical slots of a token, from the two routed logits its lanes hold (the same fp32
// subtraction as reading them from the row).
template <int PER_LANE>
__device__ __forceinline__ int token_keep(const LynxToken<PER_LANE>& x, int E, int k, float bin_width) {
  if (k < 2) return k;
  const int e0 = lane_int(x.slot_id, 0), e1 = lane_int(x.slot_id, 1);
  return lynx_keep_gap(token_logit(x, e0) - token_logit(x, e1), E, k, bin_width);
}

template <int PER_LANE>
__global__ __launch_bounds__(kLynxThreads) void lynx_kernel(
    const float* __restrict__ logits, int T, int E, int k, float bin_width, int32_t* __restrict__ ids,
    int32_t* __restrict__ remapped, uint8_t* __restrict__ critical) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kLynxThreads / 64;
  __shared__ uint32_t s_crit[(MOE_MAX_EXPERTS + 31) / 32];
  for (int w = tid; w < (E + 31) / 32; w += kLynxThreads) s_crit[w] = 0u;
  __syncthreads();
  // pass 1: critical assignments.  Each wavefront takes tokens wave, wave + 16, ..., with the
  // next token's loads issued before the current one is binned.
  LynxToken<PER_LANE> cur{}, nxt{};
  if (wave < T) load_lynx_token<PER_LANE>(logits, ids, wave, E, k, lane, cur);
  for (int t = wave; t < T; t += kWaves) {
    if (t + kWaves < T) load_lynx_token<PER_LANE>(logits, ids, t + kWaves, E, k, lane, nxt);
    const int keep = token_keep<PER_LANE>(cur, E, k, bin_width);
    if (lane < keep) atomicOr(&s_crit[cur.slot_id >> 5], 1u << (cur.slot_id & 31));
    cur = nxt;
  }
  __syncthreads();
  // pass 2: remap the other slots onto the critical set; slot values come from scalar lane
  // reads and the substitute from the routing's DPP key maximum
  if (wave < T) load_lynx_token<PER_LANE>(logits, ids, wave, E, k, lane, cur);
  for (int t = wave; t < T; t += kWaves) {
    if (t + kWaves < T) load_lynx_token<PER_LANE>(logits, ids, t + kWaves, E, k, lane, nxt);
    const int slot_id = cur.slot_id;
    uint64_t cand[PER_LANE];  // keys of the lane's critical experts (0: not a candidate)
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      const bool crit = e < E && ((s_crit[e >> 5] >> (e & 31)) & 1u);
      cand[i] = crit ? order_key(cur.lg[i], e) : 0ull;
    }
    const int keep = token_keep<PER_LANE>(cur, E, k, bin_width);
    uint32_t taken = 0;  // bit i: expert lane + 64 i is among the token's experts
    for (int j = 0; j < k; ++j) {
      const int e = lane_int(slot_id, j);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
    }
    int out_id = slot_id, out_r = -1;
    for (int j = keep; j < k; ++j) {
      const int e = lane_int(slot_id, j);
      if ((s_crit[e >> 5] >> (e & 31)) & 1u) continue;
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const uint64_t c = (taken >> i) & 1u ? 0ull : cand[i];
        best = c > best ? c : best;
      }
      const uint64_t win = wave_max_u64(best);
      if (win == 0) continue;  // no free critical expert: the slot keeps its own
      const int b = key_id(win);
      if (lane == j) {
        out_id = b;
        out_r = e;
      }
      if ((b & 63) == lane) taken |= 1u << (b >> 6);
    }
    if (lane < k) {
      const size_t base = static_cast<size_t>(t) * k;
      ids[base + lane] = out_id;
      remapped[base + lane] = out_r;
    }
    cur = nxt;
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
