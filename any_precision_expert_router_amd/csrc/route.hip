// Softmax + top-k routing and stable grouping of (token, slot) pairs by expert.
//
// Routing (LYNX, 2.2 System Components: every token keeps exactly k experts; "Which Expert
// Misses Are Worth Waiting For?", Methodology: the first choice and normalised gate weights):
// one 64-lane wavefront per token.  Each lane holds ceil(E/64) candidate keys in registers; a
// key packs the order-preserving image of the fp32 logit (with -0.0 folded onto +0.0) above the
// complemented expert id, so one unsigned 64-bit maximum picks (largest logit, lowest id).  k
// rounds of a wavefront max reduction select the experts in order; the gates are the softmax of
// the k selected logits.
//
// Grouping (LYNX, 1 Problem statement: decode loads each distinct expert the batch activates):
// one workgroup.  Counts per expert by LDS integer atomics (order-free, so deterministic), an
// exclusive scan for the CSR offsets and the ascending active-expert list, then a stable
// placement: because the k experts of one token are distinct, a pair's rank inside its expert
// is the number of earlier tokens that picked that expert.  Tokens are walked in chunks through
// an LDS token x expert slot map, one thread per expert.
#include "internal.hpp"

namespace moeapq {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread workgroup

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int PER_LANE>
__global__ __launch_bounds__(64 * kRouteWaves) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * E;
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(row[e], e) : 0ull;  // real keys are never 0
  }
  uint64_t mine = 0ull;  // lane j keeps the key chosen in round j
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (key[i] == win) key[i] = 0ull;  // unique: ids differ
    if (lane == j) mine = win;
  }
  const float l0 = key_logit(__shfl(mine, 0, 64));
  const float z = lane < k ? expf(key_logit(mine) - l0) : 0.0f;
  const float s = wave_sum_f32(z);
  if (lane < k) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    ids[o] = static_cast<int32_t>(~static_cast<uint32_t>(mine));
    gates[o] = z / s;
  }
}

constexpr int kGroupThreads = 1024;
constexpr int kGroupMapBytes = 16384;  // LDS token x expert slot map per chunk

__global__ __launch_bounds__(kGroupThreads) void group_by_expert_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pairs, int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ int32_t count[MOE_MAX_EXPERTS];
  __shared__ int32_t wave_tot[2][kGroupThreads / 64];
  __shared__ uint8_t slot_map[kGroupMapBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int TK = T * k;

  for (int e = tid; e < E; e += kGroupThreads) count[e] = 0;
  __syncthreads();
  for (int p = tid; p < TK; p += kGroupThreads) atomicAdd(&count[ids[p]], 1);
  __syncthreads();

  // exclusive scans of count[e] and of (count[e] > 0), one thread per expert (E <= 1024)
  const int c = tid < E ? count[tid] : 0;
  int a = c, f = c > 0 ? 1 : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a2 = __shfl_up(a, off, 64), f2 = __shfl_up(f, off, 64);
    if (lane >= off) { a += a2; f += f2; }
  }
  if (lane == 63) { wave_tot[0][wave] = a; wave_tot[1][wave] = f; }
  __syncthreads();
  int base_a = 0, base_f = 0;
  for (int w = 0; w < wave; ++w) { base_a += wave_tot[0][w]; base_f += wave_tot[1][w]; }
  const int excl = base_a + a - c;
  const int act_pos = base_f + f - (c > 0 ? 1 : 0);
  if (tid < E) {
    offsets[tid] = excl;
    if (c > 0) active[act_pos] = tid;
  }
  if (tid == E - 1) {
    offsets[E] = excl + c;
    n_active[0] = act_pos + (c > 0 ? 1 : 0);
  }
  __syncthreads();
  // -1 padding after the active list
  int n_act = 0;
  for (int w = 0; w < kGroupThreads / 64; ++w) n_act += wave_tot[1][w];
  for (int e = tid; e < E; e += kGroupThreads)
    if (e >= n_act) active[e] = -1;

  // stable placement, chunk by chunk over tokens
  int cursor = excl;
  const int chunk = kGroupMapBytes / E > 0 ? kGroupMapBytes / E : 1;
  for (int t0 = 0; t0 < T; t0 += chunk) {
    const int tn = min(chunk, T - t0);
    for (int i = tid; i < tn * E; i += kGroupThreads) slot_map[i] = 0;
    __syncthreads();
    for (int i = tid; i < tn * k; i += kGroupThreads) {
      const int tt = i / k, j = i - tt * k;
      slot_map[tt * E + ids[(t0 + tt) * k + j]] = static_cast<uint8_t>(j + 1);
    }
    __syncthreads();
    if (tid < E && c > 0) {
      for (int tt = 0; tt < tn; ++tt) {
        const int s = slot_map[tt * E + tid];
        if (s) pairs[cursor++] = (t0 + tt) * k + (s - 1);
      }
    }
    __syncthreads();
  }
}

}  // namespace

int launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                      hipStream_t stream) {
  if (T == 0) return MOE_OK;
  const dim3 grid((T + kRouteWaves - 1) / kRouteWaves), block(64 * kRouteWaves);
  ProfileScope prof("route_topk", stream);
#define MOE_ROUTE_CASE(PL)                                                               \
  hipLaunchKernelGGL(route_topk_kernel<PL>, grid, block, 0, stream, logits, T, E, k, ids, \
                     gates)
  if (E <= 64) MOE_ROUTE_CASE(1);
  else if (E <= 128) MOE_ROUTE_CASE(2);
  else if (E <= 256) MOE_ROUTE_CASE(4);
  else if (E <= 512) MOE_ROUTE_CASE(8);
  else MOE_ROUTE_CASE(16);
#undef MOE_ROUTE_CASE
  return check_launch("route_topk");
}

int launch_group_by_expert(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                           int32_t* pairs, int32_t* active, int32_t* n_active,
                           hipStream_t stream) {
  ProfileScope prof("group_by_expert", stream);
  hipLaunchKernelGGL(group_by_expert_kernel, dim3(1), dim3(kGroupThreads), 0, stream, ids, T, k,
                     E, offsets, pairs, active, n_active);
  return check_launch("group_by_expert");
}

}  // namespace moeapq
