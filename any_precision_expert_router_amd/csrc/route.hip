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
// one workgroup.  Per-expert counts, an exclusive scan for the CSR offsets and the ascending
// active-expert list, then a stable placement (pair id ascending inside an expert).  Routing
// output names k distinct experts per token, so a pair's rank inside its expert is the number of
// earlier pairs that picked that expert: small batches fill an LDS token x expert slot map and
// one thread per expert counts and then walks its column; large batches run a segmented
// counting sort (one wavefront per run of tokens, per-segment counts by LDS integer atomics,
// which are order-free and so deterministic).  The standalone
// grouping also accepts ids it did not produce: an id outside [0, E) is not placed, and a token
// that names an expert twice is placed in slot order.
#include "internal.hpp"
#include "wave_ops.hpp"

namespace moeapq {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread workgroup

// One wavefront routes token t: each lane holds PER_LANE candidate keys; k rounds of the
// wavefront maximum select the experts in order; the gates are the softmax of the k logits.
template <int PER_LANE>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int32_t* ids_out,
                                            float* gates_out, int32_t* ids_copy, float* gates_copy) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? order_key(row[e], e) : 0ull;  // real keys are never 0
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
  const float l0 = key_value(readlane64(mine, 0));
  // computed on every lane and selected, so that no branch (EXEC write) precedes the DPP sum
  const float ez = expf(key_value(mine) - l0);
  const float z = lane < k ? ez : 0.0f;
  const float s = wave_sum_f32(z);
  if (lane < k) {
    const int32_t id = key_id(mine);
    ids_out[lane] = id;
    gates_out[lane] = z / s;
    if (ids_copy) ids_copy[lane] = id;
    if (gates_copy) gates_copy[lane] = z / s;
  }
}

template <int PER_LANE>
__global__ __launch_bounds__(64 * kRouteWaves) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ gates) {
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t o = static_cast<size_t>(t) * k;
  route_token<PER_LANE>(logits + static_cast<size_t>(t) * E, E, k, ids + o, gates + o, nullptr, nullptr);
}

// Workgroup barrier for LDS traffic only (see lds_barrier); the routing kernels' global stores
// (ids, gates, offsets, pairs, records) stay in flight across it.
__device__ __forceinline__ void group_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

constexpr int kGroupThreads = 1024;
constexpr int kGroupMapBytes = 16384;  // LDS of the stable placement (slot map or segment counters)

struct GroupSmem {
  int32_t wave_tot[2][kGroupThreads / 64];  // per wavefront: pairs, active experts
  union {
    uint8_t slot_map[kGroupMapBytes];     // small batches: token x expert slot map
    int32_t seg_pos[kGroupMapBytes / 4];  // large batches: [segments][E] pair counts, then positions
  };
  int32_t dup_tag[kGroupMapBytes / 4];    // large batches: [segments][E] last token that named e
  int32_t offsets[MOE_MAX_EXPERTS + 1];  // LDS copies of the grouping results for the records
  int32_t active[MOE_MAX_EXPERTS];
  int32_t qslot[2][4][18];                // records: per module, class and order bucket, counts then positions
  int32_t cls_tot[2][4];                  // records: per module and class
  int32_t n_active;
};
static_assert(kFusedRouteMaxT * MOE_MAX_EXPERTS <= kGroupMapBytes, "a fused call's slot map fits");

// The records' counters start at zero; cleared with the grouping's own LDS, before its first
// barrier.
__device__ __forceinline__ void zero_record_counters(GroupSmem& sm) {
  const int tid = threadIdx.x;
  if (tid < 2 * 4 * 18) (&sm.qslot[0][0][0])[tid] = 0;
  if (tid < 8) (&sm.cls_tot[0][0])[tid] = 0;
}

// Exclusive scans of the per-expert pair counts and of (count > 0), one thread per expert
// (thread e holds c = count of expert e, 0 for e >= E), then the CSR offsets, the ascending
// active-expert list (-1 after it) and their LDS copies.  Returns the expert's first position.
// One barrier (the wavefront totals).
__device__ __forceinline__ int scan_counts(int c, int E, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                           GroupSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int a = wave_inclusive_add(c), f = wave_inclusive_add(c > 0 ? 1 : 0);
  if (lane == 63) {
    sm.wave_tot[0][wave] = a;
    sm.wave_tot[1][wave] = f;
  }
  group_barrier();
  int base_a = 0, base_f = 0, n_act = 0;
  for (int w = 0; w < kGroupThreads / 64; ++w) {
    const int ta = sm.wave_tot[0][w], tf = sm.wave_tot[1][w];
    if (w < wave) {
      base_a += ta;
      base_f += tf;
    }
    n_act += tf;
  }
  const int excl = base_a + a - c;
  const int act_pos = base_f + f - (c > 0 ? 1 : 0);
  if (tid < E) {
    offsets[tid] = excl;
    sm.offsets[tid] = excl;
    if (c > 0) {
      active[act_pos] = tid;
      sm.active[act_pos] = tid;
    }
    if (tid >= n_act) active[tid] = -1;
  }
  if (tid == E - 1) {
    offsets[E] = excl + c;
    sm.offsets[E] = excl + c;
  }
  if (tid == 0) {
    n_active[0] = n_act;
    sm.n_active = n_act;
  }
  return excl;
}

// Stable grouping by one workgroup of kGroupThreads threads (E <= kGroupThreads).  `ids` may
// have been written by this workgroup before a barrier.  SEGMENTED picks the placement: a
// segmented counting sort (large batches: every wavefront places its own run of tokens), or a
// token x expert slot map walked by one thread per expert (small batches, T * E <=
// kGroupMapBytes, where it measured faster).  Each placement counts the pairs per expert from
// its own map, so the grouping takes three barriers (slot map) or four (segmented), plus the one
// the caller places after it before anything reads the results (offsets, active, n_active,
// pairs and pairs_lds, in global memory and in LDS).  It also clears the records' counters.
template <bool SEGMENTED, bool DISTINCT = false>
__device__ __forceinline__ void group_body(const int32_t* ids, int T, int k, int E, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ pairs, int32_t* __restrict__ active,
                           int32_t* __restrict__ n_active, GroupSmem& sm, int32_t* pairs_lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // this thread's expert for the per-expert loops; threads past E read expert 0's column and
  // drop it (a select, so that no branch (EXEC write) precedes the DPP scans)
  const int e_ld = tid < E ? tid : 0;
  zero_record_counters(sm);

  if constexpr (SEGMENTED) {
    // stable placement by a segmented counting sort: the tokens are cut into S consecutive
    // segments, one per wavefront; each wavefront counts its segment's pairs per expert, a
    // per-expert prefix over the segments (starting at the expert's offset) gives each segment its
    // first position, and each wavefront then walks its tokens in order, lane j placing slot j.
    // When a token's k experts are distinct (always so for routing output), its k lanes never
    // update the same position counter; a token that names an expert twice takes an exact,
    // slower path that keeps the slot order.  An id outside [0, E) names no expert: its pair is
    // not placed (offsets[E] counts placed pairs).
    const int S = max(1, min(kGroupThreads / 64, static_cast<int>(kGroupMapBytes / (4 * E))));
    const int seg_len = (T + S - 1) / S;
    for (int i = tid; i < S * E; i += kGroupThreads) {
      sm.seg_pos[i] = 0;
      if constexpr (!DISTINCT) sm.dup_tag[i] = -1;
    }
    group_barrier();
    const int t_begin = min(T, wave * seg_len), t_end = min(T, t_begin + seg_len);
    if (wave < S) {
      for (int i = t_begin * k + lane; i < t_end * k; i += 64) {
        const int e = ids[i];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&sm.seg_pos[wave * E + e], 1);
      }
    }
    group_barrier();
    int cnt = 0;
    for (int w = 0; w < S; ++w) cnt += sm.seg_pos[w * E + e_ld];
    const int c = tid < E ? cnt : 0;
    const int excl = scan_counts(c, E, offsets, active, n_active, sm);
    if (tid < E) {
      int run = excl;
      for (int w = 0; w < S; ++w) {
        const int n = sm.seg_pos[w * E + tid];
        sm.seg_pos[w * E + tid] = run;
        run += n;
      }
    }
    group_barrier();
    if (wave < S && lane < k) {
      constexpr int kBatch = 16;  // expert ids loaded ahead of the in-order placement
      int32_t* pos_of = sm.seg_pos + wave * E;
      int32_t* tag_of = sm.dup_tag + wave * E;
      for (int t0 = t_begin; t0 < t_end; t0 += kBatch) {
        int e[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) e[u] = t0 + u < t_end ? ids[(t0 + u) * k + lane] : -1;
        // Two slots of one token naming the same expert: each valid slot swaps its token into
        // the expert's tag; the later of two such slots gets its own token back.  The swaps of
        // a token complete before the next token's (one LDS instruction each, in order).
        // (ids the caller guarantees distinct per token, DISTINCT, skip the swaps)
        bool clash[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const bool valid = static_cast<unsigned>(e[u]) < static_cast<unsigned>(E);
          clash[u] = !DISTINCT && valid && atomicExch(&tag_of[valid ? e[u] : 0], t0 + u) == t0 + u;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (t0 + u < t_end) {
            const int p = (t0 + u) * k + lane;
            const int eu = e[u];
            const bool valid = static_cast<unsigned>(eu) < static_cast<unsigned>(E);
            if (DISTINCT || __ballot(clash[u]) == 0) {
              // distinct experts: the token's slots never share a position counter
              if (valid) {
                const int pos = pos_of[eu];
                pos_of[eu] = pos + 1;
                if (pairs_lds) pairs_lds[pos] = p;
                pairs[pos] = p;
              }
            } else {
              // repeated experts: the first slot naming an expert takes positions for all of
              // them, each slot its rank among them (slot order, so the sort stays stable)
              int rank = 0, cnt2 = 0, first = lane;
              for (int j2 = 0; j2 < k; ++j2) {
                const int e2 = __shfl(eu, j2, 64);
                if (e2 == eu) {
                  if (j2 < lane) {
                    ++rank;
                    first = min(first, j2);
                  }
                  ++cnt2;
                }
              }
              int base = 0;
              if (valid && rank == 0) {
                base = pos_of[eu];
                pos_of[eu] = base + cnt2;
              }
              base = __shfl(base, first, 64);
              if (valid) {
                if (pairs_lds) pairs_lds[base + rank] = p;
                pairs[base + rank] = p;
              }
            }
          }
        }
      }
    }
  } else {
    // stable placement through a token x expert slot map (the whole call in one map): because
    // the k experts of one token are distinct, a pair's rank inside its expert is the number of
    // earlier tokens that picked it.  Thread e counts its column, then walks it again in token
    // order from its offset.
    uint32_t* map32 = reinterpret_cast<uint32_t*>(sm.slot_map);
    for (int i = tid; 4 * i < T * E; i += kGroupThreads) map32[i] = 0u;
    group_barrier();
    for (int i = tid; i < T * k; i += kGroupThreads) {
      const int tt = i / k, j = i - tt * k;
      const int e = ids[i];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
        sm.slot_map[tt * E + e] = static_cast<uint8_t>(j + 1);
    }
    group_barrier();
    int cnt = 0;
    for (int tt = 0; tt < T; ++tt) cnt += sm.slot_map[tt * E + e_ld] != 0 ? 1 : 0;
    const int c = tid < E ? cnt : 0;
    int cursor = scan_counts(c, E, offsets, active, n_active, sm);
    if (tid < E && c > 0) {
      for (int tt = 0; tt < T; ++tt) {
        const int sl = sm.slot_map[tt * E + tid];
        if (sl) {
          const int p = tt * k + (sl - 1);
          if (pairs_lds) pairs_lds[cursor] = p;
          pairs[cursor++] = p;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kGroupThreads) void group_by_expert_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pairs, int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ GroupSmem sm;
  group_body<true>(ids, T, k, E, offsets, pairs, active, n_active, sm, nullptr);
}

// The tests are combined without short-circuit, so that no field's load waits on another's test.
__device__ __forceinline__ bool block_valid(const moe_apq_block& b, int rows, int cols) {
  const uintptr_t align = reinterpret_cast<uintptr_t>(b.planes) | reinterpret_cast<uintptr_t>(b.lut);
  return (b.planes != nullptr) & (b.lut != nullptr) & ((align & 15) == 0) & (b.rows == rows) &
         (b.cols == cols) & (b.q >= 1) & (b.q <= 8) & (b.state == MOE_PAGE_GPU);
}

__device__ __forceinline__ void fill_record(ExpertRecord& rec, const moe_apq_block& gu,
                                            const moe_apq_block& dn, int inter, const RecordArgs& r) {
  rec.planes[0] = gu.planes;
  rec.planes[1] = dn.planes;
  rec.lut[0] = gu.lut;
  rec.lut[1] = dn.lut;
  const int ok = static_cast<int>(block_valid(gu, 2 * inter, r.H)) &
                 static_cast<int>(block_valid(dn, r.H, inter));
  rec.meta = record_meta(gu.q, dn.q, ok != 0);
}

// Records of the shared expert and of the routed experts, the count of routed records, and
// zeroed work counters.  One thread per active expert (blockDim >= E).  Multi-token experts'
// records come first, split into token groups in small calls, then the streaming experts'
// (split and order: see kRecGroupTok in internal.hpp).  The grouping comes from this workgroup's
// LDS copies (after a barrier, with the order counters cleared before it: zero_record_counters);
// pairs and gates from LDS when the routing ran in this workgroup, else from global memory.
__device__ void records_body(GroupSmem& sm, const int32_t* pairs, const float* gates,
                             const RecordArgs& r) {
  const int tid = threadIdx.x;
  const int n_act = sm.n_active;
  const bool split = static_cast<long>(r.T) * r.k <= kRecSplitMaxPairs;
  int e = -1, base = 0, n = 0, groups = 0;
  // Per module, the records come in four classes: the matrix-core items, then the streaming
  // items by token count, larger first (3-4, 2, 1; with the current switch at most 2 tokens
  // stream) -- a streaming workgroup keeps its ring across consecutive
  // items whose token count fits the ring's, so equal counts are kept together.  Whether an
  // item streams depends on its block's width (takes_stream), so the two modules of one expert
  // may fall in different classes; the split into token groups does not (an expert with more
  // than kRecGroupTok tokens never streams).
  ExpertRecord rec;
  int cls[2] = {0, 0}, qm[2] = {0, 0};
  const bool act_ = tid < n_act;
  if (act_) {
    e = sm.active[tid];
    base = sm.offsets[e];
    n = sm.offsets[e + 1] - base;
    groups = split && n > kRecGroupTok ? (n + kRecGroupTok - 1) / kRecGroupTok : 1;
    fill_record(rec, r.table[2 * e], r.table[2 * e + 1], r.I, r);
    const bool ok = record_ok(rec.meta);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      qm[m] = ok ? record_q(rec.meta, m) : 0;
      cls[m] = !(ok && takes_stream(n, qm[m], r.dense_threshold)) ? 0 : (n >= 3 ? 1 : (n == 2 ? 2 : 3));
    }
  }
  // Per module, each class's records are ordered roughly by cost, costliest first, so that the
  // queue hands out the longest items first and the tail once it runs dry is shorter: the
  // matrix-core records with wide passes (more than 32 tokens) first, then by that module's
  // width, widest first.  Consecutive streaming items then also share a width more often (their
  // ring continues only across items of one width).  Positions inside a bucket come from LDS
  // atomics: the order only schedules work, every item's result is the same.  The counters
  // were cleared before the grouping's first barrier.
  int bk[2] = {0, 0};
  if (act_) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bk[m] = qm[m] + (cls[m] == 0 && n > kRecDensePassTok ? 9 : 0);
      atomicAdd(&sm.qslot[m][cls[m]][bk[m]], groups);
    }
  }
  group_barrier();
  // per module and class: bucket counts -> first positions inside the class, and its total
  if (tid < 8) {
    const int m = tid >> 2, c = tid & 3;
    int run = 0;
    for (int b = 17; b >= 0; --b) {
      const int cnt = sm.qslot[m][c][b];
      sm.qslot[m][c][b] = run;
      run += cnt;
    }
    sm.cls_tot[m][c] = run;
  }
  group_barrier();
  int first[2] = {0, 0};  // per module: records of the classes before this expert's
  int tot = 0;            // records in all (the same for both modules)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    tot += sm.cls_tot[0][c];
#pragma unroll
    for (int m = 0; m < 2; ++m)
      if (c < cls[m]) first[m] += sm.cls_tot[m][c];
  }
  if (tid < n_act) {
    int pos_m[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) pos_m[m] = first[m] + atomicAdd(&sm.qslot[m][cls[m]][bk[m]], groups);
    const size_t stride = max_records(r.T, r.E, r.k);
    rec.expert = e;
    for (int g = 0; g < groups; ++g) {
      rec.src_base = base + g * kRecGroupTok;
      rec.n = groups > 1 ? min(kRecGroupTok, n - g * kRecGroupTok) : n;
#pragma unroll
      for (int t = 0; t < kRecTok; ++t) {
        const int p = t < rec.n ? pairs[rec.src_base + t] : 0;
        rec.pair[t] = p;
        rec.tok[t] = p / r.k;
        rec.gate[t] = t < rec.n ? gates[p] : 0.0f;
      }
      r.recs[1 + pos_m[0] + g] = rec;
      r.recs[stride + 1 + pos_m[1] + g] = rec;
    }
  }
  if (tid == 0) {
    r.n_recs[0] = tot;
    rec = ExpertRecord{};
    if (r.shared) {
      fill_record(rec, r.shared[0], r.shared[1], r.I_shared, r);
    } else {
      rec.meta = record_meta(0, 0, false);
    }
    rec.expert = -1;
    rec.src_base = 0;
    rec.n = r.T;
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) {
      rec.tok[t] = t < r.T ? t : 0;
      rec.pair[t] = rec.tok[t];
      rec.gate[t] = 1.0f;
    }
    r.recs[0] = rec;
    r.recs[max_records(r.T, r.E, r.k)] = rec;
  }
  for (int c = tid; c < kNumCounters; c += blockDim.x) r.counters[c] = 0u;
  if (r.err_clear && tid < 3) r.err_clear[tid] = 0;   // the FFN launches of this call set it
}

// Routing of up to kFusedRouteMaxT tokens by the 16 wavefronts of one workgroup, then grouping
// and records, without leaving the workgroup.
template <int PER_LANE>
__global__ __launch_bounds__(kGroupThreads) void route_group_records_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ gates, int32_t* __restrict__ offsets, int32_t* __restrict__ pairs,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, RecordArgs r) {
  __shared__ GroupSmem sm;
  __shared__ int32_t s_ids[kFusedRouteMaxPairs];
  __shared__ float s_gates[kFusedRouteMaxPairs];
  __shared__ int32_t s_pairs[kFusedRouteMaxPairs];
  const int wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kGroupThreads / 64) {
    const size_t o = static_cast<size_t>(t) * k;
    route_token<PER_LANE>(logits + static_cast<size_t>(t) * E, E, k, ids + o, gates + o, s_ids + o,
                          s_gates + o);
  }
  group_barrier();
  group_body<false>(s_ids, T, k, E, offsets, pairs, active, n_active, sm, s_pairs);
  group_barrier();
  records_body(sm, s_pairs, s_gates, r);
}

__global__ __launch_bounds__(kGroupThreads) void group_records_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets, int32_t* __restrict__ pairs,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, RecordArgs r) {
  __shared__ GroupSmem sm;
  // the ids come from route_topk: every token names k distinct experts
  group_body<true, true>(ids, r.T, r.k, r.E, offsets, pairs, active, n_active, sm, nullptr);
  __syncthreads();  // records_body reads the pairs stored above from global memory
  records_body(sm, pairs, r.gates, r);
}

__global__ __launch_bounds__(kGroupThreads) void records_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, RecordArgs r) {
  __shared__ GroupSmem sm;
  for (int e = threadIdx.x; e <= r.E; e += blockDim.x) sm.offsets[e] = offsets[e];
  for (int e = threadIdx.x; e < r.E; e += blockDim.x) sm.active[e] = active[e];
  if (threadIdx.x == 0) sm.n_active = n_active[0];
  zero_record_counters(sm);
  group_barrier();
  records_body(sm, pairs, r.gates, r);
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

int launch_route_group_records(const float* logits, int32_t* ids, float* gates, int32_t* offsets,
                               int32_t* pairs, int32_t* active, int32_t* n_active,
                               const RecordArgs& r, hipStream_t stream) {
  ProfileScope prof("route_group", stream);
#define MOE_RG_CASE(PL)                                                                          \
  hipLaunchKernelGGL(route_group_records_kernel<PL>, dim3(1), dim3(kGroupThreads), 0, stream,     \
                     logits, r.T, r.E, r.k, ids, gates, offsets, pairs, active, n_active, r)
  if (r.E <= 64) MOE_RG_CASE(1);
  else if (r.E <= 128) MOE_RG_CASE(2);
  else if (r.E <= 256) MOE_RG_CASE(4);
  else if (r.E <= 512) MOE_RG_CASE(8);
  else MOE_RG_CASE(16);
#undef MOE_RG_CASE
  return check_launch("route_group");
}

int launch_group_records(const int32_t* ids, int32_t* offsets, int32_t* pairs, int32_t* active,
                         int32_t* n_active, const RecordArgs& r, hipStream_t stream) {
  ProfileScope prof("group_by_expert", stream);
  hipLaunchKernelGGL(group_records_kernel, dim3(1), dim3(kGroupThreads), 0, stream, ids, offsets,
                     pairs, active, n_active, r);
  return check_launch("group_by_expert");
}

int launch_records(const int32_t* offsets, const int32_t* pairs, const int32_t* active,
                   const int32_t* n_active, const RecordArgs& r, hipStream_t stream) {
  ProfileScope prof("expert_records", stream);
  hipLaunchKernelGGL(records_kernel, dim3(1), dim3(kGroupThreads), 0, stream, offsets, pairs, active,
                     n_active, r);
  return check_launch("expert_records");
}

}  // namespace moeapq
