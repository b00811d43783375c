// Internal plumbing of libmoe_apq: error reporting, launch bookkeeping, workspace carving and
// the launchers each kernel translation unit exports to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe_apq.h"

namespace moeapq {

// ---- error reporting (thread-local message behind moe_last_error) --------------------------
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_launch(const char* kernel_name);  // hipGetLastError -> MOE_EHIP + message

// ---- optional kernel timer -----------------------------------------------------------------
// Bracket a launch with events when moe_profile_start() is active on this thread.
struct ProfileScope {
  ProfileScope(const char* name, hipStream_t stream);
  ~ProfileScope();
  const char* name_;
  hipStream_t stream_;
  int slot_;
};
// Suspends the timer on this thread for its lifetime (an entry point that must not create
// events, which the timer does on first use).
struct ProfilePause {
  ProfilePause();
  ~ProfilePause();
  bool was_on_;
};

// ---- device facts ---------------------------------------------------------------------------
int device_cu_count();  // compute units of the current device (cached per device)

// ---- constants of the block format ---------------------------------------------------------
constexpr int kRowPanel = 64;    // rows per panel: one wavefront lane per row
constexpr int kColChunk = 128;   // columns per 16-byte unit of one plane
constexpr int kGateUpTileRows = 32;  // gate rows (and as many up rows) per gate_up tile
constexpr int kWavesPerTile = 4;     // wavefronts sharing one row tile (split over columns)

// ---- per-call expert records ----------------------------------------------------------------
// What the FFN kernels need about one block pair, gathered once per call by the grouping step so
// that a work item is decoded with a few scalar loads from one place instead of a chain of
// dependent loads (active list -> offsets -> page table -> pairs -> gates).  Record 0 is the
// shared expert, record 1 + a the a-th active routed expert.
constexpr int kRecTok = 4;   // tokens described in full (the streaming path's group)
// Records and their order.  In a call with at most kRecSplitMaxPairs pairs, an expert with more
// than kRecGroupTok tokens gets one record per group of kRecGroupTok tokens (one matrix-core
// pass each), so that a hot expert's rows are spread over many workgroups instead of one
// workgroup looping over its token groups.  Records of multi-token experts come first (their
// items are the longest), then the streaming ones, each class in active-list order.
constexpr int kRecGroupTok = 64;
constexpr int kRecDensePassTok = 32;   // the most tokens one dense matrix-core pass holds
constexpr int kRecSplitMaxPairs = 1024;
__host__ __device__ inline size_t max_records(int T, int E, int k) {
  return static_cast<size_t>(E) + 2 + (static_cast<size_t>(T) * k + kRecGroupTok - 1) / kRecGroupTok;
}
struct alignas(128) ExpertRecord {
  const uint32_t* planes[2];  // gate_up, down
  const uint16_t* lut[2];
  int32_t expert;             // routed expert id, -1 for the shared expert
  int32_t src_base;           // sorted position of its first pair (0 for the shared expert)
  int32_t n;                  // tokens routed to it (T for the shared expert)
  uint32_t meta;              // committed widths and validity, see record_meta (one dword, so
                              // that a reader fetches it with a scalar load)
  int32_t tok[kRecTok];       // token rows of its first pairs (activation rows of gate_up)
  int32_t pair[kRecTok];      // their pair ids t*k + j (partial-sum rows of down)
  float gate[kRecTok];        // their gate weights
  int32_t pad[4];
};
static_assert(sizeof(ExpertRecord) == 128, "record layout");
// meta: bits 0-7 = q of gate_up, bits 8-15 = q of down, bit 16 = both page-table descriptors
// valid and GPU-resident.
__host__ __device__ constexpr uint32_t record_meta(int q_gate_up, int q_down, bool ok) {
  return static_cast<uint32_t>(q_gate_up & 0xff) | (static_cast<uint32_t>(q_down & 0xff) << 8) |
         (ok ? 1u << 16 : 0u);
}
__host__ __device__ constexpr int record_q(uint32_t meta, int module) {
  return static_cast<int>((meta >> (8 * module)) & 0xffu);
}
__host__ __device__ constexpr bool record_ok(uint32_t meta) { return ((meta >> 16) & 1u) != 0; }

// Work counters of the FFN launches (dynamic item fetch), zeroed by the step that writes the
// records: per launch, kQueues interleaved sub-queues, each counter on its own 128-byte line.
constexpr int kQueues = 8;
constexpr int kCounterStride = 32;   // uint32 per counter (128 bytes)
enum Counter : int { kCtrGateUp = 0, kCtrDown = kQueues * kCounterStride,
                     kNumCounters = 2 * kQueues * kCounterStride };

// ---- workspace layout (all sections 256-byte aligned) ----------------------------------------
struct Workspace {
  int32_t* err;          // [64]: device error word + first bad (expert, module)
  int32_t* ids;          // [T*k]   (moe_layer_forward only)
  float* gates;          // [T*k]
  int32_t* offsets;      // [E+1]
  int32_t* pairs;        // [T*k]
  int32_t* active;       // [E]
  int32_t* n_active;     // [1]
  uint16_t* act;         // fp16 [T*k][I]    SiLU-gated activations, sorted-pair order
  uint16_t* act_shared;  // fp16 [T][I_shared]
  float* part;           // fp32 [segs][T*k][H]  gate-scaled expert outputs, pair order
  float* part_shared;    // fp32 [segs_sh][T][H] scaled shared-expert outputs
  int segs, segs_shared; // down column segments (down_segments)
  ExpertRecord* recs;    // [2][max_records(T, E, k)]: one record order per module (gate_up, down)
  int32_t* n_recs;       // [1] routed records of the call
  uint32_t* counters;    // [kNumCounters]
  size_t bytes;          // total bytes the layout needs
};
Workspace carve_workspace(void* base, int T, int E, int H, int I, int k, int I_shared);

// Column segments of a down row tile.  In decode-size batches a long down row (e.g. the shared
// expert's 5632 columns) is split so that no work item carries much more than kSegChunks
// 128-column chunks; each segment writes its own fp32 partial sums, which the combine adds in a
// fixed order.  Batches with many pairs already have enough items and keep whole rows.
constexpr int kSegChunks = 16;
// The shared expert's down items carry every token of the call through the matrix-core branch, so
// they are the slowest items of a decode launch: they are cut finer (measured: a 5632-column row
// in 4 segments instead of 3 takes the Qwen1.5-shaped layer from 97.6 to 94.0 us, while cutting
// routed rows finer slows the Mixtral- and Qwen2-shaped layers).
constexpr int kSegChunksShared = 11;
constexpr int kSegMaxPairs = 512;
inline int down_segments(int cols, int pairs, int seg_chunks = kSegChunks) {
  const int nc4 = cols / kColChunk;
  if (pairs > kSegMaxPairs || nc4 <= seg_chunks + seg_chunks / 2) return 1;
  return (nc4 + seg_chunks - 1) / seg_chunks;
}

// ---- launchers (return MOE_OK or an error code with the message set) -------------------------
int launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                      hipStream_t stream);
int launch_group_by_expert(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                           int32_t* pairs, int32_t* active, int32_t* n_active, hipStream_t stream);

// Inputs of the record builder (all device pointers; shared may be null).
struct RecordArgs {
  const moe_apq_block* table;
  const moe_apq_block* shared;
  const float* gates;          // [T*k] gate weights (written by routing in the same launch or before)
  int E, H, I, I_shared, T, k;
  ExpertRecord* recs;          // [2][max_records(T, E, k)]
  uint32_t* counters;
  int32_t* n_recs;             // out: routed records written (records 1 .. n_recs)
  int dense_threshold;         // the FFN's effective threshold (orders the records)
  int32_t* err_clear = nullptr;  // non-null: the device error word, cleared at the call's start
};
// Routing, grouping and the records in one single-workgroup launch (small batches).
constexpr int kFusedRouteMaxT = 16;   // one token per wavefront of the fused workgroup
constexpr int kFusedRouteMaxPairs = kFusedRouteMaxT * MOE_MAX_TOPK;
int launch_route_group_records(const float* logits, int32_t* ids, float* gates, int32_t* offsets,
                               int32_t* pairs, int32_t* active, int32_t* n_active,
                               const RecordArgs& r, hipStream_t stream);
// Grouping then records (large batches, after launch_route_topk).
int launch_group_records(const int32_t* ids, int32_t* offsets, int32_t* pairs, int32_t* active,
                         int32_t* n_active, const RecordArgs& r, hipStream_t stream);
// Records only, from routing arrays the caller computed (moe_apq_ffn).
int launch_records(const int32_t* offsets, const int32_t* pairs, const int32_t* active,
                   const int32_t* n_active, const RecordArgs& r, hipStream_t stream);

struct FfnArgs {
  const moe_apq_block* table;  // device [E][2]
  const moe_apq_block* shared; // device [2] or nullptr
  int E, H, I, k, T, I_shared;
  const uint16_t* x;
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  const int32_t* n_active;
  const float* gates;
  const float* shared_scale;
  uint16_t* y;
  Workspace ws;
  int dense_threshold;  // <= 0: library default
  int32_t* status = nullptr;  // non-null: device int32 that receives the error word at the end
};
int launch_apq_ffn(const FfnArgs& a, hipStream_t stream);
// The whole layer on a carved workspace (moe_layer_forward and its allocation-free variant).
int layer_forward_ws(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                     const moe_apq_block* table, const moe_apq_block* shared, int I_shared,
                     const float* shared_scale, int prefill_threshold, uint16_t* y, const Workspace& ws,
                     bool clear_err, int32_t* status, hipStream_t stream);
// Argument checks shared by the layer entry points (host scalars only).
int check_layer_args(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                     const moe_apq_block* table, const moe_apq_block* shared, int I_shared, uint16_t* y);
int launch_apq_gemv(const moe_apq_block& blk, const uint16_t* x, int T, float* y,
                    int dense_threshold, hipStream_t stream);

// The product path of a tile of n tokens on a block of width q.  The packed-dot VALU path
// (streaming) takes at most 2 tokens on blocks of width <= 4, whose 2q-bit pair tables make its
// decode about half as costly as the matrix-core path's single-entry tables, and single tokens on
// wider blocks, where both paths decode alike and the matrix cores do the products for free;
// everything else takes the matrix-core (MFMA) path.  A caller's threshold (the n at or above
// which a tile must use the MFMA path) can only lower that switch.
constexpr int kDefaultDenseThreshold = 5;
inline int effective_dense_threshold(int prefill_threshold) {
  return prefill_threshold > 0 ? prefill_threshold : kDefaultDenseThreshold;
}
__host__ __device__ inline int stream_max_tokens(int q) { return q <= 4 ? 2 : 1; }
__host__ __device__ inline bool takes_stream(int n, int q, int dense_threshold) {
  return n <= stream_max_tokens(q) && n < dense_threshold;
}
int launch_decode_indices(const moe_apq_block& blk, uint8_t* idx_out, hipStream_t stream);
int launch_routing_stats(const int32_t* offsets, const int32_t* pairs, const float* gates, int E,
                         const uint8_t* resident, unsigned long long* count, double* mass,
                         double* sums, hipStream_t stream);
int launch_commit_blocks(moe_apq_block* table, const int32_t* index, const moe_apq_block* desc, int n,
                         hipStream_t stream);
int page_reload(moe_apq_block* table, int table_len, int index, const moe_apq_block* cur,
                const moe_apq_block* tgt, const void* host_planes, const void* host_lut,
                hipEvent_t copy_event, hipStream_t copy_stream, hipStream_t stream);
int page_commit(moe_apq_block* table, int table_len, int index, const moe_apq_block* tgt,
                hipEvent_t copy_event, hipStream_t stream);
int page_offload(moe_apq_block* table, int table_len, int index, const moe_apq_block* cur,
                 const moe_apq_block* tgt, void* host_planes, void* host_lut, hipEvent_t copy_event,
                 hipStream_t copy_stream, hipStream_t stream);
int launch_substitute(const float* logits, int T, int E, int k, const uint8_t* resident, int policy,
                      float gate_threshold, int32_t* ids, const float* gates, int32_t* missed,
                      uint8_t* fetch, float* admit_mass, float admit_threshold, uint8_t* admit,
                      hipStream_t stream);
int launch_lynx_remap(const float* logits, int T, int E, int k, float bin_width, int32_t* ids,
                      int32_t* remapped, uint8_t* critical, hipStream_t stream);
int launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace moeapq
