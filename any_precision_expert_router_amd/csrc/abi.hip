// C-ABI entry points of libmoe_apq: argument validation from host-visible scalars, workspace
// carving, launch sequencing on the caller's stream, the optional kernel timer and error
// messages.  No entry point allocates, frees or reads device memory back (except the explicit
// moe_check_device_error / moe_profile_stop helpers, which synchronise by contract).
#include <cfloat>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"

namespace moeapq {

namespace {
thread_local std::string g_last_error;

struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
struct ProfState {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local ProfState g_prof;

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
}  // namespace

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int check_launch(const char* kernel_name) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(MOE_EHIP, "%s: launch failed: %s", kernel_name, hipGetErrorString(e));
  return MOE_OK;
}

ProfileScope::ProfileScope(const char* name, hipStream_t stream) : name_(name), stream_(stream), slot_(-1) {
  if (!g_prof.on) return;
  ProfRec r{name, g_prof.take(), g_prof.take()};
  if (!r.start || !r.stop) return;
  (void)hipEventRecord(r.start, stream);
  slot_ = static_cast<int>(g_prof.recs.size());
  g_prof.recs.push_back(r);
}

ProfileScope::~ProfileScope() {
  if (slot_ >= 0) (void)hipEventRecord(g_prof.recs[slot_].stop, stream_);
}

ProfilePause::ProfilePause() : was_on_(g_prof.on) { g_prof.on = false; }
ProfilePause::~ProfilePause() { g_prof.on = was_on_; }

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

Workspace carve_workspace(void* base, int T, int E, int H, int I, int k, int I_shared) {
  Workspace w{};
  const size_t TK = static_cast<size_t>(T) * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t o_err = take(64 * sizeof(int32_t));
  const size_t o_ids = take(TK * sizeof(int32_t));
  const size_t o_gates = take(TK * sizeof(float));
  const size_t o_offsets = take((static_cast<size_t>(E) + 1) * sizeof(int32_t));
  const size_t o_pairs = take(TK * sizeof(int32_t));
  const size_t o_active = take(static_cast<size_t>(E) * sizeof(int32_t));
  const size_t o_nact = take(sizeof(int32_t));
  const size_t o_act = take(TK * I * sizeof(uint16_t));
  const size_t o_act_sh = take(static_cast<size_t>(T) * I_shared * sizeof(uint16_t));
  w.segs = down_segments(I, static_cast<int>(TK));
  w.segs_shared = I_shared > 0 ? down_segments(I_shared, T, kSegChunksShared) : 1;
  const size_t o_part = take(w.segs * TK * H * sizeof(float));
  const size_t o_part_sh =
      take(I_shared > 0 ? w.segs_shared * static_cast<size_t>(T) * H * sizeof(float) : 0);
  const size_t o_recs = take(2 * max_records(T, E, k) * sizeof(ExpertRecord));
  const size_t o_ctr = take(kNumCounters * sizeof(uint32_t));
  const size_t o_nrecs = take(sizeof(int32_t));
  w.bytes = off;
  if (base) {
    char* b = static_cast<char*>(base);
    w.err = reinterpret_cast<int32_t*>(b + o_err);
    w.ids = reinterpret_cast<int32_t*>(b + o_ids);
    w.gates = reinterpret_cast<float*>(b + o_gates);
    w.offsets = reinterpret_cast<int32_t*>(b + o_offsets);
    w.pairs = reinterpret_cast<int32_t*>(b + o_pairs);
    w.active = reinterpret_cast<int32_t*>(b + o_active);
    w.n_active = reinterpret_cast<int32_t*>(b + o_nact);
    w.act = reinterpret_cast<uint16_t*>(b + o_act);
    w.act_shared = reinterpret_cast<uint16_t*>(b + o_act_sh);
    w.part = reinterpret_cast<float*>(b + o_part);
    w.part_shared = reinterpret_cast<float*>(b + o_part_sh);
    w.recs = reinterpret_cast<ExpertRecord*>(b + o_recs);
    w.counters = reinterpret_cast<uint32_t*>(b + o_ctr);
    w.n_recs = reinterpret_cast<int32_t*>(b + o_nrecs);
  }
  return w;
}

namespace {

int check_route_args(int T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0) return set_error(MOE_EINVAL, "need T >= 0, E > 0, k > 0 (T=%d E=%d k=%d)", T, E, k);
  if (k > E) return set_error(MOE_EINVAL, "k=%d exceeds E=%d", k, E);
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || T > MOE_MAX_TOKENS)
    return set_error(MOE_EUNSUPPORTED, "outside bounds: E<=%d, k<=%d, T<=%d (got E=%d k=%d T=%d)",
                     MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_TOKENS, E, k, T);
  return MOE_OK;
}

int check_ffn_dims(int H, int I, int I_shared, bool has_shared) {
  if (H <= 0 || I <= 0 || H % kColChunk || I % kColChunk)
    return set_error(MOE_EINVAL, "need H %% 128 == 0 and I %% 128 == 0 (H=%d I=%d)", H, I);
  if (has_shared && (I_shared <= 0 || I_shared % kColChunk))
    return set_error(MOE_EINVAL, "need I_shared %% 128 == 0 (I_shared=%d)", I_shared);
  return MOE_OK;
}

int check_block_host(const moe_apq_block* b) {
  if (!b) return set_error(MOE_EINVAL, "block descriptor is NULL");
  if (!b->planes || !b->lut) return set_error(MOE_EINVAL, "block planes/lut pointer is NULL");
  if (b->rows <= 0 || b->cols <= 0 || b->rows % kRowPanel || b->cols % kColChunk)
    return set_error(MOE_EINVAL, "block needs rows %% 64 == 0 and cols %% 128 == 0 (rows=%d cols=%d)",
                     b->rows, b->cols);
  if (b->q < 1 || b->q > 8) return set_error(MOE_EINVAL, "block width q=%d outside 1..8", b->q);
  if ((reinterpret_cast<uintptr_t>(b->planes) | reinterpret_cast<uintptr_t>(b->lut)) & 15)
    return set_error(MOE_EINVAL, "block planes/lut must be 16-byte aligned");
  return MOE_OK;
}

// The FFN kernels address activation rows (x [T][H], act [T*k][I], act_shared [T][I_shared], a
// plain block's x [T][cols]) through buffer resources whose size and offsets are 32-bit byte
// counts, so every such array must stay below 4 GiB.
int check_act_range(const char* what, size_t rows, size_t cols) {
  const size_t bytes = rows * cols * sizeof(uint16_t);
  if (bytes >= (static_cast<size_t>(1) << 32))
    return set_error(MOE_EUNSUPPORTED, "%s of %zu x %zu fp16 values is %zu bytes: activation arrays "
                     "must stay below 4 GiB", what, rows, cols, bytes);
  return MOE_OK;
}

int check_ffn_range(int T, int H, int I, int k, int I_shared) {
  if (int rc = check_act_range("x", static_cast<size_t>(T), static_cast<size_t>(H))) return rc;
  if (int rc = check_act_range("act", static_cast<size_t>(T) * k, static_cast<size_t>(I))) return rc;
  if (I_shared > 0)
    if (int rc = check_act_range("act_shared", static_cast<size_t>(T), static_cast<size_t>(I_shared))) return rc;
  return MOE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

int check_layer_args(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                     const moe_apq_block* table, const moe_apq_block* shared, int I_shared, uint16_t* y) {
  if (int rc = check_route_args(T, E, k)) return rc;
  if (int rc = check_ffn_dims(H, I, I_shared, shared != nullptr)) return rc;
  if (T == 0) return MOE_OK;
  if (!logits || !x || !table || !y) return set_error(MOE_EINVAL, "NULL pointer argument");
  return check_ffn_range(T, H, I, k, shared ? I_shared : 0);
}

int layer_forward_ws(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                     const moe_apq_block* table, const moe_apq_block* shared, int I_shared,
                     const float* shared_scale, int prefill_threshold, uint16_t* y, const Workspace& ws,
                     bool clear_err, int32_t* status, hipStream_t s) {
  const int ish = shared ? I_shared : 0;
  RecordArgs ra{table, shared, ws.gates, E, H, I, ish, T, k, ws.recs, ws.counters, ws.n_recs,
                effective_dense_threshold(prefill_threshold)};
  ra.err_clear = clear_err ? ws.err : nullptr;
  if (T <= kFusedRouteMaxT && static_cast<long>(T) * k <= kFusedRouteMaxPairs) {
    if (int rc = launch_route_group_records(logits, ws.ids, ws.gates, ws.offsets, ws.pairs, ws.active,
                                            ws.n_active, ra, s))
      return rc;
  } else {
    if (int rc = launch_route_topk(logits, T, E, k, ws.ids, ws.gates, s)) return rc;
    if (int rc = launch_group_records(ws.ids, ws.offsets, ws.pairs, ws.active, ws.n_active, ra, s))
      return rc;
  }
  FfnArgs a{table, shared, E, H, I, k, T, ish, x, ws.offsets, ws.pairs, ws.active, ws.n_active,
            ws.gates, shared_scale, y, ws, prefill_threshold};
  a.status = status;
  return launch_apq_ffn(a, s);
}
}  // namespace moeapq

using namespace moeapq;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_bytes(int T, int E, int H, int I, int k, int I_shared) {
  if (T < 0 || E <= 0 || H <= 0 || I <= 0 || k <= 0 || I_shared < 0) return 0;
  return carve_workspace(nullptr, T, E, H, I, k, I_shared).bytes;
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_gates,
                   void* stream) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_gates) return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_route_topk(logits, T, E, k, topk_ids, topk_gates, as_stream(stream));
}

int moe_group_by_expert(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                        int32_t* sorted_pairs, int32_t* active_experts, int32_t* n_active,
                        void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (!expert_offsets || !active_experts || !n_active || (T > 0 && (!topk_ids || !sorted_pairs)))
    return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_group_by_expert(topk_ids, T, k, E, expert_offsets, sorted_pairs, active_experts,
                                n_active, as_stream(stream));
}

int moe_apq_ffn(const moe_apq_block* table, int E, int H, int I, const uint16_t* x, int T, int k,
                const int32_t* expert_offsets, const int32_t* sorted_pairs,
                const int32_t* active_experts, const int32_t* n_active, const float* topk_gates,
                const moe_apq_block* shared, int I_shared, const float* shared_scale,
                int prefill_threshold, uint16_t* y, void* workspace, size_t ws_bytes,
                void* stream) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (int rc = check_ffn_dims(H, I, I_shared, shared != nullptr)) return rc;
  if (T == 0) return MOE_OK;
  if (!table || !x || !expert_offsets || !sorted_pairs || !active_experts || !n_active ||
      !topk_gates || !y)
    return set_error(MOE_EINVAL, "NULL pointer argument");
  const int ish = shared ? I_shared : 0;
  if (int rc = check_ffn_range(T, H, I, k, ish)) return rc;
  const Workspace ws = carve_workspace(workspace, T, E, H, I, k, ish);
  if (!workspace || ws_bytes < ws.bytes)
    return set_error(MOE_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                     ws.bytes);
  hipStream_t s = as_stream(stream);
  const RecordArgs ra{table, shared, topk_gates, E, H, I, ish, T, k, ws.recs, ws.counters, ws.n_recs,
                      effective_dense_threshold(prefill_threshold)};
  if (int rc = launch_records(expert_offsets, sorted_pairs, active_experts, n_active, ra, s)) return rc;
  FfnArgs a{table, shared, E, H, I, k, T, ish, x, expert_offsets, sorted_pairs, active_experts,
            n_active, topk_gates, shared_scale, y, ws, prefill_threshold};
  return launch_apq_ffn(a, s);
}

int moe_layer_forward(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                      const moe_apq_block* table, const moe_apq_block* shared, int I_shared,
                      const float* shared_scale, int prefill_threshold, uint16_t* y,
                      void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_layer_args(logits, x, T, E, H, I, k, table, shared, I_shared, y)) return rc;
  if (T == 0) return MOE_OK;
  const int ish = shared ? I_shared : 0;
  const Workspace ws = carve_workspace(workspace, T, E, H, I, k, ish);
  if (!workspace || ws_bytes < ws.bytes)
    return set_error(MOE_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                     ws.bytes);
  return layer_forward_ws(logits, x, T, E, H, I, k, table, shared, I_shared, shared_scale, prefill_threshold,
                          y, ws, false, nullptr, as_stream(stream));
}

int moe_apq_gemv(const moe_apq_block* blk_host, const uint16_t* x, int T, float* y,
                 int dense_threshold, void* stream) {
  clear_error();
  if (int rc = check_block_host(blk_host)) return rc;
  if (T < 0 || T > MOE_MAX_TOKENS) return set_error(MOE_EUNSUPPORTED, "T=%d outside 0..%d", T, MOE_MAX_TOKENS);
  if (T == 0) return MOE_OK;
  if (!x || !y) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (int rc = check_act_range("x", static_cast<size_t>(T), static_cast<size_t>(blk_host->cols))) return rc;
  moe_apq_block b = *blk_host;
  b.state = MOE_PAGE_GPU;
  return launch_apq_gemv(b, x, T, y, dense_threshold, as_stream(stream));
}

int moe_apq_decode_indices(const moe_apq_block* blk_host, uint8_t* idx_out, void* stream) {
  clear_error();
  if (int rc = check_block_host(blk_host)) return rc;
  if (!idx_out) return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_decode_indices(*blk_host, idx_out, as_stream(stream));
}

int moe_check_device_error(void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!workspace || ws_bytes < 256) return set_error(MOE_EWORKSPACE, "workspace too small");
  hipStream_t s = as_stream(stream);
  int32_t word[4] = {0, 0, 0, 0};
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return set_error(MOE_EHIP, "could not read the device error word");
  if (word[0] == 0) return MOE_OK;
  const int32_t zero[4] = {0, 0, 0, 0};
  if (hipMemcpy(workspace, zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
    return set_error(MOE_EHIP, "could not clear the device error word");
  return set_error(MOE_EDEVICE,
                   "invalid block descriptor (expert %d, module %s): wrong rows/cols, q outside 1..8, "
                   "misaligned or NULL pointers, or page not GPU-resident",
                   word[1], word[2] == 0 ? "gate_up" : "down");
}

int moe_routing_stats(const int32_t* expert_offsets, const int32_t* sorted_pairs,
                      const float* topk_gates, int T, int k, int E, const uint8_t* resident,
                      uint64_t* count, double* mass, double* mass_sums, void* stream) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (!expert_offsets || !count || !mass || !mass_sums) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (T > 0 && (!sorted_pairs || !topk_gates)) return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_routing_stats(expert_offsets, sorted_pairs, topk_gates, E, resident,
                              reinterpret_cast<unsigned long long*>(count), mass, mass_sums,
                              as_stream(stream));
}

int moe_substitute(const float* logits, int T, int E, int k, const uint8_t* resident, int policy,
                   float gate_threshold, int32_t* topk_ids, const float* topk_gates,
                   int32_t* missed, uint8_t* fetch, float* admit_mass, float admit_threshold,
                   uint8_t* admit, void* stream) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (policy < MOE_POLICY_FETCH_ALL || policy > MOE_POLICY_FIRST_CHOICE)
    return set_error(MOE_EINVAL, "unknown policy %d", policy);
  if (!resident || !fetch) return set_error(MOE_EINVAL, "NULL pointer argument");
  if ((admit_mass == nullptr) != (admit == nullptr))
    return set_error(MOE_EINVAL, "admit_mass and admit must both be given or both be NULL");
  if (T > 0 && (!logits || !topk_ids || !topk_gates || !missed))
    return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_substitute(logits, T, E, k, resident, policy, gate_threshold, topk_ids, topk_gates,
                           missed, fetch, admit_mass, admit_threshold, admit, as_stream(stream));
}

int moe_lynx_remap(const float* logits, int T, int E, int k, float bin_width, int32_t* topk_ids,
                   int32_t* remapped, uint8_t* critical, void* stream) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (!(bin_width <= FLT_MAX))
    return set_error(MOE_EINVAL, "bin_width must be finite (<= 0 selects k/E)");
  // AffinityBinning's bins follow from the sparsity ratio k/N alone: the default width is k/E,
  // one fp32 division
  if (bin_width <= 0.0f) bin_width = static_cast<float>(k) / static_cast<float>(E);
  if (!critical) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (T > 0 && (!logits || !topk_ids || !remapped)) return set_error(MOE_EINVAL, "NULL pointer argument");
  return launch_lynx_remap(logits, T, E, k, bin_width, topk_ids, remapped, critical, as_stream(stream));
}

int moe_commit_blocks(moe_apq_block* table, int table_len, const int32_t* index,
                      const moe_apq_block* desc, int n, void* stream) {
  clear_error();
  if (n < 0) return set_error(MOE_EINVAL, "n=%d < 0", n);
  if (table_len <= 0) return set_error(MOE_EINVAL, "table_len=%d must be positive", table_len);
  if (n == 0) return MOE_OK;
  if (!table || !index || !desc) return set_error(MOE_EINVAL, "NULL pointer argument");
  std::vector<uint8_t> seen(static_cast<size_t>(table_len), 0);
  for (int i = 0; i < n; ++i) {
    if (index[i] < 0 || index[i] >= table_len)
      return set_error(MOE_EINVAL, "index[%d]=%d outside the table [0, %d)", i, index[i], table_len);
    if (seen[index[i]]++)
      return set_error(MOE_EINVAL, "index[%d]=%d repeats an earlier entry of the same commit", i, index[i]);
    const moe_apq_block& b = desc[i];
    if (b.q < 1 || b.q > 8) return set_error(MOE_EINVAL, "desc[%d]: q=%d outside 1..8", i, b.q);
    if (b.rows <= 0 || b.cols <= 0 || b.rows % kRowPanel || b.cols % kColChunk)
      return set_error(MOE_EINVAL, "desc[%d]: need rows %% 64 == 0 and cols %% 128 == 0", i);
  }
  return launch_commit_blocks(table, index, desc, n, as_stream(stream));
}

int moe_page_reload(moe_apq_block* table, int table_len, int index, const moe_apq_block* current,
                    const moe_apq_block* target, const void* host_planes, const void* host_lut,
                    void* copy_event, void* copy_stream, void* stream) {
  clear_error();
  return page_reload(table, table_len, index, current, target, host_planes, host_lut,
                     static_cast<hipEvent_t>(copy_event), as_stream(copy_stream), as_stream(stream));
}

int moe_page_commit(moe_apq_block* table, int table_len, int index, const moe_apq_block* target,
                    void* copy_event, void* stream) {
  clear_error();
  return page_commit(table, table_len, index, target, static_cast<hipEvent_t>(copy_event), as_stream(stream));
}

int moe_page_offload(moe_apq_block* table, int table_len, int index, const moe_apq_block* current,
                     const moe_apq_block* target, void* host_planes, void* host_lut, void* copy_event,
                     void* copy_stream, void* stream) {
  clear_error();
  return page_offload(table, table_len, index, current, target, host_planes, host_lut,
                      static_cast<hipEvent_t>(copy_event), as_stream(copy_stream), as_stream(stream));
}

int moe_workspace_routing(void* workspace, size_t ws_bytes, int T, int E, int H, int I, int k,
                          int I_shared, int32_t** topk_ids, float** topk_gates,
                          int32_t** expert_offsets, int32_t** sorted_pairs) {
  clear_error();
  if (int rc = check_route_args(T, E, k)) return rc;
  if (int rc = check_ffn_dims(H, I, I_shared, I_shared > 0)) return rc;
  if (!topk_ids || !topk_gates || !expert_offsets || !sorted_pairs)
    return set_error(MOE_EINVAL, "NULL pointer argument");
  const Workspace ws = carve_workspace(workspace, T, E, H, I, k, I_shared);
  if (!workspace || ws_bytes < ws.bytes)
    return set_error(MOE_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                     ws.bytes);
  *topk_ids = ws.ids;
  *topk_gates = ws.gates;
  *expert_offsets = ws.offsets;
  *sorted_pairs = ws.pairs;
  return MOE_OK;
}

int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  clear_error();
  if (!buf || !sink) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (bytes == 0 || bytes % 1024 || bytes > (size_t(1) << 40))
    return set_error(MOE_EINVAL, "bytes must be a positive multiple of 1024, at most 2^40");
  if (reinterpret_cast<uintptr_t>(buf) & 15) return set_error(MOE_EINVAL, "buf must be 16-byte aligned");
  return launch_hbm_read_probe(buf, bytes, sink, as_stream(stream));
}

int moe_profile_start(void) {
  clear_error();
  for (auto& r : g_prof.recs) {
    g_prof.pool.push_back(r.start);
    g_prof.pool.push_back(r.stop);
  }
  g_prof.recs.clear();
  g_prof.on = true;
  return MOE_OK;
}

int moe_profile_stop(int max_kernels, char* names_out, double* total_ms_out, int32_t* launches_out) {
  clear_error();
  g_prof.on = false;
  std::vector<std::string> names;
  std::vector<double> ms;
  std::vector<int32_t> cnt;
  for (auto& r : g_prof.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return set_error(MOE_EHIP, "event sync failed");
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return set_error(MOE_EHIP, "event timing failed");
    size_t i = 0;
    while (i < names.size() && names[i] != r.name) ++i;
    if (i == names.size()) {
      names.emplace_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
  }
  for (size_t i = 0; i < names.size() && static_cast<int>(i) < max_kernels; ++i) {
    if (names_out) {
      std::strncpy(names_out + 64 * i, names[i].c_str(), 63);
      names_out[64 * i + 63] = '\0';
    }
    if (total_ms_out) total_ms_out[i] = ms[i];
    if (launches_out) launches_out[i] = cnt[i];
  }
  return static_cast<int>(names.size());
}

}  // extern "C"
