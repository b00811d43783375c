// Launch sequence of the fused Any-Precision expert FFN: gate_up + SiLU, down, combine.  The
// kernels live in apq_gate_up.hip / apq_down.hip (one tile engine, apq_engine.hpp).
#include "apq_engine.hpp"

namespace moeapq {
namespace apq {
int launch_gate_up(const KArgs& k, int max_items, hipStream_t stream);
int launch_down(const KArgs& k, int max_items, hipStream_t stream);
int launch_combine(const float* part, const float* part_shared, int T, int H, int k, int segs,
                   int segs_shared, uint16_t* y, const int32_t* err, int32_t* status,
                   hipStream_t stream);
int launch_plain(const KArgs& k, int max_items, hipStream_t stream);
int launch_decode(const moe_apq_block& blk, uint8_t* idx_out, hipStream_t stream);
}  // namespace apq

int launch_apq_ffn(const FfnArgs& a, hipStream_t stream) {
  apq::KArgs k{};
  k.table = a.table;
  k.shared = a.shared;
  k.E = a.E; k.H = a.H; k.I = a.I; k.k = a.k; k.T = a.T; k.I_shared = a.shared ? a.I_shared : 0;
  k.x = a.x;
  k.offsets = a.offsets; k.pairs = a.pairs; k.active = a.active; k.n_active = a.n_active;
  k.gates = a.gates;
  k.shared_scale = a.shared_scale;
  k.act = a.ws.act; k.act_shared = a.ws.act_shared;
  k.part = a.ws.part; k.part_shared = a.ws.part_shared;
  k.err = a.ws.err;
  k.dense_threshold = effective_dense_threshold(a.dense_threshold);
  k.n_recs = a.ws.n_recs;
  k.recs = a.ws.recs;
  const int sh = a.shared ? 1 : 0;
  const int routed = static_cast<int>(max_records(a.T, a.E, a.k)) - 2;  // routed records at most
  const int gu_items = sh * (a.I_shared / kGateUpTileRows) + routed * (a.I / kGateUpTileRows);
  k.counter = a.ws.counters + kCtrGateUp;
  if (int rc = apq::launch_gate_up(k, gu_items, stream)) return rc;
  k.counter = a.ws.counters + kCtrDown;
  k.recs = a.ws.recs + max_records(a.T, a.E, a.k);   // the down kernel's record order
  k.segs = a.ws.segs;
  k.segs_shared = sh ? a.ws.segs_shared : 1;
  const int dn_items = (sh * k.segs_shared + routed * k.segs) * (a.H / kRowPanel);
  if (int rc = apq::launch_down(k, dn_items, stream)) return rc;
  return apq::launch_combine(a.ws.part, sh ? a.ws.part_shared : nullptr, a.T, a.H, a.k, k.segs,
                             k.segs_shared, a.y, a.ws.err, a.status, stream);
}

int launch_apq_gemv(const moe_apq_block& blk, const uint16_t* x, int T, float* y,
                    int dense_threshold, hipStream_t stream) {
  apq::KArgs k{};
  k.plain = blk;
  k.T = T;
  k.x = x;
  k.y_plain = y;
  k.segs = k.segs_shared = 1;
  k.dense_threshold = effective_dense_threshold(dense_threshold);
  return apq::launch_plain(k, blk.rows / kRowPanel, stream);
}

int launch_decode_indices(const moe_apq_block& blk, uint8_t* idx_out, hipStream_t stream) {
  return apq::launch_decode(blk, idx_out, stream);
}

}  // namespace moeapq
