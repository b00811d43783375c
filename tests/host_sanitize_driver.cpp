// Host-side checks of libmoe_apq built with AddressSanitizer and UndefinedBehaviorSanitizer: the
// plane packer, the width planner, workspace carving and the C-ABI argument validation.  The
// device launchers are replaced by recorders (no GPU is touched), so an accepted call reports
// MOE_OK and the arguments it would launch with can be checked.  Prints "ok" and exits 0 when
// every check holds; a sanitizer finding aborts the process.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "internal.hpp"

namespace moeapq {
namespace {
int g_launches = 0;
float g_bin_width = -1.0f;
int g_ffn_threshold = -1;
}  // namespace

int launch_route_topk(const float*, int, int, int, int32_t*, float*, hipStream_t) { return ++g_launches, MOE_OK; }
int launch_group_by_expert(const int32_t*, int, int, int, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_route_group_records(const float*, int32_t*, float*, int32_t*, int32_t*, int32_t*, int32_t*,
                               const RecordArgs&, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_group_records(const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, const RecordArgs&, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_records(const int32_t*, const int32_t*, const int32_t*, const int32_t*, const RecordArgs&, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_apq_ffn(const FfnArgs& a, hipStream_t) {
  g_ffn_threshold = a.dense_threshold;
  return ++g_launches, MOE_OK;
}
int launch_apq_gemv(const moe_apq_block&, const uint16_t*, int, float*, int, hipStream_t) { return ++g_launches, MOE_OK; }
int launch_decode_indices(const moe_apq_block&, uint8_t*, hipStream_t) { return ++g_launches, MOE_OK; }
int launch_routing_stats(const int32_t*, const int32_t*, const float*, int, const uint8_t*, unsigned long long*,
                         double*, double*, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_substitute(const float*, int, int, int, const uint8_t*, int, float, int32_t*, const float*, int32_t*,
                      uint8_t*, float*, float, uint8_t*, hipStream_t) {
  return ++g_launches, MOE_OK;
}
int launch_lynx_remap(const float*, int, int, int, float bin_width, int32_t*, int32_t*, uint8_t*, hipStream_t) {
  g_bin_width = bin_width;
  return ++g_launches, MOE_OK;
}
int launch_hbm_read_probe(const void*, size_t, uint32_t*, hipStream_t) { return ++g_launches, MOE_OK; }
}  // namespace moeapq

using namespace moeapq;

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// The q-bit index of (r, c) read back from packed planes by the layout the header documents.
static int read_index(const std::vector<uint32_t>& planes, int rows, int cols, int q, int r, int c) {
  const size_t plane_words = static_cast<size_t>(rows) * cols / 32;
  const int nc4 = cols / 128, P = r / 64, l = r % 64, c4 = c / 128, j = (c % 128) / 32, cc = c % 32;
  const size_t unit = (static_cast<size_t>(P) * nc4 + c4) * 64 + l;
  const int o = ((cc >> 1) & 3) + 4 * (cc & 1);
  int v = 0;
  for (int p = 0; p < q; ++p) {
    const int bit = ((8 * (cc >> 3) + 7 - p - o) % 32 + 32) % 32;
    v = (v << 1) | ((planes[p * plane_words + unit * 4 + j] >> bit) & 1u);
  }
  return v;
}

static void check_packer() {
  std::mt19937 rng(5);
  const int shapes[][2] = {{64, 128}, {128, 384}, {1024, 2048}};  // the last one packs on threads
  for (auto& s : shapes) {
    const int rows = s[0], cols = s[1];
    std::vector<uint8_t> idx(static_cast<size_t>(rows) * cols);
    for (auto& v : idx) v = static_cast<uint8_t>(rng() & 0xff);
    std::vector<uint32_t> p8(static_cast<size_t>(8) * rows * cols / 32);
    CHECK(moe_apq_pack(idx.data(), rows, cols, 8, p8.data()) == MOE_OK);
    for (int q = 1; q <= 8; ++q) {
      std::vector<uint32_t> pq(static_cast<size_t>(q) * rows * cols / 32);
      CHECK(moe_apq_pack(idx.data(), rows, cols, q, pq.data()) == MOE_OK);
      CHECK(std::memcmp(pq.data(), p8.data(), pq.size() * 4) == 0);  // planes nest
      for (int t = 0; t < 2000; ++t) {
        const int r = static_cast<int>(rng() % rows), c = static_cast<int>(rng() % cols);
        CHECK(read_index(pq, rows, cols, q, r, c) == idx[static_cast<size_t>(r) * cols + c] >> (8 - q));
      }
    }
  }
  std::vector<uint32_t> out(64);
  CHECK(moe_apq_pack(nullptr, 64, 128, 4, out.data()) == MOE_EINVAL);
  CHECK(moe_apq_pack(reinterpret_cast<const uint8_t*>(out.data()), 64, 96, 4, out.data()) == MOE_EINVAL);
}

static void check_planner() {
  std::mt19937 rng(11);
  for (int trial = 0; trial < 300; ++trial) {
    const int n = static_cast<int>(rng() % 14);
    std::vector<uint8_t> qc(n), fl(n), qn(n);
    std::vector<int32_t> rows(n), cols(n);
    std::vector<float> dmg(static_cast<size_t>(n) * 8), mult(n);
    int64_t full = 0;
    for (int i = 0; i < n; ++i) {
      qc[i] = static_cast<uint8_t>(1 + rng() % 8);
      fl[i] = static_cast<uint8_t>(1 + rng() % qc[i]);
      rows[i] = 64 * static_cast<int32_t>(1 + rng() % 40);
      cols[i] = 128 * static_cast<int32_t>(1 + rng() % 20);
      float acc = 0.0f;
      for (int w = 8; w >= 1; --w) dmg[i * 8 + w - 1] = (acc += static_cast<float>(rng() % 1000) / 997.0f);
      mult[i] = 0.5f + static_cast<float>(rng() % 100) / 40.0f;
      for (int q = qc[i]; q > fl[i]; --q)
        full += (int64_t(rows[i]) * cols[i] / 8 + int64_t(rows[i]) * 2 * (1 << (q - 1)));
    }
    const int64_t target = trial % 5 ? static_cast<int64_t>(rng() % (full + 4000)) : full + 1;
    int64_t saved = -1;
    CHECK(moe_plan_widths(n, qc.data(), fl.data(), rows.data(), cols.data(), dmg.data(), mult.data(), target,
                          qn.data(), &saved) == MOE_OK);
    int64_t sum = 0;
    for (int i = 0; i < n; ++i) {
      CHECK(qn[i] >= fl[i] && qn[i] <= qc[i]);
      for (int q = qc[i]; q > qn[i]; --q) sum += int64_t(rows[i]) * cols[i] / 8 + int64_t(rows[i]) * 2 * (1 << (q - 1));
    }
    CHECK(sum == saved);
    CHECK(saved >= target || saved == full);
  }
}

static void check_abi() {
  void* fake = reinterpret_cast<void*>(0x1000);
  const float* lg = static_cast<const float*>(fake);
  int32_t* ip = static_cast<int32_t*>(fake);
  float* fp = static_cast<float*>(fake);
  uint16_t* hp = static_cast<uint16_t*>(fake);
  const moe_apq_block* tb = static_cast<const moe_apq_block*>(fake);

  // routing bounds
  CHECK(moe_route_topk(lg, 4, 8, 9, ip, fp, nullptr) == MOE_EINVAL);
  CHECK(moe_route_topk(lg, 4, 2048, 2, ip, fp, nullptr) == MOE_EUNSUPPORTED);
  CHECK(moe_route_topk(lg, 65537, 64, 2, ip, fp, nullptr) == MOE_EUNSUPPORTED);
  int before = g_launches;
  CHECK(moe_route_topk(lg, 65536, 1024, 32, ip, fp, nullptr) == MOE_OK);
  CHECK(g_launches == before + 1);
  CHECK(moe_group_by_expert(ip, 3, 2, 8, ip, ip, ip, ip, nullptr, 0, nullptr) == MOE_OK);

  // workspace carving over many shapes: sizes are 256-byte multiples, grow with T, and the
  // routing views lie inside
  for (int T : {1, 7, 16, 128, 2048, 65536})
    for (int E : {1, 8, 60, 512, 1024})
      for (int k : {1, 2, 8, 32}) {
        if (k > E) continue;
        const size_t n = moe_workspace_bytes(T, E, 2048, 1408, k, T <= 2048 ? 5632 : 0);
        CHECK(n > 0 && n % 256 == 0);
        int32_t *ids, *off, *pairs;
        float* gates;
        const uintptr_t base = uintptr_t(1) << 40;
        CHECK(moe_workspace_routing(reinterpret_cast<void*>(base), n, T, E, 2048, 1408, k, T <= 2048 ? 5632 : 0,
                                    &ids, &gates, &off, &pairs) == MOE_OK);
        CHECK(reinterpret_cast<uintptr_t>(pairs) + 4ull * T * k <= base + n);
      }

  // the layer: accepted shapes reach the FFN launcher with the caller's threshold
  const size_t ws = moe_workspace_bytes(16, 60, 2048, 1408, 4, 5632);
  std::vector<char> wsbuf(1);  // never touched: launchers are recorders
  void* wsp = reinterpret_cast<void*>(uintptr_t(1) << 40);
  (void)wsbuf;
  CHECK(moe_layer_forward(lg, hp, 16, 60, 2048, 1408, 4, tb, tb, 5632, nullptr, 7, hp, wsp, ws, nullptr) == MOE_OK);
  CHECK(g_ffn_threshold == 7);
  CHECK(moe_layer_forward(lg, hp, 16, 60, 2048, 1408, 4, tb, tb, 5632, nullptr, 0, hp, wsp, ws - 1, nullptr) ==
        MOE_EWORKSPACE);
  CHECK(moe_layer_forward(lg, hp, 65536, 64, 32768, 128, 2, tb, nullptr, 0, nullptr, 0, hp, wsp, ws, nullptr) ==
        MOE_EUNSUPPORTED);
  CHECK(moe_apq_ffn(tb, 64, 4096, 8192, hp, 65536, 8, ip, ip, ip, ip, fp, nullptr, 0, nullptr, 0, hp, wsp,
                    size_t(1) << 40, nullptr) == MOE_EUNSUPPORTED);

  // LYNX: the default bin width is k/E in fp32, computed by the library
  CHECK(moe_lynx_remap(lg, 4, 60, 4, 0.0f, ip, ip, static_cast<uint8_t*>(fake), nullptr) == MOE_OK);
  CHECK(g_bin_width == static_cast<float>(4) / static_cast<float>(60));
  CHECK(moe_lynx_remap(lg, 4, 512, 10, -1.0f, ip, ip, static_cast<uint8_t*>(fake), nullptr) == MOE_OK);
  CHECK(g_bin_width == 10.0f / 512.0f);
  CHECK(moe_lynx_remap(lg, 4, 60, 4, 0.3f, ip, ip, static_cast<uint8_t*>(fake), nullptr) == MOE_OK);
  CHECK(g_bin_width == 0.3f);
  CHECK(moe_lynx_remap(lg, 4, 60, 4, NAN, ip, ip, static_cast<uint8_t*>(fake), nullptr) == MOE_EINVAL);
  CHECK(moe_lynx_remap(lg, 4, 60, 4, INFINITY, ip, ip, static_cast<uint8_t*>(fake), nullptr) == MOE_EINVAL);

  // commits: indices outside the table and repeats
  moe_apq_block d{};
  d.planes = static_cast<const uint32_t*>(fake);
  d.lut = static_cast<const uint16_t*>(fake);
  d.rows = 64;
  d.cols = 128;
  d.q = 4;
  moe_apq_block descs[3] = {d, d, d};
  const int32_t rep[3] = {1, 2, 1}, past[1] = {8};
  CHECK(moe_commit_blocks(static_cast<moe_apq_block*>(fake), 8, rep, descs, 3, nullptr) == MOE_EINVAL);
  CHECK(moe_commit_blocks(static_cast<moe_apq_block*>(fake), 8, past, descs, 1, nullptr) == MOE_EINVAL);

  // page moves refused before any device call
  moe_apq_block cur = d, tgt = d;
  cur.state = MOE_PAGE_IN_TRANSFER;
  tgt.q = 6;
  CHECK(moe_page_reload(static_cast<moe_apq_block*>(fake), 4, 1, &cur, &tgt, fake, fake, fake, nullptr, nullptr) ==
        MOE_EINVAL);
  cur.state = MOE_PAGE_CPU;
  CHECK(moe_page_offload(static_cast<moe_apq_block*>(fake), 4, 1, &cur, &tgt, fake, fake, fake, nullptr, nullptr) ==
        MOE_EINVAL);
  CHECK(std::strlen(moe_last_error()) > 0);
}

int main() {
  check_packer();
  check_planner();
  check_abi();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
