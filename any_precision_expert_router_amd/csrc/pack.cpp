// Host packer: logical 8-bit parent indices -> the bit-plane layout read by the kernels.
//
// Plane p (0 <= p < q) stores bit 7-p of every parent index (the Any-Precision nesting: the q-bit
// index is the top-q-bit prefix, so planes at width q' < q are the first q' planes at width q;
// PagedWeight, Key Components 1).  Inside a plane, 64-row panels and 128-column chunks form
// 16-byte units, one per (panel, chunk, row-in-panel), so a wavefront whose lanes own the 64
// rows of a panel loads a chunk of one plane as one contiguous 1-KiB run.  Inside a 32-bit word,
// column c sits at bit (8*(c/8) + 7 - p - o(c)) mod 32, o(c) = ((c >> 1) & 3) + 4*(c & 1): the
// bits one decode step needs for a given output byte are then one rotation away in every plane.
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "moe_apq.h"

namespace moeapq {
int set_error(int code, const char* fmt, ...);
void clear_error();
}  // namespace moeapq

namespace {

int bit_pos(int p, int c) {
  const int o = ((c >> 1) & 3) + 4 * (c & 1);
  return ((8 * (c >> 3) + 7 - p - o) % 32 + 32) % 32;
}

void pack_panels(const uint8_t* idx8, int rows, int cols, int q, uint32_t* planes, int panel_lo,
                 int panel_hi) {
  int pos[8][32];
  for (int p = 0; p < 8; ++p)
    for (int c = 0; c < 32; ++c) pos[p][c] = bit_pos(p, c);
  const int nc4 = cols / 128;
  const size_t plane_words = static_cast<size_t>(rows) * cols / 32;
  for (int P = panel_lo; P < panel_hi; ++P) {
    for (int l = 0; l < 64; ++l) {
      const uint8_t* src_row = idx8 + static_cast<size_t>(P * 64 + l) * cols;
      for (int c4 = 0; c4 < nc4; ++c4) {
        const size_t unit = (static_cast<size_t>(P) * nc4 + c4) * 64 + l;
        for (int j = 0; j < 4; ++j) {
          const uint8_t* s = src_row + c4 * 128 + 32 * j;
          for (int p = 0; p < q; ++p) {
            uint32_t w = 0;
            const int sh = 7 - p;
            for (int c = 0; c < 32; ++c) w |= static_cast<uint32_t>((s[c] >> sh) & 1u) << pos[p][c];
            planes[p * plane_words + unit * 4 + j] = w;
          }
        }
      }
    }
  }
}

}  // namespace

extern "C" int moe_apq_pack(const uint8_t* idx8_host, int rows, int cols, int q,
                            uint32_t* planes_host) {
  moeapq::clear_error();
  if (!idx8_host || !planes_host) return moeapq::set_error(MOE_EINVAL, "NULL pointer argument");
  if (rows <= 0 || cols <= 0 || rows % 64 || cols % 128)
    return moeapq::set_error(MOE_EINVAL, "need rows %% 64 == 0 and cols %% 128 == 0 (rows=%d cols=%d)",
                             rows, cols);
  if (q < 1 || q > 8) return moeapq::set_error(MOE_EINVAL, "q=%d outside 1..8", q);
  const int panels = rows / 64;
  const size_t work = static_cast<size_t>(rows) * cols * q;
  unsigned nthreads = std::thread::hardware_concurrency();
  if (nthreads == 0) nthreads = 1;
  if (nthreads > 16) nthreads = 16;
  if (work < (size_t{1} << 22) || panels < 2) nthreads = 1;
  if (nthreads > static_cast<unsigned>(panels)) nthreads = panels;
  if (nthreads == 1) {
    pack_panels(idx8_host, rows, cols, q, planes_host, 0, panels);
    return MOE_OK;
  }
  std::vector<std::thread> pool;
  for (unsigned i = 0; i < nthreads; ++i) {
    const int lo = static_cast<int>(static_cast<long>(panels) * i / nthreads);
    const int hi = static_cast<int>(static_cast<long>(panels) * (i + 1) / nthreads);
    pool.emplace_back(pack_panels, idx8_host, rows, cols, q, planes_host, lo, hi);
  }
  for (auto& t : pool) t.join();
  return MOE_OK;
}
