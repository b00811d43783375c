// Greedy bit-width planner (PagedWeight, Key Components 2: the runtime planner scores the damage
// of bit-width reductions and, when a memory target must be met, takes greedily the reductions
// of lowest damage per byte saved; hot experts are protected by width floors and damage
// multipliers).
//
// A reduction is one step q -> q-1 of one block, allowed while q-1 >= its floor.  Its cost is
// mult * (damage(q-1) - damage(q)) / (bytes the step frees), in double; the cheapest step is
// taken (ties: the lower block index) and the block's next step becomes a candidate, until the
// bytes freed reach the target or no step is left.  A block's bytes at width q are its q planes
// (rows*cols/8 bytes each) plus an fp16 LUT of 2^q entries per row.
#include <cstdint>
#include <queue>
#include <vector>

#include "moe_apq.h"

namespace moeapq {
int set_error(int code, const char* fmt, ...);
void clear_error();
}  // namespace moeapq

namespace {

int64_t block_bytes(int64_t rows, int64_t cols, int q) {
  return rows * cols * q / 8 + rows * (int64_t{1} << q) * 2;
}

struct Step {
  double cost;
  int block;
  bool operator>(const Step& o) const { return cost > o.cost || (cost == o.cost && block > o.block); }
};

}  // namespace

extern "C" int moe_plan_widths(int n, const uint8_t* q_cur, const uint8_t* q_floor,
                               const int32_t* rows, const int32_t* cols, const float* damage,
                               const float* mult, int64_t target_bytes, uint8_t* q_new,
                               int64_t* bytes_saved) {
  using moeapq::set_error;
  moeapq::clear_error();
  if (n < 0) return set_error(MOE_EINVAL, "n=%d < 0", n);
  if (!bytes_saved || (n > 0 && (!q_cur || !q_floor || !rows || !cols || !damage || !mult || !q_new)))
    return set_error(MOE_EINVAL, "NULL pointer argument");
  for (int i = 0; i < n; ++i) {
    if (q_cur[i] < 1 || q_cur[i] > 8 || q_floor[i] < 1 || q_floor[i] > q_cur[i])
      return set_error(MOE_EINVAL, "block %d: need 1 <= q_floor <= q_cur <= 8 (got %d, %d)", i,
                       q_floor[i], q_cur[i]);
    if (rows[i] <= 0 || cols[i] <= 0 || rows[i] % 64 || cols[i] % 128)
      return set_error(MOE_EINVAL, "block %d: rows %% 64 == 0 and cols %% 128 == 0 needed", i);
    if (!(mult[i] > 0.0f)) return set_error(MOE_EINVAL, "block %d: damage multiplier must be > 0", i);
  }
  std::priority_queue<Step, std::vector<Step>, std::greater<Step>> heap;
  auto push = [&](int i) {
    const int q = q_new[i];
    if (q - 1 < q_floor[i]) return;
    const int64_t step = block_bytes(rows[i], cols[i], q) - block_bytes(rows[i], cols[i], q - 1);
    const double d = static_cast<double>(damage[static_cast<size_t>(i) * 8 + (q - 2)]) -
                     static_cast<double>(damage[static_cast<size_t>(i) * 8 + (q - 1)]);
    heap.push(Step{static_cast<double>(mult[i]) * d / static_cast<double>(step), i});
  };
  for (int i = 0; i < n; ++i) {
    q_new[i] = q_cur[i];
    push(i);
  }
  int64_t saved = 0;
  while (saved < target_bytes && !heap.empty()) {
    const Step s = heap.top();
    heap.pop();
    const int i = s.block;
    saved += block_bytes(rows[i], cols[i], q_new[i]) - block_bytes(rows[i], cols[i], q_new[i] - 1);
    q_new[i] = static_cast<uint8_t>(q_new[i] - 1);
    push(i);
  }
  *bytes_saved = saved;
  return MOE_OK;
}
