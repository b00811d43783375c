// Width commits: new descriptors written into the device weight page table in stream order, so
// every call issued before on the stream runs with the descriptors it started with and every
// call issued after runs with the new ones -- the "safe boundary" at which PagedWeight commits
// bit-width changes (Key Components 3: commits happen only once a plan has fully run).  The
// descriptors travel by value in the launch arguments: nothing is allocated and no host memory
// has to stay alive after the call.
#include "internal.hpp"

namespace moeapq {
namespace {
constexpr int kCommitBatch = 64;

struct CommitBatch {
  int32_t index[kCommitBatch];
  moe_apq_block desc[kCommitBatch];
};

__global__ __launch_bounds__(64) void commit_blocks_kernel(moe_apq_block* __restrict__ table,
                                                           CommitBatch b, int n) {
  const int i = threadIdx.x;
  if (i < n) table[b.index[i]] = b.desc[i];
}
}  // namespace

int launch_commit_blocks(moe_apq_block* table, const int32_t* index, const moe_apq_block* desc, int n,
                         hipStream_t stream) {
  ProfileScope prof("commit_blocks", stream);
  for (int b0 = 0; b0 < n; b0 += kCommitBatch) {
    CommitBatch b;
    const int m = n - b0 < kCommitBatch ? n - b0 : kCommitBatch;
    for (int i = 0; i < m; ++i) {
      b.index[i] = index[b0 + i];
      b.desc[i] = desc[b0 + i];
    }
    hipLaunchKernelGGL(commit_blocks_kernel, dim3(1), dim3(64), 0, stream, table, b, m);
    if (int rc = check_launch("commit_blocks")) return rc;
  }
  return MOE_OK;
}
}  // namespace moeapq
