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

// ---- page movement between device and host (PagedWeight, Key Components 1: pages are
// GPU-resident, CPU-resident or in transfer; Key Components 3: offload and reload run
// asynchronously and a changed width is committed only at a safe boundary) ------------------
namespace moeapq {
namespace {
size_t plane_bytes(const moe_apq_block& b) { return static_cast<size_t>(b.rows) * b.cols / 8; }
size_t lut_bytes(const moe_apq_block& b) { return static_cast<size_t>(b.rows) * (size_t(2) << b.q); }

int check_shape(const char* what, const moe_apq_block& b) {
  if (!b.planes || !b.lut) return set_error(MOE_EINVAL, "%s: planes/lut pointer is NULL", what);
  if ((reinterpret_cast<uintptr_t>(b.planes) | reinterpret_cast<uintptr_t>(b.lut)) & 15)
    return set_error(MOE_EINVAL, "%s: planes/lut must be 16-byte aligned", what);
  if (b.rows <= 0 || b.cols <= 0 || b.rows % kRowPanel || b.cols % kColChunk)
    return set_error(MOE_EINVAL, "%s: need rows %% 64 == 0 and cols %% 128 == 0", what);
  if (b.q < 1 || b.q > 8) return set_error(MOE_EINVAL, "%s: q=%d outside 1..8", what, b.q);
  return MOE_OK;
}

int hip_rc(hipError_t e, const char* what) {
  return e == hipSuccess ? MOE_OK : set_error(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int commit_one(moe_apq_block* table, int32_t index, const moe_apq_block& d, hipStream_t s) {
  return launch_commit_blocks(table, &index, &d, 1, s);
}
}  // namespace

int page_reload(moe_apq_block* table, int table_len, int index, const moe_apq_block* cur,
                const moe_apq_block* tgt, const void* host_planes, const void* host_lut,
                hipEvent_t copy_event, hipStream_t copy_stream, hipStream_t stream) {
  if (!table || !cur || !tgt || !host_planes || !host_lut || !copy_event)
    return set_error(MOE_EINVAL, "NULL pointer argument");
  if (index < 0 || index >= table_len)
    return set_error(MOE_EINVAL, "index=%d outside the table [0, %d)", index, table_len);
  if (int rc = check_shape("target", *tgt)) return rc;
  if (tgt->state != MOE_PAGE_GPU) return set_error(MOE_EINVAL, "target state must be MOE_PAGE_GPU");
  if (tgt->rows != cur->rows || tgt->cols != cur->cols)
    return set_error(MOE_EINVAL, "target shape %dx%d differs from the current %dx%d", tgt->rows, tgt->cols,
                     cur->rows, cur->cols);
  int first = 0;  // first plane to copy
  if (cur->state == MOE_PAGE_GPU) {
    // raising the width of a resident block: its first cur->q planes stay in use meanwhile
    if (tgt->planes != cur->planes)
      return set_error(MOE_EINVAL, "a resident block keeps its planes: the target must name the same planes");
    if (tgt->q <= cur->q)
      return set_error(MOE_EINVAL, "a reload raises the width (current q=%d, target q=%d)", cur->q, tgt->q);
    if (tgt->lut == cur->lut)
      return set_error(MOE_EINVAL, "the target LUT must be a new buffer: the current one is read until the commit");
    first = cur->q;
  } else if (cur->state == MOE_PAGE_CPU) {
    first = 0;
  } else {
    return set_error(MOE_EINVAL, "block %d is already in transfer (state %d)", index, cur->state);
  }
  const size_t pb = plane_bytes(*tgt);
  if (cur->state == MOE_PAGE_CPU) {
    // calls issued from here on skip the block (and report it) until the copy has landed
    moe_apq_block mid = *tgt;
    mid.state = MOE_PAGE_IN_TRANSFER;
    if (int rc = commit_one(table, index, mid, stream)) return rc;
  }
  char* dst = reinterpret_cast<char*>(const_cast<uint32_t*>(tgt->planes)) + first * pb;
  const char* src = static_cast<const char*>(host_planes) + first * pb;
  if (int rc = hip_rc(hipMemcpyAsync(dst, src, (tgt->q - first) * pb, hipMemcpyHostToDevice, copy_stream),
                      "plane copy"))
    return rc;
  if (int rc = hip_rc(hipMemcpyAsync(const_cast<uint16_t*>(tgt->lut), host_lut, lut_bytes(*tgt),
                                     hipMemcpyHostToDevice, copy_stream),
                      "LUT copy"))
    return rc;
  // calls issued on `stream` from here on keep the old width (or skip a block in transfer) until
  // page_commit: the copy overlaps them
  return hip_rc(hipEventRecord(copy_event, copy_stream), "event record");
}

int page_commit(moe_apq_block* table, int table_len, int index, const moe_apq_block* tgt,
                hipEvent_t copy_event, hipStream_t stream) {
  if (!table || !tgt || !copy_event) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (index < 0 || index >= table_len)
    return set_error(MOE_EINVAL, "index=%d outside the table [0, %d)", index, table_len);
  if (int rc = check_shape("target", *tgt)) return rc;
  if (tgt->state != MOE_PAGE_GPU) return set_error(MOE_EINVAL, "target state must be MOE_PAGE_GPU");
  // the safe boundary: every call issued on `stream` after this point sees the whole new width
  if (int rc = hip_rc(hipStreamWaitEvent(stream, copy_event, 0), "stream wait")) return rc;
  return commit_one(table, index, *tgt, stream);
}

int page_offload(moe_apq_block* table, int table_len, int index, const moe_apq_block* cur,
                 const moe_apq_block* tgt, void* host_planes, void* host_lut, hipEvent_t copy_event,
                 hipStream_t copy_stream, hipStream_t stream) {
  if (!table || !cur || !tgt || !copy_event) return set_error(MOE_EINVAL, "NULL pointer argument");
  if (index < 0 || index >= table_len)
    return set_error(MOE_EINVAL, "index=%d outside the table [0, %d)", index, table_len);
  if (cur->state != MOE_PAGE_GPU) return set_error(MOE_EINVAL, "only a GPU-resident block can be offloaded");
  if (int rc = check_shape("current", *cur)) return rc;
  int first = 0;       // first plane that leaves the device
  bool with_lut = false;
  if (tgt->state == MOE_PAGE_CPU) {
    first = 0;
    with_lut = true;
  } else if (tgt->state == MOE_PAGE_GPU) {
    // lowering the width: the first tgt->q planes stay, with the LUT of width tgt->q
    if (int rc = check_shape("target", *tgt)) return rc;
    if (tgt->planes != cur->planes || tgt->rows != cur->rows || tgt->cols != cur->cols)
      return set_error(MOE_EINVAL, "a lowered block keeps its planes and shape");
    if (tgt->q >= cur->q)
      return set_error(MOE_EINVAL, "an offload lowers the width (current q=%d, target q=%d)", cur->q, tgt->q);
    first = tgt->q;
  } else {
    return set_error(MOE_EINVAL, "target state must be MOE_PAGE_CPU or MOE_PAGE_GPU");
  }
  // the commit comes first: calls issued after it no longer read the planes that leave
  if (int rc = commit_one(table, index, *tgt, stream)) return rc;
  // the copy waits for every call issued before the commit, so once copy_event has completed
  // the freed device memory may be reused
  if (int rc = hip_rc(hipEventRecord(copy_event, stream), "event record")) return rc;
  if (int rc = hip_rc(hipStreamWaitEvent(copy_stream, copy_event, 0), "stream wait")) return rc;
  const size_t pb = plane_bytes(*cur);
  if (host_planes) {
    const char* src = reinterpret_cast<const char*>(cur->planes) + first * pb;
    char* dst = static_cast<char*>(host_planes) + first * pb;
    if (int rc = hip_rc(hipMemcpyAsync(dst, src, (cur->q - first) * pb, hipMemcpyDeviceToHost, copy_stream),
                        "plane copy"))
      return rc;
  }
  if (with_lut && host_lut) {
    if (int rc = hip_rc(hipMemcpyAsync(host_lut, cur->lut, lut_bytes(*cur), hipMemcpyDeviceToHost, copy_stream),
                        "LUT copy"))
      return rc;
  }
  return hip_rc(hipEventRecord(copy_event, copy_stream), "event record");
}
}  // namespace moeapq
