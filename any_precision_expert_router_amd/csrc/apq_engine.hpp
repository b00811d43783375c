// The fused mixed-width Any-Precision expert FFN (PagedWeight, Key Components 3: one fused
// kernel reads bit-planes and per-row LUTs of blocks whose committed widths differ).
//
// Work decomposition.  A work item is one row tile of one linear block: 64 rows of a down (or
// plain) block, or 32 gate rows plus the matching 32 up rows of a gate_up block, so that the
// SiLU gate can be applied in the epilogue.  A 256-thread workgroup owns one item at a time; its
// four wavefronts split the columns, and inside a wavefront every lane owns one row.  With the
// row-panel layout of the planes, a lane's 16-byte unit of a 128-column chunk sits next to its
// neighbours', so each plane load of a wavefront is one contiguous 1-KiB (or two 512-B) run:
// every HBM byte is fetched once, in full 128-byte lines.  The grid is persistent and walks a
// device-side item list (shared-expert tiles first, then the routed experts' tiles), so no host
// synchronisation is needed between routing and the FFN.
//
// Decoding.  For each 32-column word a lane holds q plane words.  Masked merges of the planes
// followed by one rotation ("bit-gather") produce words whose bytes are ready-made LDS table
// indices; the mask/rotation constants depend on (q, output word) only, because plane p's bit
// for a column is stored at a position chosen so that one rotation serves all planes at once:
//   * q <= 4 (PAIR): byte = idx(even column) << 4 | idx(odd column); the row's 2^(2q)-entry pair
//     table in LDS returns both fp16 weights as one packed half2.
//   * q >= 5 (SINGLE): byte = idx of one column; the row's 2^q-entry table returns one fp16.
// Tables are stored entry-major with one 4-byte slot per lane ([entry][64 lanes]), so a lookup
// is conflict-free whatever the indices, and the LDS address is one v_perm of the index byte
// next to the lane offset.
//
// Products.  Tiles of 1 token, and of 2 tokens at widths <= 4 (takes_stream), stream:
// v_dot2c_f32_f16 (two MACs, fp32 accumulate) against the token activations, broadcast across
// each 16-lane row by DPP.  Other tiles use the matrix cores (v_mfma_f32_32x32x16_f16) on the
// decoded fp16 weights: the dense branch takes 16 or 32 tokens per decode of the weights, the
// wide branch (prefill chunks) 64.
// Weights are never expanded to a dense matrix in memory.
#pragma once
#include "internal.hpp"

namespace moeapq {
namespace apq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Address-space qualified views: plane and LUT reads are per-lane global loads; activation rows
// and the routing arrays, read at wavefront-uniform addresses and never written during the
// kernel, go through the scalar unit as constant-space loads.
#define AS_GLOBAL __attribute__((address_space(1)))
#define AS_CONST __attribute__((address_space(4)))
#define AS_LDS __attribute__((address_space(3)))
#define MOE_INLINE __device__ __attribute__((always_inline)) inline

template <class T>
MOE_INLINE const AS_GLOBAL T* gview(const void* p) { return (const AS_GLOBAL T*)p; }
template <class T>
MOE_INLINE const AS_CONST T* cview(const void* p) { return (const AS_CONST T*)p; }

// Buffer resource over `bytes` bytes at `base` (both wavefront-uniform; below 4 GiB: the host
// refuses larger activation arrays and weight blocks).  Loads past the end return zeros.
//
// The matrix-core branches load everything they stream (plane words, LUT rows, the token indices
// of their rows, and the activations they stage straight into LDS) with buffer instructions, and
// only those, while a tile's loads are in flight.  Their waits are partial counts ("all but the
// next chunk's loads"), which hold only if the loads they count complete in issue order; the
// staging loads have to be buffer loads (the global-address form is a FLAT-family instruction that
// also accesses LDS, after which the compiler waits for every outstanding load at the next use of
// a loaded register, draining the chunk ring every iteration), and mixing them with global-address
// loads in flight gave stale staged activations.
MOE_INLINE __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}
MOE_INLINE uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

constexpr int kThreads = 64 * kWavesPerTile;
constexpr int kMaxTokGroup = 2;                  // tokens sharing one VALU pass over the weights
constexpr int kDenseGroup = 16;                  // tokens of the smaller dense MFMA pass (32x32 tile)

// LDS map of a tile workgroup (bytes):
//   [0, 64K)        lookup tables, 4-byte slots [entry][64 lanes] unless noted.  Streaming (VALU)
//                   tiles: the pair table (q <= 4, entries a << 4 | b) or the single table
//                   (q >= 5).  Dense (MFMA) tiles keep their table below 32K: the pair table for
//                   q <= 3, the single table for q = 4..7, the single table with 2-byte slots
//                   for q = 8.
//   [32K, 64K)      matrix-core tiles only: each wavefront's 8K ring of two staged activation
//                   chunks of 4K, [8-column pieces][tokens][16 bytes] fp16 (16 pieces x 16
//                   tokens, 8 x 32, or for wide passes 4 x 64), filled by loads straight to LDS;
//                   after the tile's columns it holds that wavefront's partial sums for the
//                   cross-wavefront reduction.
//   [64K, 67K)      streaming tiles: cross-wavefront reduction (4 floats per lane, waves 1-3).
//   [67K, 67K+16)   the work queue's next item index.
constexpr uint32_t kTblBytes = 65536;
constexpr uint32_t kXRingBase = 32768;
constexpr uint32_t kXSlotBytes = kDenseGroup * kColChunk * 2;   // 4 KiB
constexpr uint32_t kXWaveBytes = 2 * kXSlotBytes;
constexpr uint32_t kRedBase = kTblBytes;
constexpr uint32_t kRedBytes = (kWavesPerTile - 1) * kMaxTokGroup * 64 * 4;
constexpr uint32_t kQueueBase = kRedBase + kRedBytes;   // the next item index, published by thread 0
constexpr uint32_t kLdsBytes = kQueueBase + 16;
static_assert(kXRingBase + kWavesPerTile * kXWaveBytes <= kTblBytes, "activation ring overlaps");
static_assert(32 * 64 * 4 <= kXWaveBytes, "dense partial sums do not fit a ring");

// The only LDS object of the tile kernels, so it starts at LDS address 0: a table address is
// exactly entry*256 + lane*4 and an LDS byte offset is an LDS address.
static __shared__ uint32_t g_lds[kLdsBytes / 4];

enum Mode : int { kGateUp = 0, kDown = 1, kPlain = 2 };

__host__ __device__ constexpr uint32_t rotr32(uint32_t v, int s) {
  return (s & 31) ? ((v >> (s & 31)) | (v << (32 - (s & 31)))) : v;
}
// Bits of plane p's word that hold the columns of output word o.
__host__ __device__ constexpr uint32_t plane_mask(int p, int o) { return rotr32(0x80808080u, p + o); }

MOE_INLINE uint32_t rot(uint32_t v, int s) {
  return __builtin_amdgcn_alignbit(v, v, static_cast<uint32_t>(s & 31));
}

// (a & m) | (b & ~m) in one v_bfi_b32 (the compiler would otherwise split it into and + or).
MOE_INLINE uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(a), "v"(b));
  return r;
}

// Byte b of the result = q-bit index of column 8b + 2(o&3) + (o>>2) of this 32-column word.
template <int Q>
MOE_INLINE uint32_t single_word(const uint32_t (&w)[Q], int o) {
  // the masks of planes 0..7 partition the word, so a chain of bit-field inserts merges them; with
  // all eight planes every bit of the last plane outside its mask is overwritten by another plane
  uint32_t z = Q == 8 ? w[Q - 1] : w[Q - 1] & plane_mask(Q - 1, o);
#pragma unroll
  for (int p = Q - 2; p >= 0; --p) z = bfi(plane_mask(p, o), w[p], z);
  return rot(z, 8 - Q - o);
}

// Byte b of the result = idx(8b + 2j) << 4 | idx(8b + 2j + 1)   (q <= 4).
template <int Q>
MOE_INLINE uint32_t pair_word(const uint32_t (&w)[Q], int j) {
  // with four planes the eight masks (two per plane) partition the word, as in single_word at 8
  uint32_t z = Q == 4 ? w[Q - 1] : w[Q - 1] & (plane_mask(Q - 1, j) | plane_mask(Q - 1, j + 4));
#pragma unroll
  for (int p = Q - 2; p >= 0; --p) z = bfi(plane_mask(p, j) | plane_mask(p, j + 4), w[p], z);
  return rot(z, 4 - Q - j);
}

// LDS byte address of the table entry held in byte b of `word`, for this lane: entry*256 + lane*4.
MOE_INLINE uint32_t tbl_addr(uint32_t word, uint32_t lane4, int b) {
  return __builtin_amdgcn_perm(word, lane4, 0x0c0c0000u | static_cast<uint32_t>((4 + b) << 8));
}

MOE_INLINE uint32_t lds_load(uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(g_lds) + byte_addr);
}

MOE_INLINE int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier for LDS traffic: every wavefront's LDS reads and writes (ds_*) complete
// before it, while its vector-memory loads and stores stay in flight.  The tile kernels share data
// between wavefronts only through LDS (tables, partial sums, the queue slot); a __syncthreads, and
// a release fence on LDS alone once loads that write LDS directly are in flight, would wait for
// every outstanding vector-memory operation too: the ring's prefetched chunks at the table
// barrier, the tile's output stores at the reduction barriers.  Staged activations are never
// read across wavefronts, and each wavefront waits for its own staging loads before it reads or
// reuses its ring.  The memory clobbers keep the compiler from moving LDS accesses across.
MOE_INLINE void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

MOE_INLINE uint32_t word_of(const u32x4& v, int jw) {
  return jw == 0 ? v.x : jw == 1 ? v.y : jw == 2 ? v.z : v.w;
}
MOE_INLINE uint32_t word_of(const u32x2& v, int jw) { return jw == 0 ? v.x : v.y; }

constexpr int kLutRegs = 8;  // 16-byte LUT registers one thread prefetches for an item

// Depth of the per-wavefront ring of in-flight 128-column chunks (all q planes of a chunk).
// Two chunks per wavefront, with eight wavefronts per CU, keep 16 chunks per CU in flight; a
// deeper ring measured slower (it costs 32 VGPRs per slot and doubles the unrolled loop body).
template <int Q>
constexpr int ring_depth() { return 2; }

struct Item {
  const uint32_t* planes;
  const uint16_t* lut;
  int rows, cols, q;
  int r0;        // row of lane 0 (first gate row for gate_up)
  int row_hi;    // row of lane 32 (gate_up: first up row)
  int n;         // tokens routed to the tile
  int src_base;  // sorted position of the expert's first pair (routed), 0 (shared/plain)
  int expert;    // routed expert id, -1 for the shared expert / plain block
  int c0, nc;    // the item's column chunks [c0, c0 + nc) (a segment of a long down row)
  int seg;       // segment index (selects the partial-sum buffer of a down item)
  int tok[kRecTok];     // activation rows of the first tokens (gate_up)
  int pair[kRecTok];    // their pair ids (down partial-sum rows)
  float gate[kRecTok];  // their gate weights (down)
  bool shared;
};

struct KArgs {
  const moe_apq_block* table;   // device [E][2]
  const moe_apq_block* shared;  // device [2] or null
  moe_apq_block plain;          // kPlain: the block, by value
  int E, H, I, k, T, I_shared;
  const uint16_t* x;            // fp16 [T][H] (gate_up), [T][cols] (plain)
  const int32_t* offsets;
  const int32_t* pairs;
  const int32_t* active;
  const int32_t* n_active;
  const float* gates;
  const float* shared_scale;
  uint16_t* act;                // fp16 [T*k][I]   written by gate_up, read by down
  uint16_t* act_shared;         // fp16 [T][I_shared]
  float* part;                  // fp32 [T*k][H]
  float* part_shared;           // fp32 [T][H]
  float* y_plain;               // fp32 [T][rows]
  int32_t* err;
  int dense_threshold;          // tiles with at least this many tokens take the MFMA path
  int segs, segs_shared;        // column segments per down row tile (routed, shared expert)
  const ExpertRecord* recs;     // shared expert, then the routed records (see internal.hpp)
  const int32_t* n_recs;        // [1] routed records
  uint32_t* counter;            // work counter of this launch (null: static round-robin)
};

// Work queue of a workgroup.  Its first item is blockIdx.x; its second is 2 gridDim.x - 1 -
// blockIdx.x when the launch has at least two items per workgroup (the records are ordered
// costliest first, so a workgroup whose first item is among the longest gets a second one among
// the shorter), else blockIdx.x + gridDim.x; the later ones come from its sub-queue's counter, requested by thread 0 one item ahead and
// published to the workgroup through LDS at the current item's reduction barrier, so the
// atomic's latency hides behind a whole item.  Without a counter the queue is static
// round-robin.  Everything the publish step needs is computed once here, so that step reads no
// memory (a reload of a kernel argument there costs a scalar-load round trip per item).
struct Queue {
  int nxt;            // the item after the current one (uniform)
  int base, stride;   // dynamic: item = base + stride * counter value; static: nxt + stride
  bool dynamic;       // a counter exists
  uint32_t* counter;  // this workgroup's sub-queue counter (thread 0 only)
  uint32_t pending;   // thread 0: counter value fetched for the item after nxt
};

// The dynamic items (from 2 * gridDim.x on) are dealt to min(kQueues, gridDim.x) interleaved
// sub-queues, each with its own counter, so that no single address takes every fetch.
MOE_INLINE void queue_init(const KArgs& A, Queue& Qu, int total) {
  const int grid = static_cast<int>(gridDim.x);
  const int nsub = min(kQueues, grid);
  const int sub = static_cast<int>(blockIdx.x) % nsub;
  const int b = static_cast<int>(blockIdx.x);
  Qu.nxt = total >= 2 * grid ? 2 * grid - 1 - b : b + grid;
  Qu.dynamic = A.counter != nullptr;
  Qu.base = Qu.dynamic ? 2 * grid + sub : 0;
  Qu.stride = Qu.dynamic ? nsub : grid;
  Qu.counter = Qu.dynamic ? A.counter + sub * kCounterStride : nullptr;
  Qu.pending = 0;
}
MOE_INLINE void queue_request(Queue& Qu) {
  if (Qu.dynamic && threadIdx.x == 0) Qu.pending = atomicAdd(Qu.counter, 1u);
}
// Before the barrier: thread 0 publishes the item after nxt.
MOE_INLINE void queue_publish(const Queue& Qu) {
  if (threadIdx.x == 0) {
    const int after = Qu.dynamic ? Qu.base + Qu.stride * static_cast<int>(Qu.pending) : Qu.nxt + Qu.stride;
    g_lds[kQueueBase / 4] = static_cast<uint32_t>(after);
  }
}
// After the barrier: every thread reads it, the queue moves one item on and requests the next.
// Returns the item that becomes current.
MOE_INLINE int queue_advance(Queue& Qu) {
  const int after = uniform(static_cast<int>(g_lds[kQueueBase / 4]));
  const int cur = Qu.nxt;
  Qu.nxt = after;
  queue_request(Qu);
  return cur;
}

MOE_INLINE int lane_row(const Item& it, int lane) {
  return lane < 32 ? it.r0 + lane : it.row_hi + (lane - 32);
}

// Each thread prefetches LUT bytes of its lane's row into registers (only those it needs):
//   q <= 4: the whole row (2^q fp16, at most 32 bytes), every wavefront;
//   q >= 5: quarter `wave` of the row (2^(q-2) fp16, at most 128 bytes).
template <int Q, bool BUF = false>
MOE_INLINE void prefetch_lut_q(const Item& it, int lane, int wave, u32x4 (&L)[kLutRegs]) {
  if constexpr (BUF) {   // the same bytes through buffer loads (matrix-core branches)
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(it.lut, static_cast<size_t>(it.rows) * (2u << Q));
    const uint32_t o = static_cast<uint32_t>(lane_row(it, lane)) * (2u << Q);
    if constexpr (Q == 1) {
      L[0].x = buf_u32(r, o);
    } else if constexpr (Q == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
      L[0].x = v.x;
      L[0].y = v.y;
    } else if constexpr (Q <= 4) {
#pragma unroll
      for (int q = 0; q < (1 << (Q - 3)); ++q) L[q] = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16u * q, 0, 0);
    } else {
      constexpr int n4 = 1 << (Q - 5);
      const uint32_t ow = o + static_cast<uint32_t>(wave) * (16u * n4);
#pragma unroll
      for (int q = 0; q < n4; ++q) L[q] = __builtin_amdgcn_raw_buffer_load_b128(r, ow + 16u * q, 0, 0);
    }
    return;
  }
  const AS_GLOBAL char* g = gview<char>(reinterpret_cast<const char*>(it.lut) +
                                        static_cast<size_t>(lane_row(it, lane)) * (2u << Q));
  if constexpr (Q == 1) {
    L[0].x = *reinterpret_cast<const AS_GLOBAL uint32_t*>(g);
  } else if constexpr (Q == 2) {
    const uint64_t v = *reinterpret_cast<const AS_GLOBAL uint64_t*>(g);
    L[0].x = static_cast<uint32_t>(v);
    L[0].y = static_cast<uint32_t>(v >> 32);
  } else if constexpr (Q <= 4) {
#pragma unroll
    for (int r = 0; r < (1 << (Q - 3)); ++r) L[r] = reinterpret_cast<const AS_GLOBAL u32x4*>(g)[r];
  } else {
    constexpr int n4 = 1 << (Q - 5);
    const AS_GLOBAL u32x4* src = reinterpret_cast<const AS_GLOBAL u32x4*>(g) + wave * n4;
#pragma unroll
    for (int r = 0; r < n4; ++r) L[r] = src[r];
  }
}

// fp16 number h (0-based) of the prefetched registers, as the byte pair a v_perm selects.
MOE_INLINE uint32_t lut_dword(const u32x4 (&L)[kLutRegs], int h) { return word_of(L[h >> 3], (h >> 1) & 3); }

// Write this thread's part of the row tile's table from the prefetched registers.
//   PAIR  (q <= 4): entry (a << 4 | b) = LUT[a] | LUT[b] << 16; wave w writes the a in its quarter.
//   SINGLE (q >= 5): entry v = LUT[v] in both halves; wave w writes its quarter of v.
// Addresses are lane*4 + constant, so every write is one ds_write_b32 with an immediate offset.
template <int Q, int W>
MOE_INLINE void write_pair_rows(const u32x4 (&L)[kLutRegs], char* base) {
  constexpr int NE = 1 << Q;
  constexpr int APW = NE >= 4 ? NE / 4 : 1;  // first indices per wavefront
  if constexpr (W * APW < NE) {
#pragma unroll
    for (int ai = 0; ai < APW; ++ai) {
      const int a = W * APW + ai;
      const uint32_t da = lut_dword(L, a);
#pragma unroll
      for (int b = 0; b < NE; ++b) {
        const uint32_t db = lut_dword(L, b);
        const uint32_t sel = ((a & 1) ? 0x0302u : 0x0100u) | ((b & 1) ? 0x07060000u : 0x05040000u);
        *reinterpret_cast<uint32_t*>(base + (((a << 4) | b) << 8)) = __builtin_amdgcn_perm(db, da, sel);
      }
    }
  }
}

template <int Q>
MOE_INLINE void write_table(const u32x4 (&L)[kLutRegs], int lane, int wave) {
  constexpr int NE = 1 << Q;
  char* base = reinterpret_cast<char*>(g_lds) + lane * 4;
  if constexpr (Q <= 4) {
    switch (wave) {
      case 0: write_pair_rows<Q, 0>(L, base); break;
      case 1: write_pair_rows<Q, 1>(L, base); break;
      case 2: write_pair_rows<Q, 2>(L, base); break;
      default: write_pair_rows<Q, 3>(L, base); break;
    }
  } else {
    constexpr int VPW = NE / 4;  // entries per wavefront
    char* wbase = base + wave * (VPW << 8);
#pragma unroll
    for (int vi = 0; vi < VPW; ++vi) {
      const uint32_t d = lut_dword(L, vi);
      const uint32_t dup = __builtin_amdgcn_perm(d, d, (vi & 1) ? 0x03020302u : 0x01000100u);
      *reinterpret_cast<uint32_t*>(wbase + (vi << 8)) = dup;
    }
  }
}

// One 32-column word: the row's 32 weights as 16 packed (even, odd) fp16 pairs, dword d = 4b + j
// covering columns 8b + 2j and 8b + 2j + 1.
template <int Q>
MOE_INLINE void decode_word(const uint32_t (&w)[Q], uint32_t lane4, uint32_t (&wv)[16]) {
  if constexpr (Q <= 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pw = pair_word<Q>(w, j);
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[4 * b + j] = lds_load(tbl_addr(pw, lane4, b));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t we = single_word<Q>(w, j), wo = single_word<Q>(w, j + 4);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t ve = lds_load(tbl_addr(we, lane4, b));
        const uint32_t vo = lds_load(tbl_addr(wo, lane4, b));
        wv[4 * b + j] = __builtin_amdgcn_perm(vo, ve, 0x05040100u);  // (even lo, odd hi)
      }
    }
  }
}

// The 16 products of one 32-column word for one token, with the activations broadcast across
// each 16-lane row by DPP row_newbcast: every lane of a row holds 4 dwords of the chunk's
// activations (one 16-byte load per lane), so dword 4g + c of word JW sits in component c of
// lane 4 JW + g.  a[g] += dot(w[4g + c], x.c broadcast from lane 4 JW + g).
//
// Two hazards the compiler cannot see inside the asm are covered here:
//   * a DPP instruction must come at least two wait states after any VALU write of a VGPR it
//     reads (its accumulator included): the block opens with s_nop 1;
//   * the result of a DOT instruction may be read by another instruction only three wait
//     states later (the same DOT opcode may take it back as its accumulator at once): the
//     block closes with s_nop 2, and the four accumulators rotate so that each is written by
//     a product and read again by the same opcode four instructions later.
template <int JW>
MOE_INLINE void dot16_bcast(float (&a)[4], const uint32_t (&w)[16], const u32x4& x) {
  asm("s_nop 1\n\t"
      "v_dot2c_f32_f16_dpp %0, %4, %8 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %4, %12 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %2, %4, %16 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %3, %4, %20 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %0, %5, %9 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %5, %13 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %2, %5, %17 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %3, %5, %21 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %0, %6, %10 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %6, %14 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %2, %6, %18 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %3, %6, %22 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %0, %7, %11 row_newbcast:%24 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %1, %7, %15 row_newbcast:%25 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %2, %7, %19 row_newbcast:%26 row_mask:0xf bank_mask:0xf\n\t"
      "v_dot2c_f32_f16_dpp %3, %7, %23 row_newbcast:%27 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 2"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
      : "v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w),
        "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]),
        "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]),
        "i"(4 * JW), "i"(4 * JW + 1), "i"(4 * JW + 2), "i"(4 * JW + 3));
}

// SiLU(g) * u in fp32 with the hardware exponential and reciprocal (about 1 ulp each); the result
// is rounded to fp16, whose half-ulp (2^-11) is far larger.
MOE_INLINE float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Reduce the four wavefronts' partial sums (fixed order: wave 0 + 1 + 2 + 3) and apply the
// epilogue of the mode for the ng real tokens of the group starting at g0.
template <int MODE, int NT>
MOE_INLINE void reduce_and_store(const KArgs& A, const Item& it, int g0, int ng, float (&acc)[NT],
                                 const Queue& Qu) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  float* red = reinterpret_cast<float*>(reinterpret_cast<char*>(g_lds) + kRedBase);
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((wave - 1) * kMaxTokGroup + t) * 64 + lane] = acc[t];
  }
  queue_publish(Qu);
  lds_barrier();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int w = 1; w < kWavesPerTile; ++w) acc[t] += red[((w - 1) * kMaxTokGroup + t) * 64 + lane];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float h = acc[t];
      if constexpr (MODE == kGateUp) {
        const float up = __shfl_down(h, 32, 64);
        if (t < ng && lane < 32) {
          const float a = silu_mul(h, up);
          const int Iw = it.shared ? A.I_shared : A.I;
          uint16_t* dst = it.shared ? A.act_shared + static_cast<size_t>(g0 + t) * Iw
                                    : A.act + static_cast<size_t>(it.src_base + g0 + t) * Iw;
          dst[it.r0 + lane] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(a));
        }
      } else if constexpr (MODE == kDown) {
        if (t < ng) {
          if (it.shared) {
            const float s = A.shared_scale ? cview<float>(A.shared_scale)[g0 + t] : 1.0f;
            A.part_shared[(static_cast<size_t>(it.seg) * A.T + g0 + t) * A.H + it.r0 + lane] = s * h;
          } else {
            // the streaming path holds at most kRecTok tokens, all described by the record
            const int p = it.pair[t];
            A.part[(static_cast<size_t>(it.seg) * A.T * A.k + p) * A.H + it.r0 + lane] = it.gate[t] * h;
          }
        }
      } else {
        if (t < ng) A.y_plain[static_cast<size_t>(g0 + t) * it.rows + it.r0 + lane] = h;
      }
    }
  }
  lds_barrier();
}

// Item i of the launch's list: shared-expert tiles first (they carry every token), then the
// routed experts' tiles, each described by its expert record.  Decoding is split in three steps
// so that a caller can issue the record's scalar loads early and use them later: locate_item
// (index arithmetic only), load_record (the loads) and fill_item (the uses).
struct ItemLoc {
  int slot;   // record slot: 0 = shared expert, 1 + a = a-th active routed expert
  int nseg;   // column segments of the block's rows
  int inter;  // intermediate size of the expert
};

template <int MODE>
MOE_INLINE ItemLoc locate_item(const KArgs& A, int i, int sh_tiles, int tiles, Item& it) {
  constexpr int kTileRows = MODE == kGateUp ? kGateUpTileRows : kRowPanel;
  // segments exist for down items only (the SiLU epilogue of gate_up needs whole rows)
  const int ssh = MODE == kDown ? A.segs_shared : 1;
  const int srt = MODE == kDown ? A.segs : 1;
  ItemLoc loc;
  if (i < sh_tiles * ssh) {
    loc.slot = 0;
    it.shared = true;
    it.r0 = (i / ssh) * kTileRows;
    it.seg = i - (i / ssh) * ssh;
    loc.nseg = ssh;
    loc.inter = A.I_shared;
  } else {
    const int r = i - sh_tiles * ssh;
    const int per = tiles * srt;
    const int a = r / per, rem = r - a * per, tile = rem / srt;
    loc.slot = 1 + a;
    it.shared = false;
    it.r0 = tile * kTileRows;
    it.seg = rem - tile * srt;
    loc.nseg = srt;
    loc.inter = A.I;
  }
  return loc;
}

// The fields of an expert record that an item uses, held in registers.
struct RecFields {
  const uint32_t* planes;
  const uint16_t* lut;
  int q, expert, src_base, n;
  int tok[kRecTok], pair[kRecTok];
  float gate[kRecTok];
  bool ok;
};

template <int MODE>
MOE_INLINE RecFields load_record(const KArgs& A, int slot) {
  const AS_CONST ExpertRecord& rec = cview<ExpertRecord>(A.recs)[slot];
  RecFields f;
  f.planes = rec.planes[MODE];
  f.lut = rec.lut[MODE];
  const uint32_t meta = rec.meta;
  f.q = record_q(meta, MODE);
  f.expert = rec.expert;
  f.src_base = rec.src_base;
  f.n = rec.n;
#pragma unroll
  for (int t = 0; t < kRecTok; ++t) {
    f.tok[t] = rec.tok[t];
    f.pair[t] = rec.pair[t];
    f.gate[t] = rec.gate[t];
  }
  f.ok = record_ok(meta);
  return f;
}

// Returns false if the record says a page-table descriptor is invalid.
template <int MODE>
MOE_INLINE bool fill_item(const KArgs& A, const RecFields& f, const ItemLoc& loc, Item& it) {
  it.planes = f.planes;
  it.lut = f.lut;
  it.q = f.q;
  it.expert = f.expert;
  it.src_base = f.src_base;
  it.n = f.n;
#pragma unroll
  for (int t = 0; t < kRecTok; ++t) {
    it.tok[t] = f.tok[t];
    it.pair[t] = f.pair[t];
    it.gate[t] = f.gate[t];
  }
  it.rows = MODE == kGateUp ? 2 * loc.inter : A.H;
  it.cols = MODE == kGateUp ? A.H : loc.inter;
  it.row_hi = MODE == kGateUp ? loc.inter + it.r0 : it.r0 + 32;
  if (!f.ok) return false;
  const int nc4 = it.cols / kColChunk;
  it.c0 = uniform(it.seg * nc4 / loc.nseg);
  it.nc = uniform((it.seg + 1) * nc4 / loc.nseg) - it.c0;
  return true;
}

template <int MODE>
MOE_INLINE bool decode_item(const KArgs& A, int i, int sh_tiles, int tiles, Item& it) {
  it.expert = -1;
  if constexpr (MODE == kPlain) {
    const moe_apq_block& b = A.plain;
    it.r0 = i * kRowPanel;
    it.n = A.T;
    it.src_base = 0;
    it.shared = false;
    it.seg = 0;
    it.c0 = 0;
    it.nc = b.cols / kColChunk;
    it.planes = b.planes;
    it.lut = b.lut;
    it.rows = b.rows;
    it.cols = b.cols;
    it.q = b.q;
#pragma unroll
    for (int t = 0; t < kRecTok; ++t) {
      it.tok[t] = t;
      it.pair[t] = t;
      it.gate[t] = 1.0f;
    }
    it.row_hi = it.r0 + 32;
    return true;
  } else {
    const ItemLoc loc = locate_item<MODE>(A, i, sh_tiles, tiles, it);
    return fill_item<MODE>(A, load_record<MODE>(A, loc.slot), loc, it);
  }
}

// ---------------------------------------------------------------------------------------------
// Dense tiles (many tokens on one block: the shared expert, hot experts, prefill): matrix cores.
//
// The weights are decoded as in the streaming path, one row per lane, 64 rows.  For a pair of
// 8-column octets (o, o + 1) a lane holds X = its row's octet o and Y = its row's octet o + 1;
// one v_permlane32_swap per register turns them into the two A operands of
// v_mfma_f32_32x32x16_f16: [X of lanes 0-31, Y of lanes 0-31] = rows 0-31 with k 0-7 = octet o
// and k 8-15 = octet o + 1, and [X of lanes 32-63, Y of lanes 32-63] = rows 32-63 likewise.
// The B operand is the same for both: lane n < 32 holds token n % 16's octet o, lane 32 + n its
// octet o + 1 (columns 16-31 repeat tokens 0-15 and are dropped).  Two MFMAs per octet pair
// therefore compute all 64 rows for 16 tokens with no zero padding.
//
// Activations are staged per 128-column chunk into the wavefront's LDS ring by buffer loads
// that write LDS directly, issued just before the same chunk's plane loads: vector memory
// completes in order, so one wait covers both.  The ring is piece-major ([piece][token]), so a
// B operand is one contiguous 1-KiB ds_read_b128 with no bank conflicts.
// ---------------------------------------------------------------------------------------------

// Table kind of dense tiles: 0 = pair (q <= 3), 1 = single with 4-byte slots (q = 4..7),
// 2 = single with 2-byte slots (q = 8).
template <int Q>
constexpr int dense_table_kind() { return Q <= 3 ? 0 : (Q <= 7 ? 1 : 2); }

// q <= 4 single table: every wavefront holds the whole row; wavefront W writes entries
// [W VPW, (W+1) VPW).
template <int Q, int W>
MOE_INLINE void write_small_single_rows(const u32x4 (&L)[kLutRegs], int lane) {
  constexpr int NE = 1 << Q;
  constexpr int VPW = NE >= 4 ? NE / 4 : 1;
  char* base = reinterpret_cast<char*>(g_lds) + lane * 4;
  if constexpr (W * VPW < NE) {
#pragma unroll
    for (int vi = 0; vi < VPW; ++vi) {
      const int v = W * VPW + vi;
      const uint32_t d = lut_dword(L, v);
      const uint32_t dup = __builtin_amdgcn_perm(d, d, (v & 1) ? 0x03020302u : 0x01000100u);
      *reinterpret_cast<uint32_t*>(base + (v << 8)) = dup;
    }
  }
}

// Every address is a per-lane base plus a compile-time offset (one ds_write with an immediate).
template <int Q>
MOE_INLINE void write_dense_table(const u32x4 (&L)[kLutRegs], int lane, int wave) {
  constexpr int NE = 1 << Q;
  if constexpr (dense_table_kind<Q>() == 0) {
    write_table<Q>(L, lane, wave);
  } else if constexpr (dense_table_kind<Q>() == 2) {
    // registers hold this wavefront's quarter: entries [64 wave, 64 wave + 64), at v*128 + lane*2
    char* base = reinterpret_cast<char*>(g_lds) + lane * 2 + wave * (64 * 128);
#pragma unroll
    for (int vi = 0; vi < 64; ++vi) {
      const uint32_t d = lut_dword(L, vi);
      *reinterpret_cast<uint16_t*>(base + vi * 128) = static_cast<uint16_t>((vi & 1) ? d >> 16 : d);
    }
  } else if constexpr (Q >= 5) {
    constexpr int VPW = NE / 4;  // registers hold this wavefront's quarter
    char* base = reinterpret_cast<char*>(g_lds) + lane * 4 + wave * (VPW << 8);
#pragma unroll
    for (int vi = 0; vi < VPW; ++vi) {
      const uint32_t d = lut_dword(L, vi);
      *reinterpret_cast<uint32_t*>(base + (vi << 8)) =
          __builtin_amdgcn_perm(d, d, (vi & 1) ? 0x03020302u : 0x01000100u);
    }
  } else {
    switch (wave) {
      case 0: write_small_single_rows<Q, 0>(L, lane); break;
      case 1: write_small_single_rows<Q, 1>(L, lane); break;
      case 2: write_small_single_rows<Q, 2>(L, lane); break;
      default: write_small_single_rows<Q, 3>(L, lane); break;
    }
  }
}

MOE_INLINE uint32_t lds_u16(uint32_t byte_addr) {
  return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(g_lds) + byte_addr);
}

// One 32-column word through the dense table, in two phases so that a word's LDS lookups can be
// in flight while other work issues: dense_lookup issues every lookup of the word (16 for the
// pair table, 32 for the single tables) into `v`, dense_finish turns them into the 16 dwords
// wv[4b + j] = (column 8b + 2j, column 8b + 2j + 1).  Keeping the lookups together matters: when
// they are interleaved with their uses, every pair of lookups waits out the full LDS latency.
template <int Q>
MOE_INLINE void dense_lookup(const uint32_t (&w)[Q], uint32_t lane4, uint32_t (&v)[32]) {
  if constexpr (dense_table_kind<Q>() == 0) {
    uint32_t pw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pw[j] = pair_word<Q>(w, j);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) v[4 * b + j] = lds_load(tbl_addr(pw[j], lane4, b));
  } else {
    uint32_t sw[8];
#pragma unroll
    for (int o = 0; o < 8; ++o) sw[o] = single_word<Q>(w, o);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if constexpr (dense_table_kind<Q>() == 2) {
          v[4 * b + j] = lds_u16(tbl_addr(sw[j], lane4, b) >> 1);
          v[16 + 4 * b + j] = lds_u16(tbl_addr(sw[j + 4], lane4, b) >> 1);
        } else {
          v[4 * b + j] = lds_load(tbl_addr(sw[j], lane4, b));
          v[16 + 4 * b + j] = lds_load(tbl_addr(sw[j + 4], lane4, b));
        }
      }
    }
  }
}

template <int Q>
MOE_INLINE void dense_finish(const uint32_t (&v)[32], uint32_t (&wv)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (dense_table_kind<Q>() == 0) {
      wv[i] = v[i];
    } else if constexpr (dense_table_kind<Q>() == 2) {
      wv[i] = v[i] | (v[16 + i] << 16);
    } else {
      wv[i] = __builtin_amdgcn_perm(v[16 + i], v[i], 0x05040100u);  // (even lo, odd hi)
    }
  }
}

template <int Q>
MOE_INLINE void decode_word_dense(const uint32_t (&w)[Q], uint32_t lane4, uint32_t (&wv)[16]) {
  uint32_t v[32];
  dense_lookup<Q>(w, lane4, v);
  __builtin_amdgcn_sched_barrier(0);
  dense_finish<Q>(v, wv);
}

// 16 bytes per lane from byte voff + soff of the buffer `rsrc` straight into LDS at lds_addr +
// 16 * lane (a buffer load in its LDS-DMA form).  The compiler sees it as a vector-memory load, so
// its own waits for later-used registers count it; what it does not model is the LDS write, so
// readers of the staged bytes wait by hand (dense_wait / wide_wait) and a slot is refilled only
// after an lgkmcnt(0).  The global-address form of this load belongs to the FLAT family and also
// accesses LDS; after one of those the compiler waits for every outstanding vector-memory
// operation at the next use of a loaded register, which drained the chunk ring at every loop
// iteration.  The buffer form keeps the compiler's waits exact.
MOE_INLINE void lds_dma16(uint32_t lds_addr, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (AS_LDS void*)(static_cast<uintptr_t>(lds_addr)), 16, voff,
                                           soff, 0, 0);
}


// The LDS reads of a ring slot's previous chunk have returned (it is about to be refilled).
MOE_INLINE void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Keeps the loads issued before it ahead of those issued after it.  The partial waits count a
// slot's loads as one group in slot order: if the compiler interleaved two slots' loads (it
// scheduled both slots' plane loads ahead of both slots' staging loads once), "all but the next
// slot's loads" would no longer cover the current slot's staging.
MOE_INLINE void issue_order() {
  asm volatile("" : : : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// A dense pass holds NT = 16 or 32 tokens.  Its chunk is 128 columns (a lane's 16-byte plane
// unit, 4 words) for 16 tokens and 64 columns (half a unit, 2 words) for 32 tokens, so that a
// staged chunk is 4 KiB either way: [8-column pieces][NT tokens][16 bytes].
template <int NT>
struct PlaneUnit;
template <>
struct PlaneUnit<16> {
  typedef u32x4 type;
  static constexpr int kWords = 4;
};
template <>
struct PlaneUnit<32> {
  typedef u32x2 type;
  static constexpr int kWords = 2;
};

template <int Q, int NT>
struct DenseStream {
  static constexpr int D = 2;       // chunks in flight per wavefront
  static constexpr int kDma = 4;    // LDS loads per staged chunk (4 KiB)
  static constexpr int kWords = PlaneUnit<NT>::kWords;   // 32-column words per chunk
  static constexpr uint32_t kPieceBytes = NT * 16;       // one 8-column piece of every token
  typedef typename PlaneUnit<NT>::type unit_t;
  unit_t buf[D][Q];                 // plane words of a chunk
  __amdgpu_buffer_rsrc_t prsrc;     // the block's first Q bit planes
  uint32_t poff;                    // per lane: byte of its unit in chunk 0 of plane 0
  uint32_t plane_bytes;             // plane stride
  int cb, ce;                       // this wavefront's chunks [cb, ce)
  __amdgpu_buffer_rsrc_t xrsrc;     // the activation rows
  uint32_t xoff;                    // per lane: DMA 0's source byte in chunk 0
  uint32_t xring;                   // LDS address of this wavefront's ring
  uint32_t bx;                      // per lane: B-operand address in slot 0, piece 0

  // Loads are issued unconditionally (a chunk past the end re-reads the last one, a cache hit)
  // so that the number of loads in flight is always the same.
  MOE_INLINE int clamp(int c) const { return c < ce ? c : (ce > cb ? ce - 1 : cb); }
  // Byte offset of chunk c from the lane's unit of chunk 0 (a 128-column chunk is one 1-KiB run of
  // the 64 rows' units; a 64-column chunk is half c & 1 of every unit of run c >> 1).
  MOE_INLINE uint32_t chunk_off(int c) const {
    if constexpr (NT == 16) {
      return static_cast<uint32_t>(c) * 1024u;
    } else {
      return static_cast<uint32_t>(c >> 1) * 1024u + static_cast<uint32_t>(c & 1) * 8u;
    }
  }
  // The refill of slot `slot` with chunk c: its Q plane loads (registers), then its kDma staged
  // activation loads (LDS), on every path.  The plane loads may go out as soon as the slot's
  // plane words are consumed; the staging waits until the slot's B reads have returned.
  MOE_INLINE void issue_planes(int slot, int c) {
    const uint32_t co = chunk_off(c);
#pragma unroll
    for (int p = 0; p < Q; ++p) {
      if constexpr (NT == 16) {
        buf[slot][p] = __builtin_amdgcn_raw_buffer_load_b128(prsrc, poff, co + p * plane_bytes, 0);
      } else {
        buf[slot][p] = __builtin_amdgcn_raw_buffer_load_b64(prsrc, poff, co + p * plane_bytes, 0);
      }
    }
  }
  MOE_INLINE void issue_stage(int slot, int c) {
    lds_reads_done();
    constexpr int kDmaStep = 4 * 16 * 16 / NT;                 // bytes of a token row per DMA
    constexpr int kChunkBytes = kWords * 32 * 2;               // bytes of a token row per chunk
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      lds_dma16(xring + slot * kXSlotBytes + i * 1024, xrsrc, xoff, i * kDmaStep + static_cast<uint32_t>(c) * kChunkBytes);
  }
  MOE_INLINE void issue(int slot, int c) {
    issue_order();
    issue_planes(slot, c);
    issue_order();
    issue_stage(slot, c);
    issue_order();
  }
  MOE_INLINE void prologue() {
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s, clamp(cb + s));
  }
};

// The chunk about to be consumed has landed (its staged activations and its planes): only the
// next chunk's kDma + Q loads may still be in flight.
template <int Q, int NT>
MOE_INLINE void dense_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q + DenseStream<Q, NT>::kDma) : "memory");
}

// A word's operands in flight: its two B operands (the staged activations of octets 4 JW ..
// 4 JW + 3) and its table lookups.  The B reads go first: LDS operations complete in order, so
// the products of this word then never wait for the lookups of the word issued after them.
template <int Q>
struct DenseWordOps {
  u32x4 b[2];
  uint32_t v[32];
};

template <int Q, int NT, int JW>
MOE_INLINE void dense_word_lookup(const DenseStream<Q, NT>& S, int s, uint32_t lane4, DenseWordOps<Q>& o) {
  const char* xb = reinterpret_cast<const char*>(g_lds) + S.bx + s * kXSlotBytes;
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
    o.b[pr] = *reinterpret_cast<const u32x4*>(xb + (JW * 4 + 2 * pr) * DenseStream<Q, NT>::kPieceBytes);
  uint32_t w[Q];
#pragma unroll
  for (int p = 0; p < Q; ++p) w[p] = word_of(S.buf[s][p], JW);
  dense_lookup<Q>(w, lane4, o.v);
}

template <int Q>
MOE_INLINE void dense_word_mma(const DenseWordOps<Q>& o, f32x16& lo, f32x16& hi) {
  uint32_t wv[16];
  dense_finish<Q>(o.v, wv);
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    // octets o = 2 pr and o + 1 of this word: columns 16 pr .. 16 pr + 15
    uint32_t a1[4], a2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto sw = __builtin_amdgcn_permlane32_swap(wv[8 * pr + r], wv[8 * pr + 4 + r], false, false);
      a1[r] = sw[0];
      a2[r] = sw[1];
    }
    const u32x4 va1 = {a1[0], a1[1], a1[2], a1[3]}, va2 = {a2[0], a2[1], a2[2], a2[3]};
    lo = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, va1),
                                                 __builtin_bit_cast(half8_t, o.b[pr]), lo, 0, 0, 0);
    hi = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, va2),
                                                 __builtin_bit_cast(half8_t, o.b[pr]), hi, 0, 0, 0);
  }
}

// The four words of ring slot s, software-pipelined: word j + 1's lookups are issued before
// word j's products, so the LDS latency overlaps the previous word's matrix-core work.  Once the
// last word's lookups and B reads are issued, the slot's registers and staged bytes are no
// longer needed: its refill with chunk `next` goes out there, before the last two words'
// products, which gives the refill that much more time to land.
template <int Q, int NT, bool REFILL = true>
MOE_INLINE void dense_chunk(DenseStream<Q, NT>& S, int s, int next, uint32_t lane4, f32x16& lo, f32x16& hi) {
  DenseWordOps<Q> a, b;
  dense_word_lookup<Q, NT, 0>(S, s, lane4, a);
  dense_word_lookup<Q, NT, 1>(S, s, lane4, b);
  __builtin_amdgcn_sched_barrier(0);
  dense_word_mma<Q>(a, lo, hi);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (DenseStream<Q, NT>::kWords == 4) {
    dense_word_lookup<Q, NT, 2>(S, s, lane4, a);
    __builtin_amdgcn_sched_barrier(0);
    dense_word_mma<Q>(b, lo, hi);
    __builtin_amdgcn_sched_barrier(0);
    dense_word_lookup<Q, NT, 3>(S, s, lane4, b);
    __builtin_amdgcn_sched_barrier(0);
    if (REFILL) S.issue_planes(s, next);
    __builtin_amdgcn_sched_barrier(0);
    dense_word_mma<Q>(a, lo, hi);
    __builtin_amdgcn_sched_barrier(0);
    dense_word_mma<Q>(b, lo, hi);
  } else {
    if (REFILL) S.issue_planes(s, next);
    __builtin_amdgcn_sched_barrier(0);
    dense_word_mma<Q>(b, lo, hi);
  }
  if (REFILL) {
    issue_order();
    S.issue_stage(s, next);
    issue_order();
  }
}

template <int Q, int NT>
MOE_INLINE void dense_columns(DenseStream<Q, NT>& S, uint32_t lane4, f32x16& lo, f32x16& hi) {
  static_assert(DenseStream<Q, NT>::D == 2, "the loop below walks the two ring slots in turn");
  // Two chunks per iteration with every refill unconditional, so that the loads in flight at
  // the loop head are the same on every path and the compiler's wait there keeps the ring full
  // (a refill under a condition made it wait for every load, draining the ring each chunk).
  int c = S.cb;
  for (; c + 1 < S.ce; c += 2) {
    dense_wait<Q, NT>();
    dense_chunk<Q, NT>(S, 0, S.clamp(c + 2), lane4, lo, hi);
    dense_wait<Q, NT>();
    dense_chunk<Q, NT>(S, 1, S.clamp(c + 3), lane4, lo, hi);
  }
  if (c < S.ce) {
    dense_wait<Q, NT>();
    dense_chunk<Q, NT, false>(S, 0, -1, lane4, lo, hi);
  }
}

// Geometry of the tile for this wavefront and the activation rows of tokens [g0, g0 + ng).
template <int MODE, int Q, int NT>
MOE_INLINE void make_dense_stream(const KArgs& A, const Item& it, int g0, int ng, DenseStream<Q, NT>& S) {
  constexpr int kPer = 4 / DenseStream<Q, NT>::kWords;   // chunks per 128 columns
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int C = it.cols;
  const int row = lane_row(it, lane);
  const int nc4 = C / kColChunk;
  S.plane_bytes = static_cast<uint32_t>(static_cast<size_t>(it.rows) * C / 8);
  S.prsrc = buf_rsrc(it.planes, static_cast<size_t>(S.plane_bytes) * Q);
  S.poff = static_cast<uint32_t>((row / kRowPanel) * nc4 * 64 + (row % kRowPanel)) * 16u;
  S.cb = uniform(kPer * it.c0 + (kPer * it.nc * wave) / kWavesPerTile);
  S.ce = uniform(kPer * it.c0 + (kPer * it.nc * (wave + 1)) / kWavesPerTile);
  const uint16_t* base;   // the activation rows: x (gate_up, plain) or act (down)
  int rows_total;
  if constexpr (MODE == kDown) {
    base = it.shared ? A.act_shared : A.act;
    rows_total = it.shared ? A.T : A.T * A.k;
  } else {
    base = A.x;
    rows_total = A.T;
  }
  // token lane % NT (tokens past ng re-read token g0's row: their columns are never stored)
  const int t = lane & (NT - 1);
  const int tt = g0 + (t < ng ? t : 0);
  int row_index;
  if constexpr (MODE == kGateUp) {
    row_index = it.shared ? tt
                          : static_cast<int>(buf_u32(buf_rsrc(A.pairs, static_cast<size_t>(A.T) * A.k * 4),
                                                     static_cast<uint32_t>(it.src_base + tt) * 4u)) / A.k;
  } else if constexpr (MODE == kDown) {
    row_index = it.shared ? tt : it.src_base + tt;
  } else {
    row_index = tt;
  }
  // DMA lane l: token l % NT, piece l / NT of the DMA's group of 64 / NT pieces
  S.xrsrc = buf_rsrc(base, static_cast<size_t>(rows_total) * C * 2);
  S.xoff = static_cast<uint32_t>(row_index) * static_cast<uint32_t>(C * 2) + (lane / NT) * 16;
  S.xring = kXRingBase + static_cast<uint32_t>(wave) * kXWaveBytes;
  S.bx = S.xring + static_cast<uint32_t>(lane & (NT - 1)) * 16u + static_cast<uint32_t>(lane >> 5) * DenseStream<Q, NT>::kPieceBytes;
}

// Where lane `lane`'s token of a matrix-core tile goes: the output row base and the scale
// (rows r0 + m follow), or nothing when the lane's column is not a live token.
struct TileOut {
  uint16_t* act_dst;
  float* out_dst;
  float scale;
  bool live;
};

template <int MODE>
MOE_INLINE TileOut tile_out(const KArgs& A, const Item& it, int g0, int tok, bool live) {
  TileOut o{nullptr, nullptr, 1.0f, live};
  if (!live) return o;
  if constexpr (MODE == kGateUp) {
    o.act_dst = it.shared ? A.act_shared + static_cast<size_t>(g0 + tok) * A.I_shared + it.r0
                          : A.act + static_cast<size_t>(it.src_base + g0 + tok) * A.I + it.r0;
  } else if constexpr (MODE == kDown) {
    if (it.shared) {
      if (A.shared_scale) o.scale = A.shared_scale[g0 + tok];
      o.out_dst = A.part_shared + (static_cast<size_t>(it.seg) * A.T + g0 + tok) * A.H;
    } else {
      const int p = A.pairs[it.src_base + g0 + tok];
      o.scale = A.gates[p];
      o.out_dst = A.part + (static_cast<size_t>(it.seg) * A.T * A.k + p) * A.H;
    }
    o.out_dst += it.r0;
  } else {
    o.out_dst = A.y_plain + static_cast<size_t>(g0 + tok) * it.rows + it.r0;
  }
  return o;
}

// Wavefront W's quarter of the reduction: registers i = 4W .. 4W + 3 of lo and hi (tile rows
// m = 8W + 4 (lane / 32) + i % 4 and 32 + m), summed over the four wavefronts in the fixed order
// 0 + 1 + 2 + 3 (its own values from registers, the others' from their rings), then stored.
template <int MODE, int W>
MOE_INLINE void reduce_quarter(const f32x16& lo, const f32x16& hi, const float* ring, int lane, const TileOut& o) {
  float sl[4], sh[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * W + j;
#pragma unroll
    for (int w = 0; w < kWavesPerTile; ++w) {
      const float* other = ring + w * (kXWaveBytes / 4);
      const float a = w == W ? lo[i] : other[i * 64 + lane];
      const float b = w == W ? hi[i] : other[(16 + i) * 64 + lane];
      sl[j] = w == 0 ? a : sl[j] + a;
      sh[j] = w == 0 ? b : sh[j] + b;
    }
  }
  if (!o.live) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 8 * W + 4 * (lane >> 5) + j;
    if constexpr (MODE == kGateUp) {
      // gate row r0 + m and up row row_hi + m meet in the same lane and register
      o.act_dst[m] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(silu_mul(sl[j], sh[j])));
    } else {
      o.out_dst[m] = o.scale * sl[j];
      o.out_dst[32 + m] = o.scale * sh[j];
    }
  }
}

// D layout of the 32x32 MFMA: lane l, register i holds D[m][l % 32] with
// m = 8 (i / 4) + 4 (l / 32) + i % 4; `lo` covers tile rows m, `hi` rows 32 + m.  The four
// wavefronts hold partial sums over their own columns.  Each writes the 24 registers it does not
// reduce into its own (drained) activation ring, and after one barrier each reduces and stores
// a quarter of the tile's rows (registers 4W .. 4W + 3), so the reduction and the stores are
// spread over the four wavefronts instead of serialised in one.
template <int MODE>
MOE_INLINE void reduce_tile(const KArgs& A, const Item& it, int g0, int tok, bool live, f32x16& lo,
                            f32x16& hi, const Queue* Qu) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  float* ring = reinterpret_cast<float*>(reinterpret_cast<char*>(g_lds) + kXRingBase);
  float* mine = ring + wave * (kXWaveBytes / 4);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((i >> 2) != wave) {
      mine[i * 64 + lane] = lo[i];
      mine[(16 + i) * 64 + lane] = hi[i];
    }
  }
  if (Qu) queue_publish(*Qu);
  const TileOut o = tile_out<MODE>(A, it, g0, tok, live);
  lds_barrier();
  switch (wave) {
    case 0: reduce_quarter<MODE, 0>(lo, hi, ring, lane, o); break;
    case 1: reduce_quarter<MODE, 1>(lo, hi, ring, lane, o); break;
    case 2: reduce_quarter<MODE, 2>(lo, hi, ring, lane, o); break;
    default: reduce_quarter<MODE, 3>(lo, hi, ring, lane, o); break;
  }
  lds_barrier();
}

// Columns l % 32 < 16 of a 16-token pass are token l % 16 (the other 16 repeat them); a 32-token
// pass has token l % 32 in column l % 32.
template <int MODE, int NT>
MOE_INLINE void dense_reduce_and_store(const KArgs& A, const Item& it, int g0, int ng, f32x16& lo,
                                       f32x16& hi, const Queue* Qu) {
  const int lane = threadIdx.x & 63;
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // the ring's last (re-read) loads
  const int tok = lane & (NT - 1);
  const bool live = (NT == 32 || (lane & 16) == 0) && tok < ng;
  reduce_tile<MODE>(A, it, g0, tok, live, lo, hi, Qu);
}

template <int MODE, int Q, int NT>
MOE_INLINE void run_item_dense(const KArgs& A, const Item& it, const Queue& Qu) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  DenseStream<Q, NT> S;
  make_dense_stream<MODE, Q, NT>(A, it, 0, min(NT, it.n), S);
  u32x4 L[kLutRegs];
  prefetch_lut_q<Q, true>(it, lane, wave, L);
  S.prologue();
  write_dense_table<Q>(L, lane, wave);
  lds_barrier();
  for (int g0 = 0; g0 < it.n; g0 += NT) {
    const int ng = min(NT, it.n - g0);
    if (g0 > 0) {
      make_dense_stream<MODE, Q, NT>(A, it, g0, ng, S);
      S.prologue();
    }
    f32x16 lo = {}, hi = {};
    dense_columns<Q, NT>(S, static_cast<uint32_t>(lane) * 4u, lo, hi);
    dense_reduce_and_store<MODE, NT>(A, it, g0, ng, lo, hi, g0 + NT >= it.n ? &Qu : nullptr);
  }
}

// ---------------------------------------------------------------------------------------------
// Wide tiles (more tokens than one 32-token dense pass: prefill chunks, where an expert meets
// hundreds of tokens).  The dense passes decode the weights once per 16 or 32 tokens; here each
// decode serves kWideTok tokens.
//
// The four wavefronts take one 32-column word each of every 128-column chunk (wavefront w: word
// w), so a wavefront needs the activations of its own 32 columns only: its LDS ring slot holds
// [4 octets][kWideTok tokens][16 bytes] = 4 KiB, filled by buffer loads straight to LDS, and two
// slots fit the same 8 KiB per wavefront as the dense ring.  A lane loads its row's 32-bit word
// of each plane (the four wavefronts' loads of one 1-KiB run share its cache lines).
// The decoded word gives the A operands of two 16-column k steps exactly as in the dense path
// (one v_permlane32_swap per register: rows 0-31 and rows 32-63); B is 32 distinct tokens
// (lane n < 32: token n's first octet of the step, lane 32 + n: its second), so every output
// column is a real token: per k step, 2 MFMAs per 32-token tile.  Each wavefront holds partial
// sums over its quarter of the columns; they are reduced across wavefronts in LDS, one 32-token
// tile at a time, through the drained rings.
// ---------------------------------------------------------------------------------------------
constexpr int kWideTok = 64;                                      // tokens per pass
constexpr int kWideTiles = kWideTok / 32;                         // 32-token MFMA tiles
constexpr uint32_t kWideSlotBytes = 4 * kWideTok * 16;            // 4 octets x tokens x 16 B
static_assert(2 * kWideSlotBytes == kXWaveBytes, "wide ring slots must fill the dense ring");
static_assert(kWideTok == kRecGroupTok, "a split record holds one wide matrix-core pass");

template <int Q>
struct WideStream {
  static constexpr int D = 2;       // chunks in flight per wavefront
  static constexpr int kDma = 4;    // staged loads per chunk: one per octet (lane = token)
  uint32_t buf[D][Q];               // this wavefront's plane word of the chunk, per plane
  __amdgpu_buffer_rsrc_t prsrc;     // the block's first Q bit planes
  uint32_t poff;                    // per lane: byte of its word in chunk 0 of plane 0
  uint32_t plane_bytes;             // plane stride
  int cb, ce;                       // the item's chunks [cb, ce)
  __amdgpu_buffer_rsrc_t xrsrc;     // the activation rows
  uint32_t xoff;                    // per lane: its token's first staged octet of chunk 0
  uint32_t xring;                   // LDS address of this wavefront's ring
  uint32_t bx;                      // per lane: B-operand address in slot 0, octet 0, tile 0

  MOE_INLINE int clamp(int c) const { return c < ce ? c : (ce > cb ? ce - 1 : cb); }
  // The refill of slot `slot` with chunk c (see DenseStream).
  MOE_INLINE void issue_planes(int slot, int c) {
#pragma unroll
    for (int p = 0; p < Q; ++p) buf[slot][p] = buf_u32(prsrc, poff, static_cast<uint32_t>(c) * 1024u + p * plane_bytes);
  }
  MOE_INLINE void issue_stage(int slot, int c) {
    lds_reads_done();
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      lds_dma16(xring + slot * kWideSlotBytes + i * 1024, xrsrc, xoff, i * 16 + static_cast<uint32_t>(c) * 256);
  }
  MOE_INLINE void issue(int slot, int c) {
    issue_order();
    issue_planes(slot, c);
    issue_order();
    issue_stage(slot, c);
    issue_order();
  }
  MOE_INLINE void prologue() {
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s, clamp(cb + s));
  }
};

// The chunk about to be consumed has landed: only the next chunk's kDma + Q loads may still be
// in flight.
template <int Q>
MOE_INLINE void wide_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q + WideStream<Q>::kDma) : "memory");
}

// Geometry of the item for this wavefront and the activation rows of tokens [g0, g0 + ng).
template <int MODE, int Q>
MOE_INLINE void make_wide_stream(const KArgs& A, const Item& it, int g0, int ng, WideStream<Q>& S) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int C = it.cols;
  const int row = lane_row(it, lane);
  const int nc4 = C / kColChunk;
  // unit (panel, chunk 0, row) of plane 0, then this wavefront's 32-bit word inside it
  S.plane_bytes = static_cast<uint32_t>(static_cast<size_t>(it.rows) * C / 8);
  S.prsrc = buf_rsrc(it.planes, static_cast<size_t>(S.plane_bytes) * Q);
  S.poff = static_cast<uint32_t>((row / kRowPanel) * nc4 * 64 + (row % kRowPanel)) * 16u + wave * 4u;
  S.cb = it.c0;
  S.ce = it.c0 + it.nc;
  const uint16_t* base;   // the activation rows: x (gate_up, plain) or act (down)
  int rows_total;
  if constexpr (MODE == kDown) {
    base = it.shared ? A.act_shared : A.act;
    rows_total = it.shared ? A.T : A.T * A.k;
  } else {
    base = A.x;
    rows_total = A.T;
  }
  // the lane's token (tokens past ng re-read token g0's row: their columns are never stored)
  const int t = lane;
  const int tt = g0 + (t < ng ? t : 0);
  int row_index;
  if constexpr (MODE == kGateUp) {
    row_index = it.shared ? tt
                          : static_cast<int>(buf_u32(buf_rsrc(A.pairs, static_cast<size_t>(A.T) * A.k * 4),
                                                     static_cast<uint32_t>(it.src_base + tt) * 4u)) / A.k;
  } else if constexpr (MODE == kDown) {
    row_index = it.shared ? tt : it.src_base + tt;
  } else {
    row_index = tt;
  }
  S.xrsrc = buf_rsrc(base, static_cast<size_t>(rows_total) * C * 2);
  S.xoff = static_cast<uint32_t>(row_index) * static_cast<uint32_t>(C * 2) + wave * 64;
  S.xring = kXRingBase + static_cast<uint32_t>(wave) * kXWaveBytes;
  S.bx = S.xring + static_cast<uint32_t>(lane >> 5) * (kWideTok * 16) + static_cast<uint32_t>(lane & 31) * 16u;
}

// One chunk of ring slot s: this wavefront's 32-column word of it for the pass's tokens.  The B
// reads are issued ahead of the table lookups (LDS operations complete in order), and the
// lookups together (see dense_lookup).
template <int Q, bool REFILL = true>
MOE_INLINE void wide_chunk(WideStream<Q>& S, int s, int next, uint32_t lane4, int ntiles,
                           f32x16 (&lo)[kWideTiles], f32x16 (&hi)[kWideTiles]) {
  const char* xb = reinterpret_cast<const char*>(g_lds) + S.bx + s * kWideSlotBytes;
  u32x4 b[2][kWideTiles];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int g = 0; g < kWideTiles; ++g)
      if (g < ntiles) b[st][g] = *reinterpret_cast<const u32x4*>(xb + (2 * st) * (kWideTok * 16) + g * 512);
  uint32_t w[Q];
#pragma unroll
  for (int p = 0; p < Q; ++p) w[p] = S.buf[s][p];
  uint32_t v[32];
  dense_lookup<Q>(w, lane4, v);
  __builtin_amdgcn_sched_barrier(0);
  if (REFILL) S.issue_planes(s, next);   // the slot's plane words are consumed
  __builtin_amdgcn_sched_barrier(0);
  uint32_t wv[16];
  dense_finish<Q>(v, wv);
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    // k step st: octets 2 st and 2 st + 1 of the word (columns 16 st .. 16 st + 15)
    uint32_t a1[4], a2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto sw = __builtin_amdgcn_permlane32_swap(wv[8 * st + r], wv[8 * st + 4 + r], false, false);
      a1[r] = sw[0];
      a2[r] = sw[1];
    }
    const u32x4 va1 = {a1[0], a1[1], a1[2], a1[3]}, va2 = {a2[0], a2[1], a2[2], a2[3]};
#pragma unroll
    for (int g = 0; g < kWideTiles; ++g) {
      if (g >= ntiles) continue;   // a pass of at most 32 tokens fills one tile
      lo[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, va1),
                                                    __builtin_bit_cast(half8_t, b[st][g]), lo[g], 0, 0, 0);
      hi[g] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, va2),
                                                    __builtin_bit_cast(half8_t, b[st][g]), hi[g], 0, 0, 0);
    }
  }
  if (REFILL) {
    issue_order();
    S.issue_stage(s, next);
    issue_order();
  }
}

template <int Q>
MOE_INLINE void wide_columns(WideStream<Q>& S, uint32_t lane4, int ntiles, f32x16 (&lo)[kWideTiles],
                             f32x16 (&hi)[kWideTiles]) {
  static_assert(WideStream<Q>::D == 2, "the loop below walks the two ring slots in turn");
  // two chunks per iteration, every refill unconditional (see dense_columns)
  int c = S.cb;
  for (; c + 1 < S.ce; c += 2) {
    wide_wait<Q>();
    wide_chunk<Q>(S, 0, S.clamp(c + 2), lane4, ntiles, lo, hi);
    wide_wait<Q>();
    wide_chunk<Q>(S, 1, S.clamp(c + 3), lane4, ntiles, lo, hi);
  }
  if (c < S.ce) {
    wide_wait<Q>();
    wide_chunk<Q, false>(S, 0, -1, lane4, ntiles, lo, hi);
  }
}

// Reduce the four wavefronts' partial sums of one 32-token tile (tokens g0 + 32 g ..) and store
// them (reduce_tile).  D layout: lane l holds token 32 g + l % 32.
template <int MODE>
MOE_INLINE void wide_reduce_tile(const KArgs& A, const Item& it, int g0, int ng, int g, f32x16& lo,
                                 f32x16& hi, const Queue* Qu) {
  const int lane = threadIdx.x & 63;
  const int tok = 32 * g + (lane & 31);
  reduce_tile<MODE>(A, it, g0, tok, tok < ng, lo, hi, Qu);
}

template <int MODE, int Q>
MOE_INLINE void run_item_wide(const KArgs& A, const Item& it, const Queue& Qu) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  WideStream<Q> S;
  make_wide_stream<MODE, Q>(A, it, 0, min(kWideTok, it.n), S);
  u32x4 L[kLutRegs];
  prefetch_lut_q<Q, true>(it, lane, wave, L);
  S.prologue();
  write_dense_table<Q>(L, lane, wave);
  lds_barrier();
  for (int g0 = 0; g0 < it.n; g0 += kWideTok) {
    const int ng = min(kWideTok, it.n - g0);
    if (g0 > 0) {
      make_wide_stream<MODE, Q>(A, it, g0, ng, S);
      S.prologue();
    }
    f32x16 lo[kWideTiles], hi[kWideTiles];
#pragma unroll
    for (int g = 0; g < kWideTiles; ++g) lo[g] = hi[g] = f32x16{};
    wide_columns<Q>(S, static_cast<uint32_t>(lane) * 4u, (ng + 31) / 32, lo, hi);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // the ring's last (re-read) loads
    const bool last = g0 + kWideTok >= it.n;
#pragma unroll
    for (int g = 0; g < kWideTiles; ++g)
      if (32 * g < ng) wide_reduce_tile<MODE>(A, it, g0, ng, g, lo[g], hi[g], last && g == 0 ? &Qu : nullptr);
  }
}

// A tile that does not stream (at least as many tokens as the dense threshold, or more than 4):
// matrix-core path, in one 16- or 32-token dense pass, else in 64-token wide passes.
template <int MODE, int Q>
MOE_INLINE void run_item(const KArgs& A, const Item& it, const Queue& Qu) {
  if (it.n > 2 * kDenseGroup) run_item_wide<MODE, Q>(A, it, Qu);
  else if (it.n > kDenseGroup) run_item_dense<MODE, Q, 32>(A, it, Qu);
  else run_item_dense<MODE, Q, 16>(A, it, Qu);
}

// ---------------------------------------------------------------------------------------------
// Streaming across items (VALU tiles of 1 or 2 tokens).  Each wavefront keeps one ring of
// in-flight chunks (planes + the tokens' activations) running across consecutive items of the
// same width: while item i computes, the ring slots it frees are refilled with item i+1's
// first chunks and item i+1's LUT rows are fetched into registers, so HBM stays busy through
// every tile boundary instead of alternating between a load burst and an idle compute phase.
// ---------------------------------------------------------------------------------------------

// One item's share of the columns for this wavefront.
struct Geo {
  const AS_GLOBAL u32x4* pbase;
  const AS_GLOBAL u32x4* xbase[kMaxTokGroup];
  size_t plane_u4;
  int cb, n;  // first chunk and chunk count of this wavefront
  int ng;     // tokens (1..4)
};

template <int MODE>
MOE_INLINE void make_geo(const KArgs& A, const Item& it, Geo& G) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int C = it.cols;
  const int row = lane_row(it, lane);
  const int nc4 = C / kColChunk;
  G.pbase = gview<u32x4>(it.planes) + static_cast<size_t>(row / kRowPanel) * nc4 * 64 + (row % kRowPanel);
  G.plane_u4 = static_cast<size_t>(it.rows) * C / 128;
  G.cb = uniform(it.c0 + (it.nc * wave) / kWavesPerTile);
  G.n = uniform(it.c0 + (it.nc * (wave + 1)) / kWavesPerTile) - G.cb;
  G.ng = it.n;
#pragma unroll
  for (int t = 0; t < kMaxTokGroup; ++t) {
    const int tt = t < it.n ? t : 0;  // unused slots repeat slot 0 (never loaded)
    const uint16_t* rowp;
    if constexpr (MODE == kGateUp) {
      rowp = A.x + static_cast<size_t>(it.tok[tt]) * C;
    } else if constexpr (MODE == kDown) {
      rowp = it.shared ? A.act_shared + static_cast<size_t>(tt) * C
                       : A.act + static_cast<size_t>(it.src_base + tt) * C;
    } else {
      rowp = A.x + static_cast<size_t>(tt) * C;
    }
    G.xbase[t] = gview<u32x4>(rowp) + (lane & 15);
  }
}

// NT: activation rows the ring loads per chunk (1 or 2: the stream's largest token count).
template <int Q, int NT>
struct Ring {
  static constexpr int D = ring_depth<Q>();
  u32x4 buf[D][Q];
  u32x4 xbuf[D][NT];

  // Chunk k (0-based within the wavefront's share) of geometry g into `slot` (compile-time).
  // Every call issues exactly Q + NT loads: unused token slots re-read token 0's activations,
  // so the number of loads in flight never depends on run-time branches and the compiler's
  // wait counts stay exact.
  MOE_INLINE void issue(int slot, const Geo& g, int k) {
    const size_t c = static_cast<size_t>(g.cb + k);
    // planes stream through once: non-temporal loads keep them from displacing the cached
    // activations and tables (measured 1-2 % faster than ordinary loads)
#pragma unroll
    for (int p = 0; p < Q; ++p) buf[slot][p] = __builtin_nontemporal_load(&g.pbase[p * g.plane_u4 + c * 64]);
#pragma unroll
    for (int t = 0; t < NT; ++t) xbuf[slot][t] = g.xbase[t][c * 16];
  }
};

// Branch-free choice of the chunk a freed slot takes next: chunk w of the current item, else
// chunk w - m of the next item, else (nothing left) a filler whose Q + NT loads all read the
// first 256 bytes of token 0's activation row.  That row is hot in cache, so a filler never
// reaches HBM; re-reading a plane chunk instead would, because plane loads are non-temporal.
MOE_INLINE void pick_refill(const Geo& cur, const Geo& nxt, bool cont, int w, int m, Geo& g, int& k) {
  const bool use_cur = w < cur.n;
  const bool use_nxt = !use_cur && cont && w >= m && (w - m) < nxt.n;
  const bool filler = !use_cur && !use_nxt;
  g.pbase = filler ? cur.xbase[0] : (use_nxt ? nxt.pbase : cur.pbase);
  g.plane_u4 = filler ? 0 : (use_nxt ? nxt.plane_u4 : cur.plane_u4);
  g.cb = filler ? 0 : (use_nxt ? nxt.cb : cur.cb);
#pragma unroll
  for (int t = 0; t < kMaxTokGroup; ++t) g.xbase[t] = use_nxt ? nxt.xbase[t] : cur.xbase[t];
  k = use_cur ? w : (use_nxt ? w - m : 0);
}

// Table lookups of one 32-column word of ring slot s.
template <int Q, int NT, int JW>
MOE_INLINE void ring_decode(const Ring<Q, NT>& R, int s, uint32_t lane4, uint32_t (&wv)[16]) {
  uint32_t w[Q];
#pragma unroll
  for (int p = 0; p < Q; ++p) w[p] = word_of(R.buf[s][p], JW);
  decode_word<Q>(w, lane4, wv);
  __builtin_amdgcn_sched_barrier(0);
}

// Products of one decoded 32-column word for the ng (<= 4) tokens of ring slot s.
template <int Q, int NT, int JW>
MOE_INLINE void ring_dots(const Ring<Q, NT>& R, int s, int ng, const uint32_t (&wv)[16],
                          float (&acc)[NT][4]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (t < ng) dot16_bcast<JW>(acc[t], wv, R.xbuf[s][t]);
  __builtin_amdgcn_sched_barrier(0);
}

// The four words of ring slot s.  For q <= 4 the lookups of word j + 1 are issued before the
// products of word j, so the LDS latency is exposed once per chunk instead of once per word
// (q >= 5 merges each looked-up pair with VALU work of its own and keeps the plain order).
template <int Q, int NT>
MOE_INLINE void ring_chunk(const Ring<Q, NT>& R, int s, int ng, uint32_t lane4,
                           float (&acc)[NT][4]) {
  uint32_t wa[16], wb[16];
  if constexpr (Q <= 4) {
    ring_decode<Q, NT, 0>(R, s, lane4, wa);
    ring_decode<Q, NT, 1>(R, s, lane4, wb);
    ring_dots<Q, NT, 0>(R, s, ng, wa, acc);
    ring_decode<Q, NT, 2>(R, s, lane4, wa);
    ring_dots<Q, NT, 1>(R, s, ng, wb, acc);
    ring_decode<Q, NT, 3>(R, s, lane4, wb);
    ring_dots<Q, NT, 2>(R, s, ng, wa, acc);
    ring_dots<Q, NT, 3>(R, s, ng, wb, acc);
  } else {
    ring_decode<Q, NT, 0>(R, s, lane4, wa);
    ring_dots<Q, NT, 0>(R, s, ng, wa, acc);
    ring_decode<Q, NT, 1>(R, s, lane4, wa);
    ring_dots<Q, NT, 1>(R, s, ng, wa, acc);
    ring_decode<Q, NT, 2>(R, s, lane4, wa);
    ring_dots<Q, NT, 2>(R, s, ng, wa, acc);
    ring_decode<Q, NT, 3>(R, s, lane4, wa);
    ring_dots<Q, NT, 3>(R, s, ng, wa, acc);
  }
}

template <int MODE>
MOE_INLINE bool streamable(const KArgs& A, const Item& it) {
  return takes_stream(it.n, it.q, A.dense_threshold);
}
static_assert(kMaxTokGroup >= 2, "the streaming ring holds the largest streamed token count");

MOE_INLINE void report_invalid(const KArgs& A, const Item& it, int mode) {
  if (threadIdx.x == 0) {
    atomicOr(&A.err[0], 1);
    A.err[1] = it.expert;
    A.err[2] = mode;
  }
}

// A skipped down item (its record names an invalid block) still owns its rows of the partial
// sums: they are written as zeros, so that the combine adds nothing for the skipped expert and
// y stays defined for its tokens.
template <int MODE>
MOE_INLINE void zero_skipped_rows(const KArgs& A, const Item& it) {
  if constexpr (MODE == kDown) {
    for (int i = static_cast<int>(threadIdx.x); i < it.n * kRowPanel; i += kThreads) {
      const int t = i / kRowPanel, l = i - t * kRowPanel;
      float* dst = it.shared
                       ? A.part_shared + (static_cast<size_t>(it.seg) * A.T + t) * A.H
                       : A.part + (static_cast<size_t>(it.seg) * A.T * A.k + A.pairs[it.src_base + t]) * A.H;
      dst[it.r0 + l] = 0.0f;
    }
  }
}

// Process item `it` (index i) and every following item of the same width that is streamable
// with at most NT tokens.  On return, (i, it, ok) describe the first item not processed
// (i >= total: none left).
template <int MODE, int Q, int NT>
MOE_INLINE void valu_stream(const KArgs& A, Queue& Qu, int& i, Item& it, bool& ok, int total,
                            int sh_tiles, int tiles) {
  constexpr int D = Ring<Q, NT>::D;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;
  Ring<Q, NT> R;
  Geo cur, nxt;
  u32x4 L[kLutRegs];
  prefetch_lut_q<Q>(it, lane, wave, L);
  make_geo<MODE>(A, it, cur);
#pragma unroll
  for (int s = 0; s < D; ++s) {
    Geo g;
    int k;
    pick_refill(cur, cur, false, s, D, g, k);
    R.issue(s, g, k);
  }
  while (true) {
    Item next;
    const int j = Qu.nxt;
    const bool in_range = j < total;
    bool next_ok, cont;
    if constexpr (MODE == kPlain) {
      next_ok = in_range && decode_item<MODE>(A, j, sh_tiles, tiles, next);
      write_table<Q>(L, lane, wave);
    } else {
      // the next record's scalar loads are issued before the table is written and used after
      // (an index past the end locates item 0, whose record always exists)
      const ItemLoc loc = locate_item<MODE>(A, in_range ? j : 0, sh_tiles, tiles, next);
      const RecFields f = load_record<MODE>(A, loc.slot);
      write_table<Q>(L, lane, wave);
      next.expert = -1;
      next_ok = in_range && fill_item<MODE>(A, f, loc, next);
    }
    cont = next_ok && next.q == Q && streamable<MODE>(A, next) && next.n <= NT;
    if (cont) make_geo<MODE>(A, next, nxt);
    lds_barrier();
    if (cont) prefetch_lut_q<Q>(next, lane, wave, L);
    float acc[NT][4] = {};
    // the wavefront walks its chunks padded to a multiple of D, so the next item's chunk k
    // always lands in slot k % D
    const int m = (cur.n + D - 1) / D * D;
    for (int v0 = 0; v0 < m; v0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        const int v = v0 + s;
        if (v < cur.n) ring_chunk<Q, NT>(R, s, cur.ng, lane4, acc);
        Geo g;
        int k;
        pick_refill(cur, nxt, cont, v + D, m, g, k);
        R.issue(s, g, k);
      }
    }
    float tot[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tot[t] = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
    reduce_and_store<MODE, NT>(A, it, 0, it.n, tot, Qu);
    i = queue_advance(Qu);
    it = next;
    ok = next_ok;
    if (!cont) {
      // the ring's filler loads (global-address form) land before a matrix-core item's buffer
      // loads are issued: the partial waits there count only loads that complete in order
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      return;
    }
    cur = nxt;
  }
}

template <int MODE, int NT>
MOE_INLINE void stream_q(const KArgs& A, Queue& Qu, int& i, Item& it, bool& ok, int total, int sh_tiles,
                         int tiles) {
  switch (it.q) {
    case 1: valu_stream<MODE, 1, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 2: valu_stream<MODE, 2, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 3: valu_stream<MODE, 3, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 4: valu_stream<MODE, 4, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 5: valu_stream<MODE, 5, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 6: valu_stream<MODE, 6, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    case 7: valu_stream<MODE, 7, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
    default: valu_stream<MODE, 8, NT>(A, Qu, i, it, ok, total, sh_tiles, tiles); break;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void apq_tile_kernel(KArgs A) {
  constexpr int kTileRows = MODE == kGateUp ? kGateUpTileRows : kRowPanel;
  int sh_tiles = 0, tiles = 0, n_routed = 0;
  if constexpr (MODE == kPlain) {
    tiles = A.plain.rows / kRowPanel;
    n_routed = 1;
  } else {
    if (A.shared) sh_tiles = (MODE == kGateUp ? A.I_shared : A.H) / kTileRows;
    tiles = (MODE == kGateUp ? A.I : A.H) / kTileRows;
    n_routed = uniform(cview<int32_t>(A.n_recs)[0]);
  }
  const int ssh = MODE == kDown ? A.segs_shared : 1;
  const int srt = MODE == kDown ? A.segs : 1;
  const int total = sh_tiles * ssh + n_routed * tiles * srt;
  Queue Qu;
  queue_init(A, Qu, total);
  queue_request(Qu);
  int i = static_cast<int>(blockIdx.x);
  Item it;
  bool ok = i < total && decode_item<MODE>(A, i, sh_tiles, tiles, it);
  while (i < total) {
    if (!ok) {  // skip an item whose page-table descriptor is invalid
      report_invalid(A, it, MODE);
      zero_skipped_rows<MODE>(A, it);
      queue_publish(Qu);
      lds_barrier();
      i = queue_advance(Qu);
      ok = i < total && decode_item<MODE>(A, i, sh_tiles, tiles, it);
      continue;
    }
    if (streamable<MODE>(A, it)) {
      // the ring loads as many activation rows as the item has tokens (1 or 2)
      if (it.n <= 1) stream_q<MODE, 1>(A, Qu, i, it, ok, total, sh_tiles, tiles);
      else stream_q<MODE, 2>(A, Qu, i, it, ok, total, sh_tiles, tiles);
    } else {
      switch (it.q) {
        case 1: run_item<MODE, 1>(A, it, Qu); break;
        case 2: run_item<MODE, 2>(A, it, Qu); break;
        case 3: run_item<MODE, 3>(A, it, Qu); break;
        case 4: run_item<MODE, 4>(A, it, Qu); break;
        case 5: run_item<MODE, 5>(A, it, Qu); break;
        case 6: run_item<MODE, 6>(A, it, Qu); break;
        case 7: run_item<MODE, 7>(A, it, Qu); break;
        default: run_item<MODE, 8>(A, it, Qu); break;
      }
      i = queue_advance(Qu);
      ok = i < total && decode_item<MODE>(A, i, sh_tiles, tiles, it);
    }
  }
}

inline int persistent_grid(int max_items) {
  const int slots = device_cu_count() * 2;  // two 78-KiB-LDS workgroups fit one CU
  return max_items < slots ? (max_items > 0 ? max_items : 1) : slots;
}

}  // namespace apq
}  // namespace moeapq
