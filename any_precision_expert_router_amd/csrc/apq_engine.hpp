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
// next to the lane offset.  The products use v_dot2_f32_f16 (two MACs, fp32 accumulate) against
// the token activations, which are uniform across the wavefront and so read through the scalar
// unit.  Weights are never expanded to a dense matrix in memory.
#pragma once
#include "internal.hpp"

namespace moeapq {
namespace apq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Address-space qualified views: plane and LUT reads are per-lane global loads; activation rows
// and the routing arrays, read at wavefront-uniform addresses and never written during the
// kernel, go through the scalar unit as constant-space loads.
#define AS_GLOBAL __attribute__((address_space(1)))
#define AS_CONST __attribute__((address_space(4)))
#define MOE_INLINE __device__ __attribute__((always_inline)) inline

template <class T>
MOE_INLINE const AS_GLOBAL T* gview(const void* p) { return (const AS_GLOBAL T*)p; }
template <class T>
MOE_INLINE const AS_CONST T* cview(const void* p) { return (const AS_CONST T*)p; }

constexpr int kThreads = 64 * kWavesPerTile;
constexpr int kMaxTokGroup = 16;                 // tokens sharing one pass over the weights
constexpr int kTblWords = 256 * 64;              // [256 entries][64 lanes] uint32
constexpr int kRawWords = 16 * 64 / 2;           // PAIR staging: [16 entries][64 lanes] fp16
constexpr int kRedWords = (kWavesPerTile - 1) * kMaxTokGroup * 64;
constexpr int kLdsWords = kTblWords + kRawWords + kRedWords;

// The only LDS object of the tile kernels, so the table starts at LDS address 0 and a table
// address is exactly entry*256 + lane*4.
static __shared__ uint32_t g_lds[kLdsWords];

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
  // the masks of planes 0..7 partition the word, so a chain of bit-field inserts merges them
  uint32_t z = w[Q - 1] & plane_mask(Q - 1, o);
#pragma unroll
  for (int p = Q - 2; p >= 0; --p) z = bfi(plane_mask(p, o), w[p], z);
  return rot(z, 8 - Q - o);
}

// Byte b of the result = idx(8b + 2j) << 4 | idx(8b + 2j + 1)   (q <= 4).
template <int Q>
MOE_INLINE uint32_t pair_word(const uint32_t (&w)[Q], int j) {
  uint32_t z = w[Q - 1] & (plane_mask(Q - 1, j) | plane_mask(Q - 1, j + 4));
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

MOE_INLINE float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w), __builtin_bit_cast(half2_t, x),
                                acc, false);
}

MOE_INLINE int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

MOE_INLINE uint32_t word_of(const u32x4& v, int jw) {
  return jw == 0 ? v.x : jw == 1 ? v.y : jw == 2 ? v.z : v.w;
}

// One wavefront's share of the columns of a row tile: acc[t] += sum_c W[row(lane), c] x_t[c].
//   pbase: this lane's 16-byte unit of plane 0 in chunk 0; plane_u4: 16-byte units per plane.
//   xr[t]: token t's activation row as dwords (two fp16), wavefront-uniform.
template <int Q, int NT>
MOE_INLINE void tile_columns(const AS_GLOBAL u32x4* pbase, size_t plane_u4, int c_begin, int c_end,
                             const AS_CONST uint32_t* const (&xr)[NT], uint32_t lane4,
                             float (&acc)[NT]) {
  if (c_begin >= c_end) return;
  u32x4 cur[Q], nxt[Q];
#pragma unroll
  for (int p = 0; p < Q; ++p) cur[p] = pbase[p * plane_u4 + static_cast<size_t>(c_begin) * 64];
  for (int c4 = c_begin; c4 < c_end; ++c4) {
    const bool more = c4 + 1 < c_end;
    if (more) {
#pragma unroll
      for (int p = 0; p < Q; ++p) nxt[p] = pbase[p * plane_u4 + static_cast<size_t>(c4 + 1) * 64];
    }
#pragma unroll
    for (int jw = 0; jw < 4; ++jw) {
      uint32_t w[Q];
#pragma unroll
      for (int p = 0; p < Q; ++p) w[p] = word_of(cur[p], jw);
      const int xoff = c4 * 64 + jw * 16;  // dword offset of this word's 32 columns
      uint32_t wv[16];                     // packed (even, odd) weights, dword d = 4b + j
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
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int d = 0; d < 16; ++d) acc[t] = dot2(wv[d], xr[t][xoff + d], acc[t]);
      }
    }
    if (more) {
#pragma unroll
      for (int p = 0; p < Q; ++p) cur[p] = nxt[p];
    }
  }
}

struct Item {
  const uint32_t* planes;
  const uint16_t* lut;
  int rows, cols;
  int r0;        // first row of the tile (first gate row for gate_up)
  int row_hi;    // row of lane 32 (gate_up: first up row)
  int n;         // tokens routed to the tile
  int src_base;  // sorted position of the expert's first pair (routed), 0 (shared/plain)
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
};

// Build the row tile's lookup table in LDS: [entry][lane] 4-byte slots.
//   PAIR  (q <= 4): entry (a << 4 | b) = LUT_row[a] | LUT_row[b] << 16.
//   SINGLE (q >= 5): entry v = LUT_row[v] in both halves.
template <int Q>
MOE_INLINE void build_table(const uint16_t* lut, int row_lo, int row_hi) {
  const int tid = threadIdx.x;
  constexpr int NE = 1 << Q;
  constexpr int kPer = NE >= 8 ? 8 : NE;   // LUT entries one thread moves per step
  constexpr int kChunks = NE / kPer;
  uint16_t* raw = reinterpret_cast<uint16_t*>(g_lds + kTblWords);
  const AS_GLOBAL uint16_t* L = gview<uint16_t>(lut);
  for (int i = tid; i < 64 * kChunks; i += kThreads) {
    const int l = i & 63, ch = i >> 6;
    const int row = l < 32 ? row_lo + l : row_hi + (l - 32);
    const AS_GLOBAL uint16_t* src = L + static_cast<size_t>(row) * NE + ch * kPer;
    uint16_t v[8];
    if constexpr (NE >= 8) {
      const u32x4 u = *reinterpret_cast<const AS_GLOBAL u32x4*>(src);
      v[0] = u.x & 0xffff; v[1] = u.x >> 16; v[2] = u.y & 0xffff; v[3] = u.y >> 16;
      v[4] = u.z & 0xffff; v[5] = u.z >> 16; v[6] = u.w & 0xffff; v[7] = u.w >> 16;
    } else {
#pragma unroll
      for (int m = 0; m < kPer; ++m) v[m] = src[m];
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int e = ch * kPer + m;
      if constexpr (Q <= 4) raw[e * 64 + l] = v[m];
      else g_lds[e * 64 + l] = static_cast<uint32_t>(v[m]) * 0x00010001u;
    }
  }
  if constexpr (Q <= 4) {
    __syncthreads();
    for (int i = tid; i < NE * NE * 64; i += kThreads) {
      const int l = i & 63, e = i >> 6;
      const int a = e >> Q, b = e & (NE - 1);
      g_lds[((a << 4) | b) * 64 + l] =
          static_cast<uint32_t>(raw[a * 64 + l]) | (static_cast<uint32_t>(raw[b * 64 + l]) << 16);
    }
  }
}

template <int MODE, int Q, int NT>
MOE_INLINE void run_group(const KArgs& A, const Item& it, int g0, int ng) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);  // uniform per wavefront
  const int C = it.cols;
  // --- the activation rows of the group's tokens (uniform); padding slots repeat slot 0 ---
  const AS_CONST uint32_t* xr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tt = g0 + (t < ng ? t : 0);
    const uint16_t* row;
    if constexpr (MODE == kGateUp) {
      const int tok = it.shared ? tt : uniform(cview<int32_t>(A.pairs)[it.src_base + tt]) / A.k;
      row = A.x + static_cast<size_t>(tok) * C;
    } else if constexpr (MODE == kDown) {
      row = it.shared ? A.act_shared + static_cast<size_t>(tt) * C
                      : A.act + static_cast<size_t>(it.src_base + tt) * C;
    } else {
      row = A.x + static_cast<size_t>(tt) * C;
    }
    xr[t] = cview<uint32_t>(row);
  }
  // --- this lane's row and its first plane unit ---
  const int row = lane < 32 ? it.r0 + lane : it.row_hi + (lane - 32);
  const int nc4 = C / kColChunk;
  const AS_GLOBAL u32x4* pbase = gview<u32x4>(it.planes) +
                                 static_cast<size_t>(row / kRowPanel) * nc4 * 64 + (row % kRowPanel);
  const size_t plane_u4 = static_cast<size_t>(it.rows) * C / 128;
  const int c_begin = (nc4 * wave) / kWavesPerTile, c_end = (nc4 * (wave + 1)) / kWavesPerTile;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  tile_columns<Q, NT>(pbase, plane_u4, c_begin, c_end, xr, static_cast<uint32_t>(lane) * 4u, acc);

  // --- cross-wavefront reduction in a fixed order: wave 0 + 1 + 2 + 3 ---
  float* red = reinterpret_cast<float*>(g_lds + kTblWords + kRawWords);
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((wave - 1) * kMaxTokGroup + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
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
          const float a = h / (1.0f + expf(-h)) * up;  // SiLU(gate) * up
          const int Iw = it.shared ? A.I_shared : A.I;
          uint16_t* dst = it.shared ? A.act_shared + static_cast<size_t>(g0 + t) * Iw
                                    : A.act + static_cast<size_t>(it.src_base + g0 + t) * Iw;
          dst[it.r0 + lane] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(a));
        }
      } else if constexpr (MODE == kDown) {
        if (t < ng) {
          if (it.shared) {
            const float s = A.shared_scale ? cview<float>(A.shared_scale)[g0 + t] : 1.0f;
            A.part_shared[static_cast<size_t>(g0 + t) * A.H + it.r0 + lane] = s * h;
          } else {
            const int p = uniform(cview<int32_t>(A.pairs)[it.src_base + g0 + t]);
            A.part[static_cast<size_t>(p) * A.H + it.r0 + lane] = cview<float>(A.gates)[p] * h;
          }
        }
      } else {
        if (t < ng) A.y_plain[static_cast<size_t>(g0 + t) * it.rows + it.r0 + lane] = h;
      }
    }
  }
  __syncthreads();
}

template <int MODE, int Q>
MOE_INLINE void run_item(const KArgs& A, const Item& it) {
  build_table<Q>(it.lut, it.r0, it.row_hi);
  __syncthreads();
  for (int g0 = 0; g0 < it.n; g0 += kMaxTokGroup) {
    const int ng = min(kMaxTokGroup, it.n - g0);
    if (ng == 1) run_group<MODE, Q, 1>(A, it, g0, ng);
    else if (ng == 2) run_group<MODE, Q, 2>(A, it, g0, ng);
    else if (ng <= 4) run_group<MODE, Q, 4>(A, it, g0, ng);
    else if (ng <= 8) run_group<MODE, Q, 8>(A, it, g0, ng);
    else run_group<MODE, Q, 16>(A, it, g0, ng);
  }
}

MOE_INLINE bool block_ok(const moe_apq_block& b, int rows, int cols) {
  const uintptr_t align = reinterpret_cast<uintptr_t>(b.planes) | reinterpret_cast<uintptr_t>(b.lut);
  return b.planes != nullptr && b.lut != nullptr && (align & 15) == 0 && b.rows == rows &&
         b.cols == cols && b.q >= 1 && b.q <= 8 && b.state == MOE_PAGE_GPU;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void apq_tile_kernel(KArgs A) {
  constexpr int kTileRows = MODE == kGateUp ? kGateUpTileRows : kRowPanel;
  // item list: shared-expert tiles first (they carry every token), then routed tiles
  int sh_tiles = 0, tiles = 0, n_routed = 0;
  if constexpr (MODE == kPlain) {
    tiles = A.plain.rows / kRowPanel;
    n_routed = 1;
  } else {
    if (A.shared) sh_tiles = (MODE == kGateUp ? A.I_shared : A.H) / kTileRows;
    tiles = (MODE == kGateUp ? A.I : A.H) / kTileRows;
    n_routed = uniform(cview<int32_t>(A.n_active)[0]);
  }
  const int total = sh_tiles + n_routed * tiles;
  for (int i = blockIdx.x; i < total; i += gridDim.x) {
    Item it;
    moe_apq_block b;
    int expert = -1, inter = 0;
    if constexpr (MODE == kPlain) {
      b = A.plain;
      it.r0 = i * kRowPanel;
      it.n = A.T;
      it.src_base = 0;
      it.shared = false;
    } else if (i < sh_tiles) {
      b = A.shared[MODE];
      it.shared = true;
      it.r0 = i * kTileRows;
      it.n = A.T;
      it.src_base = 0;
      inter = A.I_shared;
    } else {
      const int a = (i - sh_tiles) / tiles, tile = (i - sh_tiles) - a * tiles;
      expert = uniform(cview<int32_t>(A.active)[a]);
      b = A.table[expert * 2 + MODE];
      it.shared = false;
      it.r0 = tile * kTileRows;
      it.src_base = uniform(cview<int32_t>(A.offsets)[expert]);
      it.n = uniform(cview<int32_t>(A.offsets)[expert + 1]) - it.src_base;
      inter = A.I;
    }
    it.row_hi = MODE == kGateUp ? inter + it.r0 : it.r0 + 32;
    if constexpr (MODE != kPlain) {
      const int want_rows = MODE == kGateUp ? 2 * inter : A.H;
      const int want_cols = MODE == kGateUp ? A.H : inter;
      if (!block_ok(b, want_rows, want_cols)) {
        if (threadIdx.x == 0) {
          atomicOr(&A.err[0], 1);
          A.err[1] = expert;
          A.err[2] = MODE;
        }
        continue;
      }
    }
    it.planes = b.planes;
    it.lut = b.lut;
    it.rows = b.rows;
    it.cols = b.cols;
    switch (b.q) {
      case 1: run_item<MODE, 1>(A, it); break;
      case 2: run_item<MODE, 2>(A, it); break;
      case 3: run_item<MODE, 3>(A, it); break;
      case 4: run_item<MODE, 4>(A, it); break;
      case 5: run_item<MODE, 5>(A, it); break;
      case 6: run_item<MODE, 6>(A, it); break;
      case 7: run_item<MODE, 7>(A, it); break;
      default: run_item<MODE, 8>(A, it); break;
    }
  }
}

inline int persistent_grid(int max_items) {
  const int slots = device_cu_count() * 2;  // two 78-KiB-LDS workgroups fit one CU
  return max_items < slots ? (max_items > 0 ? max_items : 1) : slots;
}

}  // namespace apq
}  // namespace moeapq
