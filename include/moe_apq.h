/*
 * moe_apq.h -- C ABI of the decode-time Mixture-of-Experts layer over Any-Precision weights,
 * native to AMD MI355X (gfx950).
 *
 * The layer: router logits -> softmax + top-k per token -> tokens grouped by expert -> one fused
 * expert FFN (gate_up, SiLU(gate) * up, down, gate-weighted combine) whose weights are held as
 * superposed bit-planes plus a per-row lookup table (LUT), with its own committed bit width per
 * (expert, module) linear block.
 *
 * Sources: PagedWeight, Key Components 1 (Paged Weight Representation): weights are managed per
 * linear block identified by (layer, expert, gate_up|down), held in the Any-Precision bit-plane +
 * LUT format, with a desired width d_i and a committed width q_i per block in a weight page table
 * and pages that are GPU-resident, CPU-resident or in transfer.  PagedWeight, Key Components 3: one
 * fused kernel reads the planes and LUTs directly and mixes blocks of different widths.  LYNX,
 * 1 Problem statement and 2.2 System Components: each token picks its own top-k experts, every
 * token activates exactly k experts, decode cost follows the number of distinct experts a batch
 * activates.  "Which Expert Misses Are Worth Waiting For?", Methodology: the router's first choice
 * and normalised gate weights.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every device call is
 *     asynchronous on `stream`; none reads device memory back to the host, so a sequence of calls
 *     can be captured in a HIP graph.
 *   - The caller owns every buffer (inputs, outputs, workspace).  Nothing is allocated or freed
 *     inside a call, and no state is kept between calls (except the optional profiler below).
 *   - Return value: MOE_OK (0) or a negative MOE_E* code; moe_last_error() then gives a message
 *     (thread-local).  Arguments are validated from host-visible scalars only.  No C++ exception
 *     crosses the ABI.
 *   - Numbers: fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 */
#ifndef MOE_APQ_H
#define MOE_APQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* bad scalar argument (k > E, bad shape, q outside 1..8, NULL) */
#define MOE_EUNSUPPORTED (-2) /* outside the instantiated bounds below, or an activation array
                                 (x [T][H], act [T*k][I], act_shared [T][I_shared]) of 4 GiB or
                                 more: the kernels address them with 32-bit byte offsets        */
#define MOE_EWORKSPACE (-3)   /* workspace missing or smaller than moe_workspace_bytes()       */
#define MOE_EHIP (-4)         /* a HIP launch or runtime call failed                           */
#define MOE_EDEVICE (-5)      /* a kernel found an invalid block descriptor (see below)        */

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_TOKENS 65536

/* Substitution policies of moe_substitute ("Which Expert Misses Are Worth Waiting For?"). */
#define MOE_POLICY_FETCH_ALL 0     /* fetch every miss (no substitution)                     */
#define MOE_POLICY_GATE_RULE 1     /* fetch a miss if first choice or gate >= gate_threshold */
#define MOE_POLICY_FIRST_CHOICE 2  /* fetch a miss only if it is the first choice            */

/* Page states of the weight page table (PagedWeight, Key Components 1). */
#define MOE_PAGE_GPU 0
#define MOE_PAGE_CPU 1
#define MOE_PAGE_IN_TRANSFER 2

/*
 * One weight-page-table entry = one (expert, module) linear block, rows x cols, read as
 * y_r = sum_c W[r, c] x_c with W[r, c] = LUT_r[ idx_q(r, c) ].
 *
 *   gate_up block: rows = 2*I, cols = H; rows 0..I-1 are the gate projection, I..2I-1 the up one.
 *   down block:    rows = H,   cols = I.
 *   Shape rules:   rows % 64 == 0, cols % 128 == 0.
 *
 * planes: q bit-planes of the 8-bit parent index, plane p (0 <= p < q) holding bit 7-p, so the
 *   q-bit index is the top-q-bit prefix of the parent index and lowering q only drops trailing
 *   planes (no re-encoding).  Plane p is rows*cols/8 bytes at byte offset p*rows*cols/8.  Inside
 *   a plane, the 16-byte unit of (row panel P = r/64, column chunk c4 = c/128, row-in-panel
 *   l = r%64) sits at byte ((P*(cols/128) + c4)*64 + l)*16 and holds four little-endian words;
 *   word j covers columns c4*128 + 32j + [0, 32), column c of a word (0..31) at bit
 *   (8*(c/8) + 7 - p - o(c)) mod 32 with o(c) = ((c >> 1) & 3) + 4*(c & 1).  (So one wavefront
 *   reads a row panel with 1-KiB coalesced loads and every lane owns one row.)  Write them with
 *   moe_apq_pack().
 * lut: fp16 [rows][2^q] row-major, entry v of row r = weight value of q-bit index v.
 * q: committed width q_i, 1..8.  desired: d_i, carried, not read here.  state: must be
 *   MOE_PAGE_GPU for every block a call reads (precondition; see MOE_EDEVICE).
 * The table is an immutable snapshot for the duration of a call: width commits and page moves
 * happen between calls, at safe boundaries (PagedWeight, Key Components 3).
 */
typedef struct moe_apq_block {
  const uint32_t* planes;
  const uint16_t* lut;
  int32_t rows;
  int32_t cols;
  uint8_t q;
  uint8_t desired;
  uint8_t state;
  uint8_t reserved0;
  int32_t reserved1;
} moe_apq_block; /* 32 bytes */

/*
 * Softmax + top-k per token (LYNX 2.2; "Which Expert Misses...", Methodology).
 *   logits     fp32 [T][E], finite (NaN/inf: undefined result).
 *   topk_ids   out int32 [T][k]: the k largest logits ordered by (logit desc, expert id asc);
 *              -0.0 == +0.0, so equal values tie to the lower id.  Slot 0 is the first choice.
 *   topk_gates out fp32 [T][k]: softmax over the k selected logits (the full softmax
 *              renormalised over them); sums to 1 up to fp32 rounding.
 *   Bounds: 1 <= k <= E <= MOE_MAX_EXPERTS, k <= MOE_MAX_TOPK, 0 <= T <= MOE_MAX_TOKENS (T = 0 is
 *   a no-op).
 */
int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_gates,
                   void* stream);

/*
 * Group the T*k (token, slot) pairs p = t*k + j by expert (LYNX 1: the set of distinct experts is
 * what a decode batch loads).  Stable counting sort.
 *   topk_ids       int32 [T][k].  Routing output names k distinct experts in [0, E) per token;
 *                  other ids are accepted with a defined result: a pair whose id is outside
 *                  [0, E) names no expert and is not placed, and a token that names one expert
 *                  in several slots has each of those pairs placed (in slot order).
 *   expert_offsets out int32 [E+1]: expert e's pairs are sorted_pairs[offsets[e] .. offsets[e+1]);
 *                  offsets[E] = number of placed pairs (T*k when every id is in [0, E)).
 *   sorted_pairs   out int32 [T*k]: pair ids, expert ascending, p ascending inside an expert;
 *                  entries from offsets[E] on are not written.
 *   active_experts out int32 [E]: experts with >= 1 pair, ascending, then -1 padding.
 *   n_active       out int32 [1].
 *   workspace/ws_bytes: unused (may be NULL/0); kept for ABI stability.
 */
int moe_group_by_expert(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                        int32_t* sorted_pairs, int32_t* active_experts, int32_t* n_active,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * The fused Any-Precision expert FFN over the grouped tokens (PagedWeight, Key Components 3):
 *   for every active expert e and every pair p routed to it (token t = p / k, slot j = p % k):
 *     h = W_gu(e) x_t;  a = SiLU(h[0:I]) * h[I:2I];  o = W_d(e) a
 *   y_t = fp16( sum_j g_tj o_tj  +  s_t * FFN_shared(x_t) )
 *   table        device moe_apq_block [E][2] (index e*2 + 0 = gate_up, e*2 + 1 = down).  Blocks
 *                may each have a different q.
 *   x            fp16 [T][H].
 *   expert_offsets, sorted_pairs, active_experts, n_active: from moe_group_by_expert, with
 *                every pair placed (every id in [0, E)); a pair left out has no term in y.
 *   topk_gates   fp32 [T][k] from moe_route_topk.
 *   shared       device moe_apq_block [2] (gate_up [2*I_shared x H], down [H x I_shared]) or
 *                NULL (then I_shared is ignored); shared_scale fp32 [T] or NULL (= 1).
 *   prefill_threshold: the token count n_e at or above which an expert's tiles (and the shared
 *                expert's, with n = T) must use the matrix-core (MFMA) product path instead of
 *                the packed-dot VALU path; <= 0 selects no lowering.  By default a tile streams
 *                through the VALU path only when n_e <= 2 on a block of width q <= 4 or n_e = 1
 *                on a wider block (the VALU path's pair tables make q <= 4 cheap to decode), so
 *                a threshold can only lower that switch: 1 sends every tile to the MFMA path, 2
 *                streams single tokens only, and values above 2 change nothing.  Results agree
 *                up to fp32 summation order.
 *   y            out fp16 [T][H].
 *   workspace    >= moe_workspace_bytes(T, E, H, I, k, I_shared) bytes, 256-byte aligned.
 *   Device checks: a routed block whose descriptor does not match (rows, cols) of its module, has
 *   q outside 1..8 or is not MOE_PAGE_GPU is skipped and recorded in the workspace error word;
 *   moe_check_device_error() reports it.  The skipped expert contributes zero to y (its tokens
 *   keep their other experts' terms), so y stays defined.  Host checks: MOE_EUNSUPPORTED when
 *   T*H, T*k*I or T*I_shared fp16 values reach 4 GiB.  Accuracy: fp32 accumulation, the SiLU-gated activation
 *   rounded once to fp16, y rounded to fp16.
 */
int moe_apq_ffn(const moe_apq_block* table, int E, int H, int I, const uint16_t* x, int T, int k,
                const int32_t* expert_offsets, const int32_t* sorted_pairs,
                const int32_t* active_experts, const int32_t* n_active, const float* topk_gates,
                const moe_apq_block* shared, int I_shared, const float* shared_scale,
                int prefill_threshold, uint16_t* y, void* workspace, size_t ws_bytes,
                void* stream);

/*
 * The whole layer: moe_route_topk + moe_group_by_expert + moe_apq_ffn, with the routing arrays
 * kept inside the workspace.  Same arguments and rules as above.
 */
int moe_layer_forward(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                      const moe_apq_block* table, const moe_apq_block* shared, int I_shared,
                      const float* shared_scale, int prefill_threshold, uint16_t* y,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * The whole layer without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Same arguments and results as moe_layer_forward; the workspace is a fixed device array of
 *   MOE_NOALLOC_WORKSPACE_BYTES inside the library (one per GPU, held until the process ends),
 *   so the call allocates nothing.  A call whose moe_workspace_bytes() exceeds that size is
 *   refused with MOE_EWORKSPACE before anything is issued (every decode shape of the pages'
 *   models fits; a 2048-token prefill chunk does not: use moe_layer_forward).
 *   status: device int32 [1] or NULL.  The call clears its device error word when it starts and
 *   writes it to *status when it ends (0 = clean; nonzero = a routed block was skipped, as
 *   moe_check_device_error reports for moe_layer_forward).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 *   other threads) race and their results are undefined; order them on one stream.  The array
 *   keeps the last call's contents.  Errors: as moe_layer_forward, MOE_EWORKSPACE above the limit,
 *   MOE_EHIP if the array's device address cannot be obtained.
 */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
int moe_layer_forward_noalloc(const float* logits, const uint16_t* x, int T, int E, int H, int I, int k,
                              const moe_apq_block* table, const moe_apq_block* shared, int I_shared,
                              const float* shared_scale, int prefill_threshold, uint16_t* y,
                              int32_t* status, void* stream);

/* Workspace bytes moe_apq_ffn / moe_layer_forward need for these sizes (0 on bad arguments). */
size_t moe_workspace_bytes(int T, int E, int H, int I, int k, int I_shared);

/*
 * Host-side, synchronous: pack logical 8-bit parent indices into the plane layout above.
 *   idx8_host   host uint8 [rows][cols];  planes_host out host uint32 [q * rows * cols / 32].
 *   Only the top q bits of each index are stored.  Packing at q and keeping the first
 *   q' * rows*cols/32 words gives exactly the packing at q' < q.
 */
int moe_apq_pack(const uint8_t* idx8_host, int rows, int cols, int q, uint32_t* planes_host);

/*
 * Debug / parity: the decode GEMV engine alone on one block, no routing.
 *   y[t][r] = sum_c W[r, c] x[t][c] for all T tokens, fp32 accumulate (the same kernel and table
 *   lookups moe_apq_ffn uses, in its plain mode).
 *   blk_host  host pointer to the descriptor (planes/lut are device pointers, 16-byte aligned).
 *   x         fp16 [T][cols];  y out fp32 [T][rows].
 *   dense_threshold: the tile streams through the VALU path when T < dense_threshold (<= 0: no
 *             limit) and T <= 2 (q <= 4) or T = 1 (q >= 5), else takes the matrix-core path,
 *             so that both product paths can be checked on the same block.
 */
int moe_apq_gemv(const moe_apq_block* blk_host, const uint16_t* x, int T, float* y,
                 int dense_threshold, void* stream);

/*
 * Debug / parity: decode one block's q-bit indices on the GPU.
 *   blk_host  host pointer to the descriptor (its planes pointer is a device pointer).
 *   idx_out   device uint8 [rows][cols], row-major.
 */
int moe_apq_decode_indices(const moe_apq_block* blk_host, uint8_t* idx_out, void* stream);

/*
 * Synchronise `stream` and read the device error word that moe_apq_ffn / moe_layer_forward keep
 * in `workspace`: MOE_OK if clean, MOE_EDEVICE (with a message naming the first bad block)
 * otherwise.  Clears the word.
 */
int moe_check_device_error(void* workspace, size_t ws_bytes, void* stream);

/*
 * Optional kernel timer (tracing).  moe_profile_start() makes every later device call on this
 * thread bracket each kernel it launches with HIP events on the call's stream.
 * moe_profile_stop() synchronises those streams, stops recording and returns the number of
 * distinct kernels; for each (up to max_kernels) it writes the name (NUL-terminated, at most 63
 * chars, into names_out + 64*i), the summed milliseconds and the launch count.
 */
int moe_profile_start(void);
int moe_profile_stop(int max_kernels, char* names_out, double* total_ms_out,
                     int32_t* launches_out);

/*
 * Online routing statistics of one call, added to caller-owned accumulators.
 *
 * Source: PagedWeight, Key Components 2 (online routing statistics): an expert's routing mass is
 * how often and with what weight it is selected.  "Which Expert Misses Are Worth Waiting For?",
 * Methodology: the substituted gate mass m is the normalised sum of the gate weights of the
 * substituted experts; here, with every non-resident expert substituted,
 * m = mass_sums[0] / mass_sums[1].
 *
 * Inputs are one call's grouping and gates (device): expert_offsets [E+1] and sorted_pairs [T*k]
 * as written by moe_group_by_expert (or left by moe_layer_forward, see moe_workspace_routing),
 * topk_gates [T*k] fp32 in pair order p = t*k + j.  resident: device uint8 [E], 0 = the expert
 * is not GPU-resident; NULL = all resident.
 * Accumulators (device, caller-owned, never reset by the library -- zero them to start a
 * window; no decay): count [E] uint64 += pairs routed to expert e; mass [E] double += the sum of
 * their gates; mass_sums[0] double += gate mass of pairs whose expert is not resident,
 * mass_sums[1] += the total gate mass (T when every token's gates sum to 1).
 * Sums are taken in double, per expert in ascending pair order, then across experts in a fixed
 * order: the results do not depend on timing.  Calls that share accumulators must be ordered
 * (one stream).  Errors: MOE_EINVAL for bad T/E/k or NULL arguments.
 */
int moe_routing_stats(const int32_t* expert_offsets, const int32_t* sorted_pairs,
                      const float* topk_gates, int T, int k, int E, const uint8_t* resident,
                      uint64_t* count, double* mass, double* mass_sums, void* stream);

/*
 * Device addresses of the routing results that moe_layer_forward leaves in its workspace:
 * topk ids [T*k] int32, gates [T*k] fp32, expert offsets [E+1] int32 and sorted pairs [T*k]
 * int32 (same layouts as moe_route_topk / moe_group_by_expert).  They are valid after the
 * layer call on the workspace's stream and until the workspace is used again.  Host-only: no
 * device access.  The shape arguments are those of moe_workspace_bytes.  Errors: MOE_EINVAL,
 * MOE_EWORKSPACE (workspace NULL or smaller than moe_workspace_bytes()).
 */
int moe_workspace_routing(void* workspace, size_t ws_bytes, int T, int E, int H, int I, int k,
                          int I_shared, int32_t** topk_ids, float** topk_gates,
                          int32_t** expert_offsets, int32_t** sorted_pairs);

/*
 * Residency-aware substitution of routed experts, and background admission.
 *
 * Source: "Which Expert Misses Are Worth Waiting For?", Methodology: a routed expert that is not
 * GPU-resident (a miss) is fetched or substituted by a resident expert according to a policy
 * (MOE_POLICY_*: fetch every miss; the 0.15 rule -- fetch a miss if it is the router's first
 * choice or its gate weight is >= gate_threshold, e.g. 0.15; the first-choice rule); background
 * admission accumulates an expert's substituted gate weight over calls and admits it to the
 * cache once it reaches a threshold (e.g. 0.5).  Readings: slots are processed in order j =
 * 0..k-1; a substituted slot gets the token's highest-logit resident expert not already among
 * its experts (ties: lower id), keeps its gate weight, and each token keeps exactly k distinct
 * experts; a miss with no such expert left is fetched.  Admission adds the gates of the slots
 * substituted away from each expert in pair order (fp32), admits at the threshold and restarts
 * the accumulator at 0.  Runs between moe_route_topk and moe_group_by_expert.
 * Device arguments: logits fp32 [T,E] (finite); resident uint8 [E] (0 = not resident);
 * topk_ids int32 [T,k] (in: routing, out: after substitution); topk_gates fp32 [T,k] (read);
 * missed int32 [T,k] (out: the original expert of a substituted slot, else -1); fetch uint8 [E]
 * (out: 1 = a non-resident expert still routed, to be fetched).  admit_mass float [E]
 * (accumulators, in/out) and admit uint8 [E] (out: admitted this call): both NULL for no
 * admission.  Errors: MOE_EINVAL (bad T/E/k, policy, NULL), MOE_EUNSUPPORTED (bounds).
 */
int moe_substitute(const float* logits, int T, int E, int k, const uint8_t* resident, int policy,
                   float gate_threshold, int32_t* topk_ids, const float* topk_gates,
                   int32_t* missed, uint8_t* fetch, float* admit_mass, float admit_threshold,
                   uint8_t* admit, void* stream);

/*
 * Batch-aware expert remapping onto a critical expert set.
 *
 * Source: LYNX, 2.2 System Components: a confidence analyser cuts each token's router
 * confidence, taken from the gap between the logits of its top-ranked experts, into bins whose
 * width and count are set by the sparsity ratio k/N alone (AffinityBinning); an expert remapper
 * redirects low-affinity token-expert assignments to the surviving critical set of experts, and
 * every token still activates exactly k experts.  Readings: confidence c = l(slot 0) - l(slot 1)
 * in fp32; bin b = min(floor(c / bin_width), ceil(E/k) - 1), at least 0, with the quotient an
 * IEEE fp32 division; a token in bin b keeps its first min(k, b + 1) slots as critical
 * assignments and the critical set is the union of their experts; each other slot whose expert
 * is not critical takes the token's highest-logit critical expert not already among its experts
 * (ties: lower id), slots in order j = 0..k-1, and keeps its gate weight (gates are not touched);
 * with no such expert left it keeps its own.  Runs between moe_route_topk and
 * moe_group_by_expert, like moe_substitute.
 * Device arguments: logits fp32 [T,E] (finite); topk_ids int32 [T,k] (in: routing output in
 * routing order; out: after remapping); remapped int32 [T,k] (out: the original expert of a
 * remapped slot, else -1); critical uint8 [E] (out: 1 = expert in the critical set).  bin_width
 * is a host scalar; bin_width <= 0 selects the page's default, k/E computed as one fp32
 * division (float)k / (float)E.  One workgroup; nothing is allocated.
 * Errors: MOE_EINVAL (bad T/E/k, bin_width NaN or infinite, NULL), MOE_EUNSUPPORTED (bounds),
 * MOE_EHIP.
 */
int moe_lynx_remap(const float* logits, int T, int E, int k, float bin_width, int32_t* topk_ids,
                   int32_t* remapped, uint8_t* critical, void* stream);

/*
 * Commit new descriptors into the device weight page table, in stream order.
 *
 * Source: PagedWeight, Key Components 1 (a committed width q_i per block in the page table) and
 * Key Components 3 (bit-width commits are applied only at safe boundaries, once a plan has run).
 * Every call issued earlier on `stream` uses the old descriptors, every later one the new
 * ones.  Lowering a block's width is a commit of the same planes pointer with a smaller q (the
 * planes of width q' are the first q' planes) and the LUT of width q'; raising it is a commit
 * after the missing planes and the new LUT have been copied in (e.g. an asynchronous copy from
 * pinned host memory on another stream, which `stream` waits for with an event).
 * table: device page table of table_len entries (2*E for a layer's [E][2] table, 2 for a shared
 * pair); index (host) [n]: entries to overwrite, each in [0, table_len) and none repeated;
 * desc (host) [n]: the new descriptors, copied by value into the launch (both host arrays may
 * be reused on return).  Nothing is allocated on the device.  Errors: MOE_EINVAL (n < 0,
 * table_len <= 0, NULL, an index outside the table or repeated, q outside 1..8, rows % 64 or
 * cols % 128), MOE_EHIP.  For page moves (offload to the host, reload from it) see
 * moe_page_offload / moe_page_reload, which commit through this same stream-ordered write.
 */
int moe_commit_blocks(moe_apq_block* table, int table_len, const int32_t* index,
                      const moe_apq_block* desc, int n, void* stream);

/*
 * Asynchronous page movement between device and host memory.
 *
 * Source: PagedWeight, Key Components 1 (a block's pages are GPU-resident, CPU-resident or in
 * transfer) and Key Components 3 (offload and reload run asynchronously beside the computation;
 * a changed bit width is committed only at a safe boundary).  Because the q-bit planes are a
 * prefix of the wider ones, lowering a width drops trailing planes and raising it copies only
 * the missing ones.
 *
 * Both calls take the page table (device, table_len entries) and the entry `index`, the entry's
 * descriptor as committed now (`current`, host) and the one to commit (`target`, host), a
 * caller-owned hipEvent_t `copy_event`, a side stream `copy_stream` for the copies and the
 * compute `stream` on which the layer calls run.  Host buffers are pinned host memory
 * (hipHostMalloc) holding the planes plane-major as moe_apq_pack writes them (plane p at byte
 * p*rows*cols/8) and the LUT [rows][2^q] fp16; pageable memory makes the copies synchronous.
 * Nothing is allocated.  Host-side state rules (checked before anything is issued, MOE_EINVAL):
 *
 * moe_page_reload: target->state is MOE_PAGE_GPU and target has the current shape.
 *   current GPU-resident at width q' (raise the width): target names the same planes, q > q',
 *     and a new LUT buffer; planes q'..q-1 and the LUT are copied; calls issued before the
 *     final commit keep running at width q'.
 *   current MOE_PAGE_CPU (bring back): the entry is committed as MOE_PAGE_IN_TRANSFER on
 *     `stream` first (later calls skip the block and report MOE_EDEVICE), then all q planes and
 *     the LUT are copied.
 *   current MOE_PAGE_IN_TRANSFER: refused (a reload is already in flight).
 *   Copies run on copy_stream, then copy_event is recorded there.  The call does not commit
 *   target: layer calls issued on `stream` afterwards keep running at width q' (or skip the
 *   block in transfer) while the copy proceeds beside them.
 * moe_page_commit: the safe boundary of a reload.  `stream` waits for copy_event, then target
 *   (the descriptor given to the moe_page_reload that recorded copy_event; state MOE_PAGE_GPU)
 *   is committed: no call ever reads a width whose planes have not all landed, and every call
 *   issued after it reads the new width.
 * moe_page_offload: current must be MOE_PAGE_GPU.
 *   target MOE_PAGE_CPU (evict): all planes and the LUT are copied to host_planes / host_lut
 *     (each may be NULL when the host already holds them).
 *   target MOE_PAGE_GPU with the same planes and 1 <= q < q' (lower the width; its LUT of width
 *     q must be on the device already): planes q..q'-1 go to host_planes (may be NULL).
 *   The commit of target is issued on `stream` first; the copies wait for every call issued
 *   before it, so once copy_event has completed the host copies are whole and the device memory
 *   that left may be reused.
 * Errors: MOE_EINVAL (the rules above, NULL, index outside the table, bad shape or q), MOE_EHIP.
 */
int moe_page_reload(moe_apq_block* table, int table_len, int index, const moe_apq_block* current,
                    const moe_apq_block* target, const void* host_planes, const void* host_lut,
                    void* copy_event, void* copy_stream, void* stream);
int moe_page_commit(moe_apq_block* table, int table_len, int index, const moe_apq_block* target,
                    void* copy_event, void* stream);
int moe_page_offload(moe_apq_block* table, int table_len, int index, const moe_apq_block* current,
                     const moe_apq_block* target, void* host_planes, void* host_lut, void* copy_event,
                     void* copy_stream, void* stream);

/*
 * Greedy bit-width plan (host, synchronous; no device access).
 *
 * Source: PagedWeight, Key Components 2 (quality-aware runtime planner: damage scores of
 * bit-width reductions; when a memory target must be met, the reductions of lowest damage per
 * byte saved are taken greedily; frequently routed experts get width floors and damage
 * multipliers).  Readings: a reduction is one step q -> q-1 of one block, allowed while
 * q-1 >= q_floor; its cost is mult * (damage(q-1) - damage(q)) / (bytes the step frees), in
 * double; the cheapest is taken (ties: lower block index) until the bytes freed reach
 * target_bytes or no step is left.  A block's bytes at width q: rows*cols*q/8 + rows*2^q*2.
 * Inputs (host) [n]: q_cur (1..8), q_floor (1..q_cur), rows (% 64), cols (% 128), mult (> 0);
 * damage [n*8]: damage[i*8 + w-1] = score of block i at width w.  Outputs: q_new [n],
 * *bytes_saved.  Errors: MOE_EINVAL.
 */
int moe_plan_widths(int n, const uint8_t* q_cur, const uint8_t* q_floor, const int32_t* rows,
                    const int32_t* cols, const float* damage, const float* mult,
                    int64_t target_bytes, uint8_t* q_new, int64_t* bytes_saved);

/*
 * Diagnostic: read `bytes` of device memory at `buf` once, with the access pattern that streams
 * fastest on this device (every wavefront reads one contiguous run in 1-KiB non-temporal loads,
 * 16 in flight), and XOR every 32-bit word of it into `*sink` (device, 4 bytes, stream-ordered
 * atomic: the caller clears it first to read the XOR of the buffer).  bytes must be a positive
 * multiple of 1024, at most 2^40, and buf 16-byte aligned; otherwise MOE_EINVAL and nothing is
 * launched.  Timing this call gives the achievable HBM read rate that the layer's bandwidth is
 * compared with.
 */
int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_APQ_H */
