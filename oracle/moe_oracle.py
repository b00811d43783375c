"""CPU oracle of the decode-time MoE layer over Any-Precision bit-plane weights.

TEST INFRASTRUCTURE -- not part of the product path.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import or call
anything in ``oracle/``.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators) and imports nothing from it; the only thing both sides
take is the seeded inputs from ``workloads``.

It is the plain, slow definition of what the layer computes, in float64 NumPy:

1. ``route_topk``   per token, the k largest router logits ordered by (logit desc, id asc);
                    gates = softmax over those k logits.  Every token activates exactly k
                    experts (LYNX, 2.2 System Components, expert remapper keeps top-k
                    semantics); slot 0 is the router's first choice and gate weights are
                    normalised quantities ("Which Expert Misses Are Worth Waiting For?",
                    Methodology: the 0.15 rule and the first-choice rule).
2. ``group_by_expert`` the (token, slot) pairs p = t*k + j grouped by expert, expert
                    ascending, p ascending inside an expert (stable); the set of distinct
                    experts is what the batch must load (LYNX, 1 Problem statement).
3. ``unpack_planes`` / ``dequantize``  the Any-Precision weight of one (expert, module)
                    linear block: superposed bit-planes plus a per-row lookup table, at the
                    block's committed width q (PagedWeight, Key Components 1: Paged Weight
                    Representation -- blocks per (layer, expert, gate_up|down), bit-plane + LUT
                    format, committed width q_i per block in the weight page table).
4. ``expert_ffn``   gate_up -> SiLU(gate) * up -> down for the tokens routed to one expert.
5. ``layer_forward`` the gate-weighted combine y_t = sum_j g_tj o_tj, plus an optional
                    always-on shared expert (PagedWeight, Key Components 3: one fused kernel
                    reads the planes and LUTs of blocks of different widths).
6. ``routing_stats`` per-expert selection count and routing mass of a call, and the gate mass
                    on non-resident experts (PagedWeight, Key Components 2; "Which Expert
                    Misses Are Worth Waiting For?", Methodology: substituted gate mass).
7. ``plan_widths``  the greedy width planner: lowest damage per byte saved until a memory
                    target is met (PagedWeight, Key Components 2).
8. ``substitute`` / ``admit``  residency-aware substitution (fetch every miss, the 0.15 rule,
                    the first-choice rule) and background admission ("Which Expert Misses
                    Are Worth Waiting For?", Methodology).
9. ``lynx_bins`` / ``lynx_remap``  confidence bins from the top-logit gap and batch-aware
                    remapping of low-affinity slots onto the critical expert set (LYNX, 2.2
                    System Components).

Readings where the pages are silent (all listed in the design notes of the repository):
the parent width is 8 bits and plane p holds bit 7-p of the parent index, so the q-bit index
is the top-q-bit prefix idx8 >> (8-q); the LUT of a row has 2**q fp16 entries indexed by that
prefix; gate_up is one [2I x H] block whose rows 0..I-1 are the gate and I..2I-1 the up
projection; SiLU(z) = z / (1 + e^-z); the shared expert is added with weight 1 (or a given
per-token scale).

Physical bit-plane layout (a choice of this library, fixed for every width so that lowering
q only drops trailing planes):
  * a block of R rows x C columns needs R % 64 == 0 and C % 128 == 0;
  * plane p (0 <= p < q) occupies R*C/8 bytes; plane p starts at byte p*R*C/8;
  * inside a plane, rows form panels of 64 and columns form chunks of 128; the 16-byte unit
    of (panel P, chunk c4, row-in-panel l) starts at byte ((P*(C/128) + c4)*64 + l)*16 and
    holds 4 little-endian 32-bit words, word j covering columns c4*128 + 32*j + [0, 32);
  * inside a word, column c (0..31) sits at bit (8*(c//8) + 7 - p - o(c)) mod 32 with
    o(c) = ((c >> 1) & 3) + 4*(c & 1).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` (brute force,
closed forms, invariants, library routines); nothing is "parity unpinned" except behaviour
on real checkpoints, which the container does not have.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

PARENT_BITS = 8
ROW_PANEL = 64
COL_CHUNK = 128
GATE_UP = 0
DOWN = 1


# --------------------------------------------------------------------------------------------
# 1. Routing: softmax + top-k
# --------------------------------------------------------------------------------------------
def route_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts per token and their gate weights.

    ids[t]   : the k experts with the largest logits, ordered by (logit descending, expert id
               ascending); -0.0 and +0.0 are equal and so tie to the lower id.
    gates[t] : g_j = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0) in float64, i.e. the full
               softmax renormalised over the selected experts; it sums to 1.
    """
    logits = np.asarray(logits)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(logits)):
        raise ValueError("router logits must be finite")
    l64 = logits.astype(np.float64)
    ids = np.zeros((T, k), dtype=np.int32)
    gates = np.zeros((T, k), dtype=np.float64)
    expert_ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert_ids, -l64[t]))  # last key is primary: -logit, then id
        sel = order[:k]
        ids[t] = sel
        z = np.exp(l64[t, sel] - l64[t, sel[0]])
        gates[t] = z / z.sum()
    return ids, gates


# --------------------------------------------------------------------------------------------
# 2. Grouping tokens by expert
# --------------------------------------------------------------------------------------------
def group_by_expert(ids: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """CSR of the pairs p = t*k + j by expert.

    offsets[e]..offsets[e+1] bounds expert e's pairs inside ``pairs``; pairs ascend inside an
    expert; ``active`` lists the experts with at least one pair in ascending order (padded
    with -1 to length E); n_active is their count.
    """
    flat = np.asarray(ids).reshape(-1)
    offsets = np.zeros(E + 1, dtype=np.int32)
    chunks = []
    active = []
    for e in range(E):
        pe = np.flatnonzero(flat == e).astype(np.int32)
        chunks.append(pe)
        offsets[e + 1] = offsets[e] + len(pe)
        if len(pe):
            active.append(e)
    pairs = np.concatenate(chunks) if chunks else np.zeros(0, dtype=np.int32)
    act = np.full(E, -1, dtype=np.int32)
    act[: len(active)] = active
    return offsets, pairs.astype(np.int32), act, len(active)


# --------------------------------------------------------------------------------------------
# 3. Any-Precision block: bit-planes + per-row LUT
# --------------------------------------------------------------------------------------------
def bit_position(p: int, c: np.ndarray) -> np.ndarray:
    """Bit of plane p's 32-bit word that holds column c (0..31) of that word."""
    c = np.asarray(c)
    o = ((c >> 1) & 3) + 4 * (c & 1)
    return (8 * (c // 8) + 7 - p - o) % 32


def _plane_words_as_matrix(words: np.ndarray, R: int, C: int) -> np.ndarray:
    """One plane's words (flat, storage order) -> [R, C/32] with word (r, w) for columns 32w.."""
    u = words.reshape(R // ROW_PANEL, C // COL_CHUNK, ROW_PANEL, 4)
    return u.transpose(0, 2, 1, 3).reshape(R, C // 32)


def _matrix_as_plane_words(mat: np.ndarray, R: int, C: int) -> np.ndarray:
    u = mat.reshape(R // ROW_PANEL, ROW_PANEL, C // COL_CHUNK, 4)
    return np.ascontiguousarray(u.transpose(0, 2, 1, 3)).reshape(-1)


def check_block_dims(R: int, C: int) -> None:
    if R <= 0 or C <= 0 or R % ROW_PANEL or C % COL_CHUNK:
        raise ValueError("block needs rows % 64 == 0 and cols % 128 == 0")


def pack_planes(idx8: np.ndarray, q: int) -> np.ndarray:
    """Oracle's own writer of the plane layout: uint32 [q * R * C / 32]."""
    R, C = idx8.shape
    check_block_dims(R, C)
    if not 1 <= q <= PARENT_BITS:
        raise ValueError("q must be in 1..8")
    idx8 = idx8.astype(np.uint32).reshape(R, C // 32, 32)
    out = []
    cols = np.arange(32)
    for p in range(q):
        bit = (idx8 >> (PARENT_BITS - 1 - p)) & 1                     # [R, C/32, 32]
        word = (bit << bit_position(p, cols).astype(np.uint32)).sum(axis=2, dtype=np.uint64)
        out.append(_matrix_as_plane_words(word.astype(np.uint32), R, C))
    return np.concatenate(out).astype(np.uint32)


def unpack_planes(planes: np.ndarray, R: int, C: int, q: int) -> np.ndarray:
    """Oracle's own reader: the q-bit index of every weight, uint8 [R, C]."""
    check_block_dims(R, C)
    planes = np.asarray(planes).view(np.uint32).reshape(-1)
    per_plane = R * C // 32
    if planes.size < q * per_plane:
        raise ValueError("not enough plane words for this width")
    idx = np.zeros((R, C // 32, 32), dtype=np.uint32)
    cols = np.arange(32)
    for p in range(q):
        mat = _plane_words_as_matrix(planes[p * per_plane:(p + 1) * per_plane], R, C)
        bit = (mat[:, :, None] >> bit_position(p, cols)[None, None, :].astype(np.uint32)) & 1
        idx |= bit << (q - 1 - p)
    return idx.reshape(R, C).astype(np.uint8)


def committed_index(idx8: np.ndarray, q: int) -> np.ndarray:
    """The q-bit index is the top-q-bit prefix of the 8-bit parent index."""
    return (np.asarray(idx8) >> (PARENT_BITS - q)).astype(np.uint8)


def dequantize(idx_q: np.ndarray, lut: np.ndarray, rows: Optional[slice] = None) -> np.ndarray:
    """W[r, c] = LUT_r[idx_q[r, c]] in float64 (optionally for a row range only)."""
    if rows is not None:
        idx_q, lut = idx_q[rows], lut[rows]
    return np.take_along_axis(lut.astype(np.float64), idx_q.astype(np.int64), axis=1)


def apq_matvec(idx_q: np.ndarray, lut: np.ndarray, X: np.ndarray, row_chunk: int = 4096) -> np.ndarray:
    """Y = W X for X float64 [C, n]; W dequantised in row chunks to bound memory -> [R, n]."""
    R = idx_q.shape[0]
    X = np.asarray(X, dtype=np.float64)
    Y = np.empty((R, X.shape[1]), dtype=np.float64)
    for r0 in range(0, R, row_chunk):
        sl = slice(r0, min(R, r0 + row_chunk))
        Y[sl] = dequantize(idx_q, lut, sl) @ X
    return Y


# --------------------------------------------------------------------------------------------
# 4. Expert FFN
# --------------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(gu_idx_q: np.ndarray, gu_lut: np.ndarray, d_idx_q: np.ndarray, d_lut: np.ndarray,
               X: np.ndarray) -> np.ndarray:
    """FFN of one expert on tokens X [n, H] -> [n, H]: down(SiLU(gate) * up)."""
    I = gu_idx_q.shape[0] // 2
    h = apq_matvec(gu_idx_q, gu_lut, np.asarray(X, dtype=np.float64).T)   # [2I, n]
    act = silu(h[:I]) * h[I:]
    return apq_matvec(d_idx_q, d_lut, act).T                              # [n, H]


# --------------------------------------------------------------------------------------------
# 5. The layer
# --------------------------------------------------------------------------------------------
BlockGetter = Callable[[int, int], Tuple[np.ndarray, int, np.ndarray]]
"""(expert, module) -> (idx8 uint8 [R, C], q, lut fp16 [R, 2**q])."""


def _ffn_from_getter(get: BlockGetter, expert: int, X: np.ndarray) -> np.ndarray:
    gi, gq, gl = get(expert, GATE_UP)
    di, dq, dl = get(expert, DOWN)
    return expert_ffn(committed_index(gi, gq), gl, committed_index(di, dq), dl, X)


def layer_forward(x: np.ndarray, logits: np.ndarray, k: int, get_block: BlockGetter,
                  shared: Optional[BlockGetter] = None, shared_scale: Optional[np.ndarray] = None,
                  tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Route, group and run the expert FFNs; y in float64 [T, H].

    ``tokens`` restricts the FFN work to those token rows (the routing and grouping are still
    computed for the whole batch); rows of y outside it are left at zero.
    """
    x = np.asarray(x)
    T, H = x.shape
    E = logits.shape[1]
    ids, gates = route_topk(logits, k)
    offsets, pairs, active, n_active = group_by_expert(ids, E)
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), tokens)
    y = np.zeros((T, H), dtype=np.float64)
    x64 = x.astype(np.float64)
    for e in active[:n_active]:
        pe = pairs[offsets[e]:offsets[e + 1]]
        t, j = pe // k, pe % k
        keep = want[t]
        t, j = t[keep], j[keep]
        if len(t) == 0:
            continue
        o = _ffn_from_getter(get_block, int(e), x64[t])                   # [n, H]
        y[t] += gates[t, j][:, None] * o          # a token picks an expert at most once
    if shared is not None:
        rows = np.flatnonzero(want)
        s = np.ones(T) if shared_scale is None else np.asarray(shared_scale, dtype=np.float64)
        y[rows] += s[rows, None] * _ffn_from_getter(shared, 0, x64[rows])
    return dict(ids=ids, gates=gates, offsets=offsets, pairs=pairs, active=active,
                n_active=n_active, y=y)


# --------------------------------------------------------------------------------------------
# 6. Online routing statistics and the substituted gate mass
# --------------------------------------------------------------------------------------------
def routing_stats(ids: np.ndarray, gates: np.ndarray, E: int,
                  resident: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, float, float]:
    """Routing mass of one call and the gate mass that would be substituted.

    PagedWeight, Key Components 2 (online routing statistics): an expert's routing mass is how
    often and with what weight the router selects it -- here count[e] = number of (token, slot)
    pairs routed to e and mass[e] = the sum of their gate weights.  "Which Expert Misses Are
    Worth Waiting For?", Methodology: the substituted gate mass m is the normalised sum of the
    gate weights of the substituted experts; with a resident set and every miss substituted
    (no policy fetches any), substituted = sum of g over pairs whose expert is not resident and
    m = substituted / total, total = sum of every g.  Sums run over the pairs p = t*k + j in
    ascending order.  Returns (count int64 [E], mass float64 [E], substituted, total).
    """
    flat_ids = np.asarray(ids).reshape(-1)
    flat_g = np.asarray(gates, dtype=np.float64).reshape(-1)
    assert flat_ids.shape == flat_g.shape
    res = np.ones(E, dtype=bool) if resident is None else np.asarray(resident).reshape(-1) != 0
    count = np.zeros(E, dtype=np.int64)
    mass = np.zeros(E, dtype=np.float64)
    substituted = 0.0
    total = 0.0
    for p in range(flat_ids.size):
        e = int(flat_ids[p])
        assert 0 <= e < E
        g = float(flat_g[p])
        count[e] += 1
        mass[e] += g
        total += g
        if not res[e]:
            substituted += g
    return count, mass, substituted, total


# --------------------------------------------------------------------------------------------
# 7. Width planning: greedy lowest-damage-per-byte reductions
# --------------------------------------------------------------------------------------------
def block_bytes(rows: int, cols: int, q: int) -> int:
    """Resident bytes of a block at width q: q planes of rows*cols/8 bytes + an fp16 LUT of
    2**q entries per row (PagedWeight, Key Components 1: bit-planes + LUTs)."""
    rows, cols, q = int(rows), int(cols), int(q)
    return rows * cols * q // 8 + rows * (1 << q) * 2


def plan_widths(q_cur, q_floor, rows, cols, damage, mult, target_bytes: int):
    """Greedy width plan (PagedWeight, Key Components 2: the planner scores the damage of
    bit-width reductions and, when a memory target must be met, picks greedily the reductions
    of lowest damage per byte saved).  Reading of the unstated details: a reduction is one step
    q -> q-1 of one block, allowed while q-1 >= q_floor[i]; its cost is
    mult[i] * (damage[i][q-1] - damage[i][q]) / (bytes saved by the step), damage[i][w] being
    the block's damage score at width w (index w-1 of a row of 8); the cheapest step is taken
    (ties: lower block index), the block's next step becomes a candidate, and steps are taken
    until the bytes saved reach target_bytes or none is left.  Costs are compared in float64.
    Returns (q_new, bytes_saved).
    """
    q = [int(v) for v in q_cur]
    n = len(q)
    saved = 0
    while saved < target_bytes:
        best, best_cost = -1, None
        for i in range(n):
            if q[i] - 1 < max(1, int(q_floor[i])):
                continue
            step = block_bytes(rows[i], cols[i], q[i]) - block_bytes(rows[i], cols[i], q[i] - 1)
            cost = float(mult[i]) * (float(damage[i][q[i] - 2]) - float(damage[i][q[i] - 1])) / step
            if best < 0 or cost < best_cost:
                best, best_cost = i, cost
        if best < 0:
            break
        saved += block_bytes(rows[best], cols[best], q[best]) - block_bytes(rows[best], cols[best], q[best] - 1)
        q[best] -= 1
    return np.array(q, dtype=np.uint8), saved


# --------------------------------------------------------------------------------------------
# 8. Residency-aware substitution policies and background admission
# --------------------------------------------------------------------------------------------
POLICY_FETCH_ALL = 0     # fetch every miss (the baseline)
POLICY_GATE_RULE = 1     # fetch a miss if it is the first choice or its gate >= threshold
POLICY_FIRST_CHOICE = 2  # fetch a miss only if it is the first choice


def substitute(logits: np.ndarray, ids: np.ndarray, gates: np.ndarray, resident: np.ndarray,
               policy: int, gate_threshold: float = 0.15):
    """Substitution of non-resident experts ("Which Expert Misses Are Worth Waiting For?",
    Methodology: fetch every miss; the 0.15 rule fetches a missed expert if it is the router's
    first choice or its gate weight is >= 0.15 and substitutes the others; the first-choice rule
    fetches only a missed first choice).  Readings where the page is silent: slots are taken in
    order j = 0..k-1; a substituted slot gets the token's highest-logit resident expert that is
    not already among its experts (ties: lower id), keeps its gate weight, and the token keeps
    exactly k distinct experts; with no such expert left the miss is fetched.
    Returns (new ids [T,k], missed [T,k] = original expert of a substituted slot else -1,
    fetch [E] bool = a non-resident expert some token still uses)."""
    T, k = ids.shape
    E = logits.shape[1]
    res = np.asarray(resident).reshape(-1) != 0
    new = np.array(ids, dtype=np.int64, copy=True)
    missed = np.full((T, k), -1, dtype=np.int64)
    fetch = np.zeros(E, dtype=bool)
    lg = np.asarray(logits, dtype=np.float64)
    for t in range(T):
        taken = set(int(v) for v in ids[t])
        for j in range(k):
            e = int(ids[t, j])
            if res[e]:
                continue
            keep = (policy == POLICY_FETCH_ALL or
                    (policy == POLICY_GATE_RULE and (j == 0 or gates[t, j] >= gate_threshold)) or
                    (policy == POLICY_FIRST_CHOICE and j == 0))
            cands = [c for c in range(E) if res[c] and c not in taken]
            if keep or not cands:
                fetch[e] = True
                continue
            best = min(cands, key=lambda c: (-lg[t, c], c))
            new[t, j] = best
            missed[t, j] = e
            taken.add(best)
    return new, missed, fetch


def admit(missed: np.ndarray, gates: np.ndarray, acc: np.ndarray, threshold: float = 0.5):
    """Background admission ("Which Expert Misses Are Worth Waiting For?", Methodology: the
    substituted gate weight of an expert accumulates over time and the expert is admitted to
    the cache once it reaches a threshold, e.g. 0.5).  Reading: per expert, the gates of this
    call's slots substituted away from it are added in pair order (fp32, as the accumulator is
    stored), then compared with the threshold; an admitted expert's accumulator restarts at 0.
    Returns (new accumulators float32 [E], admitted bool [E])."""
    acc = np.array(acc, dtype=np.float32, copy=True)
    flat_m = np.asarray(missed).reshape(-1)
    flat_g = np.asarray(gates, dtype=np.float32).reshape(-1)
    for p in range(flat_m.size):
        if flat_m[p] >= 0:
            acc[flat_m[p]] = np.float32(acc[flat_m[p]] + flat_g[p])
    admitted = acc >= np.float32(threshold)
    acc[admitted] = 0.0
    return acc, admitted


def lynx_bins(logits: np.ndarray, ids: np.ndarray, bin_width: float):
    """AffinityBinning (LYNX, 2.2 System Components, confidence analyser: each token's router
    confidence, taken from the gap between its top-ranked logits, is cut into bins whose width
    and count follow from the sparsity ratio k/N alone).  Readings where the page is silent:
    confidence c_t = l(ids[t,0]) - l(ids[t,1]), the gap between the token's two best logits,
    as one fp32 subtraction; bin width w = k/N (fp32, passed in) and ceil(N/k) bins, so
    b_t = min(floor(c_t / w), ceil(N/k) - 1), at least 0, with the quotient rounded once to fp32; a token in
    bin b keeps its first min(k, b + 1) slots as critical assignments.  For k = 1 every slot is
    critical.  Returns (confidence float32 [T], bin int [T], kept slots int [T])."""
    T, k = ids.shape
    E = logits.shape[1]
    lg = np.asarray(logits, dtype=np.float32)
    w = np.float32(bin_width)
    nbins = -(-E // k)
    conf = np.zeros(T, dtype=np.float32)
    bins = np.full(T, nbins - 1, dtype=np.int64)
    keep = np.full(T, k, dtype=np.int64)
    if k < 2:
        return conf, bins, keep
    for t in range(T):
        c = np.float32(lg[t, ids[t, 0]] - lg[t, ids[t, 1]])
        conf[t] = c
        q = np.float32(c / w)
        b = max(0, min(int(np.floor(q)), nbins - 1))
        bins[t] = b
        keep[t] = min(k, b + 1)
    return conf, bins, keep


def lynx_remap(logits: np.ndarray, ids: np.ndarray, bin_width: float):
    """Batch-aware expert remapping (LYNX, 2.2 System Components, expert remapper: low-affinity
    token-expert assignments are redirected to the surviving critical set of experts; every
    token still activates exactly k experts while the batch activates fewer distinct ones).
    Readings: the critical set is the set of experts of the critical assignments of every token
    (its first ``keep`` slots, ``lynx_bins``); a non-critical slot whose expert is outside the
    critical set takes the token's highest-logit critical expert not already among its experts
    (ties: lower id), slots taken in order j = 0..k-1, and keeps its gate weight; with no such
    expert left the slot keeps its own expert.
    Returns (new ids [T,k], remapped [T,k] = original expert of a remapped slot else -1,
    critical [E] bool)."""
    T, k = ids.shape
    E = logits.shape[1]
    _, _, keep = lynx_bins(logits, ids, bin_width)
    critical = np.zeros(E, dtype=bool)
    for t in range(T):
        for j in range(int(keep[t])):
            critical[int(ids[t, j])] = True
    lg = np.asarray(logits, dtype=np.float64)
    new = np.array(ids, dtype=np.int64, copy=True)
    remapped = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        taken = set(int(v) for v in ids[t])
        for j in range(int(keep[t]), k):
            e = int(ids[t, j])
            if critical[e]:
                continue
            cands = [c for c in range(E) if critical[c] and c not in taken]
            if not cands:
                continue
            best = min(cands, key=lambda c: (-lg[t, c], c))
            new[t, j] = best
            remapped[t, j] = e
            taken.add(best)
    return new, remapped, critical


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 over the whole array, in float64."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))
