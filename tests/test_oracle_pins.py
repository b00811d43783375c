"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks one oracle function against something other than its own formula: brute
force on tiny inputs, an independent library routine, a closed form, an invariant of the
method, or a hand-derived case under tests/golden/.  A plausible mistake in the oracle (a
dropped term, a wrong sign, index or bit order, a transposed operand) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------
def _bruteforce_route(logits, k):
    """Rank of e = #experts strictly larger + #equal experts with a lower id."""
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        for e in range(E):
            rank = sum(1 for f in range(E) if row[f] > row[e] or (row[f] == row[e] and f < e))
            if rank < k:
                ids[t, rank] = e
    return ids


@pytest.mark.parametrize("E,k", [(8, 2), (13, 5), (16, 16), (5, 1)])
def test_route_ids_match_bruteforce_rank(E, k):
    r = _rng(E * 100 + k)
    # fp16-grid values create many exact ties
    logits = (r.standard_normal((9, E)) * 2).astype(np.float16).astype(np.float32)
    logits[0, :] = 0.5                     # a fully tied row
    logits[1, ::2] = -0.0
    logits[1, 1::2] = 0.0                  # signed zeros
    ids, gates = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids, _bruteforce_route(logits, k))


def test_route_first_choice_is_numpy_argmax():
    r = _rng(1)
    logits = r.integers(-3, 4, size=(64, 17)).astype(np.float32)  # heavy ties
    ids, _ = oracle.route_topk(logits, 4)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(logits, axis=1))  # first max = lowest id


def test_route_exactly_k_distinct_in_range_and_k_equals_E_is_full_order():
    r = _rng(2)
    logits = r.standard_normal((20, 11)).astype(np.float32)
    for k in (1, 3, 11):
        ids, gates = oracle.route_topk(logits, k)
        assert ids.shape == (20, k)
        for t in range(20):
            assert len(set(ids[t].tolist())) == k
            assert ids[t].min() >= 0 and ids[t].max() < 11
    ids, _ = oracle.route_topk(logits, 11)
    np.testing.assert_array_equal(ids, np.argsort(-logits.astype(np.float64), axis=1, kind="stable"))


def test_route_gates_equal_full_softmax_renormalised():
    r = _rng(3)
    logits = (r.standard_normal((30, 40)) * 3).astype(np.float32)
    k = 7
    ids, gates = oracle.route_topk(logits, k)
    l = logits.astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)                       # full-E softmax
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(gates, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(gates, axis=1) <= 1e-15)         # non-increasing along the slots


def test_route_golden_cases():
    with open(os.path.join(GOLDEN, "routing_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        logits = np.array([[float(v) for v in c["logits"]]], dtype=np.float32)
        ids, gates = oracle.route_topk(logits, c["k"])
        assert ids[0].tolist() == c["ids"], c["note"]
        np.testing.assert_allclose(gates[0], c["gates"], rtol=0, atol=c["tol"] + 1e-16,
                                   err_msg=c["note"])


def test_route_rejects_non_finite_and_bad_k():
    with pytest.raises(ValueError):
        oracle.route_topk(np.array([[0.0, np.nan]], dtype=np.float32), 1)
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((1, 3), dtype=np.float32), 4)


def test_route_empty_batch():
    ids, gates = oracle.route_topk(np.zeros((0, 6), dtype=np.float32), 2)
    assert ids.shape == (0, 2) and gates.shape == (0, 2)


# ------------------------------------------------------------------------------------------
# grouping
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (33, 16, 5), (1, 3, 3), (50, 64, 8)])
def test_group_matches_stable_argsort_and_inverts(T, E, k):
    r = _rng(T * E + k)
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 3.0                              # a hot expert
    ids, _ = oracle.route_topk(logits, k)
    offsets, pairs, active, n_active = oracle.group_by_expert(ids, E)
    flat = ids.reshape(-1)
    np.testing.assert_array_equal(pairs, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert offsets[-1] == T * k
    assert sorted(pairs.tolist()) == list(range(T * k))            # bijection
    rebuilt = np.empty(T * k, dtype=np.int64)
    for e in range(E):
        rebuilt[pairs[offsets[e]:offsets[e + 1]]] = e
    np.testing.assert_array_equal(rebuilt, flat)
    uniq = np.unique(flat)
    assert n_active == len(uniq)
    np.testing.assert_array_equal(active[:n_active], uniq)
    assert np.all(active[n_active:] == -1)


def test_group_empty():
    offsets, pairs, active, n_active = oracle.group_by_expert(np.zeros((0, 2), dtype=np.int32), 5)
    assert n_active == 0 and len(pairs) == 0 and np.all(offsets == 0)


# ------------------------------------------------------------------------------------------
# bit-plane format
# ------------------------------------------------------------------------------------------
def test_bit_position_is_a_bijection_per_plane():
    for p in range(8):
        pos = oracle.bit_position(p, np.arange(32))
        assert sorted(pos.tolist()) == list(range(32))


@pytest.mark.parametrize("q", range(1, 9))
def test_pack_unpack_round_trip_gives_top_q_bit_prefix(q):
    r = _rng(q)
    idx8 = r.integers(0, 256, size=(128, 384), dtype=np.uint8)
    planes = oracle.pack_planes(idx8, q)
    assert planes.dtype == np.uint32 and planes.size == q * 128 * 384 // 32
    got = oracle.unpack_planes(planes, 128, 384, q)
    np.testing.assert_array_equal(got, idx8 >> (8 - q))
    np.testing.assert_array_equal(oracle.committed_index(idx8, q), idx8 >> (8 - q))


def test_dropping_tail_planes_equals_repacking_at_lower_width():
    r = _rng(11)
    idx8 = r.integers(0, 256, size=(64, 256), dtype=np.uint8)
    full = oracle.pack_planes(idx8, 8)
    per_plane = 64 * 256 // 32
    for q in range(1, 8):
        np.testing.assert_array_equal(full[: q * per_plane], oracle.pack_planes(idx8, q))


def test_plane_p_holds_bit_7_minus_p_row_by_row():
    """Popcount of plane p, per row, equals the count of parent indices with bit 7-p set."""
    r = _rng(12)
    R, C = 128, 256
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    planes = oracle.pack_planes(idx8, 8).reshape(8, -1)
    for p in range(8):
        total = int(np.unpackbits(planes[p].view(np.uint8)).sum())
        assert total == int(((idx8 >> (7 - p)) & 1).sum())
    # a single full-scale index lights exactly one bit in every plane, none elsewhere
    one = np.zeros((R, C), dtype=np.uint8)
    one[70, 201] = 0xFF
    pl = oracle.pack_planes(one, 8).reshape(8, -1)
    loc = [np.flatnonzero(pl[p]) for p in range(8)]
    assert all(len(l) == 1 for l in loc)
    assert len({int(l[0]) for l in loc}) == 1          # same word offset in every plane
    bits = [int(pl[p][loc[p][0]]) for p in range(8)]
    assert all(b and (b & (b - 1)) == 0 for b in bits)  # one bit each
    # all-0x80 -> plane 0 all ones, other planes empty
    msb = np.full((R, C), 0x80, dtype=np.uint8)
    pl = oracle.pack_planes(msb, 3).reshape(3, -1)
    assert np.all(pl[0] == 0xFFFFFFFF) and not pl[1:].any()


def test_format_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.pack_planes(np.zeros((64, 96), dtype=np.uint8), 4)
    with pytest.raises(ValueError):
        oracle.pack_planes(np.zeros((32, 128), dtype=np.uint8), 4)


# ------------------------------------------------------------------------------------------
# dequantised GEMV
# ------------------------------------------------------------------------------------------
def _naive_matvec(idx_q, lut, X):
    R, C = idx_q.shape
    n = X.shape[1]
    Y = np.zeros((R, n))
    for r in range(R):
        for c in range(C):
            w = float(lut[r, idx_q[r, c]])
            for j in range(n):
                Y[r, j] += w * float(X[c, j])
    return Y


def test_apq_matvec_matches_naive_loops():
    r = _rng(20)
    q = 3
    idx8 = r.integers(0, 256, size=(64, 128), dtype=np.uint8)
    lut = (r.standard_normal((64, 1 << q)) * 0.02).astype(np.float16)
    X = r.standard_normal((128, 3))
    idx_q = oracle.committed_index(idx8, q)
    Y = oracle.apq_matvec(idx_q, lut, X)
    np.testing.assert_allclose(Y, _naive_matvec(idx_q, lut, X), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.apq_matvec(idx_q, lut, X, row_chunk=7), Y, rtol=1e-13, atol=1e-15)


def test_apq_matvec_closed_forms():
    r = _rng(21)
    R, C, q = 64, 256, 5
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    idx_q = oracle.committed_index(idx8, q)
    X = r.integers(-4, 5, size=(C, 2)).astype(np.float64)          # integers: exact sums
    # constant LUT row: y_r = a * sum(x)
    a = np.float16(0.375)
    lut = np.full((R, 1 << q), a, dtype=np.float16)
    np.testing.assert_array_equal(oracle.apq_matvec(idx_q, lut, X), np.broadcast_to(float(a) * X.sum(0), (R, 2)))
    # affine LUT lut[v] = a + b v (fp16-exact): y_r = a sum(x) + b sum(idx x)
    b = np.float16(0.125)
    lut = (float(a) + float(b) * np.arange(1 << q))[None, :].repeat(R, 0).astype(np.float16)
    expect = float(a) * X.sum(0)[None, :] + float(b) * (idx_q.astype(np.float64) @ X)
    np.testing.assert_array_equal(oracle.apq_matvec(idx_q, lut, X), expect)


def test_one_hot_probe_reads_the_lut_entry():
    r = _rng(22)
    R, C, q = 64, 128, 6
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    lut = (r.standard_normal((R, 1 << q))).astype(np.float16)
    idx_q = oracle.committed_index(idx8, q)
    for c in (0, 37, 127):
        X = np.zeros((C, 1))
        X[c] = 1.0
        y = oracle.apq_matvec(idx_q, lut, X)[:, 0]
        np.testing.assert_array_equal(y, lut[np.arange(R), idx_q[:, c]].astype(np.float64))


def test_silu_identities():
    z = np.linspace(-30, 30, 1001)
    s = oracle.silu(z)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - oracle.silu(-z), z, atol=1e-12)
    np.testing.assert_allclose(s, z * expit(z), rtol=1e-13, atol=1e-300)


# ------------------------------------------------------------------------------------------
# the layer
# ------------------------------------------------------------------------------------------
def _tiny_layer(shape, seed=0):
    inputs = wl.gen_layer_inputs(shape, seed)
    blocks = {}

    def get(e, m):
        if (e, m) not in blocks:
            b = wl.gen_block(shape, e, m, int(inputs.widths[e, m]))
            blocks[(e, m)] = (b.idx8, b.q, b.lut)
        return blocks[(e, m)]
    return inputs, get


def _dense_W(idx8, q, lut):
    R, C = idx8.shape
    W = np.zeros((R, C))
    for r in range(R):
        W[r] = [float(lut[r, v >> (8 - q)]) for v in idx8[r]]
    return W


def test_layer_equals_dense_bruteforce_over_all_experts():
    """Every expert on every token, weighted by a dense gate matrix (no grouping logic)."""
    shape = wl.TINY.replace(T=6)
    inputs, get = _tiny_layer(shape)
    res = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get)
    T, E, H, I = shape.T, shape.E, shape.H, shape.I
    G = np.zeros((T, E))
    l = inputs.logits.astype(np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))[: shape.k]
        w = np.array([math.exp(l[t, e] - l[t, order[0]]) for e in order])
        G[t, order] = w / w.sum()
    y = np.zeros((T, H))
    x = inputs.x.astype(np.float64)
    for e in range(E):
        Wgu = _dense_W(*get(e, 0))
        Wd = _dense_W(*get(e, 1))
        h = x @ Wgu.T
        act = h[:, :I] * expit(h[:, :I]) * h[:, I:]
        y += G[:, e:e + 1] * (act @ Wd.T)
    np.testing.assert_allclose(res["y"], y, rtol=1e-10, atol=1e-12)


def test_identical_experts_make_output_routing_invariant():
    shape = wl.TINY.replace(T=5, E=6, k=3)
    inputs, get = _tiny_layer(shape)
    fixed = {m: get(0, m) for m in (0, 1)}
    same = lambda e, m: fixed[m]
    y1 = oracle.layer_forward(inputs.x, inputs.logits, 3, same)["y"]
    r = _rng(5)
    y2 = oracle.layer_forward(inputs.x, r.standard_normal(inputs.logits.shape).astype(np.float32), 3, same)["y"]
    ffn = oracle.expert_ffn(oracle.committed_index(fixed[0][0], fixed[0][1]), fixed[0][2],
                            oracle.committed_index(fixed[1][0], fixed[1][1]), fixed[1][2], inputs.x)
    np.testing.assert_allclose(y1, ffn, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y2, ffn, rtol=1e-12, atol=1e-14)


def test_k1_output_is_the_first_choice_ffn_and_shared_adds_linearly():
    shape = wl.TINY.replace(T=4, k=1)
    inputs, get = _tiny_layer(shape)
    res = oracle.layer_forward(inputs.x, inputs.logits, 1, get)
    for t in range(shape.T):
        e = int(res["ids"][t, 0])
        gi, gq, gl = get(e, 0)
        di, dq, dl = get(e, 1)
        yt = oracle.expert_ffn(oracle.committed_index(gi, gq), gl, oracle.committed_index(di, dq), dl,
                               inputs.x[t:t + 1])
        np.testing.assert_allclose(res["y"][t], yt[0], rtol=1e-12, atol=1e-14)
    # a shared expert adds s_t * FFN_shared(x_t); scale 0 removes it, scale 2 doubles it
    sh = lambda e, m: get(3, m)
    base = res["y"]
    ffn_sh = oracle.layer_forward(inputs.x, inputs.logits, 1, get, shared=sh)["y"] - base
    s = np.array([0.0, 1.0, 2.0, -0.5])
    y_s = oracle.layer_forward(inputs.x, inputs.logits, 1, get, shared=sh, shared_scale=s)["y"]
    np.testing.assert_allclose(y_s - base, s[:, None] * ffn_sh, rtol=1e-10, atol=1e-13)


def test_token_subset_matches_full_rows():
    shape = wl.TINY.replace(T=7)
    inputs, get = _tiny_layer(shape, seed=3)
    full = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get)["y"]
    part = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, tokens=[1, 5])["y"]
    np.testing.assert_allclose(part[[1, 5]], full[[1, 5]], rtol=1e-12, atol=1e-16)
    assert not part[[0, 2, 3, 4, 6]].any()


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert oracle.rel_l2(a, a) == 0.0
    assert abs(oracle.rel_l2(a * 1.001, a) - 1e-3) < 1e-12


# ------------------------------------------------------------------------------------------
# the seeded generators (determinism and the stated distributions)
# ------------------------------------------------------------------------------------------
def test_generators_are_deterministic_and_luts_nested():
    shape = wl.TINY
    a = wl.gen_block(shape, 3, 1)
    b = wl.gen_block(shape, 3, 1)
    np.testing.assert_array_equal(a.idx8, b.idx8)
    np.testing.assert_array_equal(a.lut, b.lut)
    assert a.q in shape.widths and a.lut.shape == (shape.H, 1 << a.q)
    assert np.all(np.diff(a.lut.astype(np.float64), axis=1) >= 0)           # sorted rows
    l3 = wl.gen_lut(shape, 3, 1, 3).astype(np.float64)
    l4 = wl.gen_lut(shape, 3, 1, 4).astype(np.float64)
    np.testing.assert_allclose(l3, l4.reshape(-1, 8, 2).mean(2), atol=4e-5)  # nested prefixes
    w = wl.gen_widths(wl.QWEN3_NEXT_80B_A3B)
    assert (w[:, 0] == 8).sum() >= 128 and set(np.unique(w).tolist()) <= {3, 4, 5, 6, 8}
    assert np.all(wl.gen_widths(wl.QWEN15_MOE_A27B) == 4)


# ---- routing statistics --------------------------------------------------------------------
def test_routing_stats_match_bincount_and_mass_sums_to_tokens():
    """count = numpy.bincount of the ids, mass = bincount weighted by the gates (library
    routines), the counts add up to T*k and, since each token's gates sum to 1, the masses add
    up to T."""
    r = np.random.default_rng(11)
    T, E, k = 29, 13, 3
    ids, gates = oracle.route_topk(r.standard_normal((T, E)), k)
    count, mass, sub, tot = oracle.routing_stats(ids, gates, E)
    np.testing.assert_array_equal(count, np.bincount(ids.ravel(), minlength=E))
    np.testing.assert_allclose(mass, np.bincount(ids.ravel(), weights=gates.ravel(), minlength=E),
                               rtol=1e-15, atol=1e-15)
    assert count.sum() == T * k
    assert abs(mass.sum() - T) < 1e-12 and abs(tot - T) < 1e-12
    assert sub == 0.0   # every expert resident


def test_substituted_mass_special_cases_and_hand_example():
    """No expert resident: everything is substituted (m = 1); all resident: m = 0.  Hand case:
    token 0 picks experts (2, 0) with gates (0.7, 0.3), token 1 picks (1, 2) with (0.6, 0.4);
    with only expert 2 resident, the substituted mass is 0.3 + 0.6 of a total 2.0."""
    ids = np.array([[2, 0], [1, 2]])
    gates = np.array([[0.7, 0.3], [0.6, 0.4]])
    count, mass, sub, tot = oracle.routing_stats(ids, gates, 4, resident=np.array([0, 0, 1, 0]))
    np.testing.assert_array_equal(count, [1, 1, 2, 0])
    np.testing.assert_allclose(mass, [0.3, 0.6, 1.1, 0.0], rtol=0, atol=1e-15)
    assert abs(sub - 0.9) < 1e-15 and abs(tot - 2.0) < 1e-15
    _, _, sub0, tot0 = oracle.routing_stats(ids, gates, 4, resident=np.zeros(4))
    assert sub0 == tot0
    _, _, sub1, _ = oracle.routing_stats(ids, gates, 4, resident=np.ones(4))
    assert sub1 == 0.0


# ---- width planner -------------------------------------------------------------------------
def test_block_bytes_closed_form():
    """q planes of R*C/8 bytes plus an fp16 LUT of 2**q entries per row."""
    assert oracle.block_bytes(64, 128, 4) == 64 * 128 * 4 // 8 + 64 * 16 * 2
    assert oracle.block_bytes(2816, 2048, 8) == 2816 * 2048 + 2816 * 256 * 2


def test_planner_hand_example():
    """Two blocks of one shape (each step saves the same bytes); block 0's step 4->3 costs 1.0,
    block 1's 4->3 costs 0.5 and its 3->2 costs 3.0.  A target of two steps takes block 1's
    4->3 (0.5), then block 0's 4->3 (1.0) rather than block 1's 3->2 (3.0)."""
    R, C = 64, 128
    step43 = oracle.block_bytes(R, C, 4) - oracle.block_bytes(R, C, 3)
    dmg = np.zeros((2, 8))
    dmg[0, 2] = 1.0 * step43            # damage at width 3 (index 2), width 4 has damage 0
    dmg[1, 2] = 0.5 * step43
    dmg[1, 1] = dmg[1, 2] + 3.0 * (oracle.block_bytes(R, C, 3) - oracle.block_bytes(R, C, 2))
    q, saved = oracle.plan_widths([4, 4], [1, 1], [R, R], [C, C], dmg, [1.0, 1.0], 2 * step43)
    np.testing.assert_array_equal(q, [3, 3])
    assert saved == 2 * step43
    # one step only: the cheaper block
    q, _ = oracle.plan_widths([4, 4], [1, 1], [R, R], [C, C], dmg, [1.0, 1.0], 1)
    np.testing.assert_array_equal(q, [4, 3])
    # a damage multiplier of 3 on block 1 (a hot expert) makes block 0 the cheaper first step
    q, _ = oracle.plan_widths([4, 4], [1, 1], [R, R], [C, C], dmg, [1.0, 3.0], 1)
    np.testing.assert_array_equal(q, [3, 4])


def test_planner_invariants_and_exhaustive_optimality_of_each_step():
    """Random instances: floors are respected, the plan stops as soon as the target is met, an
    unreachable target reduces every block to its floor, and (definition of the greedy rule)
    replaying the plan step by step, each taken step is no more costly than any step available
    at that moment (checked by enumerating all of them)."""
    r = np.random.default_rng(5)
    for _ in range(40):
        n = int(r.integers(1, 7))
        rows = r.choice([64, 128], n)
        cols = r.choice([128, 256], n)
        qc = r.integers(2, 9, n)
        fl = np.minimum(qc, r.integers(1, 5, n))
        dmg = np.cumsum(r.random((n, 8))[:, ::-1], axis=1)[:, ::-1]   # non-increasing in width
        mult = r.uniform(0.5, 3.0, n)
        full = sum(oracle.block_bytes(rows[i], cols[i], qc[i]) - oracle.block_bytes(rows[i], cols[i], fl[i])
                   for i in range(n))
        target = int(r.integers(0, full + 2000))
        q, saved = oracle.plan_widths(qc, fl, rows, cols, dmg, mult, target)
        assert np.all(q >= fl) and np.all(q <= qc)
        assert saved == sum(oracle.block_bytes(rows[i], cols[i], qc[i]) - oracle.block_bytes(rows[i], cols[i], q[i])
                            for i in range(n))
        if target > full:
            np.testing.assert_array_equal(q, fl)
        else:
            assert saved >= target
        # replay: every taken step is a minimum-cost available step at its time
        cur = [int(v) for v in qc]
        done = 0
        while done < saved:
            costs = {}
            for i in range(n):
                if cur[i] - 1 >= max(1, fl[i]):
                    st = oracle.block_bytes(rows[i], cols[i], cur[i]) - oracle.block_bytes(rows[i], cols[i], cur[i] - 1)
                    costs[i] = mult[i] * (dmg[i][cur[i] - 2] - dmg[i][cur[i] - 1]) / st
            i = min(costs, key=lambda j: (costs[j], j))
            assert q[i] < cur[i]     # the plan took this block's step
            done += oracle.block_bytes(rows[i], cols[i], cur[i]) - oracle.block_bytes(rows[i], cols[i], cur[i] - 1)
            cur[i] -= 1
        np.testing.assert_array_equal(cur, q)


# ---- substitution policies and background admission ----------------------------------------
def _subst_case(seed, T=20, E=24, k=4):
    r = np.random.default_rng(seed)
    logits = r.standard_normal((T, E))
    ids, gates = oracle.route_topk(logits, k)
    resident = r.random(E) < 0.4
    return logits, ids, gates, resident


def test_substitution_rules_keep_what_they_must_and_choose_the_best_resident():
    """For every policy: all-resident changes nothing; every token keeps k distinct experts;
    every substituted slot held a non-resident expert and now holds a resident one that is the
    highest-logit resident expert not among the token's experts at that point (brute force over
    the experts); the fetch set is exactly the non-resident experts still in use.  Policy
    specifics: fetch-every-miss substitutes nothing; the first-choice rule never substitutes
    slot 0; the gate rule never substitutes slot 0 or a gate >= 0.15."""
    for seed in range(6):
        logits, ids, gates, res = _subst_case(seed)
        T, k = ids.shape
        for pol in (oracle.POLICY_FETCH_ALL, oracle.POLICY_GATE_RULE, oracle.POLICY_FIRST_CHOICE):
            same, none, _ = oracle.substitute(logits, ids, gates, np.ones(len(res)), pol)
            np.testing.assert_array_equal(same, ids)
            assert np.all(none == -1)
            new, missed, fetch = oracle.substitute(logits, ids, gates, res, pol)
            for t in range(T):
                assert len(set(new[t])) == k
                taken = set(ids[t])
                for j in range(k):
                    if missed[t, j] >= 0:
                        assert missed[t, j] == ids[t, j] and not res[ids[t, j]] and res[new[t, j]]
                        cands = [c for c in range(len(res)) if res[c] and c not in taken]
                        assert new[t, j] == max(cands, key=lambda c: (logits[t, c], -c))
                        taken.add(new[t, j])
                    else:
                        assert new[t, j] == ids[t, j]
            used = {int(e) for e in new.ravel() if not res[e]}
            assert set(np.flatnonzero(fetch)) == used
            if pol == oracle.POLICY_FETCH_ALL:
                assert np.all(missed == -1)
            if pol in (oracle.POLICY_FIRST_CHOICE, oracle.POLICY_GATE_RULE):
                assert np.all(missed[:, 0] == -1)
            if pol == oracle.POLICY_GATE_RULE:
                assert np.all(missed[gates >= 0.15] == -1)


def test_substitution_hand_example_and_admission():
    """One token, experts 0..4, logits [5, 4, 3, 2, 1], k = 3 -> ids (0, 1, 2); only experts 2
    and 4 resident.  First-choice rule: slot 0 (expert 0) is fetched, slot 1 (expert 1) is
    substituted by the best free resident expert, 4 (2 is already taken).  Admission: expert 1's
    substituted gate accumulates across calls and is admitted when it reaches 0.5."""
    logits = np.array([[5.0, 4.0, 3.0, 2.0, 1.0]])
    ids, gates = oracle.route_topk(logits, 3)
    np.testing.assert_array_equal(ids, [[0, 1, 2]])
    res = np.array([0, 0, 1, 0, 1])
    new, missed, fetch = oracle.substitute(logits, ids, gates, res, oracle.POLICY_FIRST_CHOICE)
    np.testing.assert_array_equal(new, [[0, 4, 2]])
    np.testing.assert_array_equal(missed, [[-1, 1, -1]])
    np.testing.assert_array_equal(fetch, [True, False, False, False, False])
    g1 = np.float32(gates[0, 1])              # e^-1 / (1 + e^-1 + e^-2) ~ 0.2447
    assert abs(float(g1) - math.exp(-1) / (1 + math.exp(-1) + math.exp(-2))) < 1e-7
    acc, adm = oracle.admit(missed, gates, np.zeros(5, np.float32))
    assert acc[1] == g1 and not adm.any()
    acc, adm = oracle.admit(missed, gates, acc)          # 0.489 < 0.5: not yet
    assert acc[1] == np.float32(g1 + g1) and not adm.any()
    acc, adm = oracle.admit(missed, gates, acc)          # 0.734 >= 0.5: admitted, restarts at 0
    assert acc[1] == 0.0 and adm[1] and adm.sum() == 1


def test_lynx_hand_example():
    """Three tokens over experts 0..5, k = 2, so the bin width is k/N = 1/3 (fp32) and there are
    3 bins.  Token 0: logits (2, 1, ...) -> ids (0, 1), gap 1 -> bin 2 -> both slots critical.
    Token 1: ids (2, 3), gap 0.125 -> bin 0 -> only slot 0 critical; expert 3 is outside the
    critical set {0, 1, 2, 4}, so slot 1 takes the best free critical expert, 0 (logit 0.5).
    Token 2: ids (4, 5), gap 0.25 -> bin 0; slot 1 (expert 5) takes expert 1 (logit 0.25).
    The batch goes from 6 distinct experts to 4."""
    logits = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -1.0],
                       [0.5, -1.0, 3.0, 2.875, 0.0, -1.0],
                       [-1.0, 0.25, -1.0, -1.0, 1.5, 1.25]], dtype=np.float32)
    ids, _ = oracle.route_topk(logits, 2)
    np.testing.assert_array_equal(ids, [[0, 1], [2, 3], [4, 5]])
    w = np.float32(2) / np.float32(6)
    conf, bins, keep = oracle.lynx_bins(logits, ids, w)
    np.testing.assert_array_equal(conf, np.float32([1.0, 0.125, 0.25]))
    np.testing.assert_array_equal(bins, [2, 0, 0])
    np.testing.assert_array_equal(keep, [2, 1, 1])
    new, remapped, critical = oracle.lynx_remap(logits, ids, w)
    np.testing.assert_array_equal(new, [[0, 1], [2, 0], [4, 1]])
    np.testing.assert_array_equal(remapped, [[-1, -1], [-1, 3], [-1, 5]])
    np.testing.assert_array_equal(critical, [True, True, True, False, True, False])
    assert len(set(ids.ravel())) == 6 and len(set(new.ravel())) == 4


def test_lynx_bin_boundaries_and_quotient_rounding():
    """A gap equal to the bin width lands in bin 1, the next fp32 value below it in bin 0; the
    clamp puts very large gaps in the last bin, ceil(N/k) - 1.  The fp32 quotient equals the
    double quotient rounded once to fp32 (exact for fp32 operands), on random gaps."""
    E, k = 6, 2
    w = np.float32(k) / np.float32(E)
    below = np.nextafter(w, np.float32(0))
    logits = np.full((3, E), -5.0, dtype=np.float32)
    logits[0, 0], logits[0, 1] = w, 0.0
    logits[1, 0], logits[1, 1] = below, 0.0
    logits[2, 0], logits[2, 1] = 100.0, 0.0
    ids, _ = oracle.route_topk(logits, k)
    conf, bins, keep = oracle.lynx_bins(logits, ids, w)
    assert conf[0] == w and conf[1] == below
    np.testing.assert_array_equal(bins, [1, 0, 2])
    np.testing.assert_array_equal(keep, [2, 1, 2])
    r = np.random.default_rng(5)
    for _ in range(2000):
        c = np.float32(abs(r.standard_normal()))
        ww = np.float32(r.integers(1, 33)) / np.float32(r.integers(33, 1025))
        assert np.float32(c / ww) == np.float32(float(c) / float(ww))


def test_lynx_negative_gap_counts_as_bin_zero():
    """Slots handed over out of routing order (the caller's ids, e.g. after its own edits) give a
    negative top-2 gap; the reading takes such a token as least confident: bin 0, one critical
    slot (its slot 0).  Hand-derived: E = 6, k = 2, w = 1/3.  Token 0 names [1, 0] with logits
    1.0 and 2.0: gap -1.0, quotient -3 -> bin 0, keeps slot 0 (expert 1).  Token 1 names [2, 3]
    (logits 3.0, 2.875): gap 0.125 -> bin 0, keeps expert 2.  Critical set {1, 2}.  Token 0's
    slot 1 (expert 0, not critical) takes the best critical expert it does not hold: 2; token
    1's slot 1 (expert 3) takes 1."""
    logits = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -1.0],
                       [0.5, -1.0, 3.0, 2.875, 0.0, -1.0]], dtype=np.float32)
    ids = np.array([[1, 0], [2, 3]], dtype=np.int32)
    w = np.float32(2) / np.float32(6)
    conf, bins, keep = oracle.lynx_bins(logits, ids, w)
    np.testing.assert_array_equal(conf, np.array([-1.0, 0.125], dtype=np.float32))
    np.testing.assert_array_equal(bins, [0, 0])
    np.testing.assert_array_equal(keep, [1, 1])
    new, remapped, critical = oracle.lynx_remap(logits, ids, w)
    np.testing.assert_array_equal(new, [[1, 2], [2, 1]])
    np.testing.assert_array_equal(remapped, [[-1, 0], [-1, 3]])
    np.testing.assert_array_equal(critical, [False, True, True, False, False, False])


def test_lynx_remap_invariants_and_brute_force_choice():
    """Random batches: every token keeps k distinct experts; its first `keep` slots are
    unchanged; a remapped slot held a non-critical expert and now holds the highest-logit
    critical expert not among the token's experts at that point (brute force); a slot that is
    not remapped is unchanged; the critical set is exactly the experts of the kept slots; the
    batch never activates more distinct experts than before.  k = 1, and a bin width so small
    that every token keeps all its slots, change nothing."""
    for seed in range(8):
        r = np.random.default_rng(100 + seed)
        T, E, k = int(r.integers(1, 40)), int(r.integers(8, 80)), int(r.integers(2, 7))
        logits = (r.standard_normal((T, E)) * 0.3).astype(np.float32)
        ids, _ = oracle.route_topk(logits, k)
        w = np.float32(k) / np.float32(E)
        _, _, keep = oracle.lynx_bins(logits, ids, w)
        new, remapped, critical = oracle.lynx_remap(logits, ids, w)
        crit_ref = np.zeros(E, dtype=bool)
        for t in range(T):
            crit_ref[ids[t, :keep[t]]] = True
        np.testing.assert_array_equal(critical, crit_ref)
        for t in range(T):
            assert len(set(new[t])) == k
            np.testing.assert_array_equal(new[t, :keep[t]], ids[t, :keep[t]])
            taken = set(ids[t])
            for j in range(k):
                if remapped[t, j] >= 0:
                    assert j >= keep[t] and remapped[t, j] == ids[t, j] and not critical[ids[t, j]]
                    cands = [c for c in range(E) if critical[c] and c not in taken]
                    assert new[t, j] == max(cands, key=lambda c: (float(logits[t, c]), -c))
                    taken.add(int(new[t, j]))
                else:
                    assert new[t, j] == ids[t, j]
        assert len(set(new.ravel())) <= len(set(ids.ravel()))
        if -(-E // k) >= k:   # the last bin keeps every slot
            same, none, _ = oracle.lynx_remap(logits, ids, np.float32(1e-30))
            np.testing.assert_array_equal(same, ids)
            assert np.all(none == -1)
        ids1, _ = oracle.route_topk(logits, 1)
        one, none1, _ = oracle.lynx_remap(logits, ids1, w)
        np.testing.assert_array_equal(one, ids1)
        assert np.all(none1 == -1)
