"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: top-k ids, the grouping (offsets, pairs, active list), decoded indices and one-hot
GEMV probes.  Floating point: gates within 1e-6 absolute (fp32 softmax of the same fp32 logits),
the single-block GEMV within 1e-5 relative L2 (fp32 accumulation of exact fp16 products), and
layer outputs within 1e-3 relative L2 (fp32 accumulation, the SiLU-gated activation rounded
once to fp16, y rounded to fp16: about 4e-4 expected).
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import any_precision_expert_router_amd as apq  # noqa: E402  (fails loudly if not built)
from workloads import device as gpu_layers  # noqa: E402

DEV = "cuda"
LAYER_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def _route_gpu(logits, k):
    T, E = logits.shape
    lt = _t(logits.astype(np.float32))
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, k), dtype=torch.float32, device=DEV)
    apq.moe_route_topk(lt, k, ids, gates)
    return ids, gates


def _group_gpu(ids, E):
    T, k = ids.shape
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pairs = torch.empty(max(T * k, 1), dtype=torch.int32, device=DEV)
    act = torch.empty(E, dtype=torch.int32, device=DEV)
    nact = torch.empty(1, dtype=torch.int32, device=DEV)
    apq.moe_group_by_expert(ids, E, off, pairs, act, nact)
    return off, pairs[: T * k], act, nact


# ------------------------------------------------------------------------------------------
# routing and grouping: bit-exact
# ------------------------------------------------------------------------------------------
ROUTE_CASES = [(4, 8, 2), (16, 60, 4), (64, 512, 10), (33, 64, 8), (7, 1024, 32), (5, 3, 3),
               (2048, 64, 8), (1, 1, 1), (9, 128, 1)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
def test_route_topk_bit_exact(T, E, k):
    say(f"route T={T} E={E} k={k}")
    r = np.random.default_rng(T * 7 + E + k)
    logits = (r.standard_normal((T, E)) * 2).astype(np.float16).astype(np.float32)  # ties
    if T > 2:
        logits[0] = 0.25
        logits[1, ::2] = -0.0
        logits[1, 1::2] = 0.0
    ids, gates = _route_gpu(logits, k)
    ref_ids, ref_g = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    g = gates.cpu().numpy()
    np.testing.assert_allclose(g, ref_g, rtol=0, atol=1e-6)
    np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-6)


def test_route_zipf_router_bit_exact():
    shape = wl.QWEN3_NEXT_80B_A3B
    inp = wl.gen_layer_inputs(shape)
    ids, gates = _route_gpu(inp.logits, shape.k)
    ref_ids, ref_g = oracle.route_topk(inp.logits, shape.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), ref_g, atol=1e-6)


@pytest.mark.parametrize("T,E,k", ROUTE_CASES + [(0, 8, 2), (40, 16, 16)])
def test_group_by_expert_bit_exact(T, E, k):
    say(f"group T={T} E={E} k={k}")
    r = np.random.default_rng(T + 3 * E + k)
    logits = r.standard_normal((T, E)).astype(np.float32)
    if T:
        logits[:, 0] += 4.0   # a hot expert
    ref_ids, _ = oracle.route_topk(logits, k)
    ids = _t(ref_ids.astype(np.int32))
    off, pairs, act, nact = _group_gpu(ids, E)
    r_off, r_pairs, r_act, r_n = oracle.group_by_expert(ref_ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    np.testing.assert_array_equal(pairs.cpu().numpy(), r_pairs)
    np.testing.assert_array_equal(act.cpu().numpy(), r_act)
    assert int(nact.item()) == r_n


def test_group_single_expert_takes_every_token():
    T, E, k = 300, 64, 1
    ids = np.full((T, k), 5, dtype=np.int32)
    off, pairs, act, nact = _group_gpu(_t(ids), E)
    r_off, r_pairs, r_act, r_n = oracle.group_by_expert(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    np.testing.assert_array_equal(pairs.cpu().numpy(), r_pairs)
    assert int(nact.item()) == 1 and int(act[0].item()) == 5


@pytest.mark.parametrize("T,E,k", [(5, 8, 4), (300, 64, 8), (3000, 64, 8), (40, 1024, 32), (700, 16, 16)])
def test_group_by_expert_repeated_and_foreign_ids(T, E, k):
    """Ids the routing never writes: a token naming one expert in several slots, and ids outside
    [0, E) (-1, E, a large value).  The oracle's definition places every pair whose id names an
    expert, stably by pair id (repeats in slot order), and leaves the others out; the kernel must
    give the same offsets, placed pairs, active list and count."""
    say(f"group foreign T={T} E={E} k={k}")
    r = np.random.default_rng(T + E + 5 * k)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    rep = r.random((T, k)) < 0.3                                    # repeats inside tokens
    for j in range(1, k):
        ids[rep[:, j], j] = ids[rep[:, j], j - 1]
    ids[r.random((T, k)) < 0.05] = -1
    ids[r.random((T, k)) < 0.05] = E
    ids[r.random((T, k)) < 0.02] = 1 << 20
    ids[0, :] = ids[0, 0] if (0 <= ids[0, 0] < E) else 0            # one token naming one expert k times
    ids[-1, -1] = -1                                                # at least one id of each foreign kind
    ids[T // 2, 0] = E
    ids[T // 2, k - 1] = 1 << 20
    off, pairs, act, nact = _group_gpu(_t(ids), E)
    r_off, r_pairs, r_act, r_n = oracle.group_by_expert(ids, E)
    np.testing.assert_array_equal(off.cpu().numpy(), r_off)
    n_placed = int(r_off[E])
    assert n_placed < T * k
    np.testing.assert_array_equal(pairs.cpu().numpy()[:n_placed], r_pairs)
    np.testing.assert_array_equal(act.cpu().numpy(), r_act)
    assert int(nact.item()) == r_n


# ------------------------------------------------------------------------------------------
# bit-plane decoding and the decode GEMV engine
# ------------------------------------------------------------------------------------------
def _upload_block(idx8, q, lut):
    planes = apq.moe_apq_pack(idx8, q)
    pt = _t(planes.view(np.int32))
    lt = _t(np.ascontiguousarray(lut, dtype=np.float16).view(np.int16))
    blk = apq.ApqBlock(pt.data_ptr(), lt.data_ptr(), idx8.shape[0], idx8.shape[1], q, q, 0, 0, 0)
    return blk, (pt, lt)


@pytest.mark.parametrize("q", range(1, 9))
def test_decode_indices_bit_exact(q):
    r = np.random.default_rng(q)
    idx8 = r.integers(0, 256, size=(192, 384), dtype=np.uint8)
    lut = r.standard_normal((192, 1 << q)).astype(np.float16)
    blk, keep = _upload_block(idx8, q, lut)
    out = torch.empty((192, 384), dtype=torch.uint8, device=DEV)
    apq.moe_apq_decode_indices(blk, out)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.committed_index(idx8, q))


@pytest.mark.parametrize("dense", [0, 1], ids=["auto", "mfma"])
@pytest.mark.parametrize("q", range(1, 9))
@pytest.mark.parametrize("T", [1, 2, 3, 5, 16, 17, 40])
@pytest.mark.parametrize("C", [640, 2176])
def test_gemv_matches_oracle(q, T, dense, C):
    """Both product paths (packed-dot VALU below the dense threshold, MFMA at or above it).
    C = 2176 gives every wavefront 4 or 5 chunks, more than the deepest chunk ring holds."""
    say(f"gemv q={q} T={T} dense={dense} C={C}")
    R = 128
    r = np.random.default_rng(q * 100 + T)
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    lut = (np.sort(r.standard_normal((R, 1 << q)), axis=1) * 0.02).astype(np.float16)
    x = r.standard_normal((T, C)).astype(np.float16)
    blk, keep = _upload_block(idx8, q, lut)
    y = torch.empty((T, R), dtype=torch.float32, device=DEV)
    apq.moe_apq_gemv(blk, _t(x), y, dense_threshold=1 if dense else 0)
    ref = oracle.apq_matvec(oracle.committed_index(idx8, q), lut, x.astype(np.float64).T).T
    assert oracle.rel_l2(y.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("q", range(1, 9))
@pytest.mark.parametrize("T", [17, 32, 33, 64, 65, 130])
def test_gemv_wide_passes_match_oracle(q, T):
    """More tokens than one 16-token matrix-core pass: the wide path (one decode of the weights per
    pass, 32-token MFMA tiles, one 32-column word of each chunk per wavefront).  17 and 32 tokens
    take the 32-token pass (two staged loads per chunk, one tile); more take 64-token passes.
    Token counts cover a barely used and a full 32-token pass, one partly used tile of a 64-token
    pass, exactly one pass, one token into a second pass and a ragged third pass; C = 2176 gives 17
    chunks (an odd count for the two-slot ring)."""
    say(f"gemv wide q={q} T={T}")
    R, C = 128, 2176
    r = np.random.default_rng(q * 1000 + T)
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    lut = (np.sort(r.standard_normal((R, 1 << q)), axis=1) * 0.02).astype(np.float16)
    x = r.standard_normal((T, C)).astype(np.float16)
    blk, keep = _upload_block(idx8, q, lut)
    y = torch.empty((T, R), dtype=torch.float32, device=DEV)
    apq.moe_apq_gemv(blk, _t(x), y)
    ref = oracle.apq_matvec(oracle.committed_index(idx8, q), lut, x.astype(np.float64).T).T
    assert oracle.rel_l2(y.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("dense", [1000, 1], ids=["valu", "mfma"])
@pytest.mark.parametrize("q", range(1, 9))
@pytest.mark.parametrize("C", [256, 2048])
def test_gemv_one_hot_probe_is_exact_lut_read(q, dense, C):
    """x = e_c gives y_r = LUT_r[idx_q(r, c)] exactly: pins the decode through the GEMV.
    At C = 2048 every wavefront walks 4 chunks; every column of its last chunk is probed."""
    R = 64
    r = np.random.default_rng(50 + q)
    idx8 = r.integers(0, 256, size=(R, C), dtype=np.uint8)
    lut = r.standard_normal((R, 1 << q)).astype(np.float16)
    if C == 256:
        cols = [0, 1, 31, 32, 77, 128, 200, 255]
    else:
        cols = list(range(384, 512)) + list(range(1920, 2048)) + [0, 1, 700, 1100]
    x = np.zeros((len(cols), C), dtype=np.float16)
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    blk, keep = _upload_block(idx8, q, lut)
    y = torch.empty((len(cols), R), dtype=torch.float32, device=DEV)
    if dense == 1:
        apq.moe_apq_gemv(blk, _t(x), y, dense_threshold=1)
    else:  # the VALU path takes at most 2 tokens per tile at q <= 4, 1 above
        step = 2 if q <= 4 else 1
        for t0 in range(0, len(cols), step):
            apq.moe_apq_gemv(blk, _t(x[t0:t0 + step]), y[t0:t0 + step], dense_threshold=dense)
    idx = oracle.committed_index(idx8, q)
    expect = np.stack([lut[np.arange(R), idx[:, c]].astype(np.float32) for c in cols])
    np.testing.assert_array_equal(y.cpu().numpy(), expect)


# ------------------------------------------------------------------------------------------
# the layer
# ------------------------------------------------------------------------------------------
def _run_layer(shape, inputs, dl, shared_scale=None, threshold=0):
    T = shape.T
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    ss = None if shared_scale is None else _t(shared_scale.astype(np.float32))
    apq.moe_layer_forward(_t(inputs.logits), _t(inputs.x), shape.E, shape.H, shape.I, shape.k, dl.table,
                          y, ws, shared=dl.shared, I_shared=shape.I_shared, shared_scale=ss,
                          prefill_threshold=threshold)
    apq.moe_check_device_error(ws)
    return y.float().cpu().numpy().astype(np.float64), ws


def _check_layer(shape, q_override=None, shared_scale=None, tokens=None, seed=0, threshold=0):
    inputs = wl.gen_layer_inputs(shape, seed)
    dl = gpu_layers.device_layer(shape, q_override=q_override)
    y, _ = _run_layer(shape, inputs, dl, shared_scale, threshold)
    get, sh = gpu_layers.oracle_getters(shape, q_override)
    ref = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh,
                               shared_scale=shared_scale, tokens=tokens)
    rows = slice(None) if tokens is None else list(tokens)
    err = oracle.rel_l2(y[rows], ref["y"][rows])
    say(f"  {shape.name} T={shape.T}: rel L2 = {err:.3e}")
    assert err <= LAYER_TOL
    return y, ref


def test_layer_tiny():
    _check_layer(wl.TINY)


@pytest.mark.parametrize("threshold", [0, 1, 1000], ids=["auto", "all-mfma", "valu-max"])
def test_layer_every_width_in_one_call_ragged_tokens(threshold):
    shape = wl.TINY.replace(H=256, E=12, I=384, k=3, T=21, name="mixed widths 1..8")
    q = np.array([[1 + (2 * e + m) % 8 for m in range(2)] for e in range(shape.E)], dtype=np.uint8)
    _check_layer(shape, q_override=q, threshold=threshold)


@pytest.mark.parametrize("threshold", [0, 1, 1000], ids=["auto", "all-mfma", "valu-max"])
def test_layer_with_shared_expert_and_scale(threshold):
    shape = wl.TINY.replace(H=256, E=8, I=256, k=2, T=19, I_shared=512, q_shared=8, name="shared")
    r = np.random.default_rng(3)
    _check_layer(shape, shared_scale=r.uniform(-1, 2, size=shape.T), threshold=threshold)


@pytest.mark.parametrize("threshold", [0, 1, 1000], ids=["auto", "all-mfma", "valu-max"])
def test_layer_long_down_rows_split_into_segments(threshold):
    """Down rows long enough to be cut into column segments (routed: 26 chunks of 128 columns ->
    2 segments of 13; shared: 41 chunks -> 4 segments of 10/10/10/11, every wavefront share
    ragged), each with its own partial sums, summed by the combine."""
    shape = wl.TINY.replace(H=128, E=6, I=26 * 128, k=2, T=7, I_shared=41 * 128, q_shared=8,
                            name="segmented down rows")
    q = np.array([[3 + (e + m) % 6 for m in range(2)] for e in range(shape.E)], dtype=np.uint8)
    _check_layer(shape, q_override=q, threshold=threshold)


def test_layer_output_at_an_unaligned_address():
    """y given 2 bytes past an 8-byte boundary: the combine stores it element by element, with the
    same values as into an aligned buffer."""
    shape = wl.TINY.replace(H=256, E=8, I=256, k=2, T=9, I_shared=512, q_shared=8, name="unaligned y")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    y_aligned, _ = _run_layer(shape, inputs, dl)
    T = shape.T
    buf = torch.zeros(T * shape.H + 4, dtype=torch.float16, device=DEV)
    y = buf[1:1 + T * shape.H].view(T, shape.H)
    assert y.data_ptr() % 8 == 2
    ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    apq.moe_layer_forward(_t(inputs.logits), _t(inputs.x), shape.E, shape.H, shape.I, shape.k, dl.table,
                          y, ws, shared=dl.shared, I_shared=shape.I_shared)
    apq.moe_check_device_error(ws)
    got = buf.cpu().numpy()
    assert got[0] == 0 and got[-3:].tolist() == [0, 0, 0]   # nothing written outside y
    np.testing.assert_array_equal(y.float().cpu().numpy().astype(np.float64), y_aligned)


def test_layer_k1_and_k_equals_E():
    _check_layer(wl.TINY.replace(k=1, T=9, name="k=1"))
    _check_layer(wl.TINY.replace(k=8, T=6, name="k=E"))


@pytest.mark.parametrize("T", [70, 300, 600], ids=["one-pass", "split-records", "whole-records"])
@pytest.mark.parametrize("threshold", [0, 1000], ids=["auto", "valu-max"])
def test_layer_many_tokens_on_one_expert(threshold, T):
    """More tokens per expert than one matrix-core pass takes.  70 tokens x top-2 over 4 experts
    (about 35 per expert): one wide pass per item, second MFMA tile live.  300 tokens (600 pairs,
    at most the split limit): each hot expert's record is split into 64-token groups, one wide
    pass each, the last group ragged.  600 tokens (1200 pairs, above the split limit): one record
    per expert whose items loop over 64-token passes."""
    shape = wl.TINY.replace(E=4, k=2, T=T, name="hot experts")
    _check_layer(shape, threshold=threshold)


def test_layer_prefill_chunk_every_width_and_shared_expert():
    """A prefill-sized call (530 tokens x top-2 = 1060 pairs, above the record split limit): every
    routed expert and the shared expert meet far more than 16 tokens and run the wide
    matrix-core path over passes of 64 tokens, at every width 1..8, with a shared-expert scale."""
    shape = wl.TINY.replace(H=256, E=6, I=384, k=2, T=530, I_shared=256, q_shared=8,
                            name="prefill chunk")
    q = np.array([[1 + (2 * e + m) % 8 for m in range(2)] for e in range(shape.E)], dtype=np.uint8)
    r = np.random.default_rng(11)
    _check_layer(shape, q_override=q, shared_scale=r.uniform(-1, 2, size=shape.T))


def test_layer_is_deterministic():
    shape = wl.TINY.replace(T=13, name="determinism")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    y1, _ = _run_layer(shape, inputs, dl)
    y2, _ = _run_layer(shape, inputs, dl)
    np.testing.assert_array_equal(y1, y2)


def test_layer_components_match_layer_forward():
    """route -> group -> ffn through the separate entry points equals moe_layer_forward."""
    shape = wl.TINY.replace(T=11, name="components")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    y_full, _ = _run_layer(shape, inputs, dl)
    ids, gates = _route_gpu(inputs.logits, shape.k)
    off, pairs, act, nact = _group_gpu(ids, shape.E)
    y = torch.empty((shape.T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(shape.T, shape.E, shape.H, shape.I, shape.k, 0),
                     dtype=torch.uint8, device=DEV)
    apq.moe_apq_ffn(dl.table, shape.E, shape.H, shape.I, _t(inputs.x), shape.k, off, pairs, act, nact,
                    gates, y, ws)
    np.testing.assert_array_equal(y.float().cpu().numpy(), y_full)


def test_invalid_descriptor_is_reported_not_read():
    shape = wl.TINY.replace(T=4, name="bad descriptor")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    table = dl.table.clone().view(torch.uint8).reshape(shape.E * 2, 32)
    table[:, 24] = 9          # q = 9 on every block
    y = torch.empty((shape.T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(shape.T, shape.E, shape.H, shape.I, shape.k, 0),
                     dtype=torch.uint8, device=DEV)
    apq.moe_layer_forward(_t(inputs.logits), _t(inputs.x), shape.E, shape.H, shape.I, shape.k,
                          table.reshape(-1), y, ws)
    with pytest.raises(apq.MoeError) as ei:
        apq.moe_check_device_error(ws)
    assert ei.value.code == apq.MOE_EDEVICE
    apq.moe_check_device_error(ws)    # cleared by the read


_ws_layers = {}


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 60, 4), (11, 512, 10), (13, 1024, 32), (16, 60, 4),
                                   (16, 1024, 32), (16, 8, 8), (17, 60, 4), (64, 512, 10), (2048, 64, 8),
                                   (1, 1, 1), (9, 128, 1), (5, 3, 3), (16, 2, 2), (40, 1, 1)])
@pytest.mark.parametrize("ties", [False, True], ids=["matmul", "ties"])
def test_layer_workspace_routing_bit_exact(T, E, k, ties):
    """The routing and grouping a moe_layer_forward call computes and leaves in its workspace --
    top-k ids, gates, expert offsets and sorted pairs -- against the oracle, bit for bit (gates
    within 1e-6).  Calls of at most 16 tokens run routing, grouping and the expert records in one
    fused single-workgroup kernel (token x expert slot map); larger ones use the separate routing
    and segmented grouping kernels.  Shapes cover both paths, E from 1 to 1024, k from 1 to 32
    and k = E (every expert active); "ties" rounds the logits to the fp16 grid and plants equal
    and signed-zero logits."""
    say(f"layer workspace routing T={T} E={E} k={k} ties={ties}")
    shape = wl.TINY.replace(H=128, E=E, I=128, k=k, T=T, name="workspace routing")
    if E not in _ws_layers:
        _ws_layers.clear()
        _ws_layers[E] = gpu_layers.device_layer(shape)
    dl = _ws_layers[E]
    inputs = wl.gen_layer_inputs(shape)
    logits = inputs.logits
    if ties:
        r = np.random.default_rng(T * 31 + E)
        logits = (r.standard_normal((T, E)) * 2).astype(np.float16).astype(np.float32)
        logits[0, : min(E, 3 * k)] = 0.5
        if T > 1:
            logits[1, ::2] = -0.0
            logits[1, 1::2] = 0.0
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, E, shape.H, shape.I, k, 0), dtype=torch.uint8, device=DEV)
    apq.moe_layer_forward(_t(logits), _t(inputs.x), E, shape.H, shape.I, k, dl.table, y, ws)
    apq.moe_check_device_error(ws)
    view = apq.moe_workspace_routing(ws, T, E, shape.H, shape.I, k, 0)
    ref_ids, ref_g = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(view["ids"].cpu().numpy().reshape(T, k), ref_ids)
    np.testing.assert_allclose(view["gates"].cpu().numpy().reshape(T, k), ref_g, rtol=0, atol=1e-6)
    r_off, r_pairs, _, _ = oracle.group_by_expert(ref_ids, E)
    np.testing.assert_array_equal(view["offsets"].cpu().numpy(), r_off)
    np.testing.assert_array_equal(view["pairs"].cpu().numpy(), r_pairs)


def _expert_share(shape, inputs, get, e):
    """Gate-weighted output of expert e for the tokens routed to it (float64 [T, H])."""
    ids, gates = oracle.route_topk(inputs.logits, shape.k)
    out = np.zeros((shape.T, shape.H))
    t, j = np.nonzero(ids == e)
    if len(t):
        gi, gq, gl = get(e, wl.GATE_UP)
        di, dq, dl_ = get(e, wl.DOWN)
        o = oracle.expert_ffn(oracle.committed_index(gi, gq), gl, oracle.committed_index(di, dq), dl_,
                              inputs.x[t].astype(np.float64))
        out[t] = gates[t, j][:, None] * o
    return out


@pytest.mark.parametrize("threshold", [0, 1, 1000], ids=["auto", "all-mfma", "valu-max"])
def test_skipped_expert_contributes_zero(threshold):
    """A routed expert whose down block is not GPU-resident is skipped and reported; its tokens
    keep their other experts' terms and the skipped expert adds exactly nothing, so y equals the
    oracle's layer minus that expert's gate-weighted output."""
    shape = wl.TINY.replace(H=256, E=8, I=256, k=2, T=21, I_shared=256, q_shared=8, name="skipped expert")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    e = int(np.bincount(ids.ravel(), minlength=shape.E).argmax())   # the busiest expert
    table = dl.table.clone().view(torch.uint8).reshape(shape.E * 2, 32)
    table[2 * e + 1, 26] = apq.MOE_PAGE_CPU                          # state byte of its down block
    y = torch.empty((shape.T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.full((apq.moe_workspace_bytes(shape.T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),),
                    0x7F, dtype=torch.uint8, device=DEV)   # stale partial sums would show as NaN-like garbage
    ws[:256].zero_()
    apq.moe_layer_forward(_t(inputs.logits), _t(inputs.x), shape.E, shape.H, shape.I, shape.k,
                          table.reshape(-1), y, ws, shared=dl.shared, I_shared=shape.I_shared,
                          prefill_threshold=threshold)
    with pytest.raises(apq.MoeError) as ei:
        apq.moe_check_device_error(ws)
    assert ei.value.code == apq.MOE_EDEVICE
    get, sh = gpu_layers.oracle_getters(shape)
    ref = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh)["y"]
    ref = ref - _expert_share(shape, inputs, get, e)
    err = oracle.rel_l2(y.float().cpu().numpy(), ref)
    say(f"  expert {e} skipped: rel L2 {err:.2e}")
    assert err <= LAYER_TOL


def test_layer_replays_from_a_hip_graph():
    """moe_layer_forward issues no host synchronisation and no memset, so it can be captured;
    every replay (with other eager work between them) equals the eager call bit for bit."""
    shape = wl.TINY.replace(H=256, E=8, I=256, k=2, T=12, I_shared=256, q_shared=8, name="graph")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    y_ref, _ = _run_layer(shape, inputs, dl)
    T = shape.T
    lg, x = _t(inputs.logits), _t(inputs.x)
    y = torch.zeros((T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            apq.moe_layer_forward(lg, x, shape.E, shape.H, shape.I, shape.k, dl.table, y, ws,
                                  shared=dl.shared, I_shared=shape.I_shared, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(3):
        y.zero_()
        ws.fill_(0x5A)          # the replay must not depend on leftovers in its workspace
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.float().cpu().numpy().astype(np.float64), y_ref)
        _run_layer(shape, inputs, dl)   # eager work between replays


@pytest.mark.parametrize("kib", [1, 37, 4096 + 3])
def test_hbm_read_probe_reads_every_word_once(kib):
    """The read-ceiling probe folds each 32-bit word into its sink exactly once: the sink equals
    the XOR of the buffer computed on the host (sizes below, at and above one unit per wavefront)."""
    g = torch.Generator().manual_seed(kib)
    host = torch.randint(-2**31, 2**31 - 1, (kib * 256,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.to(DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    apq.moe_hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


# ------------------------------------------------------------------------------------------
# online routing statistics and the substituted gate mass
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(37, 20, 3), (64, 512, 10), (16, 60, 4), (5, 3, 3), (300, 1024, 32)])
def test_routing_stats_match_oracle_and_accumulate(T, E, k):
    """Counts bit-exact; per-expert masses bit-exact against the oracle run on the same fp32
    gates (both sum in double in ascending pair order); the two totals within 1e-12 (the GPU
    adds the experts' sums in a tree).  Two calls double every accumulator; a quarter of the
    experts resident."""
    say(f"routing stats T={T} E={E} k={k}")
    r = np.random.default_rng(T * 7 + E + k)
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[:, 1] += 3.0   # a hot expert
    ids, gates = _route_gpu(logits, k)
    off, pairs, _, _ = _group_gpu(ids, E)
    resident = (r.random(E) < 0.25).astype(np.uint8)
    count = torch.zeros(E, dtype=torch.int64, device=DEV)
    mass = torch.zeros(E, dtype=torch.float64, device=DEV)
    sums = torch.zeros(2, dtype=torch.float64, device=DEV)
    for _ in range(2):
        apq.moe_routing_stats(off, pairs, gates, T, k, E, count, mass, sums, resident=_t(resident))
    torch.cuda.synchronize()
    g = gates.cpu().numpy().astype(np.float64)
    c_ref, m_ref, s_ref, t_ref = oracle.routing_stats(ids.cpu().numpy(), g, E, resident=resident)
    np.testing.assert_array_equal(count.cpu().numpy(), 2 * c_ref)
    np.testing.assert_array_equal(mass.cpu().numpy(), 2 * m_ref)
    s = sums.cpu().numpy()
    assert abs(s[0] - 2 * s_ref) <= 1e-12 * max(1.0, t_ref) and abs(s[1] - 2 * t_ref) <= 1e-12 * t_ref
    # against the oracle's own float64 routing: the fp32 gates differ by rounding only
    _, m64, s64, t64 = oracle.routing_stats(*oracle.route_topk(logits, k), E, resident=resident)
    np.testing.assert_allclose(mass.cpu().numpy(), 2 * m64, rtol=1e-6, atol=1e-6)
    assert abs(s[1] - 2 * t64) <= 1e-5 * T and abs(s[0] - 2 * s64) <= 1e-5 * T


def test_routing_stats_from_a_layer_calls_workspace():
    """The routing results a moe_layer_forward call leaves in its workspace give the same
    statistics as routing and grouping the same logits separately."""
    shape = wl.QWEN3_NEXT_80B_A3B.replace(H=256, I=256, name="stats from layer")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    _, ws = _run_layer(shape, inputs, dl)
    view = apq.moe_workspace_routing(ws, shape.T, shape.E, shape.H, shape.I, shape.k, shape.I_shared)
    E, T, k = shape.E, shape.T, shape.k
    acc = [torch.zeros(E, dtype=torch.int64, device=DEV), torch.zeros(E, dtype=torch.float64, device=DEV),
           torch.zeros(2, dtype=torch.float64, device=DEV)]
    apq.moe_routing_stats(view["offsets"], view["pairs"], view["gates"], T, k, E, *acc)
    ids, gates = _route_gpu(inputs.logits, k)
    off, pairs, _, _ = _group_gpu(ids, E)
    np.testing.assert_array_equal(view["ids"].cpu().numpy().reshape(T, k), ids.cpu().numpy())
    ref = [torch.zeros_like(a) for a in acc]
    apq.moe_routing_stats(off, pairs, gates, T, k, E, *ref)
    torch.cuda.synchronize()
    for a, b in zip(acc, ref):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
    assert acc[2][0].item() == 0.0   # no resident mask: nothing substituted


# ------------------------------------------------------------------------------------------
# page movement: width changes by a prefix of planes, eviction and return, async copies
# ------------------------------------------------------------------------------------------
def _pinned(a):
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory()


def _layer_unchecked(shape, inputs, dl):
    """One layer call; returns (y float64, device error code or 0)."""
    y = torch.empty((shape.T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(shape.T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    apq.moe_layer_forward(_t(inputs.logits), _t(inputs.x), shape.E, shape.H, shape.I, shape.k, dl.table,
                          y, ws, shared=dl.shared, I_shared=shape.I_shared)
    code = 0
    try:
        apq.moe_check_device_error(ws)
    except apq.MoeError as err:
        code = err.code
    return y.float().cpu().numpy().astype(np.float64), code


def test_page_lower_width_then_reload_beside_layer_calls():
    """A width change through the library's page calls (PagedWeight: nested widths, asynchronous
    offload and reload, commits at safe boundaries).  One routed gate_up block goes from q = 6 to
    q = 3 with moe_page_offload (same planes, the width-3 LUT already on the device): its planes
    3..5 are copied to pinned host memory on a side stream, and the layer matches the oracle at
    width 3.  Once the copy event has completed the freed planes are overwritten (reused).
    moe_page_reload copies them back with the width-6 LUT on the side stream; a layer call
    issued before the commit still runs at width 3 (bit for bit the same output); after
    moe_page_commit the layer matches the oracle at width 6."""
    shape = wl.TINY.replace(H=256, E=6, I=256, k=2, T=12, name="page width change")
    q6 = np.full((shape.E, 2), 6, dtype=np.uint8)
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape, q_override=q6)
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    e, m = int(ids[0, 0]), wl.GATE_UP
    index = 2 * e + m
    blk = dl.block(e, m)
    idx8 = wl.gen_parent_indices(shape, e, m)
    pb = blk.rows * blk.cols // 8
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()

    def check(qmap):
        y, code = _layer_unchecked(shape, inputs, dl)
        assert code == 0
        get, sh = gpu_layers.oracle_getters(shape, qmap)
        err = oracle.rel_l2(y, oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh)["y"])
        say(f"  widths of expert {e}: {qmap[e]}: rel L2 {err:.2e}")
        assert err <= LAYER_TOL
        return y

    lut3 = _t(np.ascontiguousarray(wl.gen_lut(shape, e, m, 3), dtype=np.float16).view(np.int16))
    low = apq.ApqBlock(blk.planes, lut3.data_ptr(), blk.rows, blk.cols, 3, 6, apq.MOE_PAGE_GPU, 0, 0)
    host_planes = torch.zeros(6 * pb, dtype=torch.uint8).pin_memory()
    apq.moe_page_offload(dl.table, index, blk, low, host_planes, None, ev, side)
    q3 = q6.copy()
    q3[e, m] = 3
    y3 = check(q3)
    ev.synchronize()
    packed = apq.moe_apq_pack(idx8, 6).view(np.uint8)
    np.testing.assert_array_equal(host_planes.numpy()[3 * pb:], packed[3 * pb:])
    off = blk.planes - dl.arena.data_ptr()
    dl.arena[off + 3 * pb: off + 6 * pb].fill_(0xA5)          # the freed planes are reused
    torch.cuda.synchronize()

    lut6_host = _pinned(np.ascontiguousarray(wl.gen_lut(shape, e, m, 6), dtype=np.float16).view(np.int16))
    lut6_dev = torch.empty(blk.rows * 64, dtype=torch.int16, device=DEV)
    tgt = apq.ApqBlock(blk.planes, lut6_dev.data_ptr(), blk.rows, blk.cols, 6, 6, apq.MOE_PAGE_GPU, 0, 0)
    apq.moe_page_reload(dl.table, index, low, tgt, _pinned(packed), lut6_host, ev, side)
    y3b, code = _layer_unchecked(shape, inputs, dl)          # before the commit: still width 3
    assert code == 0
    np.testing.assert_array_equal(y3b, y3)
    apq.moe_page_commit(dl.table, index, tgt, ev)
    check(q6)


def test_page_evict_to_host_and_bring_back():
    """Eviction and return of a routed down block (PagedWeight: pages GPU-resident, CPU-resident
    or in transfer).  moe_page_offload to MOE_PAGE_CPU copies its planes and LUT to pinned host
    memory; layer calls then skip the expert, report MOE_EDEVICE, and give the oracle's layer
    minus that expert's share.  The device memory is overwritten (reused), moe_page_reload brings
    the block back from the host copies: until moe_page_commit the block is in transfer (same
    skipped output, same report); after it the layer matches the oracle in full."""
    shape = wl.TINY.replace(H=256, E=6, I=256, k=2, T=12, name="page evict")
    q6 = np.full((shape.E, 2), 6, dtype=np.uint8)
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape, q_override=q6)
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    e = int(np.bincount(ids.ravel(), minlength=shape.E).argmax())
    m = wl.DOWN
    index = 2 * e + m
    blk = dl.block(e, m)
    pb = blk.rows * blk.cols // 8
    lb = blk.rows * 64 * 2
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    get, sh = gpu_layers.oracle_getters(shape, q6)
    full = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh)["y"]
    without = full - _expert_share(shape, inputs, get, e)

    host_planes = torch.zeros(6 * pb, dtype=torch.uint8).pin_memory()
    host_lut = torch.zeros(lb, dtype=torch.uint8).pin_memory()
    evicted = apq.ApqBlock(blk.planes, blk.lut, blk.rows, blk.cols, 6, 6, apq.MOE_PAGE_CPU, 0, 0)
    apq.moe_page_offload(dl.table, index, blk, evicted, host_planes, host_lut, ev, side)
    y_out, code = _layer_unchecked(shape, inputs, dl)
    assert code == apq.MOE_EDEVICE
    err = oracle.rel_l2(y_out, without)
    say(f"  expert {e} evicted: rel L2 vs the layer without it {err:.2e}")
    assert err <= LAYER_TOL
    ev.synchronize()
    np.testing.assert_array_equal(host_planes.numpy(),
                                  apq.moe_apq_pack(wl.gen_parent_indices(shape, e, m), 6).view(np.uint8))
    np.testing.assert_array_equal(host_lut.numpy().view(np.float16),
                                  np.ascontiguousarray(wl.gen_lut(shape, e, m, 6), dtype=np.float16).ravel())
    po, lo = blk.planes - dl.arena.data_ptr(), blk.lut - dl.arena.data_ptr()
    dl.arena[po: po + 6 * pb].fill_(0x5A)                     # the device pages are reused
    dl.arena[lo: lo + lb].fill_(0x5A)
    torch.cuda.synchronize()

    apq.moe_page_reload(dl.table, index, evicted, blk, host_planes, host_lut, ev, side)
    y_mid, code = _layer_unchecked(shape, inputs, dl)         # in transfer: still skipped
    assert code == apq.MOE_EDEVICE
    np.testing.assert_array_equal(y_mid, y_out)
    apq.moe_page_commit(dl.table, index, blk, ev)
    y_back, code = _layer_unchecked(shape, inputs, dl)
    assert code == 0
    err = oracle.rel_l2(y_back, full)
    say(f"  expert {e} back: rel L2 {err:.2e}")
    assert err <= LAYER_TOL


# ------------------------------------------------------------------------------------------
# residency-aware substitution and background admission
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("policy", [0, 1, 2], ids=["fetch-all", "gate-rule", "first-choice"])
@pytest.mark.parametrize("T,E,k", [(24, 32, 4), (64, 512, 10), (9, 1024, 32), (16, 60, 4), (3, 5, 3)])
def test_substitution_and_admission_bit_exact(policy, T, E, k):
    """Substituted ids, the missed and fetch outputs and three calls of background admission
    match the oracle bit for bit.  The oracle takes the GPU's fp32 gates and the fp32 threshold,
    so the 0.15 decision is made in the kernel's precision on both sides."""
    say(f"substitute policy={policy} T={T} E={E} k={k}")
    r = np.random.default_rng(policy * 1000 + T + E + k)
    logits = r.standard_normal((T, E)).astype(np.float32)
    logits[:, 2] += 2.0
    resident = (r.random(E) < 0.3).astype(np.uint8)
    thr = float(np.float32(0.15))
    lt = _t(logits)
    acc = torch.zeros(E, dtype=torch.float32, device=DEV)
    adm = torch.zeros(E, dtype=torch.uint8, device=DEV)
    acc_ref = np.zeros(E, np.float32)
    for call in range(3):
        ids, gates = _route_gpu(logits, k)
        ids0 = ids.cpu().numpy()
        missed = torch.empty((T, k), dtype=torch.int32, device=DEV)
        fetch = torch.empty(E, dtype=torch.uint8, device=DEV)
        apq.moe_substitute(lt, _t(resident), policy, ids, gates, missed, fetch, gate_threshold=thr,
                           admit_mass=acc, admit=adm)
        torch.cuda.synchronize()
        g = gates.cpu().numpy()
        new_ref, missed_ref, fetch_ref = oracle.substitute(logits, ids0, g.astype(np.float64), resident,
                                                           policy, gate_threshold=thr)
        np.testing.assert_array_equal(ids.cpu().numpy(), new_ref)
        np.testing.assert_array_equal(missed.cpu().numpy(), missed_ref)
        np.testing.assert_array_equal(fetch.cpu().numpy().astype(bool), fetch_ref)
        acc_ref, adm_ref = oracle.admit(missed_ref, g, acc_ref)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)
        np.testing.assert_array_equal(adm.cpu().numpy().astype(bool), adm_ref)


def test_substituted_layer_matches_oracle_on_substituted_routing():
    """Route, substitute (first-choice rule, a third of the experts resident), group and run the
    FFN through the component calls: the output equals the oracle's layer evaluated on the
    substituted ids with the original gates."""
    shape = wl.TINY.replace(H=256, E=12, I=256, k=3, T=10, name="substituted layer")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    T, E, k = shape.T, shape.E, shape.k
    resident = (np.arange(E) % 3 == 0).astype(np.uint8)
    ids, gates = _route_gpu(inputs.logits, k)
    missed = torch.empty((T, k), dtype=torch.int32, device=DEV)
    fetch = torch.empty(E, dtype=torch.uint8, device=DEV)
    apq.moe_substitute(_t(inputs.logits), _t(resident), apq.MOE_POLICY_FIRST_CHOICE, ids, gates,
                       missed, fetch)
    off, pairs, act, nact = _group_gpu(ids, E)
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, E, shape.H, shape.I, k, 0), dtype=torch.uint8, device=DEV)
    apq.moe_apq_ffn(dl.table, E, shape.H, shape.I, _t(inputs.x), k, off, pairs, act, nact, gates, y, ws)
    apq.moe_check_device_error(ws)
    sub_ids = ids.cpu().numpy()
    g = gates.cpu().numpy().astype(np.float64)
    assert (missed.cpu().numpy() >= 0).any()
    get, _ = gpu_layers.oracle_getters(shape)
    # the oracle layer on fixed routing: logits that select exactly sub_ids with gates g
    ref = np.zeros((T, shape.H))
    x64 = inputs.x.astype(np.float64)
    for t in range(T):
        for j in range(k):
            e = int(sub_ids[t, j])
            gi, gq, gl = get(e, wl.GATE_UP)
            di, dq, dlut = get(e, wl.DOWN)
            ref[t] += g[t, j] * oracle.expert_ffn(oracle.committed_index(gi, gq), gl,
                                                  oracle.committed_index(di, dq), dlut, x64[t:t + 1])[0]
    err = oracle.rel_l2(y.float().cpu().numpy().astype(np.float64), ref)
    say(f"  substituted layer rel L2 {err:.2e}")
    assert err <= LAYER_TOL


def _lynx_gpu(logits, ids, bin_width=None):
    T, k = ids.shape
    E = logits.shape[1]
    remapped = torch.empty((T, k), dtype=torch.int32, device=DEV)
    critical = torch.empty(E, dtype=torch.uint8, device=DEV)
    apq.moe_lynx_remap(_t(logits), ids, remapped, critical, bin_width=bin_width)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), remapped.cpu().numpy(), critical.cpu().numpy().astype(bool)


def test_lynx_negative_gap_on_gpu():
    """Ids out of routing order (a negative top-2 gap) take bin 0 in the kernel as in the oracle:
    the hand case of the oracle pins, through the kernel."""
    logits = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -1.0],
                       [0.5, -1.0, 3.0, 2.875, 0.0, -1.0]], dtype=np.float32)
    ids = _t(np.array([[1, 0], [2, 3]], dtype=np.int32))
    new, remapped, critical = _lynx_gpu(logits, ids)
    np.testing.assert_array_equal(new, [[1, 2], [2, 1]])
    np.testing.assert_array_equal(remapped, [[-1, 0], [-1, 3]])
    np.testing.assert_array_equal(critical, [False, True, True, False, False, False])


@pytest.mark.parametrize("T,E,k,kind", [(16, 60, 4, "matmul"), (64, 512, 10, "zipf"), (32, 8, 2, "matmul"),
                                        (37, 1024, 32, "normal"), (5, 64, 1, "normal"),
                                        (200, 128, 6, "flat"), (1, 3, 3, "normal")])
def test_lynx_remap_bit_exact(T, E, k, kind):
    """Remapped ids, the remapped-slot outputs and the critical set match the oracle bit for bit,
    on the GPU's own routing (itself checked against the oracle).  The bin decision is an fp32
    subtraction and an IEEE fp32 division on both sides.  Shapes: the Qwen1.5 and Qwen3-Next
    (Zipf router) decode batches, a Mixtral-like 8-expert batch, the largest E and k, k = 1
    (nothing remapped), low-confidence batches (small logit spread: many tokens in bin 0) and
    k = E."""
    say(f"lynx T={T} E={E} k={k} {kind}")
    r = np.random.default_rng(T * 7 + E + k)
    if kind == "matmul":
        shape = wl.TINY.replace(H=512, E=E, k=k, T=T, router_std=0.02, name="lynx")
        logits = wl.gen_layer_inputs(shape).logits
    elif kind == "zipf":
        logits = wl.gen_layer_inputs(wl.QWEN3_NEXT_80B_A3B).logits
    elif kind == "flat":
        logits = (r.standard_normal((T, E)) * 0.05).astype(np.float32)
    else:
        logits = r.standard_normal((T, E)).astype(np.float32)
    ids, _ = _route_gpu(logits, k)
    ids0 = ids.cpu().numpy()
    ref_ids, _ = oracle.route_topk(logits, k)
    np.testing.assert_array_equal(ids0, ref_ids)
    w = np.float32(k) / np.float32(E)
    new, remapped, critical = _lynx_gpu(logits, ids)
    new_ref, rem_ref, crit_ref = oracle.lynx_remap(logits, ids0, w)
    np.testing.assert_array_equal(new, new_ref)
    np.testing.assert_array_equal(remapped, rem_ref)
    np.testing.assert_array_equal(critical, crit_ref)
    say(f"  distinct experts {len(set(ids0.ravel()))} -> {len(set(new.ravel()))}, "
        f"remapped slots {(remapped >= 0).sum()}")


def test_lynx_hand_example_and_bin_boundaries_on_gpu():
    """The oracle's hand example (6 -> 4 distinct experts) and a gap exactly at the bin width
    (bin 1) next to the fp32 value just below it (bin 0), through the kernel."""
    logits = np.array([[2.0, 1.0, 0.5, 0.0, -1.0, -1.0],
                       [0.5, -1.0, 3.0, 2.875, 0.0, -1.0],
                       [-1.0, 0.25, -1.0, -1.0, 1.5, 1.25]], dtype=np.float32)
    ids, _ = _route_gpu(logits, 2)
    new, remapped, critical = _lynx_gpu(logits, ids)
    np.testing.assert_array_equal(new, [[0, 1], [2, 0], [4, 1]])
    np.testing.assert_array_equal(remapped, [[-1, -1], [-1, 3], [-1, 5]])
    np.testing.assert_array_equal(critical, [True, True, True, False, True, False])
    w = np.float32(2) / np.float32(6)
    lg = np.full((2, 6), -5.0, dtype=np.float32)
    lg[0, 0], lg[0, 1], lg[0, 2] = w, 0.0, -0.5
    lg[1, 3], lg[1, 4], lg[1, 2] = np.nextafter(w, np.float32(0)), 0.0, -0.25
    ids, _ = _route_gpu(lg, 2)
    ids0 = ids.cpu().numpy()
    new, remapped, critical = _lynx_gpu(lg, ids)
    new_ref, rem_ref, crit_ref = oracle.lynx_remap(lg, ids0, w)
    _, bins, _ = oracle.lynx_bins(lg, ids0, w)
    np.testing.assert_array_equal(bins, [1, 0])
    np.testing.assert_array_equal(new, new_ref)
    np.testing.assert_array_equal(remapped, rem_ref)
    np.testing.assert_array_equal(critical, crit_ref)


def test_lynx_remapped_layer_matches_oracle():
    """Route, remap (LYNX), group and run the FFN through the component calls: the output equals
    the oracle's layer evaluated on the remapped ids with the original gates."""
    shape = wl.TINY.replace(H=256, E=16, I=256, k=4, T=12, router_std=0.01, name="lynx layer")
    inputs = wl.gen_layer_inputs(shape)
    dl = gpu_layers.device_layer(shape)
    T, E, k = shape.T, shape.E, shape.k
    ids, gates = _route_gpu(inputs.logits, k)
    new, remapped, _ = _lynx_gpu(inputs.logits, ids)
    assert (remapped >= 0).any()
    off, pairs, act, nact = _group_gpu(ids, E)
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, E, shape.H, shape.I, k, 0), dtype=torch.uint8, device=DEV)
    apq.moe_apq_ffn(dl.table, E, shape.H, shape.I, _t(inputs.x), k, off, pairs, act, nact, gates, y, ws)
    apq.moe_check_device_error(ws)
    g = gates.cpu().numpy().astype(np.float64)
    get, _ = gpu_layers.oracle_getters(shape)
    ref = np.zeros((T, shape.H))
    x64 = inputs.x.astype(np.float64)
    for t in range(T):
        for j in range(k):
            e = int(new[t, j])
            gi, gq, gl = get(e, wl.GATE_UP)
            di, dq, dlut = get(e, wl.DOWN)
            ref[t] += g[t, j] * oracle.expert_ffn(oracle.committed_index(gi, gq), gl,
                                                  oracle.committed_index(di, dq), dlut, x64[t:t + 1])[0]
    err = oracle.rel_l2(y.float().cpu().numpy().astype(np.float64), ref)
    say(f"  LYNX-remapped layer rel L2 {err:.2e}")
    assert err <= LAYER_TOL


@pytest.mark.parametrize("threshold", [0, 2], ids=["auto", "mfma-from-2"])
def test_streaming_token_counts_and_ring_switches(threshold):
    """Routing built so that experts 0-3 get 1 token, 4-7 get 2, 8-11 get 3 and 12-15 get 4 (top-2
    over 20 tokens), at every width 1..8 (the two modules of an expert at different widths): the
    1-token items stream at every width, the 2-token items at widths <= 4 (the ring loads 1 or 2
    activation rows by token count) and take the matrix-core branch above, the 3- and 4-token
    items take the matrix-core branch; the record step orders each module's streaming items by
    count, so the two modules of one expert can sit in different classes, and a stream ends where
    the next item's width or count does not fit its ring.  With the switch at 2 tokens only the
    single tokens stream.  Output against the oracle."""
    E, k = 16, 2
    mult = [1] * 4 + [2] * 4 + [3] * 4 + [4] * 4
    slots = [e for e in range(E) for _ in range(mult[e])]          # 40 (token, slot) pairs
    T = len(slots) // k
    # deal the pairs to tokens so that each token's two experts differ: token t takes slots t
    # and t + T of the expert list (the list is sorted, so the two halves never coincide)
    r = np.random.default_rng(7)
    logits = (r.standard_normal((T, E)) * 0.1).astype(np.float32)
    for t in range(T):
        a, b = slots[t], slots[t + T]
        assert a != b
        logits[t, a] = 5.0
        logits[t, b] = 4.0
    ids, _ = oracle.route_topk(logits, k)
    counts = np.bincount(ids.ravel(), minlength=E)
    np.testing.assert_array_equal(counts, mult)
    shape = wl.TINY.replace(H=256, E=E, I=384, k=k, T=T, name="token-count rings")
    q = np.array([[1 + (e + 3 * m) % 8 for m in range(2)] for e in range(E)], dtype=np.uint8)
    inputs = dataclasses.replace(wl.gen_layer_inputs(shape), logits=logits)
    dl = gpu_layers.device_layer(shape, q_override=q)
    y, _ = _run_layer(shape, inputs, dl, threshold=threshold)
    get, _ = gpu_layers.oracle_getters(shape, q)
    ref = oracle.layer_forward(inputs.x, logits, k, get)
    err = oracle.rel_l2(y, ref["y"])
    say(f"  token-count rings (threshold {threshold}): rel L2 {err:.2e}")
    assert err <= LAYER_TOL
