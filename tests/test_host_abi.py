"""The C-ABI library on the CPU: it loads, exports every declared symbol, its host packer agrees
with the oracle's own writer and reader of the plane layout, and it rejects bad arguments before
touching the GPU.  No compute call here needs a GPU."""
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_apq.h")

apq = pytest.importorskip("any_precision_expert_router_amd",
                          reason="libmoe_apq.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"moe_route_topk", "moe_group_by_expert", "moe_apq_ffn", "moe_layer_forward"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", apq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(apq.EXPORTED) == set(names)
    for n in names:
        getattr(apq.lib(), n)


@pytest.mark.parametrize("q", range(1, 9))
@pytest.mark.parametrize("shape", [(64, 128), (128, 384), (192, 256)])
def test_host_packer_matches_oracle_layout(q, shape):
    r = np.random.default_rng(q * 1000 + shape[0] + shape[1])
    idx8 = r.integers(0, 256, size=shape, dtype=np.uint8)
    lib_planes = apq.moe_apq_pack(idx8, q)
    np.testing.assert_array_equal(lib_planes, oracle.pack_planes(idx8, q))
    np.testing.assert_array_equal(oracle.unpack_planes(lib_planes, *shape, q), idx8 >> (8 - q))


def test_host_packer_threaded_path_and_plane_drop():
    r = np.random.default_rng(7)
    idx8 = r.integers(0, 256, size=(1024, 2048), dtype=np.uint8)   # large enough to use threads
    p8 = apq.moe_apq_pack(idx8, 8)
    np.testing.assert_array_equal(oracle.unpack_planes(p8, 1024, 2048, 8), idx8)
    per_plane = 1024 * 2048 // 32
    np.testing.assert_array_equal(apq.moe_apq_pack(idx8, 3), p8[: 3 * per_plane])


def test_host_packer_rejects_bad_arguments():
    lib = apq.lib()
    buf = np.zeros(64 * 128, dtype=np.uint8)
    out = np.zeros(64 * 128, dtype=np.uint32)
    assert lib.moe_apq_pack(buf.ctypes.data, 64, 96, 4, out.ctypes.data) == apq.MOE_EINVAL
    assert lib.moe_apq_pack(buf.ctypes.data, 48, 128, 4, out.ctypes.data) == apq.MOE_EINVAL
    assert lib.moe_apq_pack(buf.ctypes.data, 64, 128, 0, out.ctypes.data) == apq.MOE_EINVAL
    assert lib.moe_apq_pack(buf.ctypes.data, 64, 128, 9, out.ctypes.data) == apq.MOE_EINVAL
    assert lib.moe_apq_pack(None, 64, 128, 4, out.ctypes.data) == apq.MOE_EINVAL
    assert b"rows" in lib.moe_last_error() or b"NULL" in lib.moe_last_error()


def test_argument_validation_happens_before_any_launch():
    lib = apq.lib()
    fake = 0x1000  # never dereferenced: every call below must fail validation first
    assert lib.moe_route_topk(fake, 4, 8, 9, fake, fake, None) == apq.MOE_EINVAL          # k > E
    assert lib.moe_route_topk(fake, 4, 2048, 2, fake, fake, None) == apq.MOE_EUNSUPPORTED  # E > 1024
    assert lib.moe_route_topk(fake, 4, 64, 33, fake, fake, None) == apq.MOE_EUNSUPPORTED   # k > 32
    assert lib.moe_route_topk(fake, -1, 8, 2, fake, fake, None) == apq.MOE_EINVAL
    assert lib.moe_route_topk(None, 3, 8, 2, fake, fake, None) == apq.MOE_EINVAL
    assert lib.moe_route_topk(fake, 0, 8, 2, fake, fake, None) == apq.MOE_OK              # T = 0: no-op
    # layer: H not a multiple of 128, then a too-small workspace
    assert lib.moe_layer_forward(fake, fake, 4, 8, 96, 256, 2, fake, None, 0, None, 0, fake, fake,
                                 1 << 20, None) == apq.MOE_EINVAL
    need = lib.moe_workspace_bytes(4, 8, 128, 256, 2, 0)
    assert need > 0
    assert lib.moe_layer_forward(fake, fake, 4, 8, 128, 256, 2, fake, None, 0, None, 0, fake, fake,
                                 need - 1, None) == apq.MOE_EWORKSPACE
    assert lib.moe_layer_forward(fake, fake, 4, 8, 128, 256, 2, fake, fake, 100, None, 0, fake, fake,
                                 need, None) == apq.MOE_EINVAL                           # I_shared % 128
    assert lib.moe_apq_ffn(fake, 8, 128, 256, fake, 4, 2, fake, fake, fake, fake, fake, None, 0, None, 0,
                           fake, None, 0, None) == apq.MOE_EWORKSPACE
    assert lib.moe_layer_forward(fake, fake, 0, 8, 128, 256, 2, fake, None, 0, None, 0, fake, None, 0,
                                 None) == apq.MOE_OK                                     # T = 0
    # LYNX remap: bin width must be finite (<= 0 selects k/E); outputs must be given
    assert lib.moe_lynx_remap(fake, 4, 8, 2, 0.0, fake, None, fake, None) == apq.MOE_EINVAL
    assert lib.moe_lynx_remap(fake, 4, 8, 2, float("nan"), fake, fake, fake, None) == apq.MOE_EINVAL
    assert lib.moe_lynx_remap(fake, 4, 8, 2, float("inf"), fake, fake, fake, None) == apq.MOE_EINVAL
    assert lib.moe_lynx_remap(fake, 4, 8, 2, 0.25, fake, None, fake, None) == apq.MOE_EINVAL
    assert lib.moe_lynx_remap(fake, 4, 8, 2, 0.25, fake, fake, None, None) == apq.MOE_EINVAL
    assert lib.moe_lynx_remap(fake, 4, 8, 9, 0.25, fake, fake, fake, None) == apq.MOE_EINVAL    # k > E
    assert lib.moe_lynx_remap(fake, 4, 2048, 2, 0.25, fake, fake, fake, None) == apq.MOE_EUNSUPPORTED
    blk = apq.ApqBlock(fake, fake, 64, 100, 4, 4, 0, 0, 0)
    assert lib.moe_apq_decode_indices(apq.ctypes.byref(blk), fake, None) == apq.MOE_EINVAL
    blk = apq.ApqBlock(fake, fake, 64, 128, 9, 4, 0, 0, 0)
    assert lib.moe_apq_gemv(apq.ctypes.byref(blk), fake, 1, fake, 0, None) == apq.MOE_EINVAL
    blk = apq.ApqBlock(fake + 4, fake, 64, 128, 4, 4, 0, 0, 0)
    assert lib.moe_apq_gemv(apq.ctypes.byref(blk), fake, 1, fake, 0, None) == apq.MOE_EINVAL  # alignment


def test_workspace_bytes_cover_the_sections():
    lib = apq.lib()
    T, E, H, I, k, Ish = 16, 60, 2048, 1408, 4, 5632
    n = lib.moe_workspace_bytes(T, E, H, I, k, Ish)
    need = T * k * I * 2 + T * Ish * 2 + T * k * H * 4 + T * H * 4 + 3 * T * k * 4 + (2 * E + 1) * 4
    assert n >= need and n % 256 == 0
    assert lib.moe_workspace_bytes(T, E, H, I, k, 0) < n
    assert lib.moe_workspace_bytes(-1, E, H, I, k, 0) == 0
    # the shared expert's 44-chunk down rows are cut into 4 column segments, each with its own
    # fp32 partial sums [T][H]
    assert n - lib.moe_workspace_bytes(T, E, H, I, k, 0) >= T * Ish * 2 + 4 * T * H * 4


def test_workspace_routing_addresses_lie_inside_the_workspace():
    """moe_workspace_routing is host-only: with a made-up base address it returns the addresses
    of the ids, gates, offsets and pairs sections, disjoint, 4-byte aligned and inside the
    workspace; a short workspace and bad shapes are rejected."""
    import ctypes
    lib = apq.lib()
    T, E, H, I, k, Ish = 16, 60, 2048, 1408, 4, 5632
    n = lib.moe_workspace_bytes(T, E, H, I, k, Ish)
    base = 1 << 40
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    rc = lib.moe_workspace_routing(base, n, T, E, H, I, k, Ish, *[ctypes.byref(p) for p in ptrs])
    assert rc == apq.MOE_OK
    spans = sorted((p.value, p.value + size) for p, size in
                   zip(ptrs, [4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k]))
    for lo, hi in spans:
        assert base <= lo < hi <= base + n and lo % 4 == 0
    for (lo0, hi0), (lo1, hi1) in zip(spans, spans[1:]):
        assert hi0 <= lo1
    assert lib.moe_workspace_routing(base, n - 1, T, E, H, I, k, Ish,
                                     *[ctypes.byref(p) for p in ptrs]) == apq.MOE_EWORKSPACE
    assert lib.moe_workspace_routing(base, n, T, 0, H, I, k, Ish,
                                     *[ctypes.byref(p) for p in ptrs]) == apq.MOE_EINVAL
    assert lib.moe_routing_stats(None, None, None, T, k, E, None, None, None, None, None) == apq.MOE_EINVAL


def test_native_width_planner_matches_oracle():
    """moe_plan_widths (host C++, heap) against the oracle's plain greedy loop: same plan and
    bytes saved, bit for bit, on random instances with floors, multipliers, ties and targets
    from zero to unreachable."""
    r = np.random.default_rng(8)
    for trial in range(200):
        n = int(r.integers(0, 12))
        rows = r.choice([64, 128, 2816], n).astype(np.int32)
        cols = r.choice([128, 1408, 2048], n).astype(np.int32)
        qc = r.integers(1, 9, n).astype(np.uint8)
        fl = np.minimum(qc, r.integers(1, 6, n)).astype(np.uint8)
        dmg = np.cumsum(r.random((n, 8))[:, ::-1], axis=1)[:, ::-1].astype(np.float32)
        if trial % 5 == 0 and n:
            dmg[:] = 1.0          # all steps free: ties everywhere, decided by block index
        mult = r.uniform(0.5, 3.0, n).astype(np.float32)
        full = sum(oracle.block_bytes(rows[i], cols[i], qc[i]) - oracle.block_bytes(rows[i], cols[i], fl[i])
                   for i in range(n))
        target = int(r.integers(0, full + 4000)) if trial % 7 else full + 1
        q, saved = apq.moe_plan_widths(qc, fl, rows, cols, dmg, mult, target)
        q_ref, saved_ref = oracle.plan_widths(qc, fl, rows, cols, dmg.astype(np.float64),
                                              mult.astype(np.float64), target)
        np.testing.assert_array_equal(q, q_ref)
        assert saved == saved_ref


def test_native_width_planner_rejects_bad_arguments():
    ok = dict(q_cur=[4], q_floor=[2], rows=[64], cols=[128], damage=np.zeros((1, 8)), mult=[1.0])
    apq.moe_plan_widths(**ok, target_bytes=1)
    for bad in (dict(q_floor=[5]), dict(q_cur=[9], q_floor=[1]), dict(rows=[60]), dict(cols=[100]),
                dict(mult=[0.0])):
        with pytest.raises(apq.MoeError):
            apq.moe_plan_widths(**{**ok, **bad}, target_bytes=1)


def test_activation_arrays_of_4_gib_are_refused():
    """The FFN kernels address x [T][H], act [T*k][I] and act_shared [T][I_shared] with 32-bit
    byte offsets: a call whose arrays reach 4 GiB is refused with MOE_EUNSUPPORTED before any
    launch (just below the limit it proceeds to the workspace check)."""
    lib = apq.lib()
    fake = 0x1000
    T = 65536

    def layer(H, I, k, Ish=0, shared=None):
        return lib.moe_layer_forward(fake, fake, T, 64, H, I, k, fake, shared, Ish, None, 0, fake, fake,
                                     1 << 20, None)

    assert layer(32768, 128, 2) == apq.MOE_EUNSUPPORTED                  # x: T*H*2 = 4 GiB
    assert layer(32640, 128, 2) == apq.MOE_EWORKSPACE                    # x just below
    assert layer(4096, 8192, 8) == apq.MOE_EUNSUPPORTED                  # act: 8.6 GB
    assert layer(4096, 1024, 32) == apq.MOE_EUNSUPPORTED                 # act: exactly 4 GiB
    assert layer(4096, 896, 32) == apq.MOE_EWORKSPACE                    # act: 3.76 GB
    assert layer(4096, 128, 2, Ish=32768, shared=fake) == apq.MOE_EUNSUPPORTED   # act_shared
    assert b"4 GiB" in lib.moe_last_error()
    assert lib.moe_apq_ffn(fake, 64, 4096, 8192, fake, T, 8, fake, fake, fake, fake, fake, None, 0, None,
                           0, fake, fake, 1 << 20, None) == apq.MOE_EUNSUPPORTED
    blk = apq.ApqBlock(fake, fake, 64, 32768, 4, 4, 0, 0, 0)
    assert lib.moe_apq_gemv(apq.ctypes.byref(blk), fake, T, fake, 0, None) == apq.MOE_EUNSUPPORTED


def test_commit_refuses_indices_outside_the_table_and_repeats():
    """moe_commit_blocks knows the table's length: an index past it, or one entry named twice in
    one commit (whose winner would depend on thread timing), is refused before any launch."""
    lib = apq.lib()
    fake = 0x1000
    ok = apq.ApqBlock(fake, fake, 64, 128, 4, 4, 0, 0, 0)

    def commit(index, table_len=8):
        n = len(index)
        idx = (apq.ctypes.c_int32 * n)(*index)
        arr = (apq.ApqBlock * n)(*([ok] * n))
        return lib.moe_commit_blocks(fake, table_len, idx, arr, n, None)

    assert commit([8]) == apq.MOE_EINVAL
    assert b"outside the table" in lib.moe_last_error()
    assert commit([-1]) == apq.MOE_EINVAL
    assert commit([3, 5, 3]) == apq.MOE_EINVAL
    assert b"repeats" in lib.moe_last_error()
    assert commit([0], table_len=0) == apq.MOE_EINVAL
    assert lib.moe_commit_blocks(fake, 8, None, None, 0, None) == apq.MOE_OK   # nothing to do


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except ImportError:  # pragma: no cover
        return False


def test_page_state_machine_allows_exactly_the_documented_moves():
    """The host rules of moe_page_reload / moe_page_offload over every (current state, target
    state, width step, planes, LUT) combination: a move the rules forbid is refused with
    MOE_EINVAL before anything is issued; an allowed one passes validation and reaches its first
    device call (on a machine without a GPU that call fails with MOE_EHIP, which is how the test
    tells the two apart).  Allowed: GPU -> GPU at a higher width (same planes, new LUT), CPU ->
    GPU (through IN_TRANSFER); GPU -> CPU, GPU -> GPU at a lower width (same planes).  Refused:
    anything from IN_TRANSFER, a reload to a width that does not grow or with other planes or
    the LUT still in use, an offload to a width that does not shrink, to IN_TRANSFER or of a
    block that is not resident."""
    if _gpu_visible():
        pytest.skip("the allowed moves would launch on the GPU with made-up pointers")
    lib = apq.lib()
    byref = apq.ctypes.byref
    P0, P1, L0, L1, fake = 0x10000, 0x20000, 0x30000, 0x40000, 0x1000
    GPU, CPU, XFER = apq.MOE_PAGE_GPU, apq.MOE_PAGE_CPU, apq.MOE_PAGE_IN_TRANSFER

    def blk(planes, lut, q, state):
        return apq.ApqBlock(planes, lut, 64, 128, q, q, state, 0, 0)

    def reload(cur, tgt, index=1):
        return lib.moe_page_reload(fake, 4, index, byref(cur), byref(tgt), fake, fake, fake, None, None)

    def offload(cur, tgt, index=1):
        return lib.moe_page_offload(fake, 4, index, byref(cur), byref(tgt), fake, fake, fake, None, None)

    allowed = apq.MOE_EHIP
    # reloads
    assert reload(blk(P0, L0, 3, GPU), blk(P0, L1, 6, GPU)) == allowed      # raise the width
    assert reload(blk(P0, L0, 6, CPU), blk(P0, L1, 6, GPU)) == allowed      # bring back
    assert reload(blk(P0, L0, 6, CPU), blk(P1, L1, 8, GPU)) == allowed      # to a new place
    assert reload(blk(P0, L0, 6, XFER), blk(P0, L1, 6, GPU)) == apq.MOE_EINVAL
    assert b"already in transfer" in lib.moe_last_error()
    assert reload(blk(P0, L0, 6, GPU), blk(P0, L1, 6, GPU)) == apq.MOE_EINVAL   # no growth
    assert reload(blk(P0, L0, 6, GPU), blk(P0, L1, 4, GPU)) == apq.MOE_EINVAL
    assert reload(blk(P0, L0, 3, GPU), blk(P1, L1, 6, GPU)) == apq.MOE_EINVAL   # other planes
    assert reload(blk(P0, L0, 3, GPU), blk(P0, L0, 6, GPU)) == apq.MOE_EINVAL   # LUT in use
    assert reload(blk(P0, L0, 3, CPU), blk(P0, L1, 6, CPU)) == apq.MOE_EINVAL   # target not GPU
    assert reload(blk(P0, L0, 3, CPU), blk(P0, L1, 6, XFER)) == apq.MOE_EINVAL
    assert reload(blk(P0, L0, 3, CPU), blk(P0, L1, 9, GPU)) == apq.MOE_EINVAL   # q outside 1..8
    assert reload(blk(P0, L0, 3, CPU), blk(P0, L1, 6, GPU), index=4) == apq.MOE_EINVAL
    odd = apq.ApqBlock(P0, L1, 64, 256, 6, 6, GPU, 0, 0)
    assert reload(blk(P0, L0, 3, GPU), odd) == apq.MOE_EINVAL                   # other shape
    # offloads
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L0, 6, CPU)) == allowed     # evict
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L1, 3, GPU)) == allowed     # lower the width
    assert offload(blk(P0, L0, 6, CPU), blk(P0, L0, 6, CPU)) == apq.MOE_EINVAL  # not resident
    assert offload(blk(P0, L0, 6, XFER), blk(P0, L0, 6, CPU)) == apq.MOE_EINVAL
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L1, 6, GPU)) == apq.MOE_EINVAL  # no shrink
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L1, 8, GPU)) == apq.MOE_EINVAL
    assert offload(blk(P0, L0, 6, GPU), blk(P1, L1, 3, GPU)) == apq.MOE_EINVAL  # other planes
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L1, 3, XFER)) == apq.MOE_EINVAL
    assert offload(blk(P0, L0, 6, GPU), blk(P0, L0, 6, CPU), index=-1) == apq.MOE_EINVAL
    # the commit that ends a reload: a resident target inside the table
    def commit(tgt, index=1):
        return lib.moe_page_commit(fake, 4, index, byref(tgt), fake, None)

    assert commit(blk(P0, L1, 6, GPU)) == allowed
    assert commit(blk(P0, L1, 6, CPU)) == apq.MOE_EINVAL
    assert commit(blk(P0, L1, 6, XFER)) == apq.MOE_EINVAL
    assert commit(blk(P0, L1, 6, GPU), index=4) == apq.MOE_EINVAL
    assert commit(blk(P0, L1, 0, GPU)) == apq.MOE_EINVAL
    # a full cycle of one block: GPU(6) -> GPU(3) -> CPU -> (IN_TRANSFER) -> GPU(6) -> GPU(8);
    # each step validated against the descriptor the previous step committed
    seq = [(offload, blk(P0, L0, 6, GPU), blk(P0, L1, 3, GPU)),
           (offload, blk(P0, L1, 3, GPU), blk(P0, L1, 3, CPU)),
           (reload, blk(P0, L1, 3, CPU), blk(P0, L0, 6, GPU)),
           (reload, blk(P0, L0, 6, GPU), blk(P0, L1, 8, GPU))]
    for fn, cur, tgt in seq:
        assert fn(cur, tgt) == allowed, lib.moe_last_error()
        if fn is reload:
            assert commit(tgt) == allowed, lib.moe_last_error()
