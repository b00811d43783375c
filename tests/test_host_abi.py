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
    # LYNX remap: bin width must be positive and finite; outputs must be given
    assert lib.moe_lynx_remap(fake, 4, 8, 2, 0.0, fake, fake, fake, None) == apq.MOE_EINVAL
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
