"""Thin Python binding of libmoe_apq (the MI355X decode-time Any-Precision MoE layer).

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI
declared in ``include/moe_apq.h``.  PyTorch provides device memory and the stream; the
functions here take torch tensors, pass their device pointers and the current stream, and
raise :class:`MoeError` on a non-zero return code.  There is no CPU fallback: importing this
module fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_apq.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_EHIP = -4
MOE_EDEVICE = -5
MOE_PAGE_GPU, MOE_PAGE_CPU, MOE_PAGE_IN_TRANSFER = 0, 1, 2
GATE_UP, DOWN = 0, 1

EXPORTED = (
    "moe_route_topk", "moe_group_by_expert", "moe_apq_ffn", "moe_layer_forward", "moe_layer_forward_noalloc",
    "moe_workspace_bytes", "moe_apq_pack", "moe_apq_gemv", "moe_apq_decode_indices",
    "moe_check_device_error", "moe_profile_start", "moe_profile_stop", "moe_hbm_read_probe",
    "moe_routing_stats", "moe_workspace_routing", "moe_commit_blocks", "moe_plan_widths",
    "moe_substitute", "moe_lynx_remap", "moe_page_reload", "moe_page_commit",
    "moe_page_offload",
    "moe_last_error",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


class ApqBlock(ctypes.Structure):
    """One weight-page-table entry (``moe_apq_block``, 32 bytes)."""

    _fields_ = [
        ("planes", ctypes.c_void_p),
        ("lut", ctypes.c_void_p),
        ("rows", ctypes.c_int32),
        ("cols", ctypes.c_int32),
        ("q", ctypes.c_uint8),
        ("desired", ctypes.c_uint8),
        ("state", ctypes.c_uint8),
        ("reserved0", ctypes.c_uint8),
        ("reserved1", ctypes.c_int32),
    ]


assert ctypes.sizeof(ApqBlock) == 32


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "moe_route_topk": ([P, I, I, I, P, P, S], I),
        "moe_group_by_expert": ([P, I, I, I, P, P, P, P, P, Z, S], I),
        "moe_apq_ffn": ([P, I, I, I, P, I, I, P, P, P, P, P, P, I, P, I, P, P, Z, S], I),
        "moe_layer_forward": ([P, P, I, I, I, I, I, P, P, I, P, I, P, P, Z, S], I),
        "moe_layer_forward_noalloc": ([P, P, I, I, I, I, I, P, P, I, P, I, P, P, S], I),
        "moe_workspace_bytes": ([I, I, I, I, I, I], Z),
        "moe_apq_pack": ([P, I, I, I, P], I),
        "moe_apq_gemv": ([P, P, I, P, I, S], I),
        "moe_apq_decode_indices": ([P, P, S], I),
        "moe_check_device_error": ([P, Z, S], I),
        "moe_profile_start": ([], I),
        "moe_profile_stop": ([I, P, P, P], I),
        "moe_hbm_read_probe": ([P, Z, P, S], I),
        "moe_routing_stats": ([P, P, P, I, I, I, P, P, P, P, S], I),
        "moe_workspace_routing": ([P, Z, I, I, I, I, I, I, P, P, P, P], I),
        "moe_commit_blocks": ([P, I, P, P, I, S], I),
        "moe_page_reload": ([P, I, I, P, P, P, P, P, S, S], I),
        "moe_page_commit": ([P, I, I, P, P, S], I),
        "moe_page_offload": ([P, I, I, P, P, P, P, P, S, S], I),
        "moe_substitute": ([P, I, I, I, P, I, ctypes.c_float, P, P, P, P, P, ctypes.c_float, P, S], I),
        "moe_lynx_remap": ([P, I, I, I, ctypes.c_float, P, P, P, S], I),
        "moe_plan_widths": ([I, P, P, P, P, P, P, ctypes.c_int64, P, P], I),
        "moe_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(fn, rc, _lib.moe_last_error().decode(errors="replace"))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---------------------------------------------------------------------------------------------
# The four entry points of the layer (same names as the C ABI)
# ---------------------------------------------------------------------------------------------
def moe_route_topk(logits, k: int, topk_ids, topk_gates, stream=None) -> None:
    """logits fp32 [T, E] -> topk_ids int32 [T, k], topk_gates fp32 [T, k] (device tensors)."""
    T, E = logits.shape
    _check("moe_route_topk", _lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids),
                                                 _ptr(topk_gates), _stream(stream)))


def moe_group_by_expert(topk_ids, E: int, expert_offsets, sorted_pairs, active_experts, n_active,
                        stream=None) -> None:
    T, k = topk_ids.shape
    _check("moe_group_by_expert", _lib.moe_group_by_expert(
        _ptr(topk_ids), T, k, E, _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(active_experts),
        _ptr(n_active), None, 0, _stream(stream)))


def moe_apq_ffn(table, E: int, H: int, I: int, x, k: int, expert_offsets, sorted_pairs,
                active_experts, n_active, topk_gates, y, workspace, shared=None, I_shared: int = 0,
                shared_scale=None, prefill_threshold: int = 0, stream=None) -> None:
    T = x.shape[0]
    _check("moe_apq_ffn", _lib.moe_apq_ffn(
        _ptr(table), E, H, I, _ptr(x), T, k, _ptr(expert_offsets), _ptr(sorted_pairs),
        _ptr(active_experts), _ptr(n_active), _ptr(topk_gates), _ptr(shared), I_shared,
        _ptr(shared_scale), prefill_threshold, _ptr(y), _ptr(workspace), workspace.numel(),
        _stream(stream)))


def moe_layer_forward(logits, x, E: int, H: int, I: int, k: int, table, y, workspace, shared=None,
                      I_shared: int = 0, shared_scale=None, prefill_threshold: int = 0,
                      stream=None) -> None:
    T = x.shape[0]
    _check("moe_layer_forward", _lib.moe_layer_forward(
        _ptr(logits), _ptr(x), T, E, H, I, k, _ptr(table), _ptr(shared), I_shared,
        _ptr(shared_scale), prefill_threshold, _ptr(y), _ptr(workspace), workspace.numel(),
        _stream(stream)))


NOALLOC_WORKSPACE_BYTES = 32 << 20   # MOE_NOALLOC_WORKSPACE_BYTES


def moe_layer_forward_noalloc(logits, x, E: int, H: int, I: int, k: int, table, y, status=None,
                              shared=None, I_shared: int = 0, shared_scale=None,
                              prefill_threshold: int = 0, stream=None) -> None:
    """The whole layer on the library's own device array (no workspace argument; nothing is
    allocated).  status: optional device int32 [1] that receives the call's error word."""
    T = x.shape[0]
    _check("moe_layer_forward_noalloc", _lib.moe_layer_forward_noalloc(
        _ptr(logits), _ptr(x), T, E, H, I, k, _ptr(table), _ptr(shared), I_shared,
        _ptr(shared_scale), prefill_threshold, _ptr(y), _ptr(status), _stream(stream)))


def moe_workspace_bytes(T: int, E: int, H: int, I: int, k: int, I_shared: int = 0) -> int:
    n = _lib.moe_workspace_bytes(T, E, H, I, k, I_shared)
    if n == 0:
        raise MoeError("moe_workspace_bytes", MOE_EINVAL, "bad sizes")
    return n


def moe_apq_pack(idx8: np.ndarray, q: int) -> np.ndarray:
    """Host packer: uint8 [rows, cols] parent indices -> uint32 planes [q * rows * cols / 32]."""
    idx8 = np.ascontiguousarray(idx8, dtype=np.uint8)
    rows, cols = idx8.shape
    out = np.empty(q * rows * cols // 32, dtype=np.uint32)
    _check("moe_apq_pack", _lib.moe_apq_pack(idx8.ctypes.data, rows, cols, q, out.ctypes.data))
    return out


def moe_apq_gemv(block: ApqBlock, x, y, dense_threshold: int = 0, stream=None) -> None:
    """Decode GEMV on one block: x fp16 [T, cols] -> y fp32 [T, rows]."""
    _check("moe_apq_gemv", _lib.moe_apq_gemv(ctypes.byref(block), _ptr(x), x.shape[0], _ptr(y),
                                             dense_threshold, _stream(stream)))


def moe_apq_decode_indices(block: ApqBlock, idx_out, stream=None) -> None:
    _check("moe_apq_decode_indices", _lib.moe_apq_decode_indices(ctypes.byref(block), _ptr(idx_out),
                                                                 _stream(stream)))


def moe_check_device_error(workspace, stream=None) -> None:
    _check("moe_check_device_error", _lib.moe_check_device_error(_ptr(workspace), workspace.numel(),
                                                                 _stream(stream)))


def moe_hbm_read_probe(buf, sink, stream=None) -> None:
    """Stream-read `buf` (device tensor, size a multiple of 1 KiB) once; XOR of the data into sink."""
    _check("moe_hbm_read_probe", _lib.moe_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                                         _ptr(sink), _stream(stream)))


def moe_routing_stats(expert_offsets, sorted_pairs, topk_gates, T, k, E, count, mass, mass_sums,
                      resident=None, stream=None) -> None:
    """Add one call's per-expert counts (uint64 [E] as int64 tensor), gate masses (float64 [E])
    and [non-resident mass, total mass] (float64 [2]) to the accumulators (device tensors)."""
    _check("moe_routing_stats", _lib.moe_routing_stats(
        _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(topk_gates), T, k, E,
        None if resident is None else _ptr(resident), _ptr(count), _ptr(mass), _ptr(mass_sums),
        _stream(stream)))


def moe_workspace_routing(workspace, T, E, H, I, k, I_shared=0) -> dict:
    """Views into `workspace` (uint8 device tensor) of the routing results a moe_layer_forward
    call left there: ids / pairs int32 [T*k], gates float32 [T*k], offsets int32 [E+1]."""
    import torch
    ptrs = [ctypes.c_void_p() for _ in range(4)]
    _check("moe_workspace_routing", _lib.moe_workspace_routing(
        _ptr(workspace), workspace.numel(), T, E, H, I, k, I_shared,
        *[ctypes.byref(p) for p in ptrs]))
    base = workspace.data_ptr()

    def view(p, n, dtype):
        off = p.value - base
        return workspace[off: off + n * 4].view(dtype)

    TK = T * k
    return {"ids": view(ptrs[0], TK, torch.int32), "gates": view(ptrs[1], TK, torch.float32),
            "offsets": view(ptrs[2], E + 1, torch.int32), "pairs": view(ptrs[3], TK, torch.int32)}


MOE_POLICY_FETCH_ALL, MOE_POLICY_GATE_RULE, MOE_POLICY_FIRST_CHOICE = 0, 1, 2


def moe_substitute(logits, resident, policy, topk_ids, topk_gates, missed, fetch,
                   gate_threshold=0.15, admit_mass=None, admit=None, admit_threshold=0.5,
                   stream=None) -> None:
    """Substitute non-resident routed experts in place in topk_ids (device tensors); see the
    header for the policies, the outputs and the admission accumulators."""
    T, E = logits.shape
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else topk_ids.numel() // max(T, 1)
    _check("moe_substitute", _lib.moe_substitute(
        _ptr(logits), T, E, k, _ptr(resident), int(policy), float(gate_threshold), _ptr(topk_ids),
        _ptr(topk_gates), _ptr(missed), _ptr(fetch), None if admit_mass is None else _ptr(admit_mass),
        float(admit_threshold), None if admit is None else _ptr(admit), _stream(stream)))


def moe_lynx_remap(logits, topk_ids, remapped, critical, bin_width=None, stream=None) -> None:
    """Remap low-confidence slots of topk_ids (device int32 [T,k], in place) onto the critical
    expert set; remapped gets each remapped slot's original expert (else -1), critical [E] the
    set.  bin_width None lets the library take its default, k/E in fp32.  See the header for
    the readings."""
    T, E = logits.shape
    k = topk_ids.shape[1] if topk_ids.dim() == 2 else topk_ids.numel() // max(T, 1)
    if bin_width is None:
        bin_width = 0.0
    _check("moe_lynx_remap", _lib.moe_lynx_remap(
        _ptr(logits), T, E, k, float(bin_width), _ptr(topk_ids), _ptr(remapped), _ptr(critical),
        _stream(stream)))


def _event(ev, stream) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (torch creates the event at its first record, so an
    unrecorded one is recorded once on `stream` first) or an int handle."""
    if isinstance(ev, int):
        return ev
    if not ev.cuda_event:
        ev.record(stream)
    return ev.cuda_event


def _table_len(table) -> int:
    return table.numel() * table.element_size() // ctypes.sizeof(ApqBlock)


def moe_commit_blocks(table, index, descs, stream=None) -> None:
    """Overwrite page-table entries `index` (ints) of the device table (uint8 tensor of
    32-byte entries) with `descs` (ApqBlock list), in stream order."""
    n = len(index)
    idx = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in index])
    arr = (ApqBlock * max(n, 1))(*descs)
    _check("moe_commit_blocks", _lib.moe_commit_blocks(_ptr(table), _table_len(table), idx, arr, n,
                                                       _stream(stream)))


def moe_page_reload(table, index: int, current: ApqBlock, target: ApqBlock, host_planes, host_lut,
                    copy_event, copy_stream, stream=None) -> None:
    """Copy a block's missing planes and its LUT from pinned host tensors on copy_stream and
    record copy_event there; a block coming back from the host is marked in transfer on `stream`
    first.  `target` is committed later by moe_page_commit (see the header for the rules)."""
    _check("moe_page_reload", _lib.moe_page_reload(
        _ptr(table), _table_len(table), int(index), ctypes.byref(current), ctypes.byref(target),
        _ptr(host_planes), _ptr(host_lut), _event(copy_event, copy_stream), _stream(copy_stream),
        _stream(stream)))


def moe_page_commit(table, index: int, target: ApqBlock, copy_event, stream=None) -> None:
    """The safe boundary of a reload: `stream` waits for copy_event, then `target` is committed."""
    _check("moe_page_commit", _lib.moe_page_commit(
        _ptr(table), _table_len(table), int(index), ctypes.byref(target), _event(copy_event, stream),
        _stream(stream)))


def moe_page_offload(table, index: int, current: ApqBlock, target: ApqBlock, host_planes, host_lut,
                     copy_event, copy_stream, stream=None) -> None:
    """Commit `target` (evicted to the host, or a lower width) on `stream`, then copy the planes
    (and LUT) that leave the device into pinned host tensors on copy_stream (None: no copy)."""
    _check("moe_page_offload", _lib.moe_page_offload(
        _ptr(table), _table_len(table), int(index), ctypes.byref(current), ctypes.byref(target),
        _ptr(host_planes), _ptr(host_lut), _event(copy_event, copy_stream), _stream(copy_stream),
        _stream(stream)))


def moe_plan_widths(q_cur, q_floor, rows, cols, damage, mult, target_bytes):
    """Greedy width plan on the host.  Array arguments are NumPy-convertible; damage is [n, 8]
    (damage[i, w-1] = score at width w).  Returns (q_new uint8 [n], bytes saved)."""
    import numpy as np
    q_cur = np.ascontiguousarray(q_cur, dtype=np.uint8)
    n = q_cur.size
    args = [np.ascontiguousarray(q_floor, dtype=np.uint8), np.ascontiguousarray(rows, dtype=np.int32),
            np.ascontiguousarray(cols, dtype=np.int32),
            np.ascontiguousarray(np.asarray(damage, dtype=np.float32).reshape(n * 8)),
            np.ascontiguousarray(mult, dtype=np.float32)]
    q_new = np.zeros(n, dtype=np.uint8)
    saved = ctypes.c_int64()
    _check("moe_plan_widths", _lib.moe_plan_widths(
        n, q_cur.ctypes.data, *[a.ctypes.data for a in args], int(target_bytes), q_new.ctypes.data,
        ctypes.byref(saved)))
    return q_new, int(saved.value)


def moe_profile_start() -> None:
    _check("moe_profile_start", _lib.moe_profile_start())


def moe_profile_stop(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} for the launches since moe_profile_start()."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = _lib.moe_profile_stop(max_kernels, names, ms, cnt)
    if n < 0:
        _check("moe_profile_stop", n)
    raw = names.raw
    out = {}
    for i in range(min(n, max_kernels)):
        name = raw[64 * i: 64 * i + 64].split(b"\0", 1)[0].decode()
        out[name] = (ms[i], cnt[i])
    return out


# ---------------------------------------------------------------------------------------------
# Device-resident weights: planes + LUTs per block and the weight page table
# ---------------------------------------------------------------------------------------------
class DeviceLayer:
    """Device copies of a layer's blocks and its page table ([E][2] descriptors).

    Blocks are packed on the host by ``moe_apq_pack`` and copied into one device arena per
    layer (16-byte aligned sub-buffers).  ``table`` is the device page table consumed by
    ``moe_apq_ffn``/``moe_layer_forward``; ``shared`` the optional shared-expert pair.
    """

    def __init__(self, E: int, H: int, I: int, blocks, shared_blocks=None, I_shared: int = 0,
                 device="cuda"):
        import torch
        self.E, self.H, self.I, self.I_shared = E, H, I, I_shared if shared_blocks else 0
        entries = []   # (planes ndarray uint32, lut ndarray fp16, rows, cols, q)
        for e in range(E):
            for m in (GATE_UP, DOWN):
                entries.append(blocks(e, m))
        sh_entries = [shared_blocks(m) for m in (GATE_UP, DOWN)] if shared_blocks else []
        all_entries = entries + sh_entries
        # one arena: planes and LUTs at 256-byte aligned offsets
        offs, total = [], 0
        for planes, lut, *_ in all_entries:
            po = total
            total += (planes.nbytes + 255) // 256 * 256
            lo = total
            total += (lut.nbytes + 255) // 256 * 256
            offs.append((po, lo))
        host = np.zeros(total, dtype=np.uint8)
        for (po, lo), (planes, lut, *_) in zip(offs, all_entries):
            host[po:po + planes.nbytes] = planes.view(np.uint8)
            host[lo:lo + lut.nbytes] = np.ascontiguousarray(lut).view(np.uint8).reshape(-1)
        self.arena = torch.from_numpy(host).to(device)
        base = self.arena.data_ptr()
        descs = []
        for (po, lo), (planes, lut, rows, cols, q) in zip(offs, all_entries):
            descs.append(ApqBlock(base + po, base + lo, rows, cols, q, q, MOE_PAGE_GPU, 0, 0))
        self.host_blocks = descs
        raw = np.frombuffer(b"".join(bytes(d) for d in descs), dtype=np.uint8)
        self.table = torch.from_numpy(raw[: 32 * 2 * E].copy()).to(device)
        self.shared = torch.from_numpy(raw[32 * 2 * E:].copy()).to(device) if sh_entries else None
        self.weight_bytes = int(total)

    def block(self, e: int, m: int) -> ApqBlock:
        return self.host_blocks[2 * e + m]

    def shared_block(self, m: int) -> ApqBlock:
        return self.host_blocks[2 * self.E + m]


def pack_block(idx8: np.ndarray, q: int, lut: np.ndarray):
    """(planes, lut, rows, cols, q) for DeviceLayer from parent indices and the width-q LUT."""
    rows, cols = idx8.shape
    return moe_apq_pack(idx8, q), np.ascontiguousarray(lut, dtype=np.float16), rows, cols, q
