"""The seeded synthetic layers on the device, for the GPU tests, smoke() and the benchmark: blocks
packed by the library's host packer and uploaded with their page table (device_layer), the same
blocks in the (indices, width, LUT) form the oracle takes (oracle_getters: plain data, the oracle
itself is not imported here), and the weight bytes one call reads (active_weight_bytes)."""
from __future__ import annotations

import functools

import numpy as np

import workloads as wl


def device_layer(shape: wl.LayerShape, device="cuda", q_override=None):
    """Pack and upload every block of a layer (and its shared expert) -> DeviceLayer."""
    import any_precision_expert_router_amd as apq
    widths = wl.gen_widths(shape) if q_override is None else q_override

    def routed(e, m):
        q = int(widths[e, m])
        return apq.pack_block(wl.gen_parent_indices(shape, e, m), q, wl.gen_lut(shape, e, m, q))

    shared = None
    if shape.I_shared:
        def shared(m):
            q = shape.q_shared
            return apq.pack_block(wl.gen_parent_indices(shape, wl.SHARED_EXPERT, m), q,
                                  wl.gen_lut(shape, wl.SHARED_EXPERT, m, q))
    return apq.DeviceLayer(shape.E, shape.H, shape.I, routed, shared, shape.I_shared, device=device)


def oracle_getters(shape: wl.LayerShape, q_override=None, cache_size=64):
    """(routed getter, shared getter or None) in the oracle's (idx8, q, lut) form."""
    widths = wl.gen_widths(shape) if q_override is None else q_override

    @functools.lru_cache(maxsize=cache_size)
    def get(e, m):
        q = int(widths[e, m])
        return wl.gen_parent_indices(shape, e, m), q, wl.gen_lut(shape, e, m, q)

    shared = None
    if shape.I_shared:
        @functools.lru_cache(maxsize=2)
        def shared(e, m):
            q = shape.q_shared
            return (wl.gen_parent_indices(shape, wl.SHARED_EXPERT, m), q,
                    wl.gen_lut(shape, wl.SHARED_EXPERT, m, q))
    return get, shared


def active_weight_bytes(shape: wl.LayerShape, ids: np.ndarray, widths=None):
    """(plane bytes, LUT bytes) of the blocks one call must read: active routed + shared."""
    widths = wl.gen_widths(shape) if widths is None else widths
    planes = lut = 0
    for e in np.unique(ids):
        for m in (wl.GATE_UP, wl.DOWN):
            r, c = wl.block_dims(shape, m, int(e))
            p, l = wl.algorithmic_weight_bytes(r, c, int(widths[e, m]))
            planes += p
            lut += l
    if shape.I_shared:
        for m in (wl.GATE_UP, wl.DOWN):
            r, c = wl.block_dims(shape, m, wl.SHARED_EXPERT)
            p, l = wl.algorithmic_weight_bytes(r, c, shape.q_shared)
            planes += p
            lut += l
    return planes, lut
