"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop counts behind its
effective-GB/s value and its roofline objects, and the one-GPU contract."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workloads as wl

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__))))
from workloads import device as gpu_layers  # noqa: E402

SHAPES = [wl.QWEN15_MOE_A27B, wl.MIXTRAL_8X7B, wl.QWEN3_NEXT_80B_A3B, wl.QWEN2_57B_A14B.with_tokens(8)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name.split("-shaped")[0])
def test_module_bytes_add_up_to_the_layer_and_match_the_oracle(shape):
    """gate_up + down bytes of the blocks a call reads equal the layer's active weight bytes, and
    each equals the oracle's own resident-bytes formula summed over the routed experts (and the
    shared expert)."""
    inputs = wl.gen_layer_inputs(shape)
    widths = wl.gen_widths(shape)
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    gu = bench.module_bytes(shape, ids, wl.GATE_UP, widths)
    dn = bench.module_bytes(shape, ids, wl.DOWN, widths)
    planes, lut = gpu_layers.active_weight_bytes(shape, ids, widths)
    assert gu[0] + dn[0] == planes and gu[1] + dn[1] == lut
    for module, got in ((wl.GATE_UP, gu), (wl.DOWN, dn)):
        ref = 0
        for e in np.unique(ids):
            r, c = wl.block_dims(shape, module, int(e))
            ref += oracle.block_bytes(r, c, int(widths[e, module]))
        if shape.I_shared:
            r, c = wl.block_dims(shape, module, wl.SHARED_EXPERT)
            ref += oracle.block_bytes(r, c, shape.q_shared)
        assert sum(got) == ref


def test_headline_bytes_and_prefill_flops():
    """The Qwen1.5-shaped call reads 47 active experts at 4 bits plus the 8-bit shared expert:
    the gate_up launch's algorithmic bytes are the figure its roofline is quoted on.  The
    prefill row's flops are 2 T k 3 H I."""
    shape = wl.QWEN15_MOE_A27B
    inputs = wl.gen_layer_inputs(shape)
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    n_act = len(np.unique(ids))
    gu = sum(bench.module_bytes(shape, ids, wl.GATE_UP, wl.gen_widths(shape)))
    expect = n_act * (2 * 1408 * 2048 // 2 + 2 * 1408 * 16 * 2) + (2 * 5632 * 2048 + 2 * 5632 * 256 * 2)
    assert gu == expect
    p = wl.QWEN2_57B_A14B.with_tokens(wl.QWEN2_PREFILL_TOKENS)
    assert 2.0 * p.T * p.k * 3 * p.H * p.I == 901943132160.0


def test_default_workload_is_the_largest_mixed_width_decode_shape():
    """The headline is the Qwen2-57B-A14B-shaped layer at 128 decode tokens with widths drawn from
    {3, 4, 6, 8}; every other shape of the pages' models is a sub-record of the same line."""
    shape = bench.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (shape.H, shape.E, shape.I, shape.k, shape.T) == (3584, 64, 2560, 8, 128)
    assert sorted(set(int(v) for v in np.unique(wl.gen_widths(shape)))) == [3, 4, 6, 8]
    others = set(bench.WORKLOADS) - {bench.DEFAULT_WORKLOAD, "qwen2_57b_a14b_prefill2048"}
    assert others == set(bench.SUB_WORKLOADS)
    assert "internal.hpp" in " ".join(bench.ENGINE_SOURCES)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
