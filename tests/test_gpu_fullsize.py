"""Parity at the full layer shapes of the pages' models, in the launch configuration the
benchmark times (moe_layer_forward on the whole batch).  Routing and grouping are compared
bit-exactly for every token; the layer output on a few sampled tokens, which the float64 oracle
can compute one by one (dequantising only those tokens' experts).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import any_precision_expert_router_amd as apq  # noqa: E402
import gpu_layers  # noqa: E402

DEV = "cuda"

CASES = [
    ("qwen15_moe_a27b", wl.QWEN15_MOE_A27B, [0, 7, 15]),
    ("mixtral_8x7b", wl.MIXTRAL_8X7B, [3]),
    ("qwen3_next_80b_a3b", wl.QWEN3_NEXT_80B_A3B, [0, 63]),
    ("qwen2_57b_t1", wl.QWEN2_57B_A14B.with_tokens(1), [0]),
    ("qwen2_57b_t8", wl.QWEN2_57B_A14B.with_tokens(8), [5]),
    ("qwen2_57b_t32", wl.QWEN2_57B_A14B.with_tokens(32), [31]),
    ("qwen2_57b_t128", wl.QWEN2_57B_A14B.with_tokens(128), [64]),
    ("qwen2_57b_prefill2048", wl.QWEN2_57B_A14B.with_tokens(2048), [1000]),
]

_layers = {}


def _layer(shape):
    key = (shape.workload_id, shape.E, shape.H, shape.I)
    if key not in _layers:
        _layers.clear()
        torch.cuda.empty_cache()
        _layers[key] = gpu_layers.device_layer(shape)
    return _layers[key]


@pytest.mark.parametrize("name,shape,tokens", CASES, ids=[c[0] for c in CASES])
def test_full_size_layer(name, shape, tokens):
    print(f"full-size {name}: building", flush=True)
    inputs = wl.gen_layer_inputs(shape)
    dl = _layer(shape)
    T = shape.T
    ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    apq.moe_layer_forward(torch.from_numpy(inputs.logits).to(DEV), torch.from_numpy(inputs.x).to(DEV),
                          shape.E, shape.H, shape.I, shape.k, dl.table, y, ws, shared=dl.shared,
                          I_shared=shape.I_shared)
    apq.moe_check_device_error(ws)
    print(f"full-size {name}: GPU done", flush=True)
    # routing arrays the layer kept in its workspace are checked through the separate entry points
    ids = torch.empty((T, shape.k), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, shape.k), dtype=torch.float32, device=DEV)
    apq.moe_route_topk(torch.from_numpy(inputs.logits).to(DEV), shape.k, ids, gates)
    ref_ids, ref_g = oracle.route_topk(inputs.logits, shape.k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(gates.cpu().numpy(), ref_g, atol=1e-6)
    get, sh = gpu_layers.oracle_getters(shape, cache_size=8)
    ref = oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh, tokens=tokens)
    yc = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yc))
    for t in tokens:
        err = oracle.rel_l2(yc[t], ref["y"][t])
        print(f"full-size {name}: token {t} rel L2 = {err:.3e}", flush=True)
        assert err <= 1e-3
    sys.stdout.flush()
