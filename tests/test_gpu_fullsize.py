"""Parity at the full layer shapes of the pages' models, in the launch configuration the
benchmark times (one moe_layer_forward call over the whole batch).

For every shape, the routing results the layer call itself left in its workspace (top-k ids,
gates, expert offsets, sorted pairs: read back through moe_workspace_routing) are compared
with the oracle's routing and grouping bit for bit (gates within 1e-6), so the fused
route+group+records kernel (calls of at most 16 tokens) and the split kernels (larger calls)
are both checked on the path that feeds the FFN.  The layer output is compared over the whole
[T, H] for every decode shape (relative L2 <= 1e-3 over the whole array, the metric of the
readings), and over 64 tokens spread across the batch for the 2048-token prefill chunk.
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
from workloads import device as gpu_layers  # noqa: E402

DEV = "cuda"
PREFILL_TOKENS = [int(t) for t in np.linspace(0, wl.QWEN2_PREFILL_TOKENS - 1, 64)]

CASES = [
    ("qwen15_moe_a27b", wl.QWEN15_MOE_A27B, None),
    ("mixtral_8x7b", wl.MIXTRAL_8X7B, None),
    ("qwen3_next_80b_a3b", wl.QWEN3_NEXT_80B_A3B, None),
    ("qwen2_57b_t1", wl.QWEN2_57B_A14B.with_tokens(1), None),
    ("qwen2_57b_t8", wl.QWEN2_57B_A14B.with_tokens(8), None),
    ("qwen2_57b_t32", wl.QWEN2_57B_A14B.with_tokens(32), None),
    ("qwen2_57b_t128", wl.QWEN2_57B_A14B.with_tokens(128), None),
    ("qwen2_57b_prefill2048", wl.QWEN2_57B_A14B.with_tokens(wl.QWEN2_PREFILL_TOKENS), PREFILL_TOKENS),
]

_layers = {}


def _layer(shape):
    key = (shape.workload_id, shape.E, shape.H, shape.I)
    if key not in _layers:
        _layers.clear()
        torch.cuda.empty_cache()
        _layers[key] = gpu_layers.device_layer(shape)
    return _layers[key]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,shape,tokens", CASES, ids=[c[0] for c in CASES])
def test_full_size_layer(name, shape, tokens):
    say(f"full-size {name}: building")
    inputs = wl.gen_layer_inputs(shape)
    dl = _layer(shape)
    T, E, k = shape.T, shape.E, shape.k
    ws = torch.zeros(apq.moe_workspace_bytes(T, E, shape.H, shape.I, k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty((T, shape.H), dtype=torch.float16, device=DEV)
    apq.moe_layer_forward(torch.from_numpy(inputs.logits).to(DEV), torch.from_numpy(inputs.x).to(DEV),
                          E, shape.H, shape.I, k, dl.table, y, ws, shared=dl.shared,
                          I_shared=shape.I_shared)
    apq.moe_check_device_error(ws)
    say(f"full-size {name}: GPU done")
    # routing and grouping exactly as the layer call computed them
    view = apq.moe_workspace_routing(ws, T, E, shape.H, shape.I, k, shape.I_shared)
    ref_ids, ref_g = oracle.route_topk(inputs.logits, k)
    np.testing.assert_array_equal(view["ids"].cpu().numpy().reshape(T, k), ref_ids)
    np.testing.assert_allclose(view["gates"].cpu().numpy().reshape(T, k), ref_g, rtol=0, atol=1e-6)
    r_off, r_pairs, _, _ = oracle.group_by_expert(ref_ids, E)
    np.testing.assert_array_equal(view["offsets"].cpu().numpy(), r_off)
    np.testing.assert_array_equal(view["pairs"].cpu().numpy(), r_pairs)
    # the layer output
    get, sh = gpu_layers.oracle_getters(shape, cache_size=8)
    ref = oracle.layer_forward(inputs.x, inputs.logits, k, get, shared=sh, tokens=tokens)
    yc = y.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yc))
    rows = slice(None) if tokens is None else tokens
    err = oracle.rel_l2(yc[rows], ref["y"][rows])
    per_tok = [oracle.rel_l2(yc[t], ref["y"][t]) for t in (range(T) if tokens is None else tokens)]
    say(f"full-size {name}: rel L2 over {'all' if tokens is None else len(tokens)} tokens = {err:.3e}, "
        f"worst token {max(per_tok):.3e}")
    assert err <= 1e-3
