"""moe_layer_forward_noalloc (the layer on the library's own device array, for callers that
cannot allocate) against moe_layer_forward with a caller-owned workspace, through the C ABI.

Both run the same kernels in the same order on the same inputs, so the outputs must be equal
bit for bit.  Two calls in a row, the second with fewer tokens than the first (the array keeps
the first call's contents), on a small layer (split and fused routing paths) and on the
Qwen2-57B-A14B-shaped layer at 128 tokens, the largest decode workspace; then the error word
reported through `status`, and the refusal of a call above the array's size.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import any_precision_expert_router_amd as apq  # noqa: E402
from workloads import device as gpu_layers  # noqa: E402

DEV = "cuda"


def _both(shape, dl, inputs, table=None):
    T = shape.T
    table = dl.table if table is None else table
    lg = torch.from_numpy(inputs.logits).to(DEV)
    x = torch.from_numpy(inputs.x).to(DEV)
    y_ws = torch.full((T, shape.H), 7.0, dtype=torch.float16, device=DEV)
    ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                     dtype=torch.uint8, device=DEV)
    apq.moe_layer_forward(lg, x, shape.E, shape.H, shape.I, shape.k, table, y_ws, ws, shared=dl.shared,
                          I_shared=shape.I_shared)
    y_na = torch.full((T, shape.H), -7.0, dtype=torch.float16, device=DEV)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    apq.moe_layer_forward_noalloc(lg, x, shape.E, shape.H, shape.I, shape.k, table, y_na, status=status,
                                  shared=dl.shared, I_shared=shape.I_shared)
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_na.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("base,Ts", [
    (wl.TINY.replace(H=256, E=8, I=256, k=2, I_shared=256, q_shared=8, name="noalloc small"), (40, 5)),
    (wl.QWEN2_57B_A14B, (128, 8)),
], ids=["small-shared", "qwen2-57b"])
def test_noalloc_equals_workspace_call_on_two_calls(base, Ts):
    dl = gpu_layers.device_layer(base.with_tokens(Ts[0]))
    for T in Ts:
        shape = base.with_tokens(T)
        print(f"noalloc {shape.name} T={T}", flush=True)
        inputs = wl.gen_layer_inputs(shape, seed_offset=T)
        y_ws, y_na, status = _both(shape, dl, inputs)
        assert status == 0
        assert np.all(np.isfinite(y_na.astype(np.float32)))
        np.testing.assert_array_equal(y_na.view(np.uint16), y_ws.view(np.uint16))


def test_noalloc_status_reports_and_clears_the_error_word():
    """A call with an invalid block writes a nonzero status; the next clean call clears it (the
    array keeps the earlier call's word, so clearing at the start matters); y agrees with the
    workspace entry point in both calls."""
    shape = wl.TINY.replace(H=256, E=8, I=256, k=2, T=9, name="noalloc status")
    dl = gpu_layers.device_layer(shape)
    inputs = wl.gen_layer_inputs(shape)
    bad = dl.table.clone().view(torch.uint8).reshape(shape.E * 2, 32)
    bad[:, 24] = 9                       # q = 9: every routed block is invalid
    y_ws, y_na, status = _both(shape, dl, inputs, table=bad.reshape(-1))
    assert status != 0
    np.testing.assert_array_equal(y_na.view(np.uint16), y_ws.view(np.uint16))
    y_ws, y_na, status = _both(shape, dl, inputs)
    assert status == 0
    np.testing.assert_array_equal(y_na.view(np.uint16), y_ws.view(np.uint16))


def test_noalloc_refuses_a_call_above_its_array():
    shape = wl.QWEN2_57B_A14B.with_tokens(wl.QWEN2_PREFILL_TOKENS)
    need = apq.moe_workspace_bytes(shape.T, shape.E, shape.H, shape.I, shape.k, 0)
    assert need > apq.NOALLOC_WORKSPACE_BYTES
    fake = torch.empty(1, device=DEV).data_ptr()   # never launched on: the size check comes first
    rc = apq.lib().moe_layer_forward_noalloc(fake, fake, shape.T, shape.E, shape.H, shape.I, shape.k, fake,
                                             None, 0, None, 0, fake, None, None)
    assert rc == apq.MOE_EWORKSPACE
    assert b"allocation-free" in apq.lib().moe_last_error()
