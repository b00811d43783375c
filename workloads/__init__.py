"""Seeded synthetic inputs for the decode-time MoE layer over Any-Precision weights.

This module only *draws* inputs: token activations, router logits, the 8-bit parent indices
of every linear block, the per-row lookup tables and the committed width of every
(expert, module) block.  It holds none of the layer's arithmetic (no routing, grouping,
bit-plane packing, decoding or FFN), so that the CPU oracle and the HIP path can both take
their inputs from here without sharing any of the method.

Shapes follow the MoE models the pages evaluate (PagedWeight, Results: Qwen1.5-MoE-A2.7B and
Mixtral-8x7B; "Which Expert Misses Are Worth Waiting For?", Problem statement: a 512-expert
top-10 model; LYNX, Problem statement: Qwen2-57B-A14B with 64 experts).  No checkpoint is
used: every tensor is random with the distribution stated beside it.

Every tensor has its own PCG64 stream, seeded by ``SeedSequence([2026, workload_id, tag, ...])``
so that a single block can be regenerated without drawing the rest of the layer.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

# Tensor tags used in the seed sequences.
_TAG_X = 1
_TAG_ROUTER_W = 2
_TAG_ZIPF_RANK = 3
_TAG_ZIPF_NOISE = 4
_TAG_WIDTHS = 5
_TAG_HOT = 6
_TAG_IDX = 7
_TAG_LUT = 8

GATE_UP = 0
DOWN = 1
MODULE_NAMES = ("gate_up", "down")
SHARED_EXPERT = -1  # expert id used for the always-on shared expert's blocks


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One synthetic MoE layer.

    H hidden size, E routed experts, I expert intermediate size, k experts per token, T tokens.
    ``widths`` are the candidate committed widths; ``width_rule`` says how they are drawn:
      * "uniform": i.i.d. uniform over ``widths`` per (expert, module) block;
      * "fixed":   every routed block at ``widths[0]``;
      * "hot25":   a seeded quarter of the experts at 8 bits for both modules, the rest
                   uniform over ``widths``.
    ``router`` is "matmul" (logits = x . W_r^T with W_r ~ N(0, router_std) fp16) or "zipf"
    (logits = -1.1 ln(rank_e) + N(0, 1), rank a seeded permutation of 1..E).
    ``I_shared`` > 0 adds an always-on shared expert at width ``q_shared``.
    """

    name: str
    workload_id: int
    H: int
    E: int
    I: int
    k: int
    T: int
    widths: Tuple[int, ...]
    width_rule: str = "uniform"
    router: str = "matmul"
    router_std: float = 0.02
    zipf_s: float = 1.1
    I_shared: int = 0
    q_shared: int = 8
    lut_std: float = 0.02

    def with_tokens(self, T: int) -> "LayerShape":
        return dataclasses.replace(self, T=T)

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


# The layer shapes the pages' models give (synthetic weights; no checkpoint is read).
TINY = LayerShape("tiny H128 E8 I256 top-2", 0, H=128, E=8, I=256, k=2, T=4,
                  widths=(3, 4), router_std=0.05)
QWEN15_MOE_A27B = LayerShape("Qwen1.5-MoE-A2.7B-shaped H2048 E60 I1408 top-4 + shared I5632",
                             1, H=2048, E=60, I=1408, k=4, T=16, widths=(4,),
                             width_rule="fixed", I_shared=5632, q_shared=8)
MIXTRAL_8X7B = LayerShape("Mixtral-8x7B-shaped H4096 E8 I14336 top-2", 2, H=4096, E=8,
                          I=14336, k=2, T=32, widths=(3, 4, 6, 8))
QWEN3_NEXT_80B_A3B = LayerShape("Qwen3-Next-80B-A3B-shaped H2048 E512 I512 top-10 (Zipf router)",
                                3, H=2048, E=512, I=512, k=10, T=64, widths=(3, 4, 5, 6),
                                width_rule="hot25", router="zipf")
QWEN2_57B_A14B = LayerShape("Qwen2-57B-A14B-shaped H3584 E64 I2560 top-8", 4, H=3584, E=64,
                            I=2560, k=8, T=32, widths=(3, 4, 6, 8))

PRESETS: Dict[str, LayerShape] = {
    "tiny": TINY,
    "qwen15_moe_a27b": QWEN15_MOE_A27B,
    "mixtral_8x7b": MIXTRAL_8X7B,
    "qwen3_next_80b_a3b": QWEN3_NEXT_80B_A3B,
    "qwen2_57b_a14b": QWEN2_57B_A14B,
}
# Decode batch sweep and chunked-prefill size used with the Qwen2-57B-A14B-shaped layer.
QWEN2_TOKEN_SWEEP = (1, 8, 32, 128)
QWEN2_PREFILL_TOKENS = 2048


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, *key])))


def block_dims(shape: LayerShape, module: int, expert: int = 0) -> Tuple[int, int]:
    """(rows, cols) of a linear block: gate_up is [2I x H], down is [H x I]."""
    inter = shape.I_shared if expert == SHARED_EXPERT else shape.I
    if module == GATE_UP:
        return 2 * inter, shape.H
    return shape.H, inter


def gen_x(shape: LayerShape, seed_offset: int = 0) -> np.ndarray:
    """Token activations, fp16 N(0, 1), [T, H]."""
    r = _rng(shape.workload_id, _TAG_X, shape.T, seed_offset)
    return r.standard_normal((shape.T, shape.H)).astype(np.float16)


def gen_router_weight(shape: LayerShape) -> np.ndarray:
    """Router weight W_r, fp16 N(0, router_std), [E, H]."""
    r = _rng(shape.workload_id, _TAG_ROUTER_W, shape.E, shape.H)
    return (r.standard_normal((shape.E, shape.H)) * shape.router_std).astype(np.float16)


def gen_logits(shape: LayerShape, x: np.ndarray, seed_offset: int = 0) -> np.ndarray:
    """Router logits handed to the layer, fp32 [T, E].

    "matmul": x . W_r^T evaluated in float64 from the fp16 operands, rounded once to fp32.
    "zipf":   per-expert bias -s ln(rank_e) (so that softmax(bias) follows the Zipf pmf) plus
              N(0, 1) noise per (token, expert), rounded to fp32.
    """
    if shape.router == "zipf":
        rank = _rng(shape.workload_id, _TAG_ZIPF_RANK, shape.E).permutation(shape.E) + 1
        bias = -shape.zipf_s * np.log(rank.astype(np.float64))
        noise = _rng(shape.workload_id, _TAG_ZIPF_NOISE, shape.T, seed_offset).standard_normal(
            (shape.T, shape.E))
        return (bias[None, :] + noise).astype(np.float32)
    w = gen_router_weight(shape).astype(np.float64)
    return (x.astype(np.float64) @ w.T).astype(np.float32)


def gen_widths(shape: LayerShape) -> np.ndarray:
    """Committed width q of every routed (expert, module) block, uint8 [E, 2]."""
    r = _rng(shape.workload_id, _TAG_WIDTHS, shape.E)
    cand = np.asarray(shape.widths, dtype=np.uint8)
    if shape.width_rule == "fixed":
        return np.full((shape.E, 2), cand[0], dtype=np.uint8)
    q = cand[r.integers(0, len(cand), size=(shape.E, 2))]
    if shape.width_rule == "hot25":
        hot = _rng(shape.workload_id, _TAG_HOT, shape.E).permutation(shape.E)[: shape.E // 4]
        q[hot, :] = 8
    return q.astype(np.uint8)


def gen_parent_indices(shape: LayerShape, expert: int, module: int) -> np.ndarray:
    """8-bit parent indices of one block, uint8 uniform on [0, 255], [rows, cols]."""
    rows, cols = block_dims(shape, module, expert)
    r = _rng(shape.workload_id, _TAG_IDX, expert + 1, module)
    return r.integers(0, 256, size=(rows, cols), dtype=np.uint8)


def gen_lut(shape: LayerShape, expert: int, module: int, q: int) -> np.ndarray:
    """Per-row fp16 lookup table of the committed width q, [rows, 2**q].

    Each row draws 256 N(0, lut_std) values in float64 and sorts them (the 8-bit parent
    table).  The width-w table of that row holds, for every w-bit prefix v, the mean of the
    2**(8-w) parent entries that share the prefix, rounded to fp16: the tables are sorted and
    nested by prefix, and only the committed width's table is kept.
    """
    rows, _ = block_dims(shape, module, expert)
    r = _rng(shape.workload_id, _TAG_LUT, expert + 1, module)
    parent = np.sort(r.standard_normal((rows, 256)) * shape.lut_std, axis=1)
    group = 1 << (8 - q)
    return parent.reshape(rows, 1 << q, group).mean(axis=2).astype(np.float16)


@dataclasses.dataclass
class Block:
    """Host copy of one (expert, module) linear block: parent indices, committed width, LUT."""

    expert: int
    module: int
    q: int
    idx8: np.ndarray  # uint8 [rows, cols]
    lut: np.ndarray   # fp16 [rows, 2**q]

    @property
    def rows(self) -> int:
        return self.idx8.shape[0]

    @property
    def cols(self) -> int:
        return self.idx8.shape[1]


def gen_block(shape: LayerShape, expert: int, module: int, q: Optional[int] = None) -> Block:
    """Regenerate one block deterministically (same bytes on every call)."""
    if q is None:
        q = shape.q_shared if expert == SHARED_EXPERT else int(gen_widths(shape)[expert, module])
    return Block(expert, module, int(q), gen_parent_indices(shape, expert, module),
                 gen_lut(shape, expert, module, int(q)))


@dataclasses.dataclass
class LayerInputs:
    shape: LayerShape
    x: np.ndarray        # fp16 [T, H]
    logits: np.ndarray   # fp32 [T, E]
    widths: np.ndarray   # uint8 [E, 2]


def gen_layer_inputs(shape: LayerShape, seed_offset: int = 0) -> LayerInputs:
    x = gen_x(shape, seed_offset)
    return LayerInputs(shape, x, gen_logits(shape, x, seed_offset), gen_widths(shape))


def algorithmic_weight_bytes(rows: int, cols: int, q: int) -> Tuple[int, int]:
    """(plane bytes, LUT bytes) one block occupies at committed width q."""
    return rows * cols * q // 8, rows * (1 << q) * 2
