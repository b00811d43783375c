"""CPU oracle (test infrastructure only; see ``oracle.moe_oracle``)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (apq_matvec, bit_position, committed_index, dequantize, expert_ffn,
                         group_by_expert, layer_forward, pack_planes, rel_l2, route_topk, silu,
                         unpack_planes)
