"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

The layer runs in hand-written HIP kernels behind the C ABI of
``include/moe.h``; this package holds those sources (``csrc/``), the build
script and a thin ctypes binding whose functions carry the C names.
"""
from .binding import (DECODE_MAX_TOKENS, DTYPE, MoeError, PATH, SCORE, config_from, load,  # noqa: F401
                      make_config, make_weights, moe_combine, moe_config, moe_expert_ffn,
                      moe_layer_forward, moe_layer_forward_noalloc, moe_permute, moe_prefetch_experts,
                      moe_route, moe_select, moe_status_str, moe_topk_rows, moe_workspace_bytes, workspace)
