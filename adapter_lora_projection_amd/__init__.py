"""MI355X (gfx950) multi-adapter LoRA projection: chunked-SGMV shrink/expand, the fused
single-adapter LoRA+SwiGLU MLP and the single-adapter LoRA attention projections, as hand-written
HIP kernels behind a C ABI.

``_lib`` mirrors the C entry points one to one; ``ops`` adds tensor-level helpers that infer
sizes and strides from torch tensors, allocate outputs and workspaces, and pass the current
stream. Every step runs in the HIP library; there is no CPU path.
"""

from ._lib import LoraError, Plan, lib, lora_version
from .ops import (LoraLinearFunction, LoraMlpFunction, LoraQkvFunction, check_metadata, embedding_a, expand, fast_path_eligible,
                  linear_backward, linear_prepare_backward, qkv_backward, qkv_prepare_backward,
                  fast_path_ineligibility, linear_fused, mlp_backward, mlp_fused, mlp_fused_train,
                  mlp_prepare_backward, qkv_fused, require_fast_path, schedule_tiles, shrink,
                  shrink_expand)

__all__ = ["LoraError", "Plan", "lib", "lora_version", "shrink", "expand", "shrink_expand",
           "schedule_tiles",
           "mlp_fused", "linear_fused", "qkv_fused", "embedding_a", "mlp_fused_train",
           "mlp_prepare_backward", "mlp_backward", "LoraMlpFunction", "check_metadata",
           "fast_path_eligible", "fast_path_ineligibility", "require_fast_path",
           "linear_prepare_backward", "linear_backward", "qkv_prepare_backward", "qkv_backward",
           "LoraLinearFunction", "LoraQkvFunction"]
