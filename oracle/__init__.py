"""CPU oracle for the multi-adapter LoRA projection and the fused LoRA+SwiGLU MLP.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only the tests,
the smoke check of the package entry module and the CPU-baseline leg of the benchmark may
import, call or execute it. It is a plain, slow, fp64 implementation of the definitions, written
for a reader to check against the pages by eye, and it shares no code with the HIP path.

Sources (pages as titled):
* "Decode LoRA kernels are optimized" (sgl-kernel-xpu pull request 550), Summary and Behaviour
  changes: chunked-SGMV shrink/expand driven by seg_indptr, an index range (weight_indices), a
  token permutation and a slice offset table; one segment per adapter.
* "Add optional fast lora path for qwen2/qwen3 on npu" (ms-swift pull request 9754), What this PR
  does and Compatibility checks: the single-adapter LoRA MLP with fused SwiGLU, and the
  single-adapter LoRA attention projections (query/key/value and output), dropout 0, no bias,
  not merged; review thread and Verification advice: the MLP backward (saved X and gate/up
  projections, SwiGLU backward, dX, LoRA weight gradients).

Readings where the pages are silent are listed in each function's docstring.

Parity status: every public function here is pinned by tests under tests/ (brute force on tiny
inputs, hand-worked fixtures, closed forms, invariants and library casts); none is unpinned.
"""

from .rounding import rho, DTYPE_FORMATS
from .sgmv import shrink, expand, tile_list, slice_blocks, validate_metadata
from .mlp import silu, lora_mlp, lora_mlp_rows, sigmoid, silu_grad, lora_mlp_saved, lora_mlp_backward, \
    lora_mlp_grads
from .linear import lora_linear, lora_qkv, lora_linear_rows, lora_linear_backward, lora_qkv_backward
from .embedding import embedding_lora_a

__all__ = [
    "rho", "DTYPE_FORMATS", "shrink", "expand", "tile_list", "slice_blocks",
    "validate_metadata", "silu", "lora_mlp", "lora_mlp_rows", "sigmoid", "silu_grad",
    "lora_mlp_saved", "lora_mlp_backward", "lora_mlp_grads", "lora_linear", "lora_qkv",
    "lora_linear_rows", "lora_linear_backward", "lora_qkv_backward", "embedding_lora_a",
]
