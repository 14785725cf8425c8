"""fp64 oracle of the single-adapter LoRA MLP with SwiGLU.

Test infrastructure only (see the package docstring).

Source: "Add optional fast lora path for qwen2/qwen3 on npu" (ms-swift pull request 9754). The
fast path patches the Qwen2/Qwen3 MLP forward to apply LoRA on the gate, up and down projections
with a fused SwiGLU, and applies only with dropout 0, one active adapter, no trainable base bias
and unmerged weights (Compatibility checks). The review thread names the forward SwiGLU kernel
(swiglu_fg) without showing it; the reading is the standard Qwen MLP, silu of the gate projection
times the up projection, fed to the down projection. With nn.Linear layouts ``[out][in]``:

    gate(x) = x W_g^T + s (x A_g^T) B_g^T,   up(x) likewise,   down(h) likewise,
    out = down( silu(gate(x)) * up(x) ),     silu(z) = z / (1 + exp(-z)).

Reading of the rounding points (the pages do not state them): the LoRA-A products that feed a
second matrix product are stored in the storage dtype (xa_g, xa_u, xa_d); the SwiGLU product
``hmid`` crosses from the gate/up product to the down product and is stored once; ``out`` is
stored once. Nothing else is rounded.
"""

from __future__ import annotations

import numpy as np

from .rounding import rho


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        import torch

        return a.detach().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in fp64 (exp overflow gives z/inf = -0 for very negative z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def lora_mlp(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down, scale: float,
             out_dtype: str, return_intermediates: bool = False):
    """out = rho(hmid W_d^T + s * xa_d B_d^T) with

    xa_g = rho(x A_g^T), xa_u = rho(x A_u^T),
    g = x W_g^T + s * xa_g B_g^T,  u = x W_u^T + s * xa_u B_u^T    (not rounded),
    hmid = rho(silu(g) * u),  xa_d = rho(hmid A_d^T).
    """
    x = _f64(x)
    s = float(scale)
    xa_g = rho(x @ _f64(a_gate).T, out_dtype)
    xa_u = rho(x @ _f64(a_up).T, out_dtype)
    g = x @ _f64(w_gate).T + s * (xa_g @ _f64(b_gate).T)
    u = x @ _f64(w_up).T + s * (xa_u @ _f64(b_up).T)
    hmid = rho(silu(g) * u, out_dtype)
    xa_d = rho(hmid @ _f64(a_down).T, out_dtype)
    out = rho(hmid @ _f64(w_down).T + s * (xa_d @ _f64(b_down).T), out_dtype)
    if return_intermediates:
        return out, {"xa_g": xa_g, "xa_u": xa_u, "g": g, "u": u, "hmid": hmid, "xa_d": xa_d}
    return out


def lora_mlp_rows(rows, x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down,
                  scale: float, out_dtype: str):
    """``lora_mlp`` restricted to the given token rows (each output row depends on its own input
    row only), for sampled checks at full size."""
    rows = np.asarray(rows, dtype=np.int64)
    xs = _f64(x)[rows]
    return lora_mlp(xs, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down,
                    scale, out_dtype)
