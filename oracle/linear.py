"""fp64 oracle of the single-adapter LoRA linear projections (attention Q, K, V and O).

Test infrastructure only (see the package docstring).

Source: "Add optional fast lora path for qwen2/qwen3 on npu" (ms-swift pull request 9754). What
this PR does: the fast path patches the Qwen2/Qwen3 attention forward as well as the MLP, with
the fast LoRA projection logic; the review thread names the projection helpers for the fused
query/key/value projection and for the output projection, under the same compatibility checks
(dropout 0, one active adapter, no trainable base bias, unmerged weights). With nn.Linear
layouts ``[out][in]`` each projection is

    y = x W^T + s (x A^T) B^T.

Reading of the rounding points (the pages do not state them), as for the MLP: the LoRA-A product
that feeds the second matrix product is stored in the storage dtype, and the output is stored
once. The query, key and value projections read the same x; each has its own W, A and B.

Backward (same PR, Verification advice: gradients of the projection fast paths are checked
against a reference). For dout = dL/dy of one projection, with the forward's rounding points and
the same reading as the MLP backward (a product that feeds a second product is stored once,
every returned gradient is stored once; the frozen W takes no gradient):

    xa  = rho(x A^T)                         (recomputed, as the forward stores it)
    dxa = rho(s dout B)
    dx  = rho(dout W + dxa A)
    dA  = rho(dxa^T x),   dB = rho(s dout^T xa)

For the query, key and value projections of one x, dx is the sum of the three projections'
dout W + dxa A terms, rounded once.
"""

from __future__ import annotations

import numpy as np

from .rounding import rho


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        import torch

        return a.detach().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def lora_linear(x, w, a, b, scale: float, out_dtype: str):
    """y = rho(x W^T + s * xa B^T) with xa = rho(x A^T) (``out_dtype`` 'f64' rounds nothing)."""
    x = _f64(x)
    xa = rho(x @ _f64(a).T, out_dtype)
    return rho(x @ _f64(w).T + float(scale) * (xa @ _f64(b).T), out_dtype)


def lora_qkv(x, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v, b_v, scale: float, out_dtype: str):
    """(q, k, v): the three projections of the same x, each ``lora_linear``."""
    return (lora_linear(x, w_q, a_q, b_q, scale, out_dtype),
            lora_linear(x, w_k, a_k, b_k, scale, out_dtype),
            lora_linear(x, w_v, a_v, b_v, scale, out_dtype))


def lora_linear_rows(rows, x, w, a, b, scale: float, out_dtype: str):
    """``lora_linear`` restricted to the given rows of x (each output row depends on its own
    input row only), for sampled checks at full size."""
    rows = np.asarray(rows, dtype=np.int64)
    return lora_linear(_f64(x)[rows], w, a, b, scale, out_dtype)


def lora_linear_backward(x, dout, w, a, b, scale: float, out_dtype: str):
    """Gradients of ``lora_linear`` (module docstring): dict with dx [M][K], da [r][K],
    db [N][r] (fp64 arrays holding values of ``out_dtype``; 'f64' rounds nothing)."""
    x, d, W, A, B = _f64(x), _f64(dout), _f64(w), _f64(a), _f64(b)
    s = float(scale)
    rnd = lambda t: rho(t, out_dtype)
    xa = rnd(x @ A.T)
    dxa = rnd(s * (d @ B))
    return {"dx": rnd(d @ W + dxa @ A), "da": rnd(dxa.T @ x), "db": rnd(s * (d.T @ xa))}


def lora_qkv_backward(x, dq, dk, dv, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v, b_v, scale: float,
                      out_dtype: str):
    """Gradients of ``lora_qkv``: dx [M][K] (the three projections' terms summed, rounded once)
    and da_*, db_* of each projection."""
    x = _f64(x)
    s = float(scale)
    rnd = lambda t: rho(t, out_dtype)
    out, acc = {}, 0.0
    for name, d, W, A, B in (("q", dq, w_q, a_q, b_q), ("k", dk, w_k, a_k, b_k),
                             ("v", dv, w_v, a_v, b_v)):
        d, W, A, B = _f64(d), _f64(W), _f64(A), _f64(B)
        xa = rnd(x @ A.T)
        dxa = rnd(s * (d @ B))
        acc = acc + d @ W + dxa @ A
        out["da_" + name] = rnd(dxa.T @ x)
        out["db_" + name] = rnd(s * (d.T @ xa))
    out["dx"] = rnd(acc)
    return out
