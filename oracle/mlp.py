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

Backward (same page, review thread and Verification advice: the fast path's backward takes the
saved input X and the saved gate and up projections, runs the SwiGLU backward kernel
(swiglu_DWf_DW_dfg) and forms dX as df times the up weight plus the gate term, with gradients of
the LoRA A and B weights; X must not be overwritten; gradients are to be tested). The page shows
only fragments. Reading: the training forward also stores the gate and up pre-activations
e = rho(g) and v = rho(u); the frozen W take no gradient; with d = dout,

    f = silu(e),  hmid = rho(f * v),  xa_g = rho(x A_g^T),  xa_u = rho(x A_u^T),
    xa_d = rho(hmid A_d^T),
    dxa_d = rho(s * d B_d),          dhmid = d W_d + dxa_d A_d               (not rounded),
    de = rho(dhmid * v * silu'(e)),  dv = rho(dhmid * f),
    dxa_g = rho(s * de B_g),         dxa_u = rho(s * dv B_u),
    dx = rho(de W_g + dv W_u + dxa_g A_g + dxa_u A_u),
    dA_d = rho(dxa_d^T hmid),  dB_d = rho(s * d^T xa_d),
    dA_g = rho(dxa_g^T x),     dB_g = rho(s * de^T xa_g),
    dA_u = rho(dxa_u^T x),     dB_u = rho(s * dv^T xa_u),

silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))). The products that feed a second matrix product
(dxa_*, de, dv) and every returned gradient are stored once; nothing else is rounded. With no
rounding ('f64') and e, v the exact pre-activations this is the exact gradient of ``lora_mlp``.
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


def sigmoid(z) -> np.ndarray:
    """1 / (1 + exp(-z)) in fp64 (exp overflow gives 0 for very negative z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z) -> np.ndarray:
    """d silu / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    sg = sigmoid(z)
    return sg * (1.0 + z * (1.0 - sg))


def lora_mlp_saved(x, w_gate, w_up, a_gate, b_gate, a_up, b_up, scale: float, out_dtype: str):
    """The gate and up pre-activations the training forward stores for the backward:
    (e, v) = (rho(g), rho(u)) with g and u as in ``lora_mlp``."""
    x = _f64(x)
    s = float(scale)
    xa_g = rho(x @ _f64(a_gate).T, out_dtype)
    xa_u = rho(x @ _f64(a_up).T, out_dtype)
    g = x @ _f64(w_gate).T + s * (xa_g @ _f64(b_gate).T)
    u = x @ _f64(w_up).T + s * (xa_u @ _f64(b_up).T)
    return rho(g, out_dtype), rho(u, out_dtype)


def lora_mlp_backward(x, e, v, dout, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
                      b_down, scale: float, out_dtype: str, return_intermediates: bool = False):
    """Gradients of the LoRA MLP (see the module docstring for the formulas and rounding points).

    ``e`` and ``v`` are the saved gate and up pre-activations; for the plain definition from the
    input alone they come from ``lora_mlp_saved`` (``lora_mlp_grads`` does both steps).

    Returns a dict with dx [M][H], da_gate [r][H], db_gate [I][r], da_up [r][H], db_up [I][r],
    da_down [r][I], db_down [H][r] (fp64 arrays holding values of ``out_dtype``); with
    ``return_intermediates`` also a dict of the stored intermediates (hmid, xa_*, dxa_*, de, dv)
    and the unrounded dhmid."""
    x, e, v, d = _f64(x), _f64(e), _f64(v), _f64(dout)
    Wg, Wu, Wd = _f64(w_gate), _f64(w_up), _f64(w_down)
    Ag, Bg, Au, Bu = _f64(a_gate), _f64(b_gate), _f64(a_up), _f64(b_up)
    Ad, Bd = _f64(a_down), _f64(b_down)
    s = float(scale)
    rnd = lambda t: rho(t, out_dtype)

    # recomputed forward quantities
    f = silu(e)
    hmid = rnd(f * v)
    xa_g = rnd(x @ Ag.T)
    xa_u = rnd(x @ Au.T)
    xa_d = rnd(hmid @ Ad.T)
    # down projection: out = hmid W_d^T + s (hmid A_d^T) B_d^T
    dxa_d = rnd(s * (d @ Bd))
    dhmid = d @ Wd + dxa_d @ Ad
    # SwiGLU: hmid = silu(e) * v
    de = rnd(dhmid * v * silu_grad(e))
    dv = rnd(dhmid * f)
    # gate and up projections
    dxa_g = rnd(s * (de @ Bg))
    dxa_u = rnd(s * (dv @ Bu))
    dx = rnd(de @ Wg + dv @ Wu + dxa_g @ Ag + dxa_u @ Au)
    grads = {
        "dx": dx,
        "da_gate": rnd(dxa_g.T @ x), "db_gate": rnd(s * (de.T @ xa_g)),
        "da_up": rnd(dxa_u.T @ x), "db_up": rnd(s * (dv.T @ xa_u)),
        "da_down": rnd(dxa_d.T @ hmid), "db_down": rnd(s * (d.T @ xa_d)),
    }
    if return_intermediates:
        inter = {"hmid": hmid, "xa_g": xa_g, "xa_u": xa_u, "xa_d": xa_d, "dxa_d": dxa_d,
                 "de": de, "dv": dv, "dxa_g": dxa_g, "dxa_u": dxa_u, "dhmid": dhmid}
        return grads, inter
    return grads


def lora_mlp_grads(x, dout, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down,
                   scale: float, out_dtype: str, return_intermediates: bool = False):
    """The gradients from the layer input, the upstream gradient and the weights alone: the saved
    pre-activations of ``lora_mlp_saved`` fed to ``lora_mlp_backward``."""
    e, v = lora_mlp_saved(x, w_gate, w_up, a_gate, b_gate, a_up, b_up, scale, out_dtype)
    return lora_mlp_backward(x, e, v, dout, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up,
                             a_down, b_down, scale, out_dtype, return_intermediates)
