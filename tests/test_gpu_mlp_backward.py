"""GPU parity of the LoRA MLP training forward and backward (through the C ABI) against the CPU
oracle, bf16 tolerance |err| <= 1e-2 + 1e-2 |ref|.

Each step is checked on its own inputs: the saved pre-activations e, v against the oracle's
from x; every stored intermediate of the backward (hmid, de, dv, the LoRA-A products and their
gradients) against the oracle's step applied to the GPU's own inputs of that step, and every
gradient against the oracle applied to the GPU's intermediates. A stored bf16 intermediate may
differ from the oracle's by one unit where its fp32 and fp64 values straddle a rounding
boundary; carried into a later sum with cancellation (dA = dxa^T x over the tokens) such a
difference alone can exceed the tolerance, so only the small layers are also compared end to
end (oracle from x, e, v and dout alone). Small layers compare every output; the Qwen3-8B-shaped
layer (H = 4096, I = 12288, r = 16, scale 4) compares every output on its first 160 tokens
(M = 160: one partial row tile) and, at M = 4096, sampled rows of e, v, out and dx and sampled
columns of de, dv, hmid, db_gate, db_up and da_down.
"""

import functools

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle
from oracle.mlp import silu, silu_grad
from oracle.rounding import rho
from tests.parity import assert_close_lowp

pytestmark = pytest.mark.gpu

NAMES = ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")
LORA = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def _dev(c):
    g = lambda t: t.to("cuda").contiguous()
    return {k: g(getattr(c, k)) for k in ("x", "w_gate", "w_up", "w_down") + LORA}


def _gpu(c, dout):
    alp = __import__("adapter_lora_projection_amd")
    d = _dev(c)
    out, e, v = alp.mlp_fused_train(d["x"], d["w_gate"], d["w_up"], d["w_down"], *[d[k] for k in LORA],
                                    c.scale)
    w_gu_t, w_down_t = alp.mlp_prepare_backward(d["w_gate"], d["w_up"], d["w_down"])
    x_before = d["x"].clone()
    g, inter = alp.mlp_backward(d["x"], e, v, dout.to("cuda").contiguous(), w_gu_t, w_down_t,
                                *[d[k] for k in LORA], c.scale, return_intermediates=True)
    torch.cuda.synchronize()
    assert torch.equal(d["x"], x_before)  # the saved input is only read
    # the prepared layouts are the transposes of the frozen weights, bit for bit
    assert torch.equal(w_gu_t[:, :c.I].cpu(), c.w_gate.T.contiguous())
    assert torch.equal(w_gu_t[:, c.I:].cpu(), c.w_up.T.contiguous())
    assert torch.equal(w_down_t.cpu(), c.w_down.T.contiguous())
    return (out.cpu(), e.cpu(), v.cpu(), {k: t.cpu() for k, t in g.items()},
            {k: t.cpu() for k, t in inter.items()})


def _check_all(c, dout, out, e, v, g, inter, end_to_end):
    re, rv = oracle.lora_mlp_saved(c.x, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up,
                                   c.scale, "bf16")
    assert_close_lowp(e, re, f"e {c.name}")
    assert_close_lowp(v, rv, f"v {c.name}")
    ro = oracle.lora_mlp(c.x, c.w_gate, c.w_up, c.w_down, *[getattr(c, k) for k in LORA], c.scale,
                         "bf16")
    assert_close_lowp(out, ro, f"out {c.name}")
    W = (c.w_gate, c.w_up, c.w_down, *[getattr(c, k) for k in LORA])
    # step by step: each intermediate and gradient from the GPU's own inputs of that step
    ref, own = oracle.lora_mlp_backward(c.x, e, v, dout, *W, c.scale, "bf16",
                                        return_intermediates=True, given=inter)
    for k, t in inter.items():
        assert_close_lowp(t, own[k], f"{k} {c.name}")
    for k in NAMES:
        assert_close_lowp(g[k], ref[k], f"{k} {c.name}")
    if end_to_end:
        ref = oracle.lora_mlp_backward(c.x, e, v, dout, *W, c.scale, "bf16")
        for k in NAMES:
            assert_close_lowp(g[k], ref[k], f"{k} {c.name} end to end")


@pytest.mark.parametrize("M,H,I,r,scale", [
    (96, 128, 160, 16, 4.0),
    (300, 256, 320, 7, 2.0),      # ragged M, odd rank
    (257, 128, 96, 33, 1.5),      # rank padded to 64, scale not a power of two
    (1, 32, 32, 1, 4.0),
    (512, 256, 512, 64, 0.5),
])
def test_backward_small(M, H, I, r, scale):
    c = li.config_mlp(seed=70 + M, M=M, H=H, I=I, r=r, scale=scale)
    dout = li.mlp_dout(seed=70 + M, M=M, H=H)
    print("case", c.name, flush=True)
    out, e, v, g, inter = _gpu(c, dout)
    _check_all(c, dout, out, e, v, g, inter, end_to_end=True)


def test_b_zero_gives_zero_lora_a_gradients():
    c = li.config_mlp(seed=81, M=128, H=128, I=192, r=16, scale=4.0)
    for k in ("b_gate", "b_up", "b_down"):
        setattr(c, k, torch.zeros_like(getattr(c, k)))
    dout = li.mlp_dout(seed=81, M=128, H=128)
    print("case", c.name, "B=0", flush=True)
    out, e, v, g, inter = _gpu(c, dout)
    for k in ("da_gate", "da_up", "da_down"):
        assert torch.all(g[k] == 0), k
    _check_all(c, dout, out, e, v, g, inter, end_to_end=True)


def test_autograd_function_matches_the_direct_calls():
    alp = __import__("adapter_lora_projection_amd")
    c = li.config_mlp(seed=82, M=192, H=128, I=160, r=8, scale=2.0)
    dout = li.mlp_dout(seed=82, M=192, H=128).to("cuda")
    print("case", c.name, "autograd", flush=True)
    d = _dev(c)
    w_gu_t, w_down_t = alp.mlp_prepare_backward(d["w_gate"], d["w_up"], d["w_down"])
    leaves = {k: d[k].clone().requires_grad_(True) for k in ("x",) + LORA}
    out = alp.LoraMlpFunction.apply(leaves["x"], *[leaves[k] for k in LORA], d["w_gate"], d["w_up"],
                                    d["w_down"], w_gu_t, w_down_t, c.scale)
    out.backward(dout)
    _, e, v = alp.mlp_fused_train(d["x"], d["w_gate"], d["w_up"], d["w_down"], *[d[k] for k in LORA],
                                  c.scale)
    g = alp.mlp_backward(d["x"], e, v, dout, w_gu_t, w_down_t, *[d[k] for k in LORA], c.scale)
    torch.cuda.synchronize()
    names = {"x": "dx", "a_gate": "da_gate", "b_gate": "db_gate", "a_up": "da_up", "b_up": "db_up",
             "a_down": "da_down", "b_down": "db_down"}
    for leaf, k in names.items():
        assert torch.equal(leaves[leaf].grad, g[k]), k


@functools.lru_cache(maxsize=1)
def _qwen3_8b():
    return li.config_mlp(), li.mlp_dout()


def test_qwen3_8b_layer_first_160_tokens():
    full, full_dout = _qwen3_8b()
    M = 160
    c = li.config_mlp(seed=4, M=8, H=32, I=32, r=16)  # container, overwritten below
    c.name, c.M, c.H, c.I, c.r, c.scale = "mlp_qwen3_8b_M160", M, full.H, full.I, full.r, full.scale
    for k in ("w_gate", "w_up", "w_down") + LORA:
        setattr(c, k, getattr(full, k))
    c.x = full.x[:M].contiguous()
    dout = full_dout[:M].contiguous()
    print("case", c.name, flush=True)
    out, e, v, g, inter = _gpu(c, dout)
    _check_all(c, dout, out, e, v, g, inter, end_to_end=False)


def test_qwen3_8b_layer_sampled():
    c, dout = _qwen3_8b()
    print("case", c.name, "sampled", flush=True)
    out, e, v, g, inter = _gpu(c, dout)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(c.M, size=24, replace=False))
    rows[0], rows[-1] = 0, c.M - 1
    W = [getattr(c, k) for k in LORA]
    # e, v, out on sampled rows (each row depends on its own input row only)
    re, rv = oracle.lora_mlp_saved(c.x[rows], c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up,
                                   c.scale, "bf16")
    assert_close_lowp(e[rows], re, "e rows")
    assert_close_lowp(v[rows], rv, "v rows")
    ro = oracle.lora_mlp_rows(rows, c.x, c.w_gate, c.w_up, c.w_down, *W, c.scale, "bf16")
    assert_close_lowp(out[rows], ro, "out rows")
    # every row-local step on the sampled rows, from the GPU's own inputs of each step (the
    # oracle's weight gradients are then partial sums over those rows and are not used)
    given = {k: t[rows] for k, t in inter.items()}
    rb, own = oracle.lora_mlp_backward(c.x[rows], e[rows], v[rows], dout[rows], c.w_gate, c.w_up,
                                       c.w_down, *W, c.scale, "bf16", return_intermediates=True,
                                       given=given)
    for k, t in given.items():
        assert_close_lowp(t, own[k], f"{k} rows")
    assert_close_lowp(g["dx"][rows], rb["dx"], "dx rows")
    # sampled columns i: de, dv, hmid (over all tokens) from the GPU's inputs of their step, and
    # the sums over the tokens db_gate[i], db_up[i], da_down[:, i] from the GPU's intermediates
    f64 = lambda t: t.to(torch.float64).numpy()
    d, E, V = f64(dout), f64(e), f64(v)
    s = c.scale
    dxa_d = f64(inter["dxa_d"])
    Wd, Ad = f64(c.w_down), f64(c.a_down)
    xa_g, xa_u = f64(inter["xa_g"]), f64(inter["xa_u"])
    cols = np.sort(rng.choice(c.I, size=24, replace=False))
    cols[0], cols[-1] = 0, c.I - 1
    for i in cols:
        dh = d @ Wd[:, i] + dxa_d @ Ad[:, i]
        f = silu(E[:, i])
        assert_close_lowp(inter["de"][:, i], rho(dh * V[:, i] * silu_grad(E[:, i]), "bf16"), f"de col {i}")
        assert_close_lowp(inter["dv"][:, i], rho(dh * f, "bf16"), f"dv col {i}")
        assert_close_lowp(inter["hmid"][:, i], rho(f * V[:, i], "bf16"), f"hmid col {i}")
        de, dv, hm = f64(inter["de"][:, i]), f64(inter["dv"][:, i]), f64(inter["hmid"][:, i])
        assert_close_lowp(g["db_gate"][i], rho(s * (de @ xa_g), "bf16"), f"db_gate col {i}")
        assert_close_lowp(g["db_up"][i], rho(s * (dv @ xa_u), "bf16"), f"db_up col {i}")
        assert_close_lowp(g["da_down"][:, i], rho(dxa_d.T @ hm, "bf16"), f"da_down col {i}")
