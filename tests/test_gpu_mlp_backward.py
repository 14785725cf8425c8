"""GPU parity of the LoRA MLP training forward and backward (through the C ABI) against the CPU
oracle computed from x, dout and the weights alone (oracle.lora_mlp_grads: its own saved
pre-activations, its own intermediates).

Tolerances (tests/parity.py): the saved pre-activations e, v and the output are stored values of
row-local sums, compared with the plain bf16 bar |err| <= 1e-2 + 1e-2 |ref|; the seven gradients
are sums whose terms carry bf16-stored factors and are compared with 1e-2 + 1e-2 |ref| + 2u RSS
(u = 2^-8, RSS the root-sum-square of the sum's terms from the oracle's values) and normwise
within 2u, the bar derived in tests/parity.py; the fraction outside the plain bar is printed. Small layers compare every
output; the Qwen3-8B-shaped layer (H = 4096, I = 12288, r = 16, scale 4) compares every output on
its first 160 tokens and, at M = 4096, all seven gradients in full against the oracle over all
4096 tokens (e, v and out on sampled rows).
"""

import functools

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle
from tests.parity import (assert_close_lowp, assert_close_sum_lowp, backward_rss,
                          strict_fail_fraction)

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
    g = alp.mlp_backward(d["x"], e, v, dout.to("cuda").contiguous(), w_gu_t, w_down_t,
                         *[d[k] for k in LORA], c.scale)
    torch.cuda.synchronize()
    assert torch.equal(d["x"], x_before)  # the saved input is only read
    # the prepared layouts are the transposes of the frozen weights, bit for bit
    assert torch.equal(w_gu_t[:, :c.I].cpu(), c.w_gate.T.contiguous())
    assert torch.equal(w_gu_t[:, c.I:].cpu(), c.w_up.T.contiguous())
    assert torch.equal(w_down_t.cpu(), c.w_down.T.contiguous())
    return out.cpu(), e.cpu(), v.cpu(), {k: t.cpu() for k, t in g.items()}


def _check_all(c, dout, out, e, v, g, rows=None):
    """e, v, out (on ``rows``, all when None) and the seven gradients in full, end to end."""
    sel = (lambda t: t) if rows is None else (lambda t: t[rows])
    xs = sel(c.x)
    re, rv = oracle.lora_mlp_saved(xs, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up,
                                   c.scale, "bf16")
    assert_close_lowp(sel(e), re, f"e {c.name}")
    assert_close_lowp(sel(v), rv, f"v {c.name}")
    ro = oracle.lora_mlp(xs, c.w_gate, c.w_up, c.w_down, *[getattr(c, k) for k in LORA], c.scale,
                         "bf16")
    assert_close_lowp(sel(out), ro, f"out {c.name}")
    W = {k: getattr(c, k) for k in ("w_gate", "w_up", "w_down") + LORA}
    ref, inter = oracle.lora_mlp_grads(c.x, dout, *W.values(), c.scale, "bf16",
                                       return_intermediates=True)
    rss = backward_rss(c.x, dout, W, inter, c.scale)
    fails = {k: strict_fail_fraction(g[k], ref[k]) for k in NAMES}
    print(f"{c.name}: fraction outside the plain bar {fails}", flush=True)
    for k in NAMES:
        assert_close_sum_lowp(g[k], ref[k], rss[k], f"{k} {c.name}")


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
    out, e, v, g = _gpu(c, dout)
    _check_all(c, dout, out, e, v, g)


def test_b_zero_gives_zero_lora_a_gradients():
    c = li.config_mlp(seed=81, M=128, H=128, I=192, r=16, scale=4.0)
    for k in ("b_gate", "b_up", "b_down"):
        setattr(c, k, torch.zeros_like(getattr(c, k)))
    dout = li.mlp_dout(seed=81, M=128, H=128)
    print("case", c.name, "B=0", flush=True)
    out, e, v, g = _gpu(c, dout)
    for k in ("da_gate", "da_up", "da_down"):
        assert torch.all(g[k] == 0), k
    _check_all(c, dout, out, e, v, g)


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
    out, e, v, g = _gpu(c, dout)
    _check_all(c, dout, out, e, v, g)


def test_qwen3_8b_layer_full():
    c, dout = _qwen3_8b()
    print("case", c.name, "M = 4096", flush=True)
    out, e, v, g = _gpu(c, dout)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(c.M, size=32, replace=False))
    rows[0], rows[-1] = 0, c.M - 1
    _check_all(c, dout, out, e, v, g, rows=rows)
