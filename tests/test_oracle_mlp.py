"""Pins for the fused LoRA+SwiGLU MLP oracle (CPU only).

Pins: pure-Python brute force on a tiny layer, the merge identity x (W + s B A)^T in fp64 (the
"not merged" condition of the fast path says both forms are the same function), B = 0 reducing
to the plain SwiGLU MLP computed with torch, closed-form silu values, and row sampling.
"""

import math

import numpy as np
import pytest
import torch

import lora_inputs as li
from oracle import lora_mlp, lora_mlp_rows, rho, silu


def _tiny(seed=0, M=4, H=8, I=12, r=2, scale=4.0):
    return li.config_mlp(seed=seed, M=M, H=H, I=I, r=r, scale=scale)


def _args(c):
    return (c.x, c.w_gate, c.w_up, c.w_down, c.a_gate, c.b_gate, c.a_up, c.b_up, c.a_down, c.b_down)


def _brute(c, dt):
    """Pure-Python loops with the same rounding points as the definition."""
    X = c.x.double().tolist()
    Wg, Wu, Wd = c.w_gate.double().tolist(), c.w_up.double().tolist(), c.w_down.double().tolist()
    Ag, Bg = c.a_gate.double().tolist(), c.b_gate.double().tolist()
    Au, Bu = c.a_up.double().tolist(), c.b_up.double().tolist()
    Ad, Bd = c.a_down.double().tolist(), c.b_down.double().tolist()
    s = c.scale

    def rnd(v):
        return float(rho([v], dt)[0])

    out = []
    for m in range(c.M):
        xa_g = [rnd(math.fsum(X[m][k] * Ag[j][k] for k in range(c.H))) for j in range(c.r)]
        xa_u = [rnd(math.fsum(X[m][k] * Au[j][k] for k in range(c.H))) for j in range(c.r)]
        hm = []
        for n in range(c.I):
            g = math.fsum(X[m][k] * Wg[n][k] for k in range(c.H)) + s * math.fsum(xa_g[j] * Bg[n][j] for j in range(c.r))
            u = math.fsum(X[m][k] * Wu[n][k] for k in range(c.H)) + s * math.fsum(xa_u[j] * Bu[n][j] for j in range(c.r))
            hm.append(rnd(g / (1.0 + math.exp(-g)) * u))
        xa_d = [rnd(math.fsum(hm[n] * Ad[j][n] for n in range(c.I))) for j in range(c.r)]
        row = []
        for o in range(c.H):
            v = math.fsum(hm[n] * Wd[o][n] for n in range(c.I)) + s * math.fsum(xa_d[j] * Bd[o][j] for j in range(c.r))
            row.append(rnd(v))
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_f64(seed):
    c = _tiny(seed)
    got = lora_mlp(*_args(c), c.scale, "f64")
    assert np.allclose(got, _brute(c, "f64"), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_bf16(seed):
    """With rounding points in place the two may differ only where a fp64 last-bit difference
    crosses a bf16 rounding boundary: allow at most one bf16 ulp, and require most bitwise."""
    c = _tiny(seed + 10, M=6, H=16, I=24, r=3, scale=2.0)
    got = lora_mlp(*_args(c), c.scale, "bf16")
    ref = _brute(c, "bf16")
    ulp = np.exp2(np.floor(np.log2(np.abs(ref) + 1e-300)) - 7)
    assert (np.abs(got - ref) <= ulp).all()
    assert np.mean(got == ref) > 0.99


def test_merge_identity():
    """Without rounding, LoRA on each projection equals the projection with merged weights
    W + s * B A (computed here with torch fp64 as a plain MLP)."""
    c = _tiny(3, M=5, H=10, I=14, r=3, scale=1.5)
    got = lora_mlp(*_args(c), c.scale, "f64")
    d = lambda t: t.double()
    Wg = d(c.w_gate) + c.scale * d(c.b_gate) @ d(c.a_gate)
    Wu = d(c.w_up) + c.scale * d(c.b_up) @ d(c.a_up)
    Wd = d(c.w_down) + c.scale * d(c.b_down) @ d(c.a_down)
    x = d(c.x)
    ref = (torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    assert np.allclose(got, ref.numpy(), rtol=1e-11, atol=1e-13)


def test_b_zero_is_plain_swiglu_mlp():
    c = _tiny(4, M=6, H=12, I=20, r=2)
    z = lambda t: torch.zeros_like(t)
    got = lora_mlp(c.x, c.w_gate, c.w_up, c.w_down, c.a_gate, z(c.b_gate), c.a_up, z(c.b_up), c.a_down,
                   z(c.b_down), c.scale, "bf16")
    x = c.x.double()
    hm = rho((torch.nn.functional.silu(x @ c.w_gate.double().T) * (x @ c.w_up.double().T)).numpy(), "bf16")
    ref = rho(hm @ c.w_down.double().numpy().T, "bf16")
    assert np.array_equal(got, ref)


def test_silu_closed_forms():
    assert silu([0.0])[0] == 0.0
    assert silu([1.0])[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert silu([-1.0])[0] == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert silu([50.0])[0] == pytest.approx(50.0, rel=1e-15)
    assert silu([-800.0])[0] == 0.0
    # silu(z) - silu(-z) = z
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(silu(z) - silu(-z), z, rtol=1e-14, atol=1e-14)


def test_rows_match_full():
    c = _tiny(5, M=16, H=24, I=40, r=4)
    full = lora_mlp(*_args(c), c.scale, "bf16")
    rows = [0, 3, 7, 15]
    assert np.array_equal(lora_mlp_rows(rows, *_args(c), c.scale, "bf16"), full[rows])


def test_intermediates_shapes():
    c = _tiny(6)
    out, it = lora_mlp(*_args(c), c.scale, "bf16", return_intermediates=True)
    assert out.shape == (c.M, c.H)
    assert it["hmid"].shape == (c.M, c.I) and it["xa_d"].shape == (c.M, c.r)
    assert np.array_equal(it["hmid"], rho(it["hmid"], "bf16"))
