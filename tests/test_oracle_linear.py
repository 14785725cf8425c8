"""Pins for the single-adapter LoRA linear projection oracle (CPU only).

Pins: pure-Python brute force on tiny projections with the same rounding points, the merge
identity x (W + s B A)^T in fp64 (the "not merged" condition of the fast path says both forms are
the same function), B = 0 reducing to the plain product computed with torch, the three
projections of one x, and row sampling.
"""

import math

import numpy as np
import pytest
import torch

import lora_inputs as li
from oracle import lora_linear, lora_linear_rows, lora_qkv, rho


def _tiny(seed=0, M=5, H=8, Nq=6, Nkv=4, r=3, scale=4.0):
    return li.config_qkv(seed=seed, M=M, H=H, Nq=Nq, Nkv=Nkv, r=r, scale=scale)


def _brute(x, w, a, b, s, dt):
    X, W, A, B = (t.double().tolist() for t in (x, w, a, b))
    r, H, N = len(A), len(X[0]), len(W)

    def rnd(v):
        return float(rho([v], dt)[0])

    out = []
    for m in range(len(X)):
        xa = [rnd(math.fsum(X[m][k] * A[j][k] for k in range(H))) for j in range(r)]
        out.append([rnd(math.fsum(X[m][k] * W[n][k] for k in range(H))
                        + s * math.fsum(xa[j] * B[n][j] for j in range(r))) for n in range(N)])
    return np.array(out)


@pytest.mark.parametrize("dt", ["f64", "bf16"])
@pytest.mark.parametrize("seed", range(3))
def test_brute_force(seed, dt):
    c = _tiny(seed)
    got = lora_linear(c.x, c.w_q, c.a_q, c.b_q, c.scale, dt)
    ref = _brute(c.x, c.w_q, c.a_q, c.b_q, c.scale, dt)
    if dt == "f64":
        assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)
    else:  # same rounding points: equal up to a one-ulp tie difference of the fp64 sums
        assert np.allclose(got, ref, rtol=2 ** -7, atol=1e-6)


def test_merge_identity():
    c = _tiny(7, M=6, H=16, Nq=12, r=4, scale=2.5)
    x, w, a, b = (t.double().numpy() for t in (c.x, c.w_q, c.a_q, c.b_q))
    merged = x @ (w + c.scale * (b @ a)).T
    assert np.allclose(lora_linear(c.x, c.w_q, c.a_q, c.b_q, c.scale, "f64"), merged,
                       rtol=1e-12, atol=1e-14)


def test_b_zero_is_plain_linear():
    c = _tiny(3)
    zero = torch.zeros_like(c.b_q)
    ref = rho((c.x.double() @ c.w_q.double().T).numpy(), "bf16")
    assert np.array_equal(lora_linear(c.x, c.w_q, c.a_q, zero, c.scale, "bf16"), ref)


def test_qkv_is_three_projections_and_rows():
    c = _tiny(4)
    q, k, v = lora_qkv(c.x, c.w_q, c.w_k, c.w_v, c.a_q, c.b_q, c.a_k, c.b_k, c.a_v, c.b_v,
                       c.scale, "bf16")
    assert q.shape == (c.M, c.Nq) and k.shape == (c.M, c.Nkv) and v.shape == (c.M, c.Nkv)
    assert np.array_equal(k, _brute(c.x, c.w_k, c.a_k, c.b_k, c.scale, "bf16")) or \
        np.allclose(k, _brute(c.x, c.w_k, c.a_k, c.b_k, c.scale, "bf16"), rtol=2 ** -7, atol=1e-6)
    assert np.allclose(v, _brute(c.x, c.w_v, c.a_v, c.b_v, c.scale, "f64"), rtol=2 ** -6, atol=1e-3)
    rows = [4, 0, 2]
    assert np.array_equal(lora_linear_rows(rows, c.x, c.w_q, c.a_q, c.b_q, c.scale, "bf16"), q[rows])
