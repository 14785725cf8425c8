"""Pins for the backward of the single-adapter LoRA projection oracle (CPU only).

Pins: torch.autograd in float64 on the plain forward (an independent derivation of every
gradient), central finite differences of the fp64 forward oracle, pure-Python loops with the
same rounding points on tiny projections (pins the rounding points, which the fp64 pins cannot
see), B = 0 (zero LoRA-A gradient, dx of the plain product), the query/key/value backward
against three single-projection backwards, and planted mistakes that one of these catches.
"""

import math

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle.linear as lin_mod
from oracle import lora_linear, lora_linear_backward, lora_qkv_backward, rho

NAMES = ("dx", "da", "db")


def _case(seed=0, M=5, H=8, N=6, r=3, scale=4.0):
    c = li.config_qkv(seed=seed, M=M, H=H, Nq=N, Nkv=4, r=r, scale=scale)
    (dout,) = li.projection_douts(seed=seed, M=M, widths=(N,))
    return c, dout


def _autograd(c, dout):
    """Gradients of sum(dout * y) for the unrounded forward, by torch.autograd in float64."""
    t = lambda a, g=False: a.detach().to(torch.float64).clone().requires_grad_(g)
    x, W, A, B = t(c.x, True), t(c.w_q), t(c.a_q, True), t(c.b_q, True)
    y = x @ W.T + c.scale * (x @ A.T) @ B.T
    (y * dout.to(torch.float64)).sum().backward()
    return {"dx": x.grad.numpy(), "da": A.grad.numpy(), "db": B.grad.numpy()}


def _oracle(c, dout, dt, mod=lin_mod):
    return mod.lora_linear_backward(c.x, dout, c.w_q, c.a_q, c.b_q, c.scale, dt)


def _brute(c, dout, dt):
    """Pure-Python loops over the backward's definition with its rounding points."""
    X, D, W, A, B = (t.double().tolist() for t in (c.x, dout, c.w_q, c.a_q, c.b_q))
    s, M, H, N, r = c.scale, len(X), len(X[0]), len(W), len(A)

    def rnd(v):
        return float(rho([v], dt)[0])

    xa = [[rnd(math.fsum(X[m][k] * A[j][k] for k in range(H))) for j in range(r)] for m in range(M)]
    dxa = [[rnd(s * math.fsum(D[m][n] * B[n][j] for n in range(N))) for j in range(r)]
           for m in range(M)]
    dx = [[rnd(math.fsum(D[m][n] * W[n][k] for n in range(N))
               + math.fsum(dxa[m][j] * A[j][k] for j in range(r))) for k in range(H)]
          for m in range(M)]
    da = [[rnd(math.fsum(dxa[m][j] * X[m][k] for m in range(M))) for k in range(H)]
          for j in range(r)]
    db = [[rnd(s * math.fsum(D[m][n] * xa[m][j] for m in range(M))) for j in range(r)]
          for n in range(N)]
    return {"dx": np.array(dx), "da": np.array(da), "db": np.array(db)}


@pytest.mark.parametrize("seed", range(3))
def test_f64_backward_is_the_autograd_gradient(seed):
    c, dout = _case(seed)
    got, ref = _oracle(c, dout, "f64"), _autograd(c, dout)
    for k in NAMES:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-13, err_msg=k)


def test_f64_backward_matches_finite_differences():
    c, dout = _case(3, M=4, H=6, N=5, r=2)
    d = dout.double().numpy()
    g = _oracle(c, dout, "f64")
    rng = np.random.default_rng(0)
    base = {"x": c.x.double().numpy(), "a": c.a_q.double().numpy(), "b": c.b_q.double().numpy()}

    def loss(x, a, b):
        return float(np.sum(lora_linear(x, c.w_q, a, b, c.scale, "f64") * d))

    eps = 1e-6
    for name, gk in (("x", "dx"), ("a", "da"), ("b", "db")):
        delta = rng.standard_normal(base[name].shape)
        plus = dict(base); plus[name] = base[name] + eps * delta
        minus = dict(base); minus[name] = base[name] - eps * delta
        fd = (loss(**plus) - loss(**minus)) / (2 * eps)
        assert math.isclose(fd, float(np.sum(g[gk] * delta)), rel_tol=1e-6, abs_tol=1e-9), name


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("scale", [4.0, 1.5])
def test_bf16_brute_force(seed, scale):
    c, dout = _case(seed, scale=scale)
    got, ref = _oracle(c, dout, "bf16"), _brute(c, dout, "bf16")
    for k in NAMES:
        assert np.array_equal(got[k], ref[k]), k


def test_b_zero_gives_zero_lora_a_gradient_and_the_plain_dx():
    c, dout = _case(4)
    c.b_q = torch.zeros_like(c.b_q)
    got = _oracle(c, dout, "bf16")
    assert not np.any(got["da"])
    plain = rho(dout.double().numpy() @ c.w_q.double().numpy(), "bf16")
    assert np.array_equal(got["dx"], plain)
    xa = rho(c.x.double().numpy() @ c.a_q.double().numpy().T, "bf16")
    assert np.array_equal(got["db"], rho(c.scale * (dout.double().numpy().T @ xa), "bf16"))


@pytest.mark.parametrize("dt", ["f64", "bf16"])
def test_qkv_backward_is_three_projections(dt):
    c = li.config_qkv(seed=6, M=5, H=8, Nq=6, Nkv=4, r=3, scale=2.0)
    dq, dk, dv = li.projection_douts(seed=6, M=5, widths=(6, 4, 4))
    got = lora_qkv_backward(c.x, dq, dk, dv, c.w_q, c.w_k, c.w_v, c.a_q, c.b_q, c.a_k, c.b_k,
                            c.a_v, c.b_v, c.scale, dt)
    parts = [lora_linear_backward(c.x, d, w, a, b, c.scale, "f64") for d, w, a, b in
             ((dq, c.w_q, c.a_q, c.b_q), (dk, c.w_k, c.a_k, c.b_k), (dv, c.w_v, c.a_v, c.b_v))]
    for name, p in zip("qkv", (
            lora_linear_backward(c.x, dq, c.w_q, c.a_q, c.b_q, c.scale, dt),
            lora_linear_backward(c.x, dk, c.w_k, c.a_k, c.b_k, c.scale, dt),
            lora_linear_backward(c.x, dv, c.w_v, c.a_v, c.b_v, c.scale, dt))):
        assert np.array_equal(got["da_" + name], p["da"]) and np.array_equal(got["db_" + name], p["db"])
    if dt == "f64":
        np.testing.assert_allclose(got["dx"], sum(p["dx"] for p in parts), rtol=1e-12, atol=1e-14)
    else:  # one rounding of the summed terms, not a sum of rounded ones
        lin = lambda d, w, a, b: (d.double().numpy() @ w.double().numpy()
                                  + rho(c.scale * (d.double().numpy() @ b.double().numpy()), "bf16")
                                  @ a.double().numpy())
        ref = rho(lin(dq, c.w_q, c.a_q, c.b_q) + lin(dk, c.w_k, c.a_k, c.b_k)
                  + lin(dv, c.w_v, c.a_v, c.b_v), "bf16")
        assert np.array_equal(got["dx"], ref)


MUTATIONS = [
    ("dxa = rnd(s * (d @ B))", "dxa = rnd(d @ B)"),                                   # dropped scale
    ('"dx": rnd(d @ W + dxa @ A)', '"dx": rnd(d @ W)'),                               # LoRA term lost
    ('"dx": rnd(d @ W + dxa @ A)', '"dx": rnd(d @ W - dxa @ A)'),                     # wrong sign
    ('"da": rnd(dxa.T @ x)', '"da": rnd(s * (dxa.T @ x))'),                           # extra scale
    ('"db": rnd(s * (d.T @ xa))', '"db": rnd(s * (d.T @ (x @ A.T)))'),                # rounding point
    ("xa = rnd(x @ A.T)", "xa = rnd(x @ A.T) * 0.5"),                                  # wrong operand
]


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_backward_mutation_is_caught(old, new):
    from tests.test_oracle_mutations import _mutant

    m = _mutant(lin_mod, old, new)
    c, dout = _case(5)
    got, ref = _oracle(c, dout, "f64", mod=m), _autograd(c, dout)
    caught = any(not np.allclose(got[k], ref[k], rtol=1e-10, atol=1e-12) for k in NAMES)
    got, ref = _oracle(c, dout, "bf16", mod=m), _brute(c, dout, "bf16")
    caught |= any(not np.array_equal(got[k], ref[k]) for k in NAMES)
    assert caught
