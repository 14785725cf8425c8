"""Pins for the LoRA+SwiGLU MLP backward oracle (CPU only).

Pins: torch.autograd in float64 on the plain forward (an independent derivation of every
gradient), central finite differences of the fp64 forward oracle, pure-Python loops with the same
rounding points on a tiny layer (pins the rounding points, which the fp64 pins cannot see),
B = 0 (zero LoRA-A gradients, dx of the plain SwiGLU MLP), closed-form silu' values, and planted
mistakes that one of these catches.
"""

import math

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle.mlp as mlp_mod
from oracle import lora_mlp, lora_mlp_backward, lora_mlp_grads, lora_mlp_saved, rho, silu_grad

NAMES = ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")


def _case(seed=0, M=4, H=8, I=12, r=2, scale=4.0, dtype="bf16"):
    c = li.config_mlp(seed=seed, M=M, H=H, I=I, r=r, scale=scale, dtype=dtype)
    dout = li.mlp_dout(seed=seed, M=M, H=H, dtype=dtype)
    return c, dout


def _w(c):
    return (c.w_gate, c.w_up, c.w_down, c.a_gate, c.b_gate, c.a_up, c.b_up, c.a_down, c.b_down)


def _oracle(c, dout, dt, mod=mlp_mod):
    e, v = mod.lora_mlp_saved(c.x, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up, c.scale, dt)
    return mod.lora_mlp_backward(c.x, e, v, dout, *_w(c), c.scale, dt)


def _autograd(c, dout):
    """Gradients of sum(dout * out) for the unrounded forward, by torch.autograd in float64."""
    t = lambda a, g=False: a.detach().to(torch.float64).clone().requires_grad_(g)
    x = t(c.x, True)
    Wg, Wu, Wd = t(c.w_gate), t(c.w_up), t(c.w_down)
    Ag, Bg, Au, Bu, Ad, Bd = (t(a, True) for a in (c.a_gate, c.b_gate, c.a_up, c.b_up, c.a_down, c.b_down))
    s = c.scale
    g = x @ Wg.T + s * (x @ Ag.T) @ Bg.T
    u = x @ Wu.T + s * (x @ Au.T) @ Bu.T
    h = torch.nn.functional.silu(g) * u
    out = h @ Wd.T + s * (h @ Ad.T) @ Bd.T
    (out * dout.to(torch.float64)).sum().backward()
    return {"dx": x.grad, "da_gate": Ag.grad, "db_gate": Bg.grad, "da_up": Au.grad, "db_up": Bu.grad,
            "da_down": Ad.grad, "db_down": Bd.grad}


@pytest.mark.parametrize("seed", range(3))
def test_f64_backward_is_the_autograd_gradient(seed):
    c, dout = _case(seed, M=6, H=16, I=24, r=3, scale=1.5)
    got = _oracle(c, dout, "f64")
    ref = _autograd(c, dout)
    for k in NAMES:
        assert np.allclose(got[k], ref[k].numpy(), rtol=1e-10, atol=1e-12), k


def test_f64_backward_matches_finite_differences():
    c, dout = _case(7, M=3, H=8, I=10, r=2, scale=2.0)
    got = _oracle(c, dout, "f64")
    d = dout.to(torch.float64).numpy()
    params = {"dx": "x", "da_gate": "a_gate", "db_gate": "b_gate", "da_up": "a_up", "db_up": "b_up",
              "da_down": "a_down", "db_down": "b_down"}
    rng = np.random.default_rng(0)
    for gname, pname in params.items():
        base = {k: getattr(c, k).to(torch.float64).numpy().copy() for k in
                ("x", "w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")}
        P = base[pname]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in P.shape)
            hstep = 1e-5
            vals = []
            for sgn in (1, -1):
                q = dict(base)
                q[pname] = P.copy()
                q[pname][idx] += sgn * hstep
                out = lora_mlp(q["x"], q["w_gate"], q["w_up"], q["w_down"], q["a_gate"], q["b_gate"],
                               q["a_up"], q["b_up"], q["a_down"], q["b_down"], c.scale, "f64")
                vals.append(float((out * d).sum()))
            fd = (vals[0] - vals[1]) / (2 * hstep)
            assert math.isclose(got[gname][idx], fd, rel_tol=1e-6, abs_tol=1e-8), (gname, idx)


def _brute(c, dout, dt):
    """Pure-Python loops with the rounding points of the definition."""
    L = lambda t: t.double().tolist()
    X, D = L(c.x), L(dout)
    Wg, Wu, Wd = L(c.w_gate), L(c.w_up), L(c.w_down)
    Ag, Bg, Au, Bu, Ad, Bd = (L(t) for t in (c.a_gate, c.b_gate, c.a_up, c.b_up, c.a_down, c.b_down))
    M, H, I, r, s = c.M, c.H, c.I, c.r, c.scale
    rnd = lambda v: float(rho([v], dt)[0])
    dot = lambda a, b: math.fsum(p * q for p, q in zip(a, b))
    col = lambda Mx, j: [row[j] for row in Mx]
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    xa_g = [[rnd(dot(X[m], Ag[j])) for j in range(r)] for m in range(M)]
    xa_u = [[rnd(dot(X[m], Au[j])) for j in range(r)] for m in range(M)]
    E = [[rnd(dot(X[m], Wg[n]) + s * dot(xa_g[m], Bg[n])) for n in range(I)] for m in range(M)]
    V = [[rnd(dot(X[m], Wu[n]) + s * dot(xa_u[m], Bu[n])) for n in range(I)] for m in range(M)]
    F = [[E[m][n] * sig(E[m][n]) for n in range(I)] for m in range(M)]
    hm = [[rnd(F[m][n] * V[m][n]) for n in range(I)] for m in range(M)]
    xa_d = [[rnd(dot(hm[m], Ad[j])) for j in range(r)] for m in range(M)]
    dxa_d = [[rnd(s * dot(D[m], col(Bd, j))) for j in range(r)] for m in range(M)]
    dh = [[dot(D[m], col(Wd, n)) + dot(dxa_d[m], col(Ad, n)) for n in range(I)] for m in range(M)]
    dE, dV = [], []
    for m in range(M):
        re, rv = [], []
        for n in range(I):
            z = E[m][n]
            sg = sig(z)
            re.append(rnd(dh[m][n] * V[m][n] * (sg * (1 + z * (1 - sg)))))
            rv.append(rnd(dh[m][n] * F[m][n]))
        dE.append(re)
        dV.append(rv)
    dxa_g = [[rnd(s * dot(dE[m], col(Bg, j))) for j in range(r)] for m in range(M)]
    dxa_u = [[rnd(s * dot(dV[m], col(Bu, j))) for j in range(r)] for m in range(M)]
    dx = [[rnd(dot(dE[m], col(Wg, k)) + dot(dV[m], col(Wu, k)) + dot(dxa_g[m], col(Ag, k))
               + dot(dxa_u[m], col(Au, k))) for k in range(H)] for m in range(M)]
    gT = lambda P, Q, j, k, sc=1.0: rnd(sc * math.fsum(P[m][j] * Q[m][k] for m in range(M)))
    return {
        "dx": np.array(dx),
        "da_gate": np.array([[gT(dxa_g, X, j, k) for k in range(H)] for j in range(r)]),
        "db_gate": np.array([[gT(dE, xa_g, n, j, s) for j in range(r)] for n in range(I)]),
        "da_up": np.array([[gT(dxa_u, X, j, k) for k in range(H)] for j in range(r)]),
        "db_up": np.array([[gT(dV, xa_u, n, j, s) for j in range(r)] for n in range(I)]),
        "da_down": np.array([[gT(dxa_d, hm, j, n) for n in range(I)] for j in range(r)]),
        "db_down": np.array([[gT(D, xa_d, k, j, s) for j in range(r)] for k in range(H)]),
    }


@pytest.mark.parametrize("seed,scale", [(0, 4.0), (1, 1.5), (2, 0.25)])
def test_bf16_brute_force(seed, scale):
    c, dout = _case(seed, scale=scale)
    got = _oracle(c, dout, "bf16")
    ref = _brute(c, dout, "bf16")
    for k in NAMES:
        # both sides take the same rounding decisions from fp64 sums that differ only in
        # summation order (numpy matmul vs fsum): equal up to a rare one-ulp flip
        assert np.allclose(got[k], ref[k], rtol=2 ** -7, atol=1e-30), k
        assert np.mean(got[k] == ref[k]) >= 0.95, k


def test_b_zero_gives_zero_lora_a_gradients_and_the_plain_mlp_dx():
    c, dout = _case(3, M=5, H=16, I=20, r=4)
    for k in ("b_gate", "b_up", "b_down"):
        setattr(c, k, torch.zeros_like(getattr(c, k)))
    got = _oracle(c, dout, "f64")
    for k in ("da_gate", "da_up", "da_down"):
        assert np.array_equal(got[k], np.zeros_like(got[k])), k
    # dx of the plain SwiGLU MLP by autograd
    x = c.x.to(torch.float64).clone().requires_grad_(True)
    g = x @ c.w_gate.double().T
    u = x @ c.w_up.double().T
    out = (torch.nn.functional.silu(g) * u) @ c.w_down.double().T
    (out * dout.double()).sum().backward()
    assert np.allclose(got["dx"], x.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.abs(got["db_gate"]).max() > 0 and np.abs(got["db_down"]).max() > 0


def test_silu_grad_closed_forms():
    assert silu_grad(0.0) == 0.5
    assert math.isclose(float(silu_grad(40.0)), 1.0, rel_tol=1e-15)
    assert abs(float(silu_grad(-800.0))) == 0.0
    z = np.linspace(-6, 6, 25)
    h = 1e-6
    fd = ((z + h) / (1 + np.exp(-(z + h))) - (z - h) / (1 + np.exp(-(z - h)))) / (2 * h)
    assert np.allclose(silu_grad(z), fd, rtol=1e-8, atol=1e-10)


def test_saved_preactivations_match_the_forward():
    c, _ = _case(4)
    e, v = lora_mlp_saved(c.x, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up, c.scale, "f64")
    _, inter = lora_mlp(*(c.x,) + _w(c), c.scale, "f64", return_intermediates=True)
    assert np.array_equal(e, inter["g"]) and np.array_equal(v, inter["u"])
    eb, vb = lora_mlp_saved(c.x, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up, c.scale, "bf16")
    assert np.array_equal(eb, rho(eb, "bf16"))


BWD_MUTATIONS = [
    ("return sg * (1.0 + z * (1.0 - sg))", "return sg * (1.0 + z * sg)"),           # wrong silu'
    ("rnd(dhmid * v * silu_grad(e))", "rnd(dhmid * silu_grad(e))"),                  # dropped v
    ("dv = rnd(dhmid * f)", "dv = rnd(dhmid * e)"),                                  # silu dropped
    ("rnd(s * (d @ Bd))", "rnd(d @ Bd)"),                                            # dropped scale
    ("dhmid = d @ Wd + dxa_d @ Ad", "dhmid = d @ Wd"),                               # LoRA term lost
    ("+ dxa_g @ Ag + dxa_u @ Au)", "+ dxa_g @ Ag + dxa_u @ Ag)"),                    # wrong A
    ('"db_gate": rnd(s * (de.T @ xa_g))', '"db_gate": rnd(s * (de.T @ xa_u))'),      # wrong operand
    ('"da_up": rnd(dxa_u.T @ x)', '"da_up": rnd(dxa_g.T @ x)'),                      # swapped
    ('"db_down": rnd(s * (d.T @ xa_d))', '"db_down": rnd(d.T @ xa_d)'),              # dropped scale
    ("de = rnd(dhmid * v * silu_grad(e))", "de = dhmid * v * silu_grad(e)"),        # rounding
    ("hmid = rnd(f * v)", "hmid = f * v"),                                           # rounding point
]


@pytest.mark.parametrize("old,new", BWD_MUTATIONS)
def test_backward_mutation_is_caught(old, new):
    from tests.test_oracle_mutations import _mutant

    m = _mutant(mlp_mod, old, new)
    c, dout = _case(5, M=5, H=8, I=12, r=2, scale=2.0)
    caught = False
    got = _oracle(c, dout, "f64", mod=m)
    ref = _autograd(c, dout)
    caught |= any(not np.allclose(got[k], ref[k].numpy(), rtol=1e-10, atol=1e-12) for k in NAMES)
    got = _oracle(c, dout, "bf16", mod=m)
    ref = _brute(c, dout, "bf16")
    caught |= any(np.mean(got[k] == ref[k]) < 0.95 for k in NAMES)
    assert caught


def test_grads_from_the_input_alone():
    c, dout = _case(7, M=5, H=16, I=20, r=3)
    e, v = lora_mlp_saved(c.x, c.w_gate, c.w_up, c.a_gate, c.b_gate, c.a_up, c.b_up, c.scale, "bf16")
    ref = lora_mlp_backward(c.x, e, v, dout, *_w(c), c.scale, "bf16")
    got = lora_mlp_grads(c.x, dout, *_w(c), c.scale, "bf16")
    for k in NAMES:
        assert np.array_equal(got[k], ref[k]), k
