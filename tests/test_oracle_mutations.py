"""The pins catch plausible mistakes: each test plants one mistake in a copy of the oracle's source
(on the CPU, never in the product) and checks that the hand-worked fixture or a brute-force pin
then fails."""

import importlib.util
import json
import os
import sys
import types

import numpy as np
import pytest

import oracle.sgmv as sgmv_mod
import oracle.mlp as mlp_mod
import oracle.linear as linear_mod
import oracle.embedding as emb_mod
import lora_inputs as li
from oracle import rho

HERE = os.path.dirname(__file__)


def _mutant(mod, old, new):
    src = open(mod.__file__).read()
    assert src.count(old) >= 1, old
    src = src.replace(old, new, 1)
    m = types.ModuleType(mod.__name__ + "_mutant")
    m.__dict__["__package__"] = "oracle"
    m.__dict__["__name__"] = "oracle._mutant"
    exec(compile(src, mod.__file__ + "[mutant]", "exec"), m.__dict__)
    return m


def _fixture_ok(m):
    with open(os.path.join(HERE, "golden", "sgmv_handworked.json")) as f:
        d = json.load(f)
    A = np.array([[[float(e) for e in r] for r in b] for b in d["A"]])
    B = np.array([[[float(e) for e in r] for r in b] for b in d["B"]])
    try:
        h = m.shrink(np.array(d["x"], float), A, d["seg_indptr"], d["weight_indices"], d["permutation"],
                     d["lora_ranks"], d["S"], d["R"], "bf16")
        y = m.expand(h, B, d["slice_offsets"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                     d["lora_ranks"], d["scalings"], np.array(d["y_in"], float), d["R"], "bf16")
    except Exception:
        return False
    return np.array_equal(h, np.array(d["h_expected"], float)) and np.array_equal(y, np.array(d["y_expected"], float))


SGMV_MUTATIONS = [
    ("rows = x[perm[i0:i1]]", "rows = x[i0:i1]"),  # forgot the gather
    ("block = A[a, s * R: s * R + r]", "block = A[a, s * R: s * R + R]"),  # ignores the rank
    ("block = A[a, s * R: s * R + r]", "block = A[a, s * r: s * r + r]"),  # wrong slice stride
    ("a = int(widx[g])\n        r = int(ranks[a])\n        rows = x", "a = g\n        r = int(ranks[a])\n        rows = x"),
    ("sig[a] * delta", "delta"),  # dropped scaling
    ("y_in[rows, n0:n1] + sig[a] * delta", "sig[a] * delta"),  # dropped base term
    ("y_in[rows, n0:n1] + sig[a] * delta", "y_in[rows, n0:n1] - sig[a] * delta"),  # sign
    ("rows = perm[i0:i1]", "rows = np.arange(i0, i1)"),  # forgot the scatter
    ("B[a, n0:n1, :r].T", "B[a, :n1 - n0, :r].T"),  # slice offset dropped
    ("h[i0:i1, s * R: s * R + r] @", "h[i0:i1, 0: r] @"),  # wrong h block
]


@pytest.mark.parametrize("old,new", SGMV_MUTATIONS)
def test_sgmv_mutation_is_caught(old, new):
    assert _fixture_ok(sgmv_mod)
    assert not _fixture_ok(_mutant(sgmv_mod, old, new))


MLP_MUTATIONS = [
    ("g = x @ _f64(w_gate).T + s * (xa_g @ _f64(b_gate).T)", "g = x @ _f64(w_gate).T + (xa_g @ _f64(b_gate).T)"),
    ("u = x @ _f64(w_up).T + s * (xa_u @ _f64(b_up).T)", "u = x @ _f64(w_up).T + s * (xa_g @ _f64(b_up).T)"),
    ("hmid = rho(silu(g) * u, out_dtype)", "hmid = rho(silu(u) * g, out_dtype)"),
    ("xa_d = rho(hmid @ _f64(a_down).T, out_dtype)", "xa_d = rho(hmid @ _f64(a_down).T * 0, out_dtype)"),
    ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
]


@pytest.mark.parametrize("old,new", MLP_MUTATIONS)
def test_mlp_mutation_is_caught(old, new):
    from tests.test_oracle_mlp import _args, _brute, _tiny

    c = _tiny(1)
    ref = _brute(c, "f64")
    good = mlp_mod.lora_mlp(*_args(c), c.scale, "f64")
    assert np.allclose(good, ref, rtol=1e-11, atol=1e-13)
    bad = _mutant(mlp_mod, old, new).lora_mlp(*_args(c), c.scale, "f64")
    assert not np.allclose(bad, ref, rtol=1e-11, atol=1e-13)


LINEAR_MUTATIONS = [
    ("rho(x @ _f64(w).T + float(scale) * (xa @ _f64(b).T), out_dtype)",
     "rho(x @ _f64(w).T + (xa @ _f64(b).T), out_dtype)"),  # dropped scaling
    ("rho(x @ _f64(w).T + float(scale) * (xa @ _f64(b).T), out_dtype)",
     "rho(x @ _f64(w).T - float(scale) * (xa @ _f64(b).T), out_dtype)"),  # sign
    ("xa = rho(x @ _f64(a).T, out_dtype)", "xa = rho(x @ _f64(a)[::-1].T, out_dtype)"),  # rank order
    ("rho(x @ _f64(w).T + float(scale)", "rho(float(scale)"),  # dropped base product
]


@pytest.mark.parametrize("old,new", LINEAR_MUTATIONS)
def test_linear_mutation_is_caught(old, new):
    from tests.test_oracle_linear import _brute, _tiny

    c = _tiny(2)
    ref = _brute(c.x, c.w_q, c.a_q, c.b_q, c.scale, "f64")
    good = linear_mod.lora_linear(c.x, c.w_q, c.a_q, c.b_q, c.scale, "f64")
    assert np.allclose(good, ref, rtol=1e-11, atol=1e-13)
    bad = _mutant(linear_mod, old, new).lora_linear(c.x, c.w_q, c.a_q, c.b_q, c.scale, "f64")
    assert not np.allclose(bad, ref, rtol=1e-11, atol=1e-13)


EMB_MUTATIONS = [
    ("cols = ids[perm[i0:i1]]", "cols = ids[i0:i1]"),            # forgot the permutation
    ("h[i0:i1, :r] = A[a, :r][:, cols].T", "h[i0:i1, :r] = A[a, :r][:, cols][::-1].T"),  # rank order
    ("a = int(widx[g])", "a = g % A.shape[0]"),                  # adapter of the segment ignored
    ("h[i0:i1, r:] = 0.0", "pass"),                                # rank padding not zeroed
]


@pytest.mark.parametrize("old,new", EMB_MUTATIONS)
def test_embedding_mutation_is_caught(old, new):
    from tests.test_oracle_embedding import HERE as H

    with open(os.path.join(H, "golden", "embedding_handworked.json")) as f:
        d = json.load(f)
    A = np.array([[[float(e) for e in r] for r in b] for b in d["A"]])
    args = (d["input_ids"], A, d["seg_indptr"], d["weight_indices"], d["permutation"], d["lora_ranks"], d["R"])
    exp = np.array(d["h_expected"], dtype=float)
    assert np.array_equal(emb_mod.embedding_lora_a(*args), exp)
    got = _mutant(emb_mod, old, new).embedding_lora_a(*args)
    assert not np.array_equal(got, exp, equal_nan=True)
