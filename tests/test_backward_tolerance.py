"""Why the MLP-backward weight gradients are compared with the bar 1e-2 + 1e-2 |ref| + 2u RSS
(tests/parity.py) and not the plain 1e-2 + 1e-2 |ref| (CPU only).

A straightforward fp32-accumulating evaluation of the same formulas and rounding points (torch
float32 on the CPU, written here independently of the oracle) is compared with the fp64 oracle
computed from x, dout and the weights alone, at the Qwen3-8B-shaped layer (M = 4096, H = 4096,
I = 12288, r = 16, scale 4):
* it fails the plain bar on a fraction of the entries of the weight gradients, because a sum over
  4096 tokens with cancellation carries the noise of the stored bf16 factors whose rounding went
  the other way, and entries near zero then have only the 1e-2 absolute allowance;
* it passes the bar with the 2u RSS allowance on every entry of all seven gradients.
"""

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle
from tests.parity import assert_close_sum_lowp, backward_rss, strict_fail_fraction

NAMES = ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")
LORA = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")


def _fp32_backward(c, dout):
    """Saved pre-activations and gradients with fp32 sums, rounded to bf16 where stored."""
    f = lambda t: t.to(torch.float32)
    bf = lambda t: t.to(torch.bfloat16).to(torch.float32)
    s = c.scale
    x, d = f(c.x), f(dout)
    Wg, Wu, Wd = f(c.w_gate), f(c.w_up), f(c.w_down)
    Ag, Bg, Au, Bu, Ad, Bd = (f(getattr(c, k)) for k in LORA)
    xa_g, xa_u = bf(x @ Ag.T), bf(x @ Au.T)
    e = bf(x @ Wg.T + s * (xa_g @ Bg.T))
    v = bf(x @ Wu.T + s * (xa_u @ Bu.T))
    sg = torch.sigmoid(e)
    hmid = bf(e * sg * v)
    xa_d = bf(hmid @ Ad.T)
    dxa_d = bf(s * (d @ Bd))
    dh = d @ Wd + dxa_d @ Ad
    de = bf(dh * v * sg * (1 + e * (1 - sg)))
    dv = bf(dh * e * sg)
    dxa_g, dxa_u = bf(s * (de @ Bg)), bf(s * (dv @ Bu))
    return {"dx": bf(de @ Wg + dv @ Wu + dxa_g @ Ag + dxa_u @ Au),
            "da_gate": bf(dxa_g.T @ x), "db_gate": bf(s * (de.T @ xa_g)),
            "da_up": bf(dxa_u.T @ x), "db_up": bf(s * (dv.T @ xa_u)),
            "da_down": bf(dxa_d.T @ hmid), "db_down": bf(s * (d.T @ xa_d))}


@pytest.mark.slow
def test_fp32_evaluation_needs_the_rss_allowance_and_meets_it():
    torch.manual_seed(0)
    c, dout = li.config_mlp(), li.mlp_dout()
    W = {k: getattr(c, k) for k in ("w_gate", "w_up", "w_down") + LORA}
    ref, inter = oracle.lora_mlp_grads(c.x, dout, *W.values(), c.scale, "bf16",
                                       return_intermediates=True)
    rss = backward_rss(c.x, dout, W, inter, c.scale)
    got = _fp32_backward(c, dout)
    fails = {k: strict_fail_fraction(got[k], ref[k]) for k in NAMES}
    print("plain-bar failure fractions of an fp32 evaluation:", fails)
    # the plain bar is out of reach for a correct fp32 evaluation on the token sums
    assert max(fails[k] for k in NAMES[1:]) > 1e-4
    for k in NAMES:
        assert_close_sum_lowp(got[k], ref[k], rss[k], k)
