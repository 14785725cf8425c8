"""GPU parity of the LoRA projection backward (lora_linear_prepare_backward, lora_linear_backward)
through the C ABI against the CPU oracle computed from x, dout and the weights alone.

The three gradients are sums whose terms carry bf16-stored factors (xa, dxa), so they are
compared with the bar of the MLP backward (tests/parity.py): |err| <= 1e-2 + 1e-2 |ref| + 2u RSS
per entry (u = 2^-8, RSS the root-sum-square of the sum's terms from the oracle's values) and
normwise within 2u; the fraction outside the plain bar 1e-2 + 1e-2 |ref| is printed. Small
projections (ragged token tiles, odd and full ranks, a scale that is not a power of two) and the
Qwen3-8B output projection (M = 4096, K = N = 4096, r = 16, scale 4) compare every output.
"""

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle
from tests.parity import assert_close_sum_lowp, f64, strict_fail_fraction

pytestmark = pytest.mark.gpu


def _alp():
    return __import__("adapter_lora_projection_amd")


def _case(seed, M, K, N, r, scale):
    c = li.config_qkv(seed=seed, M=M, H=K, Nq=N, Nkv=32, r=r, scale=scale)
    (dout,) = li.projection_douts(seed=seed, M=M, widths=(N,))
    return c, dout  # the projection under test: w_q [N][K], a_q [r][K], b_q [N][r]


def _gpu(c, dout):
    alp = _alp()
    g = lambda t: t.to("cuda").contiguous()
    x, w, a, b = g(c.x), g(c.w_q), g(c.a_q), g(c.b_q)
    w_t = alp.linear_prepare_backward(w)
    x_before = x.clone()
    out = alp.linear_backward(x, g(dout), w_t, a, b, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(x, x_before)  # the saved input is only read
    assert torch.equal(w_t.cpu(), c.w_q.T.contiguous())  # W^T bit for bit
    return {k: t.cpu() for k, t in out.items()}


def _rss(c, dout):
    """Root-sum-square of the terms of each gradient's sum, from the oracle's fp64 values:
    dx[m][k] = sum_n dout W + sum_j dxa A; dA[j][k] = sum_m dxa x; dB[n][j] = s sum_m dout xa."""
    X, D, W, A, B = (f64(t) for t in (c.x, dout, c.w_q, c.a_q, c.b_q))
    xa = oracle.rho(X @ A.T, "bf16")
    dxa = oracle.rho(c.scale * (D @ B), "bf16")
    sq = np.square
    return {"dx": np.sqrt(sq(D) @ sq(W) + sq(dxa) @ sq(A)),
            "da": np.sqrt(sq(dxa).T @ sq(X)),
            "db": np.sqrt(c.scale ** 2 * (sq(D).T @ sq(xa)))}


def _check(c, dout, got):
    ref = oracle.lora_linear_backward(c.x, dout, c.w_q, c.a_q, c.b_q, c.scale, "bf16")
    rss = _rss(c, dout)
    for k in ("dx", "da", "db"):
        print(f"{k}: outside the plain bar {strict_fail_fraction(got[k], ref[k]):.2e}", flush=True)
        assert_close_sum_lowp(got[k], ref[k], rss[k], k)


@pytest.mark.parametrize("M,K,N,r,scale", [(300, 256, 192, 16, 4.0), (77, 128, 320, 7, 1.5),
                                           (513, 320, 256, 64, 2.0), (16, 64, 96, 32, 0.5)])
def test_small_projections(M, K, N, r, scale):
    c, dout = _case(31, M, K, N, r, scale)
    print("case", M, K, N, r, scale, flush=True)
    _check(c, dout, _gpu(c, dout))


def test_b_zero():
    """B = 0: dA is exactly zero and dx is the plain product dout W."""
    c, dout = _case(32, 200, 256, 128, 16, 4.0)
    c.b_q = torch.zeros_like(c.b_q)
    got = _gpu(c, dout)
    assert int(got["da"].count_nonzero()) == 0
    _check(c, dout, got)


def test_qwen3_8b_output_projection():
    """The attention output projection of the Qwen3-8B layer: x [4096][4096] (the attention
    output), W_o [4096][4096], r = 16, scale 4; every output of the three gradients."""
    c, dout = _case(5, 4096, 4096, 4096, 16, 4.0)
    print("case qwen3-8b o_proj", flush=True)
    _check(c, dout, _gpu(c, dout))


def test_argument_errors():
    from adapter_lora_projection_amd import _lib

    alp = _alp()
    c, dout = _case(33, 64, 128, 96, 8, 2.0)
    g = lambda t: t.to("cuda").contiguous()
    x, d, a, b = g(c.x), g(dout), g(c.a_q), g(c.b_q)
    w_t = alp.linear_prepare_backward(g(c.w_q))
    n = _lib.lora_linear_backward_workspace_size(_lib.LORA_BF16, 64, 128, 96, 8)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    da = torch.empty((8, 128), dtype=torch.bfloat16, device="cuda")
    db = torch.empty((96, 8), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    L = _lib.lib()
    call = lambda dx, K=128, N=96, nbytes=n: L.lora_linear_backward(
        _lib.LORA_BF16, 64, K, N, 8, 2.0, x.data_ptr(), 128, d.data_ptr(), 96, w_t.data_ptr(),
        a.data_ptr(), b.data_ptr(), dx, 128, da.data_ptr(), db.data_ptr(), ws.data_ptr(), nbytes,
        stream)
    assert call(x.data_ptr()) == _lib.LORA_EINVAL          # dx aliasing the saved input
    assert call(d.data_ptr()) == _lib.LORA_EINVAL          # ... or dout
    dx = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    assert call(dx.data_ptr(), K=120) == _lib.LORA_EUNSUPPORTED  # K not a multiple of 32
    assert call(dx.data_ptr(), nbytes=n - 256) == _lib.LORA_EWORKSPACE
    torch.cuda.synchronize()
    assert call(dx.data_ptr()) == 0
    torch.cuda.synchronize()


# ------------------------------------------------------------ query, key and value in one call

def _qkv_gpu(c, douts):
    alp = _alp()
    g = lambda t: t.to("cuda").contiguous()
    w_t = alp.qkv_prepare_backward(g(c.w_q), g(c.w_k), g(c.w_v))
    ref_t = torch.cat([c.w_q.T, c.w_k.T, c.w_v.T], dim=1).contiguous()
    assert torch.equal(w_t.cpu(), ref_t)  # [W_q^T | W_k^T | W_v^T] bit for bit
    x = g(c.x)
    x_before = x.clone()
    out = alp.qkv_backward(x, *[g(d) for d in douts], w_t, g(c.a_q), g(c.b_q), g(c.a_k), g(c.b_k),
                           g(c.a_v), g(c.b_v), c.scale)
    torch.cuda.synchronize()
    assert torch.equal(x, x_before)
    return {k: t.cpu() for k, t in out.items()}


def _qkv_check(c, douts, got):
    ref = oracle.lora_qkv_backward(c.x, *douts, c.w_q, c.w_k, c.w_v, c.a_q, c.b_q, c.a_k, c.b_k,
                                   c.a_v, c.b_v, c.scale, "bf16")
    X = f64(c.x)
    sq = np.square
    dx2 = 0.0
    rss = {}
    for p, d, W, A, B in (("q", douts[0], c.w_q, c.a_q, c.b_q), ("k", douts[1], c.w_k, c.a_k, c.b_k),
                          ("v", douts[2], c.w_v, c.a_v, c.b_v)):
        D, W, A, B = f64(d), f64(W), f64(A), f64(B)
        xa = oracle.rho(X @ A.T, "bf16")
        dxa = oracle.rho(c.scale * (D @ B), "bf16")
        dx2 = dx2 + sq(D) @ sq(W) + sq(dxa) @ sq(A)
        rss["da_" + p] = np.sqrt(sq(dxa).T @ sq(X))
        rss["db_" + p] = np.sqrt(c.scale ** 2 * (sq(D).T @ sq(xa)))
    rss["dx"] = np.sqrt(dx2)
    for k in ("dx", "da_q", "db_q", "da_k", "db_k", "da_v", "db_v"):
        print(f"{k}: outside the plain bar {strict_fail_fraction(got[k], ref[k]):.2e}", flush=True)
        assert_close_sum_lowp(got[k], ref[k], rss[k], k)


@pytest.mark.parametrize("M,K,Nq,Nkv,r,scale", [(300, 256, 192, 64, 16, 4.0),
                                                (77, 128, 96, 32, 7, 1.5),
                                                (130, 64, 128, 96, 64, 0.5)])
def test_qkv_small(M, K, Nq, Nkv, r, scale):
    c = li.config_qkv(seed=34, M=M, H=K, Nq=Nq, Nkv=Nkv, r=r, scale=scale)
    douts = li.projection_douts(seed=34, M=M, widths=(Nq, Nkv, Nkv))
    print("case qkv", M, K, Nq, Nkv, r, scale, flush=True)
    _qkv_check(c, douts, _qkv_gpu(c, douts))


def test_qkv_qwen3_8b():
    """The query, key and value projections of the Qwen3-8B layer (M = 4096, K = 4096,
    Nq = 4096, Nkv = 1024, r = 16, scale 4); every output of the seven gradients."""
    c = li.config_qkv()
    douts = li.projection_douts(seed=5, M=c.M, widths=(c.Nq, c.Nkv, c.Nkv))
    print("case qwen3-8b qkv", flush=True)
    _qkv_check(c, douts, _qkv_gpu(c, douts))


# ------------------------------------------------------------ autograd wrappers

def test_autograd_functions_match_the_direct_calls():
    """LoraLinearFunction and LoraQkvFunction: forward outputs and every gradient equal the
    direct calls bit for bit, and the q/k/v gradients agree with the oracle chain."""
    alp = _alp()
    c = li.config_qkv(seed=35, M=192, H=128, Nq=160, Nkv=64, r=8, scale=2.0)
    dq, dk, dv, do = [t.to("cuda") for t in li.projection_douts(seed=35, M=192, widths=(160, 64, 64, 128))]
    g = lambda t: t.to("cuda").contiguous()
    d = {k: g(getattr(c, k)) for k in ("x", "w_q", "w_k", "w_v", "a_q", "b_q", "a_k", "b_k", "a_v",
                                       "b_v", "w_o", "a_o", "b_o")}
    print("case autograd projections", flush=True)
    # q/k/v
    w_qkv_t = alp.qkv_prepare_backward(d["w_q"], d["w_k"], d["w_v"])
    names = ("x", "a_q", "b_q", "a_k", "b_k", "a_v", "b_v")
    leaves = {k: d[k].clone().requires_grad_(True) for k in names}
    q, k, v = alp.LoraQkvFunction.apply(*[leaves[n] for n in names], d["w_q"], d["w_k"], d["w_v"],
                                        w_qkv_t, c.scale)
    torch.autograd.backward((q, k, v), (dq, dk, dv))
    q0, k0, v0 = alp.qkv_fused(d["x"], d["w_q"], d["w_k"], d["w_v"], d["a_q"], d["b_q"], d["a_k"],
                               d["b_k"], d["a_v"], d["b_v"], c.scale)
    ref = alp.qkv_backward(d["x"], dq, dk, dv, w_qkv_t, d["a_q"], d["b_q"], d["a_k"], d["b_k"],
                           d["a_v"], d["b_v"], c.scale)
    torch.cuda.synchronize()
    assert torch.equal(q.detach(), q0) and torch.equal(k.detach(), k0) and torch.equal(v.detach(), v0)
    for n, key in zip(names, ("dx", "da_q", "db_q", "da_k", "db_k", "da_v", "db_v")):
        assert torch.equal(leaves[n].grad, ref[key]), key
    # output projection, on q as its input
    w_o_t = alp.linear_prepare_backward(d["w_o"])
    lv = {n: t.clone().requires_grad_(True) for n, t in (("x", q0), ("a", d["a_o"]), ("b", d["b_o"]))}
    o = alp.LoraLinearFunction.apply(lv["x"], lv["a"], lv["b"], d["w_o"], w_o_t, c.scale)
    o.backward(do)
    ref = alp.linear_backward(q0, do, w_o_t, d["a_o"], d["b_o"], c.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), alp.linear_fused(q0, d["w_o"], d["a_o"], d["b_o"], c.scale))
    for n, key in (("x", "dx"), ("a", "da"), ("b", "db")):
        assert torch.equal(lv[n].grad, ref[key]), key


def test_qkv_fused_gradient_read_in_place():
    """dq, dk, dv as column views of one [M][Nq + 2 Nkv] gradient (read in place by the dx
    product) give the same gradients, bit for bit, as contiguous copies (copied side by side
    through the workspace)."""
    alp = _alp()
    c = li.config_qkv(seed=36, M=300, H=256, Nq=192, Nkv=64, r=16, scale=4.0)
    g = lambda t: t.to("cuda").contiguous()
    fused = torch.randn(300, 192 + 128, device="cuda").to(torch.bfloat16)
    views = (fused[:, :192], fused[:, 192:256], fused[:, 256:])
    w_t = alp.qkv_prepare_backward(g(c.w_q), g(c.w_k), g(c.w_v))
    lora = [g(t) for t in (c.a_q, c.b_q, c.a_k, c.b_k, c.a_v, c.b_v)]
    got = alp.qkv_backward(g(c.x), *views, w_t, *lora, c.scale)
    ref = alp.qkv_backward(g(c.x), *[v.contiguous() for v in views], w_t, *lora, c.scale)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    douts = [v.cpu() for v in views]
    _qkv_check(c, douts, {k: t.cpu() for k, t in got.items()})


def test_qkv_backward_graph_replay():
    """The q/k/v backward (with its side-by-side copy of the gradients) captured in a HIP graph:
    every replay, with eager work and synchronisations between them, equals the eager result bit
    for bit."""
    alp = _alp()
    c = li.config_qkv(seed=37, M=256, H=128, Nq=128, Nkv=64, r=16, scale=4.0)
    douts = [t.to("cuda") for t in li.projection_douts(seed=37, M=256, widths=(128, 64, 64))]
    g = lambda t: t.to("cuda").contiguous()
    w_t = alp.qkv_prepare_backward(g(c.w_q), g(c.w_k), g(c.w_v))
    lora = [g(t) for t in (c.a_q, c.b_q, c.a_k, c.b_k, c.a_v, c.b_v)]
    x = g(c.x)
    from adapter_lora_projection_amd import _lib
    n = _lib.lora_qkv_backward_workspace_size(_lib.LORA_BF16, 256, 128, 128, 64, 16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ref = alp.qkv_backward(x, *douts, w_t, *lora, c.scale, workspace=ws)
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        out = alp.qkv_backward(x, *douts, w_t, *lora, c.scale, workspace=ws)
    for rep in range(4):
        for t in out.values():
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (rep, k)
        del junk
