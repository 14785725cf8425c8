"""Benchmark: effective HBM bandwidth of the multi-adapter LoRA shrink+expand on one MI355X.

Workload: the decode-QKV projection shape (bf16; 4 adapters of rank 16; K = 4096; three output
slices of 4096, 1024 and 1024 columns; uniform-random segment lengths; random adapter order and
token permutation; x ~ N(0,1), A, B ~ N(0,0.02), scale 2) at the nine token counts
tok = 50, 128, 256, 512, 1024, 2048, 4096, 6144, 8192. One step = lora_shrink then lora_expand for
every token count, all inputs resident in HBM. The step is captured once into a HIP graph and
replayed; the nine cases (about 0.75 GB of distinct data) evict one another from L2 and the
Infinity Cache between reuses, so every case streams from HBM.

value = algorithmic bytes of one step / time of one step (GB/s), with algorithmic bytes counted
per call as: x rows + valid rank rows of A of the adapters used + valid h entries (shrink);
valid h entries + valid rank columns of B of the adapters used + y read and written (expand);
plus the int32 metadata.

The single-adapter fused LoRA+SwiGLU MLP (bf16, M=4096, H=4096, I=12288, r=16, scale 4) and the
single-adapter LoRA attention projections (q/k/v and o of the same layer shape) are timed in the
same run and reported in their own objects.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--no-mlp]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ESIZE = {"f32": 4, "bf16": 2, "f16": 2}


def _kernel_source_sha() -> str:
    d = os.path.join(ROOT, "adapter_lora_projection_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(c) -> dict:
    """Algorithmic bytes and flops of one shrink and one expand call on case c."""
    E = ESIZE[c.dtype]
    lens = np.diff(c.seg_indptr.numpy()).astype(np.int64)
    widx = c.weight_indices.numpy()
    ranks = c.lora_ranks.numpy().astype(np.int64)
    used = sorted({int(widx[g]) for g in range(len(widx)) if lens[g] > 0})
    rows_r = int(sum(lens[g] * ranks[widx[g]] for g in range(len(widx))))  # sum_i r_a(i)
    meta_s = 4 * (len(lens) + 1 + len(widx) + c.T + c.L)
    meta_e = meta_s + 4 * (c.S + 1) + 4 * c.L
    h_bytes = c.S * rows_r * E
    shrink_b = c.T * c.K * E + sum(c.S * int(ranks[a]) * c.K * E for a in used) + h_bytes + meta_s
    expand_b = h_bytes + sum(c.N * int(ranks[a]) * E for a in used) + 2 * c.T * c.N * E + meta_e
    return {"shrink_bytes": shrink_b, "expand_bytes": expand_b,
            "shrink_flops": 2 * c.S * rows_r * c.K, "expand_flops": 2 * c.N * rows_r}


class SgmvCaseRun:
    """Device buffers and pre-marshalled C-ABI argument tuples for one case."""

    def __init__(self, c, lib, stream):
        import torch

        self.c = c
        dt = {"f32": 0, "bf16": 1, "f16": 2}[c.dtype]
        dev = "cuda"
        self.d = {k: getattr(c, k).to(dev).contiguous() for k in
                  ("slice_offsets", "seg_indptr", "weight_indices", "permutation", "lora_ranks",
                   "scalings", "x", "A", "B", "y_in")}
        d = self.d
        self.h = torch.empty((c.T, c.S * c.R), dtype=d["x"].dtype, device=dev)
        self.y = d["y_in"].clone()
        ws_s = lib.lora_shrink_workspace_size(dt, c.T, c.K, c.S, c.R, c.G)
        ws_e = lib.lora_expand_workspace_size(dt, c.T, c.S, c.R, c.G, c.N)
        # the shrink workspace starts with arrival counters that must be zero before first use
        self.ws_s = torch.zeros(max(ws_s, 1), dtype=torch.uint8, device=dev)
        self.ws_e = torch.empty(max(ws_e, 1), dtype=torch.uint8, device=dev)
        p = lambda t: t.data_ptr()
        self.shrink_args = (dt, c.T, c.K, c.S, c.R, c.L, c.G, p(d["x"]), c.K, p(d["A"]), c.K,
                            p(d["seg_indptr"]), p(d["weight_indices"]), p(d["permutation"]),
                            p(d["lora_ranks"]), p(self.h), c.S * c.R, p(self.ws_s), ws_s, stream)
        self.expand_args = (dt, c.T, c.S, c.R, c.L, c.G, c.N, p(self.h), c.S * c.R, p(d["B"]), c.R,
                            p(d["slice_offsets"]), p(d["seg_indptr"]), p(d["weight_indices"]),
                            p(d["permutation"]), p(d["lora_ranks"]), p(d["scalings"]), p(self.y),
                            c.N, p(self.ws_e), ws_e, stream)
        # lora_shrink_expand: both steps of the case in one call (one launch at decode sizes)
        ws_p = lib.lora_shrink_expand_workspace_size(dt, c.T, c.K, c.S, c.R, c.G, c.N)
        self.ws_p = torch.zeros(max(ws_p, 1), dtype=torch.uint8, device=dev)
        self.pair_args = (dt, c.T, c.K, c.S, c.R, c.L, c.G, c.N, p(d["x"]), c.K, p(d["A"]), c.K,
                          p(d["B"]), c.R, p(d["slice_offsets"]), p(d["seg_indptr"]),
                          p(d["weight_indices"]), p(d["permutation"]), p(d["lora_ranks"]),
                          p(d["scalings"]), p(self.h), c.S * c.R, p(self.y), c.N, p(self.ws_p),
                          ws_p, stream)
        self.alg = algorithmic(c)

    def pair(self, L, stream=None):
        a = self.pair_args if stream is None else self.pair_args[:-1] + (stream,)
        st = L.lora_shrink_expand(*a)
        if st:
            raise RuntimeError(f"lora_shrink_expand status {st}")

    def shrink(self, L):
        st = L.lora_shrink(*self.shrink_args)
        if st:
            raise RuntimeError(f"lora_shrink status {st}")

    def expand(self, L):
        st = L.lora_expand(*self.expand_args)
        if st:
            raise RuntimeError(f"lora_expand status {st}")


def load_traffic() -> dict:
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter runs, keyed by
    kernel and workload; empty when the kernel sources changed since the counters were taken."""
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        tj = json.load(open(tpath))
    except (OSError, ValueError):
        return {}
    if tj.get("source_sha") != _kernel_source_sha():
        return {}
    return {k: v["hbm_bytes_per_launch"] for k, v in tj.get("kernels", {}).items()}


def mlp_flops(M: int, H: int, I: int, r: int) -> tuple[int, int]:
    """(frozen-weight flops, LoRA flops) of one fused LoRA+SwiGLU MLP forward."""
    base = 2 * M * H * I * 3
    lora = 2 * M * r * (2 * H) + 2 * M * r * (2 * I) + 2 * M * r * I + 2 * M * r * H
    return base, lora


def timed_windows(call, steps: int, windows: int = 5) -> tuple[float, list]:
    """Median over `windows` windows of `steps` calls back to back, each window between two HIP
    events on the launch stream (ms per call), and the per-window figures."""
    import torch

    n = max(steps, 1)
    per = []
    for _ in range(windows):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            call()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / n)
    return float(np.median(per)), [round(x, 4) for x in per]


def mlp_object(steps: int, warmup: int, traffic_table: dict) -> dict:
    """The single-adapter fused LoRA+SwiGLU MLP (bf16, M=4096, H=4096, I=12288, r=16, scale 4):
    K calls back to back after a warm-up, timed with HIP events on the stream they are launched
    on; roofline against dense bf16 MFMA."""
    import torch

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    c = li.config_mlp()
    g = lambda t: t.to("cuda").contiguous()
    w = [g(t) for t in (c.x, c.w_gate, c.w_up, c.w_down, c.a_gate, c.b_gate, c.a_up, c.b_up,
                        c.a_down, c.b_down)]
    out = torch.empty((c.M, c.H), dtype=torch.bfloat16, device="cuda")
    nbytes = _lib.lora_mlp_workspace_size(_lib.LORA_BF16, c.M, c.H, c.I, c.r)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    p = [t.data_ptr() for t in w]
    call = lambda: _lib.lora_mlp_fused(_lib.LORA_BF16, c.M, c.H, c.I, c.r, c.scale, p[0], c.H,
                                       *p[1:], out.data_ptr(), c.H, ws.data_ptr(), nbytes, stream)
    # the GPU's clocks take some tens of calls of this size to settle: warm up for at least 60
    for _ in range(max(warmup, 60)):
        call()
    torch.cuda.synchronize()
    # windows of K calls back to back between two events on the stream they run on; the median
    # window is reported (robust to a transient clock dip in one window)
    ms, windows = timed_windows(call, steps)
    base, lora = mlp_flops(c.M, c.H, c.I, c.r)
    tflops = (base + lora) / (ms * 1e-3) / 1e12
    return {"workload": f"fused LoRA+SwiGLU MLP bf16, M={c.M} H={c.H} I={c.I} r={c.r} "
                        f"scale={c.scale:g}", "ms_per_call": round(ms, 4),
            "flops_per_call": int(base + lora), "value": round(tflops, 1), "unit": "TFLOP/s",
            "windows_ms": windows,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_table.get("mlp_fused"),
                         "kernel": "lora_mlp_fused (all seven launches of one call)"}}


def mlp_backward_flops(M: int, H: int, I: int, r: int) -> tuple[int, int]:
    """(frozen-weight flops, LoRA flops) of the gradient arithmetic of one LoRA MLP backward:
    dhmid = d W_d (2 M I H) and dx = de W_g + dv W_u (4 M H I); the LoRA terms dxa_d, dxa_g,
    dxa_u, their products in dhmid and dx, and the six weight gradients. Recomputed forward
    quantities (hmid, xa_*) are overhead and not counted."""
    base = 2 * M * I * H + 2 * M * (2 * I) * H
    lora = (2 * M * H * r + 2 * M * I * r            # dxa_d, dxa_d A_d
            + 2 * 2 * M * I * r + 2 * M * H * 2 * r  # dxa_g, dxa_u and their A products
            + 2 * 2 * r * M * H + 2 * 2 * I * M * r  # dA_g, dA_u, dB_g, dB_u
            + 2 * r * M * I + 2 * H * M * r)         # dA_d, dB_d
    return base, lora


def projection_backward_object(steps: int, warmup: int) -> dict:
    """The LoRA attention-projection backward (bf16, the Qwen3-8B shapes of the forward object:
    M = 4096, H = 4096, Nq = 4096, Nkv = 1024, r = 16, scale 4): lora_qkv_backward for the query,
    key and value projections of x, then lora_linear_backward for the output projection; K pairs
    back to back after a warm-up, HIP events on their stream; flops of the gradient arithmetic
    (dx, dxa, dA, dB; the recomputed xa not counted), against dense bf16 MFMA. Beside it: the
    output projection alone, and the q/k/v backward on column views of one fused gradient (read
    in place instead of copied side by side)."""
    import torch

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    c = li.config_qkv()
    M, H, Nq, Nkv, r, s = c.M, c.H, c.Nq, c.Nkv, c.r, c.scale
    dq, dk, dv, do = li.projection_douts(seed=5, M=M, widths=(Nq, Nkv, Nkv, H))
    g = lambda t: t.to("cuda").contiguous()
    d = {k: g(getattr(c, k)) for k in ("x", "w_q", "w_k", "w_v", "a_q", "b_q", "a_k", "b_k", "a_v",
                                       "b_v", "w_o", "a_o", "b_o")}
    dq, dk, dv, do = g(dq), g(dk), g(dv), g(do)
    q_in = g(c.x[:, :Nq]) if Nq == H else torch.randn(M, Nq, device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream().cuda_stream
    bf = torch.bfloat16
    w_qkv_t = torch.empty((H, Nq + 2 * Nkv), dtype=bf, device="cuda")
    _lib.lora_qkv_prepare_backward(_lib.LORA_BF16, H, Nq, Nkv, d["w_q"], d["w_k"], d["w_v"], w_qkv_t,
                                   stream)
    w_o_t = torch.empty((Nq, H), dtype=bf, device="cuda")
    _lib.lora_linear_prepare_backward(_lib.LORA_BF16, Nq, H, d["w_o"], w_o_t, stream)
    e = lambda *shape: torch.empty(shape, dtype=bf, device="cuda")
    dx, da_q, da_k, da_v, db_q, db_k, db_v = e(M, H), e(r, H), e(r, H), e(r, H), e(Nq, r), e(Nkv, r), e(Nkv, r)
    dq_in, da_o, db_o = e(M, Nq), e(r, Nq), e(H, r)
    n = max(_lib.lora_qkv_backward_workspace_size(_lib.LORA_BF16, M, H, Nq, Nkv, r),
            _lib.lora_linear_backward_workspace_size(_lib.LORA_BF16, M, Nq, H, r), 1)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def o_call():  # output projection: input q_in [M][Nq] (the attention output), out [M][H]
        _lib.lora_linear_backward(_lib.LORA_BF16, M, Nq, H, r, s, q_in, Nq, do, H, w_o_t, d["a_o"],
                                  d["b_o"], dq_in, Nq, da_o, db_o, ws, n, stream)

    def call():
        _lib.lora_qkv_backward(_lib.LORA_BF16, M, H, Nq, Nkv, r, s, d["x"], H, dq, Nq, dk, Nkv, dv,
                               Nkv, w_qkv_t, d["a_q"], d["b_q"], d["a_k"], d["b_k"], d["a_v"],
                               d["b_v"], dx, H, da_q, db_q, da_k, db_k, da_v, db_v, ws, n, stream)
        o_call()

    # the same gradients as column views of one fused [M][Nq + 2 Nkv] gradient: read in place
    fused = torch.cat([dq, dk, dv], dim=1)
    fq, fk, fv = fused[:, :Nq], fused[:, Nq:Nq + Nkv], fused[:, Nq + Nkv:]
    nt = Nq + 2 * Nkv

    def qkv_fused_grad():
        _lib.lora_qkv_backward(_lib.LORA_BF16, M, H, Nq, Nkv, r, s, d["x"], H, fq.data_ptr(), nt,
                               fk.data_ptr(), nt, fv.data_ptr(), nt, w_qkv_t, d["a_q"], d["b_q"],
                               d["a_k"], d["b_k"], d["a_v"], d["b_v"], dx, H, da_q, db_q, da_k,
                               db_k, da_v, db_v, ws, n, stream)

    for _ in range(max(warmup, 30)):
        call()
    torch.cuda.synchronize()
    ms, _ = timed_windows(call, steps)
    ms_o, _ = timed_windows(o_call, steps)
    ms_f, _ = timed_windows(qkv_fused_grad, steps)
    flops_qkv = 2 * M * H * nt + 4 * M * r * nt + 12 * M * r * H
    flops_o = 2 * M * H * Nq + 4 * M * H * r + 4 * M * r * Nq
    tflops = (flops_qkv + flops_o) / (ms * 1e-3) / 1e12
    return {"workload": f"LoRA q/k/v + o projection backward bf16, M={M} H={H} Nq={Nq} Nkv={Nkv} "
                        f"r={r} scale={s:g}", "ms_per_call": round(ms, 4),
            "flops_per_call": int(flops_qkv + flops_o), "value": round(tflops, 1), "unit": "TFLOP/s",
            "o_projection_ms": round(ms_o, 4),
            "o_projection_tflops": round(flops_o / (ms_o * 1e-3) / 1e12, 1),
            "qkv_ms_fused_gradient": round(ms_f, 4),
            "qkv_ms": round(ms - ms_o, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": None,
                         "kernel": "lora_qkv_backward + lora_linear_backward (all launches)"}}


def mlp_backward_object(steps: int, warmup: int) -> dict:
    """The LoRA MLP backward (lora_mlp_backward, bf16, M=4096, H=4096, I=12288, r=16, scale 4)
    after one training forward (lora_mlp_fused_train, timed beside it): K calls back to back
    after a warm-up, HIP events on their stream; roofline against dense bf16 MFMA."""
    import torch

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    c = li.config_mlp()
    dout = li.mlp_dout().to("cuda")
    g = lambda t: t.to("cuda").contiguous()
    x, wg, wu, wd = g(c.x), g(c.w_gate), g(c.w_up), g(c.w_down)
    lo = [g(getattr(c, k)) for k in ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")]
    bf = torch.bfloat16
    out = torch.empty((c.M, c.H), dtype=bf, device="cuda")
    e = torch.empty((c.M, c.I), dtype=bf, device="cuda")
    v = torch.empty((c.M, c.I), dtype=bf, device="cuda")
    w_gu_t = torch.empty((c.H, 2 * c.I), dtype=bf, device="cuda")
    w_down_t = torch.empty((c.I, c.H), dtype=bf, device="cuda")
    grads = [torch.empty(sh, dtype=bf, device="cuda") for sh in
             ((c.M, c.H), (c.r, c.H), (c.I, c.r), (c.r, c.H), (c.I, c.r), (c.r, c.I), (c.H, c.r))]
    nf = _lib.lora_mlp_workspace_size(_lib.LORA_BF16, c.M, c.H, c.I, c.r)
    nb = _lib.lora_mlp_backward_workspace_size(_lib.LORA_BF16, c.M, c.H, c.I, c.r)
    wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    P = lambda t: t.data_ptr()
    L = [P(t) for t in lo]
    _lib.lora_mlp_prepare_backward(_lib.LORA_BF16, c.H, c.I, P(wg), P(wu), P(wd), P(w_gu_t),
                                   P(w_down_t), stream)
    fwd = lambda: _lib.lora_mlp_fused_train(_lib.LORA_BF16, c.M, c.H, c.I, c.r, c.scale, P(x), c.H,
                                            P(wg), P(wu), P(wd), *L, P(out), c.H, P(e), P(v), c.I,
                                            P(wsf), nf, stream)
    bwd = lambda: _lib.lora_mlp_backward(_lib.LORA_BF16, c.M, c.H, c.I, c.r, c.scale, P(x), c.H,
                                         P(e), P(v), c.I, P(dout), c.H, P(w_gu_t), P(w_down_t), *L,
                                         P(grads[0]), c.H, *[P(t) for t in grads[1:]], P(wsb), nb,
                                         stream)

    def timed(call):
        for _ in range(max(warmup, 40)):
            call()
        torch.cuda.synchronize()
        return timed_windows(call, max(steps // 2, 1), 3)[0]

    ms_f = timed(fwd)
    ms_b = timed(bwd)
    base, lora = mlp_backward_flops(c.M, c.H, c.I, c.r)
    fb, fl = mlp_flops(c.M, c.H, c.I, c.r)
    tflops = (base + lora) / (ms_b * 1e-3) / 1e12
    return {"workload": f"LoRA+SwiGLU MLP backward bf16, M={c.M} H={c.H} I={c.I} r={c.r} "
                        f"scale={c.scale:g}", "ms_per_call": round(ms_b, 4),
            "flops_per_call": int(base + lora), "value": round(tflops, 1), "unit": "TFLOP/s",
            "train_forward_ms": round(ms_f, 4),
            "train_forward_tflops": round((fb + fl) / (ms_f * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": None,
                         "kernel": "lora_mlp_backward (all launches of one call)"}}


def attention_object(steps: int, warmup: int) -> dict:
    """The single-adapter LoRA attention projections (bf16, Qwen3-8B shape: M=4096, H=4096,
    32 query and 8 key/value heads of 128, r=16, scale 4): lora_qkv_fused then lora_linear_fused
    for the output projection, K pairs back to back after a warm-up, HIP events on their stream;
    roofline against dense bf16 MFMA."""
    import torch

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    c = li.config_qkv()
    g = lambda t: t.to("cuda").contiguous()
    d = {k: g(getattr(c, k)) for k in ("x", "w_q", "w_k", "w_v", "a_q", "b_q", "a_k", "b_k", "a_v",
                                       "b_v", "w_o", "a_o", "b_o")}
    q = torch.empty((c.M, c.Nq), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((c.M, c.Nkv), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((c.M, c.Nkv), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((c.M, c.H), dtype=torch.bfloat16, device="cuda")
    nq = _lib.lora_qkv_workspace_size(_lib.LORA_BF16, c.M, c.H, c.Nq, c.Nkv, c.r)
    no = _lib.lora_linear_workspace_size(_lib.LORA_BF16, c.M, c.Nq, c.H, c.r)
    ws = torch.empty(max(nq, no, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    P = {kk: t.data_ptr() for kk, t in d.items()}

    def call():
        _lib.lora_qkv_fused(_lib.LORA_BF16, c.M, c.H, c.Nq, c.Nkv, c.r, c.scale, P["x"], c.H,
                            P["w_q"], P["w_k"], P["w_v"], P["a_q"], P["b_q"], P["a_k"], P["b_k"],
                            P["a_v"], P["b_v"], q.data_ptr(), c.Nq, k.data_ptr(), c.Nkv,
                            v.data_ptr(), c.Nkv, ws.data_ptr(), ws.numel(), stream)
        _lib.lora_linear_fused(_lib.LORA_BF16, c.M, c.Nq, c.H, c.r, c.scale, q.data_ptr(), c.Nq,
                               P["w_o"], P["a_o"], P["b_o"], o.data_ptr(), c.H, ws.data_ptr(),
                               ws.numel(), stream)

    for _ in range(max(warmup, 60)):
        call()
    torch.cuda.synchronize()
    ms, _ = timed_windows(call, steps)
    nqkv = c.Nq + 2 * c.Nkv
    flops = (2 * c.M * c.H * nqkv + 2 * c.M * c.r * (3 * c.H + nqkv)  # q, k, v
             + 2 * c.M * c.Nq * c.H + 2 * c.M * c.r * (c.Nq + c.H))   # o
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": f"LoRA q/k/v + o projections bf16, M={c.M} H={c.H} Nq={c.Nq} Nkv={c.Nkv} "
                        f"r={c.r} scale={c.scale:g}", "ms_per_call": round(ms, 4),
            "flops_per_call": int(flops), "value": round(tflops, 1), "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                         "traffic": None,
                         "kernel": "lora_qkv_fused + lora_linear_fused (all launches)"}}


def embedding_object(steps: int, warmup: int) -> dict:
    """The embedding LoRA-A product (lora_embedding_a) on 16,384 one-token segments (bf16,
    vocabulary 151,936, 8 adapters of rank 16), A stored [L][V][R] (unit rank stride; the
    [L][R][V] storage is timed beside it). Algorithmic bytes per call: per token its id and
    permutation entry (8 B), r values of A read and R values of h written, plus seg_indptr,
    weight_indices and lora_ranks. K calls back to back after a warm-up, HIP events on the
    launch stream; roofline against HBM peak."""
    import torch

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    c = li.make_embedding("emb_16384x1", seed=12, T=16384, V=151936, R=16, L=8, dtype="bf16",
                          lengths="ones")
    g = lambda t: t.to("cuda").contiguous()
    ids, ip, wi, pm, rk = (g(t) for t in (c.input_ids, c.seg_indptr, c.weight_indices,
                                          c.permutation, c.lora_ranks))
    a_rv = g(c.A)
    a_vr = g(c.A.permute(0, 2, 1))  # [L][V][R] storage
    h = torch.empty((c.T, c.R), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    V, R = c.V, c.R
    strides = {"vr": (V * R, 1, R), "rv": (R * V, V, 1)}
    ptrs = {"vr": a_vr.data_ptr(), "rv": a_rv.data_ptr()}
    ranks = c.lora_ranks.numpy().astype(np.int64)
    r_tok = ranks[c.weight_indices.numpy()]  # one token per segment
    algo = int(c.T * 8 + 2 * int(r_tok.sum()) + 2 * c.T * c.R + 4 * (2 * c.G + 1) + 4 * c.L)

    def run(layout):
        sl, sr, sv = strides[layout]

        def call():
            _lib.lora_embedding_a(_lib.LORA_BF16, c.T, V, R, c.L, c.G, ids.data_ptr(),
                                  ptrs[layout], sl, sr, sv, ip.data_ptr(), wi.data_ptr(),
                                  pm.data_ptr(), rk.data_ptr(), h.data_ptr(), R, stream)

        for _ in range(max(warmup, 20)):
            call()
        torch.cuda.synchronize()
        n = max(steps, 1) * 10
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    us = {lay: run(lay) * 1e3 for lay in ("vr", "rv")}
    gbps = algo / (us["vr"] * 1e-6) / 1e9
    return {"workload": "embedding LoRA-A bf16, 16384 one-token segments, V=151936, 8 adapters "
                        "r16, A stored [L][V][R]",
            "us_per_call": round(us["vr"], 2), "us_per_call_A_stored_LRV": round(us["rv"], 2),
            "algorithmic_bytes_per_call": algo, "value": round(gbps, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "kernel": "embedding_a_kernel (one launch)"}}


def cpu_baseline(min_seconds: float = 10.0, max_seconds: float = 30.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload (host cores): passes
    over the sweep's token counts in order, until at least min_seconds of oracle time."""
    import oracle
    import lora_inputs as li

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max((i["num_threads"] for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = 1
    total_b = 0
    total_t = 0.0
    done = []
    cases = {}
    while total_t < min_seconds:
        for tok in li.SWEEP_TOKENS:
            if tok not in cases:
                c = li.sweep_case(tok)
                cases[tok] = (c, algorithmic(c))
            c, alg = cases[tok]
            t0 = time.perf_counter()
            h = oracle.shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation,
                              c.lora_ranks, c.S, c.R, "bf16")
            oracle.expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation,
                          c.lora_ranks, c.scalings, c.y_in, c.R, "bf16")
            total_t += time.perf_counter() - t0
            total_b += alg["shrink_bytes"] + alg["expand_bytes"]
            done.append(tok)
            if total_t >= max_seconds or (total_t >= min_seconds and tok == li.SWEEP_TOKENS[-1]):
                break
        if total_t >= max_seconds:
            break
    cores = min(len(os.sched_getaffinity(0)), blas_threads)
    return {"value": round(total_b / total_t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"fp64 oracle shrink+expand over the same sweep, {len(done)} calls at tok "
                      f"{done[:9]}{'...' if len(done) > 9 else ''} ({total_t:.1f} s of oracle time; "
                      f"BLAS threads {blas_threads})"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp", action="store_true",
                    help="leave out every object beside the shrink+expand sweep")
    ap.add_argument("--extras", default="mlp,attention,backward,embedding",
                    help="comma list of the objects timed after the sweep (mlp, attention, "
                         "backward, embedding); counter runs keep only mlp, so that every GEMM "
                         "launch of the run belongs to the fused MLP")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every step runs on a single MI355X).", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}))
        return 0

    import lora_inputs as li
    from adapter_lora_projection_amd import _lib

    L = _lib.lib()  # raises if the HIP library is not built: there is no other path
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    runs = [SgmvCaseRun(li.sweep_case(t), L, stream) for t in li.SWEEP_TOKENS]
    print(f"[bench] {len(runs)} cases resident on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    def step():
        for r in runs:
            r.pair(L)

    # one pass of the separate calls, then one of lora_shrink_expand, before anything else: the
    # profile summaries name each dispatch by its position in these two passes
    for r in runs:
        r.shrink(L)
        r.expand(L)
    for r in runs:
        r.pair(L)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()

    # per-kernel breakdown (eager, events around every launch) -> dominant kernel
    reps = 5
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in runs]
    acc = np.zeros((len(runs), 3))  # shrink, expand (separate calls), lora_shrink_expand
    for _ in range(reps):
        for i, r in enumerate(runs):
            ev[i][0].record()
            r.shrink(L)
            ev[i][1].record()
            r.expand(L)
            ev[i][2].record()
        for i, r in enumerate(runs):
            ev[i][3].record()
            r.pair(L)
            ev[i][4].record()
        torch.cuda.synchronize()
        for i in range(len(runs)):
            acc[i, 0] += ev[i][0].elapsed_time(ev[i][1])
            acc[i, 1] += ev[i][1].elapsed_time(ev[i][2])
            acc[i, 2] += ev[i][3].elapsed_time(ev[i][4])
    acc /= reps  # ms
    dom_i, dom_op = np.unravel_index(np.argmax(acc[:, :2]), acc[:, :2].shape)

    # cold single calls: a 512 MiB device write before each of `cold_reps` repetitions evicts
    # the L2 and the Infinity Cache; the median of the event timings per call
    cold_reps = 30
    flush = torch.empty(512 << 18, dtype=torch.float32, device="cuda")
    cold = np.zeros((len(runs), 3, cold_reps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i, r in enumerate(runs):
        for k in range(cold_reps):
            for op in (0, 1, 2):
                flush.fill_(float(k))
                e0.record()
                (r.shrink, r.expand, r.pair)[op](L)
                e1.record()
                torch.cuda.synchronize()
                cold[i, op, k] = e0.elapsed_time(e1)
    del flush
    cold_us = np.median(cold, axis=2) * 1e3
    print(f"[bench] breakdown done; dominant kernel: {'shrink' if dom_op == 0 else 'expand'} "
          f"tok={runs[dom_i].c.T}", file=sys.stderr, flush=True)

    # the timed region: K steps
    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()  # warm on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=cap_stream):
            # the binding's stream argument is baked into the argument tuples: rebuild them for
            # the capture stream so every launch is recorded
            for r in runs:
                r.pair(L, cap_stream.cuda_stream)
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # The dominant kernel, live: K more steps of the same work, launched eagerly on the same
    # stream, with HIP events around that kernel's launch only; the other calls of each step run
    # between its launches exactly as in the timed region, so its caches start as cold. (Its
    # case is one that lora_shrink_expand runs as the two launches of lora_shrink and
    # lora_expand, so the dominant one is made directly.)
    dr = runs[dom_i]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in kev:
        for r in runs:
            if r is not dr:
                r.pair(L)
                continue
            if dom_op == 0:
                a.record()
            r.shrink(L)
            if dom_op == 0:
                b.record()
            if dom_op == 1:
                a.record()
            r.expand(L)
            if dom_op == 1:
                b.record()
    torch.cuda.synchronize()
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
    dom_bytes = dr.alg["shrink_bytes"] if dom_op == 0 else dr.alg["expand_bytes"]
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9

    step_bytes = sum(r.alg["shrink_bytes"] + r.alg["expand_bytes"] for r in runs)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    per_case = []
    for i, r in enumerate(runs):
        b = r.alg["shrink_bytes"] + r.alg["expand_bytes"]
        us = acc[i, 2] * 1e3
        cus = cold_us[i, 2]
        per_case.append({"tok": r.c.T, "shrink_us": round(acc[i, 0] * 1e3, 2),
                         "expand_us": round(acc[i, 1] * 1e3, 2),
                         "pair_us": round(us, 2),
                         "pair_gbps": round(b / (us * 1e-6) / 1e9, 1),
                         "pair_frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "cold_shrink_us": round(float(cold_us[i, 0]), 2),
                         "cold_expand_us": round(float(cold_us[i, 1]), 2),
                         "cold_pair_us": round(float(cus), 2),
                         "cold_pair_gbps": round(b / (cus * 1e-6) / 1e9, 1)})
    mean_case = float(np.mean([p["pair_gbps"] for p in per_case]))

    traffic_table = load_traffic()
    dom_name = f"{'shrink' if dom_op == 0 else 'expand'}_tok{dr.c.T}"
    traffic = traffic_table.get(dom_name)

    out = {
        "metric": "effective HBM GB/s (and % of peak) for LoRA shrink+expand, tok 50-8192",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the decode-QKV workload)",
        "config": {"workload": "decode-QKV bf16 LoRA shrink+expand, 4 adapters r16, K=4096, "
                               "N=4096+1024+1024, tok sweep 50..8192 (9 cases per step, each one "
                               "lora_shrink_expand call: one launch below 1024 tokens, the "
                               "lora_shrink and lora_expand launches from 1024)",
                   "tokens_per_step": int(sum(li.SWEEP_TOKENS)), "bytes_per_step": int(step_bytes),
                   "timing": "graph replay" if graph is not None else "eager",
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "mean_case_gbps": round(mean_case, 1),
                   "per_case_timing": "shrink_us / expand_us (separate calls) and pair_us "
                                      "(lora_shrink_expand, which pair_gbps uses): eager events, "
                                      "5 back-to-back sweeps; cold_*: median of 30 single calls "
                                      "each after a 512 MiB device write",
                   "per_case": per_case},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": dom_name, "avg_launch_us": round(dom_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": int(dom_bytes)},
    }
    extras = set() if args.no_mlp else {e.strip() for e in args.extras.split(",") if e.strip()}
    if "mlp" in extras:
        print("[bench] timing the fused LoRA+SwiGLU MLP", file=sys.stderr, flush=True)
        out["mlp"] = mlp_object(args.steps, args.warmup, traffic_table)
    if "attention" in extras:
        print("[bench] timing the LoRA attention projections", file=sys.stderr, flush=True)
        out["attention_projections"] = attention_object(args.steps, args.warmup)
    if "backward" in extras:
        print("[bench] timing the LoRA MLP training forward and backward", file=sys.stderr, flush=True)
        out["mlp_backward"] = mlp_backward_object(args.steps, args.warmup)
        print("[bench] timing the LoRA projection backward", file=sys.stderr, flush=True)
        out["projection_backward"] = projection_backward_object(args.steps, args.warmup)
    if "embedding" in extras:
        print("[bench] timing the embedding LoRA-A product", file=sys.stderr, flush=True)
        out["embedding_a"] = embedding_object(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
