"""Tensor-level helpers over the C ABI: sizes and strides from torch tensors, output and
workspace allocation, and the current HIP stream. Marshalling only; the work is the library's.
"""

from __future__ import annotations

import torch

from . import _lib

_DT = {torch.float32: _lib.LORA_F32, torch.bfloat16: _lib.LORA_BF16, torch.float16: _lib.LORA_F16}


def dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _meta(t: torch.Tensor, n: int | None, name: str) -> None:
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 vector")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} entries")


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride of a matrix whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _stacked(t: torch.Tensor, name: str) -> tuple[int, int]:
    """(rows per adapter, row stride) of a stacked [L][rows][cols] weight whose adapters are
    packed back to back."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{name} must be [L][rows][cols] with packed adapters and unit column stride")
    return t.shape[1], t.stride(1)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    """A fresh SGMV workspace: zero-filled, as the shrink's arrival counters require."""
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _given_workspace(ws: torch.Tensor, nbytes: int, device) -> torch.Tensor:
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or ws.device != device:
        raise ValueError("workspace must be a contiguous uint8 vector on the device of the operands")
    if ws.numel() < nbytes:
        raise ValueError(f"workspace must hold at least {nbytes} bytes")
    return ws


def _out(t: torch.Tensor, shape, dtype, device, name: str) -> None:
    """Checks a caller-provided output: shape, dtype and device (rows may be strided)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)} on {device}")


def _bf16_in(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bf16 (this operation is bf16 only)")


def shrink(x, w_a, seg_indptr, weight_indices, permutation, lora_ranks, S: int, R: int,
           h: torch.Tensor | None = None, plan: _lib.Plan | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """h = x[perm] A_a^T per segment (``lora_shrink``). x: [T][K] (row stride >= K),
    w_a: [L][S*R][K]; returns h [T][S*R] in sorted order. permutation=None: identity.
    plan: explicit kernel shape (``lora_shrink_ex``). workspace: a reusable uint8 buffer of at
    least the queried size whose first 32 KiB are zero (a fresh zeroed one otherwise)."""
    _dev(x, w_a, seg_indptr, weight_indices, permutation, lora_ranks, h, workspace)
    T, K = x.shape
    ldx = _rows(x, "x")
    rows, lda = _stacked(w_a, "w_a")
    if rows != S * R or w_a.shape[2] != K:
        raise ValueError("w_a must be [L][S*R][K]")
    G = weight_indices.numel()
    _meta(seg_indptr, G + 1, "seg_indptr")
    _meta(weight_indices, None, "weight_indices")
    if permutation is not None:  # None: identity (tokens already grouped by segment)
        _meta(permutation, T, "permutation")
    _meta(lora_ranks, w_a.shape[0], "lora_ranks")
    dt = dtype_code(x)
    if w_a.dtype != x.dtype:
        raise TypeError("x and w_a must share a dtype")
    if h is None:
        h = torch.empty((T, S * R), dtype=x.dtype, device=x.device)
    else:
        _out(h, (T, S * R), x.dtype, x.device, "h")
    ldh = _rows(h, "h")
    nbytes = _lib.lora_shrink_workspace_size_ex(dt, T, K, S, R, G, plan)
    ws = _workspace(nbytes, x.device) if workspace is None else _given_workspace(workspace, nbytes, x.device)
    _lib.lora_shrink_ex(dt, T, K, S, R, w_a.shape[0], G, x, ldx, w_a, lda, seg_indptr,
                        weight_indices, permutation, lora_ranks, h, ldh, plan, ws,
                        0 if ws is None else ws.numel(), _stream())
    return h


def expand(h, w_b, slice_offsets, seg_indptr, weight_indices, permutation, lora_ranks, scalings,
           y, S: int, R: int, plan: _lib.Plan | None = None) -> torch.Tensor:
    """y[perm[i], slice] += scale_a * h B_a^T in place (``lora_expand``). h: [T][S*R] sorted
    order, w_b: [L][N][R], y: [T][>=N] token order. Returns y. permutation=None: identity.
    plan: explicit kernel shape (``lora_expand_ex``)."""
    _dev(h, w_b, slice_offsets, seg_indptr, weight_indices, permutation, lora_ranks, scalings, y)
    T = h.shape[0]
    ldh = _rows(h, "h")
    N, ldb = _stacked(w_b, "w_b")
    if w_b.shape[2] != R:
        raise ValueError("w_b must be [L][N][R]")
    ldy = _rows(y, "y")
    if y.shape[0] != T or y.shape[1] < N:
        raise ValueError("y must be [T][>=N]")
    G = weight_indices.numel()
    _meta(slice_offsets, S + 1, "slice_offsets")
    _meta(seg_indptr, G + 1, "seg_indptr")
    _meta(weight_indices, None, "weight_indices")
    if permutation is not None:  # None: identity (tokens already grouped by segment)
        _meta(permutation, T, "permutation")
    _meta(lora_ranks, w_b.shape[0], "lora_ranks")
    if scalings.dtype != torch.float32 or scalings.numel() != w_b.shape[0]:
        raise ValueError("scalings must be float32 [L]")
    dt = dtype_code(y)
    if h.dtype != y.dtype or w_b.dtype != y.dtype:
        raise TypeError("h, w_b and y must share a dtype")
    if h.shape[1] != S * R:
        raise ValueError("h must be [T][S*R]")
    nbytes = _lib.lora_expand_workspace_size(dt, T, S, R, G, N)
    ws = _workspace(nbytes, y.device)
    _lib.lora_expand_ex(dt, T, S, R, w_b.shape[0], G, N, h, ldh, w_b, ldb, slice_offsets,
                        seg_indptr, weight_indices, permutation, lora_ranks, scalings, y, ldy, plan,
                        ws, nbytes, _stream())
    return y


def shrink_expand(x, w_a, w_b, slice_offsets, seg_indptr, weight_indices, permutation,
                  lora_ranks, scalings, y, S: int, R: int, h: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """shrink then expand in one call (``lora_shrink_expand``; one launch at decode sizes).
    x: [T][K], w_a: [L][S*R][K], w_b: [L][N][R], y: [T][>=N] updated in place. Returns (h, y).
    workspace: a reusable uint8 buffer of at least the queried size, zero-filled before its
    first use (a fresh zeroed one otherwise)."""
    _dev(x, w_a, w_b, slice_offsets, seg_indptr, weight_indices, permutation, lora_ranks,
         scalings, y, h, workspace)
    T, K = x.shape
    ldx = _rows(x, "x")
    rows, lda = _stacked(w_a, "w_a")
    if rows != S * R or w_a.shape[2] != K:
        raise ValueError("w_a must be [L][S*R][K]")
    N, ldb = _stacked(w_b, "w_b")
    if w_b.shape[2] != R or w_b.shape[0] != w_a.shape[0]:
        raise ValueError("w_b must be [L][N][R] with the adapters of w_a")
    ldy = _rows(y, "y")
    if y.shape[0] != T or y.shape[1] < N:
        raise ValueError("y must be [T][>=N]")
    G = weight_indices.numel()
    _meta(slice_offsets, S + 1, "slice_offsets")
    _meta(seg_indptr, G + 1, "seg_indptr")
    _meta(weight_indices, None, "weight_indices")
    if permutation is not None:
        _meta(permutation, T, "permutation")
    _meta(lora_ranks, w_a.shape[0], "lora_ranks")
    if scalings.dtype != torch.float32 or scalings.numel() != w_a.shape[0]:
        raise ValueError("scalings must be float32 [L]")
    dt = dtype_code(x)
    if w_a.dtype != x.dtype or w_b.dtype != x.dtype or y.dtype != x.dtype:
        raise TypeError("x, w_a, w_b and y must share a dtype")
    if h is None:
        h = torch.empty((T, S * R), dtype=x.dtype, device=x.device)
    else:
        _out(h, (T, S * R), x.dtype, x.device, "h")
    ldh = _rows(h, "h")
    nbytes = _lib.lora_shrink_expand_workspace_size(dt, T, K, S, R, G, N)
    ws = _workspace(nbytes, x.device) if workspace is None else _given_workspace(workspace, nbytes, x.device)
    _lib.lora_shrink_expand(dt, T, K, S, R, w_a.shape[0], G, N, x, ldx, w_a, lda, w_b, ldb,
                            slice_offsets, seg_indptr, weight_indices, permutation, lora_ranks,
                            scalings, h, ldh, y, ldy, ws, 0 if ws is None else ws.numel(),
                            _stream())
    return h, y


def schedule_tiles(T: int, seg_indptr, weight_indices, lora_ranks, BM: int, method: int = 0) -> torch.Tensor:
    """The device segment schedule as an int32 [count][5] tensor of (g, m0, mlen, a, r)."""
    _dev(seg_indptr, weight_indices, lora_ranks)
    G = weight_indices.numel()
    bound = (T + BM - 1) // BM + G
    dev = seg_indptr.device
    tiles = torch.full((max(bound, 1), 5), -1, dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = bound * 16 + 256
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if method == 1 else None
    _lib.lora_schedule_tiles(T, G, BM, method, seg_indptr, weight_indices, lora_ranks, tiles,
                             max(bound, 1), count, ws, nbytes if ws is not None else 0, _stream())
    n = int(count.item())
    return tiles[:n].clone()


def mlp_fused(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down, scale: float,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """out = down(silu(gate(x)) * up(x)) with LoRA on all three projections (``lora_mlp_fused``).
    x: [M][H] bf16; w_gate, w_up: [I][H]; w_down: [H][I]; a_*: [r][in]; b_*: [out][r]."""
    _dev(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down, out, workspace)
    M, H = x.shape
    I = w_gate.shape[0]
    r = a_gate.shape[0]
    for t, shape, name in ((w_gate, (I, H), "w_gate"), (w_up, (I, H), "w_up"), (w_down, (H, I), "w_down"),
                           (a_gate, (r, H), "a_gate"), (a_up, (r, H), "a_up"), (a_down, (r, I), "a_down"),
                           (b_gate, (I, r), "b_gate"), (b_up, (I, r), "b_up"), (b_down, (H, r), "b_down")):
        if tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
    _bf16_in(x, "x")
    ldx = _rows(x, "x")
    if out is None:
        out = torch.empty((M, H), dtype=x.dtype, device=x.device)
    else:
        _out(out, (M, H), torch.bfloat16, x.device, "out")
    ldo = _rows(out, "out")
    nbytes = _lib.lora_mlp_workspace_size(_lib.LORA_BF16, M, H, I, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.lora_mlp_fused(_lib.LORA_BF16, M, H, I, r, float(scale), x, ldx, w_gate, w_up, w_down,
                        a_gate, b_gate, a_up, b_up, a_down, b_down, out, ldo, workspace,
                        workspace.numel(), _stream())
    return out


def _mlp_shapes(x, w_gate, a_gate):
    M, H = x.shape
    return M, H, w_gate.shape[0], a_gate.shape[0]


def mlp_fused_train(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down,
                    scale: float, workspace: torch.Tensor | None = None):
    """The training forward (``lora_mlp_fused_train``): returns (out, e, v) where e and v are the
    gate and up pre-activations (bf16 [M][I]) the backward reads."""
    _dev(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down, workspace)
    M, H, I, r = _mlp_shapes(x, w_gate, a_gate)
    for t, shape, name in ((w_gate, (I, H), "w_gate"), (w_up, (I, H), "w_up"), (w_down, (H, I), "w_down"),
                           (a_gate, (r, H), "a_gate"), (a_up, (r, H), "a_up"), (a_down, (r, I), "a_down"),
                           (b_gate, (I, r), "b_gate"), (b_up, (I, r), "b_up"), (b_down, (H, r), "b_down")):
        _bf16_mat(t, shape, name)
    _bf16_in(x, "x")
    out = torch.empty((M, H), dtype=x.dtype, device=x.device)
    e = torch.empty((M, I), dtype=x.dtype, device=x.device)
    v = torch.empty((M, I), dtype=x.dtype, device=x.device)
    nbytes = _lib.lora_mlp_workspace_size(_lib.LORA_BF16, M, H, I, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.lora_mlp_fused_train(_lib.LORA_BF16, M, H, I, r, float(scale), x, _rows(x, "x"), w_gate,
                              w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down, out, H, e,
                              v, I, workspace, workspace.numel(), _stream())
    return out, e, v


def mlp_prepare_backward(w_gate, w_up, w_down):
    """The frozen weights as the backward reads them (``lora_mlp_prepare_backward``): returns
    (w_gu_t [H][2I] = [W_g^T | W_u^T], w_down_t [I][H] = W_d^T). Done once per layer."""
    _dev(w_gate, w_up, w_down)
    I, H = w_gate.shape
    _bf16_mat(w_gate, (I, H), "w_gate")
    _bf16_mat(w_up, (I, H), "w_up")
    _bf16_mat(w_down, (H, I), "w_down")
    w_gu_t = torch.empty((H, 2 * I), dtype=torch.bfloat16, device=w_gate.device)
    w_down_t = torch.empty((I, H), dtype=torch.bfloat16, device=w_gate.device)
    _lib.lora_mlp_prepare_backward(_lib.LORA_BF16, H, I, w_gate, w_up, w_down, w_gu_t, w_down_t,
                                   _stream())
    return w_gu_t, w_down_t


def mlp_backward(x, e, v, dout, w_gu_t, w_down_t, a_gate, b_gate, a_up, b_up, a_down, b_down,
                 scale: float, workspace: torch.Tensor | None = None,
                 return_intermediates: bool = False):
    """Gradients of the LoRA MLP (``lora_mlp_backward``): dict with dx [M][H], da_gate, da_up
    [r][H], db_gate, db_up [I][r], da_down [r][I], db_down [H][r] (bf16). x must not be the
    storage of any output (it is only read). return_intermediates: also return the stored
    intermediates (views into the workspace, ``lora_mlp_backward_intermediates``)."""
    _dev(x, e, v, dout, w_gu_t, w_down_t, a_gate, b_gate, a_up, b_up, a_down, b_down, workspace)
    M, H = x.shape
    I, r = w_down_t.shape[0], a_gate.shape[0]
    for t, shape, name in ((w_gu_t, (H, 2 * I), "w_gu_t"), (w_down_t, (I, H), "w_down_t"),
                           (a_gate, (r, H), "a_gate"), (a_up, (r, H), "a_up"), (a_down, (r, I), "a_down"),
                           (b_gate, (I, r), "b_gate"), (b_up, (I, r), "b_up"), (b_down, (H, r), "b_down"),
                           (e, (M, I), "e"), (v, (M, I), "v"), (dout, (M, H), "dout")):
        _bf16_mat(t, shape, name)
    _bf16_in(x, "x")
    dev, bf = x.device, torch.bfloat16
    g = {"dx": torch.empty((M, H), dtype=bf, device=dev),
         "da_gate": torch.empty((r, H), dtype=bf, device=dev),
         "db_gate": torch.empty((I, r), dtype=bf, device=dev),
         "da_up": torch.empty((r, H), dtype=bf, device=dev),
         "db_up": torch.empty((I, r), dtype=bf, device=dev),
         "da_down": torch.empty((r, I), dtype=bf, device=dev),
         "db_down": torch.empty((H, r), dtype=bf, device=dev)}
    nbytes = _lib.lora_mlp_backward_workspace_size(_lib.LORA_BF16, M, H, I, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _lib.lora_mlp_backward(_lib.LORA_BF16, M, H, I, r, float(scale), x, _rows(x, "x"), e, v, I,
                           dout, H, w_gu_t, w_down_t, a_gate, b_gate, a_up, b_up, a_down, b_down,
                           g["dx"], H, g["da_gate"], g["db_gate"], g["da_up"], g["db_up"],
                           g["da_down"], g["db_down"], workspace, workspace.numel(), _stream())
    if not return_intermediates:
        return g
    rp, offs = _lib.lora_mlp_backward_intermediates(M, H, I, r)

    def view(k, cols):
        return workspace[offs[k]: offs[k] + M * cols * 2].view(torch.bfloat16).view(M, cols)

    dedv, xa_gu, dxa_gu = view(1, 2 * I), view(2, 2 * rp), view(5, 2 * rp)
    inter = {"hmid": view(0, I), "de": dedv[:, :I], "dv": dedv[:, I:],
             "xa_g": xa_gu[:, :r], "xa_u": xa_gu[:, rp:rp + r], "xa_d": view(3, rp)[:, :r],
             "dxa_d": view(4, rp)[:, :r], "dxa_g": dxa_gu[:, :r], "dxa_u": dxa_gu[:, rp:rp + r]}
    return g, inter


class LoraMlpFunction(torch.autograd.Function):
    """autograd wrapper of the LoRA MLP: forward = lora_mlp_fused_train (saving x, e, v),
    backward = lora_mlp_backward. The frozen weights take no gradient; their backward layout
    (from mlp_prepare_backward) is passed in. x is saved and never written."""

    @staticmethod
    def forward(ctx, x, a_gate, b_gate, a_up, b_up, a_down, b_down, w_gate, w_up, w_down, w_gu_t,
                w_down_t, scale):
        out, e, v = mlp_fused_train(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
                                    b_down, scale)
        ctx.save_for_backward(x, e, v, a_gate, b_gate, a_up, b_up, a_down, b_down, w_gu_t, w_down_t)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        x, e, v, a_gate, b_gate, a_up, b_up, a_down, b_down, w_gu_t, w_down_t = ctx.saved_tensors
        g = mlp_backward(x, e, v, dout.contiguous(), w_gu_t, w_down_t, a_gate, b_gate, a_up, b_up,
                         a_down, b_down, ctx.scale)
        return (g["dx"], g["da_gate"], g["db_gate"], g["da_up"], g["db_up"], g["da_down"],
                g["db_down"], None, None, None, None, None, None)


class LoraLinearFunction(torch.autograd.Function):
    """autograd wrapper of one LoRA projection: forward = lora_linear_fused (saving x), backward =
    lora_linear_backward. W is frozen; its backward layout (linear_prepare_backward) is passed
    in. x is saved and never written."""

    @staticmethod
    def forward(ctx, x, a, b, w, w_t, scale):
        out = linear_fused(x, w, a, b, scale)
        ctx.save_for_backward(x, a, b, w_t)
        ctx.scale = scale
        return out

    @staticmethod
    def backward(ctx, dout):
        x, a, b, w_t = ctx.saved_tensors
        g = linear_backward(x, dout.contiguous(), w_t, a, b, ctx.scale)
        return g["dx"], g["da"], g["db"], None, None, None


class LoraQkvFunction(torch.autograd.Function):
    """autograd wrapper of the query, key and value projections of one x: forward =
    lora_qkv_fused (saving x), backward = lora_qkv_backward. The W are frozen; their backward
    layout (qkv_prepare_backward) is passed in."""

    @staticmethod
    def forward(ctx, x, a_q, b_q, a_k, b_k, a_v, b_v, w_q, w_k, w_v, w_qkv_t, scale):
        q, k, v = qkv_fused(x, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v, b_v, scale)
        ctx.save_for_backward(x, a_q, b_q, a_k, b_k, a_v, b_v, w_qkv_t)
        ctx.scale = scale
        return q, k, v

    @staticmethod
    def backward(ctx, dq, dk, dv):
        x, a_q, b_q, a_k, b_k, a_v, b_v, w_qkv_t = ctx.saved_tensors
        rm = lambda t: t if t.dim() == 2 and t.stride(1) == 1 else t.contiguous()  # row-major
        g = qkv_backward(x, rm(dq), rm(dk), rm(dv), w_qkv_t, a_q, b_q, a_k, b_k, a_v, b_v,
                         ctx.scale)
        return (g["dx"], g["da_q"], g["db_q"], g["da_k"], g["db_k"], g["da_v"], g["db_v"], None,
                None, None, None, None)


def _bf16_mat(t, shape, name):
    if tuple(t.shape) != shape or not t.is_contiguous() or t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape}")


def linear_fused(x, w, a, b, scale: float, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """out = x W^T + s (x A^T) B^T with one adapter (``lora_linear_fused``). x: [M][K] bf16;
    w: [N][K]; a: [r][K]; b: [N][r]."""
    _dev(x, w, a, b, out, workspace)
    M, K = x.shape
    N, r = w.shape[0], a.shape[0]
    for t, shape, name in ((w, (N, K), "w"), (a, (r, K), "a"), (b, (N, r), "b")):
        _bf16_mat(t, shape, name)
    _bf16_in(x, "x")
    ldx = _rows(x, "x")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _out(out, (M, N), torch.bfloat16, x.device, "out")
    nbytes = _lib.lora_linear_workspace_size(_lib.LORA_BF16, M, K, N, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.lora_linear_fused(_lib.LORA_BF16, M, K, N, r, float(scale), x, ldx, w, a, b, out,
                           _rows(out, "out"), workspace, workspace.numel(), _stream())
    return out


def linear_prepare_backward(w):
    """W^T [K][N] of a projection's frozen weight w [N][K], as the backward reads it
    (``lora_linear_prepare_backward``). Done once per layer."""
    _dev(w)
    N, K = w.shape
    _bf16_mat(w, (N, K), "w")
    w_t = torch.empty((K, N), dtype=torch.bfloat16, device=w.device)
    _lib.lora_linear_prepare_backward(_lib.LORA_BF16, K, N, w, w_t, _stream())
    return w_t


def linear_backward(x, dout, w_t, a, b, scale: float, workspace: torch.Tensor | None = None):
    """Gradients of ``linear_fused`` (``lora_linear_backward``): dict with dx [M][K], da [r][K],
    db [N][r] (bf16). x: the saved input [M][K]; dout [M][N]; w_t = W^T [K][N] from
    ``linear_prepare_backward``; a [r][K]; b [N][r]. x is only read."""
    _dev(x, dout, w_t, a, b, workspace)
    M, K = x.shape
    N, r = b.shape
    for t, shape, name in ((w_t, (K, N), "w_t"), (a, (r, K), "a"), (b, (N, r), "b"),
                           (dout, (M, N), "dout")):
        _bf16_mat(t, shape, name)
    _bf16_in(x, "x")
    dev, bf = x.device, torch.bfloat16
    g = {"dx": torch.empty((M, K), dtype=bf, device=dev), "da": torch.empty((r, K), dtype=bf, device=dev),
         "db": torch.empty((N, r), dtype=bf, device=dev)}
    nbytes = _lib.lora_linear_backward_workspace_size(_lib.LORA_BF16, M, K, N, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _lib.lora_linear_backward(_lib.LORA_BF16, M, K, N, r, float(scale), x, _rows(x, "x"), dout, N,
                              w_t, a, b, g["dx"], K, g["da"], g["db"], workspace, workspace.numel(),
                              _stream())
    return g


def qkv_prepare_backward(w_q, w_k, w_v):
    """[W_q^T | W_k^T | W_v^T] [K][Nq + 2 Nkv] as the q/k/v backward reads it
    (``lora_qkv_prepare_backward``). Done once per layer."""
    _dev(w_q, w_k, w_v)
    Nq, K = w_q.shape
    Nkv = w_k.shape[0]
    for t, shape, name in ((w_q, (Nq, K), "w_q"), (w_k, (Nkv, K), "w_k"), (w_v, (Nkv, K), "w_v")):
        _bf16_mat(t, shape, name)
    w_t = torch.empty((K, Nq + 2 * Nkv), dtype=torch.bfloat16, device=w_q.device)
    _lib.lora_qkv_prepare_backward(_lib.LORA_BF16, K, Nq, Nkv, w_q, w_k, w_v, w_t, _stream())
    return w_t


def qkv_backward(x, dq, dk, dv, w_qkv_t, a_q, b_q, a_k, b_k, a_v, b_v, scale: float,
                 workspace: torch.Tensor | None = None):
    """Gradients of ``qkv_fused`` (``lora_qkv_backward``): dict with dx [M][K] (the three
    projections' terms summed, rounded once), da_q/da_k/da_v [r][K], db_q [Nq][r], db_k, db_v
    [Nkv][r] (bf16). x is only read."""
    _dev(x, dq, dk, dv, w_qkv_t, a_q, b_q, a_k, b_k, a_v, b_v, workspace)
    M, K = x.shape
    Nq, r = b_q.shape
    Nkv = b_k.shape[0]
    for t, shape, name in ((w_qkv_t, (K, Nq + 2 * Nkv), "w_qkv_t"), (a_q, (r, K), "a_q"),
                           (a_k, (r, K), "a_k"), (a_v, (r, K), "a_v"), (b_q, (Nq, r), "b_q"),
                           (b_k, (Nkv, r), "b_k"), (b_v, (Nkv, r), "b_v")):
        _bf16_mat(t, shape, name)
    # upstream gradients: row-major with any row pitch (column views of one fused gradient are
    # read in place)
    for t, shape, name in ((dq, (M, Nq), "dq"), (dk, (M, Nkv), "dk"), (dv, (M, Nkv), "dv")):
        if tuple(t.shape) != shape or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a bf16 tensor of shape {shape}")
    lds = [_rows(t, n) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _bf16_in(x, "x")
    dev, bf = x.device, torch.bfloat16
    g = {"dx": torch.empty((M, K), dtype=bf, device=dev)}
    for p, n in (("q", Nq), ("k", Nkv), ("v", Nkv)):
        g["da_" + p] = torch.empty((r, K), dtype=bf, device=dev)
        g["db_" + p] = torch.empty((n, r), dtype=bf, device=dev)
    nbytes = _lib.lora_qkv_backward_workspace_size(_lib.LORA_BF16, M, K, Nq, Nkv, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _lib.lora_qkv_backward(_lib.LORA_BF16, M, K, Nq, Nkv, r, float(scale), x, _rows(x, "x"), dq,
                           lds[0], dk, lds[1], dv, lds[2], w_qkv_t, a_q, b_q, a_k, b_k, a_v, b_v, g["dx"], K,
                           g["da_q"], g["db_q"], g["da_k"], g["db_k"], g["da_v"], g["db_v"],
                           workspace, workspace.numel(), _stream())
    return g


def qkv_fused(x, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v, b_v, scale: float,
              workspace: torch.Tensor | None = None):
    """(q, k, v) projections of one x with one adapter each (``lora_qkv_fused``)."""
    _dev(x, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v, b_v, workspace)
    M, K = x.shape
    Nq, Nkv, r = w_q.shape[0], w_k.shape[0], a_q.shape[0]
    for t, shape, name in ((w_q, (Nq, K), "w_q"), (w_k, (Nkv, K), "w_k"), (w_v, (Nkv, K), "w_v"),
                           (a_q, (r, K), "a_q"), (a_k, (r, K), "a_k"), (a_v, (r, K), "a_v"),
                           (b_q, (Nq, r), "b_q"), (b_k, (Nkv, r), "b_k"), (b_v, (Nkv, r), "b_v")):
        _bf16_mat(t, shape, name)
    _bf16_in(x, "x")
    ldx = _rows(x, "x")
    q = torch.empty((M, Nq), dtype=x.dtype, device=x.device)
    k = torch.empty((M, Nkv), dtype=x.dtype, device=x.device)
    v = torch.empty((M, Nkv), dtype=x.dtype, device=x.device)
    nbytes = _lib.lora_qkv_workspace_size(_lib.LORA_BF16, M, K, Nq, Nkv, r)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _lib.lora_qkv_fused(_lib.LORA_BF16, M, K, Nq, Nkv, r, float(scale), x, ldx, w_q, w_k, w_v,
                        a_q, b_q, a_k, b_k, a_v, b_v, q, Nq, k, Nkv, v, Nkv, workspace,
                        workspace.numel(), _stream())
    return q, k, v


def embedding_a(input_ids, w_a, seg_indptr, weight_indices, permutation, lora_ranks,
                h: torch.Tensor | None = None) -> torch.Tensor:
    """h[i] = column input_ids[perm[i]] of the segment's adapter A, rank-padded with zeros
    (``lora_embedding_a``). input_ids: int32 [T]; w_a: [L][R][V], any strides (a transposed view
    of [L][V][R] storage is the faster layout); returns h [T][R] in sorted order.
    permutation=None: identity."""
    _dev(input_ids, w_a, seg_indptr, weight_indices, permutation, lora_ranks, h)
    T = input_ids.numel()
    _meta(input_ids, T, "input_ids")
    if w_a.dim() != 3 or min(w_a.stride()) < 0 or w_a.stride(1) < 1 or w_a.stride(2) < 1:
        raise ValueError("w_a must be a [L][R][V] tensor with positive rank and vocabulary strides")
    L, R, V = w_a.shape
    G = weight_indices.numel()
    _meta(seg_indptr, G + 1, "seg_indptr")
    _meta(weight_indices, None, "weight_indices")
    if permutation is not None:
        _meta(permutation, T, "permutation")
    _meta(lora_ranks, L, "lora_ranks")
    dt = dtype_code(w_a)
    if h is None:
        h = torch.empty((T, R), dtype=w_a.dtype, device=w_a.device)
    else:
        _out(h, (T, R), w_a.dtype, w_a.device, "h")
    sl, sr, sv = w_a.stride()
    _lib.lora_embedding_a(dt, T, V, R, L, G, input_ids, w_a, sl, sr, sv, seg_indptr,
                          weight_indices, permutation, lora_ranks, h, _rows(h, "h"), _stream())
    return h


def check_metadata(seg_indptr, weight_indices, lora_ranks, R: int, T: int, permutation=None,
                   slice_offsets=None, N: int = 0) -> int:
    """The metadata value checks (``lora_check_metadata``, synchronizing): the number of the
    first rule broken, 0 when valid. permutation / slice_offsets None: not checked."""
    _dev(seg_indptr, weight_indices, lora_ranks, permutation, slice_offsets)
    G = weight_indices.numel()
    _meta(seg_indptr, G + 1, "seg_indptr")
    _meta(weight_indices, None, "weight_indices")
    _meta(lora_ranks, None, "lora_ranks")
    if permutation is not None:
        _meta(permutation, T, "permutation")
    S = 0
    if slice_offsets is not None:
        _meta(slice_offsets, None, "slice_offsets")
        S = slice_offsets.numel() - 1
    nbytes = _lib.lora_check_metadata_workspace_size(T)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=seg_indptr.device)
    return _lib.lora_check_metadata(T, G, lora_ranks.numel(), R, S, N, seg_indptr, weight_indices,
                                    permutation, lora_ranks, slice_offsets, ws, nbytes, _stream())


def fast_path_ineligibility(dropout: float, active_adapters: int, base_bias=None,
                            merged: bool = False) -> str | None:
    """Why the single-adapter fused LoRA path (mlp_fused, mlp_fused_train / mlp_backward,
    linear_fused, qkv_fused) does not apply to a layer, or None when it does. A pure check of the
    conditions of "Add optional fast lora path for qwen2/qwen3 on npu" (Compatibility checks):
    LoRA dropout 0, exactly one active adapter, no base-layer bias, and adapter weights not merged
    into the base weights. Reading: the fused kernels add no bias term at all, so a bias of any
    kind (trainable or frozen) makes the layer ineligible, which covers the page's "no trainable
    bias". Does no arithmetic; a caller that is told no runs its own composition."""
    if not float(dropout) == 0.0:
        return f"LoRA dropout is {dropout}, the fused path needs 0"
    if int(active_adapters) != 1:
        return f"{active_adapters} active adapters, the fused path takes exactly one"
    if base_bias is not None:
        return "the base layer has a bias, the fused path adds none"
    if merged:
        return "the adapter is merged into the base weights"
    return None


def fast_path_eligible(dropout: float, active_adapters: int, base_bias=None,
                       merged: bool = False) -> bool:
    """True when every fast-path condition holds (see fast_path_ineligibility)."""
    return fast_path_ineligibility(dropout, active_adapters, base_bias, merged) is None


def require_fast_path(dropout: float, active_adapters: int, base_bias=None,
                      merged: bool = False) -> None:
    """Raises ValueError naming the first fast-path condition that fails."""
    why = fast_path_ineligibility(dropout, active_adapters, base_bias, merged)
    if why is not None:
        raise ValueError(f"fused LoRA path not applicable: {why}")
