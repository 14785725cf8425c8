"""ctypes binding of ``liblora_mi355x.so`` (argument marshalling only).

The functions named like the C entry points take plain integers or torch tensors (passed as
device pointers) and raise :class:`LoraError` on a non-OK status. There is no fallback: if the
library is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora_mi355x.so")

LORA_OK, LORA_EINVAL, LORA_EUNSUPPORTED, LORA_EWORKSPACE, LORA_EHIP, LORA_EVALUE = range(6)
LORA_F32, LORA_BF16, LORA_F16 = 0, 1, 2
LORA_SHRINK_RING_SHAPES, LORA_SHRINK_LDS_SHAPES, LORA_EXPAND_SHAPES = 5, 13, 10


class Plan(ctypes.Structure):
    """``lora_plan``: explicit kernel-shape choices of one call (-1 = the library's choice)."""

    _fields_ = [("shrink_kernel", ctypes.c_int32), ("shrink_shape", ctypes.c_int32),
                ("shrink_split", ctypes.c_int32), ("shrink_finish", ctypes.c_int32),
                ("expand_shape", ctypes.c_int32), ("expand_block_n", ctypes.c_int32)]

    def __init__(self, shrink_kernel=-1, shrink_shape=-1, shrink_split=-1, shrink_finish=-1,
                 expand_shape=-1, expand_block_n=-1):
        super().__init__(shrink_kernel, shrink_shape, shrink_split, shrink_finish, expand_shape,
                         expand_block_n)

# Every symbol the public header declares, with (restype, argtypes).
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "lora_status_str": (ctypes.c_char_p, [_i32]),
    "lora_version": (ctypes.c_char_p, []),
    "lora_shrink": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _i64,
                           _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz, _vp]),
    "lora_shrink_workspace_size": (_sz, [_i32, _i64, _i64, _i32, _i32, _i32]),
    "lora_expand": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i64, _vp, _i64, _vp, _i64,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz, _vp]),
    "lora_expand_workspace_size": (_sz, [_i32, _i64, _i32, _i32, _i32, _i64]),
    "lora_shrink_expand": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, _i64, _vp, _i64, _vp,
                                  _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                                  _i64, _vp, _sz, _vp]),
    "lora_shrink_expand_workspace_size": (_sz, [_i32, _i64, _i64, _i32, _i32, _i32, _i64]),
    "lora_linear_prepare_backward": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp]),
    "lora_linear_backward": (_i32, [_i32, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp,
                                    _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "lora_linear_backward_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "lora_qkv_prepare_backward": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "lora_qkv_backward": (_i32, [_i32, _i64, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64,
                                 _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lora_qkv_backward_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i64, _i32]),
    "lora_schedule_tiles": (_i32, [_i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                   _sz, _vp]),
    "lora_shrink_ex": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _i64,
                              _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lora_shrink_workspace_size_ex": (_sz, [_i32, _i64, _i64, _i32, _i32, _i32, _vp]),
    "lora_shrink_noalloc": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _i64,
                                   _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "lora_shrink_noalloc_max_workspace": (_sz, []),
    "lora_expand_ex": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i64, _vp, _i64, _vp, _i64,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "lora_mlp_fused": (_i32, [_i32, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz, _vp]),
    "lora_mlp_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "lora_mlp_fused_train": (_i32, [_i32, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                    _i64, _vp, _sz, _vp]),
    "lora_mlp_prepare_backward": (_i32, [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "lora_mlp_backward": (_i32, [_i32, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp, _vp,
                                 _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "lora_mlp_backward_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "lora_mlp_backward_intermediates": (_i32, [_i64, _i64, _i64, _i32, _vp]),
    "lora_check_metadata": (_i32, [_i64, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _sz, _vp]),
    "lora_check_metadata_workspace_size": (_sz, [_i64]),
    "lora_linear_fused": (_i32, [_i32, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp, _vp,
                                 _vp, _vp, _i64, _vp, _sz, _vp]),
    "lora_linear_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "lora_qkv_fused": (_i32, [_i32, _i64, _i64, _i64, _i64, _i32, ctypes.c_float, _vp, _i64, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                              _i64, _vp, _sz, _vp]),
    "lora_qkv_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i64, _i32]),
    "lora_embedding_a": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _i64, _i64, _i64,
                                _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
}


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(t) -> int | None:
    """Device pointer of a tensor (or an int / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(fn: str, st: int) -> None:
    if st != LORA_OK:
        raise LoraError(fn, st)


def status_str(st: int) -> str:
    return lib().lora_status_str(st).decode()


def lora_version() -> str:
    return lib().lora_version().decode()


def lora_shrink(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                permutation, lora_ranks, h, ldh, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_shrink(dtype, T, K, S, R, L, G, _p(x), ldx, _p(w_a), lda, _p(seg_indptr),
                           _p(weight_indices), _p(permutation), _p(lora_ranks), _p(h), ldh,
                           _p(workspace), workspace_bytes, stream)
    _check("lora_shrink", st)


def lora_shrink_workspace_size(dtype, T, K, S, R, G) -> int:
    return int(lib().lora_shrink_workspace_size(dtype, T, K, S, R, G))


def _plan(plan):
    return None if plan is None else ctypes.addressof(plan)


def lora_shrink_ex(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                   permutation, lora_ranks, h, ldh, plan, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_shrink_ex(dtype, T, K, S, R, L, G, _p(x), ldx, _p(w_a), lda, _p(seg_indptr),
                              _p(weight_indices), _p(permutation), _p(lora_ranks), _p(h), ldh,
                              _plan(plan), _p(workspace), workspace_bytes, stream)
    _check("lora_shrink_ex", st)


def lora_shrink_noalloc(dtype, T, K, S, R, L, G, x, ldx, w_a, lda, seg_indptr, weight_indices,
                        permutation, lora_ranks, h, ldh, stream) -> None:
    st = lib().lora_shrink_noalloc(dtype, T, K, S, R, L, G, _p(x), ldx, _p(w_a), lda,
                                   _p(seg_indptr), _p(weight_indices), _p(permutation),
                                   _p(lora_ranks), _p(h), ldh, stream)
    _check("lora_shrink_noalloc", st)


def lora_shrink_noalloc_max_workspace() -> int:
    return int(lib().lora_shrink_noalloc_max_workspace())


def lora_shrink_workspace_size_ex(dtype, T, K, S, R, G, plan) -> int:
    return int(lib().lora_shrink_workspace_size_ex(dtype, T, K, S, R, G, _plan(plan)))


def lora_expand_ex(dtype, T, S, R, L, G, N, h, ldh, w_b, ldb, slice_offsets, seg_indptr,
                   weight_indices, permutation, lora_ranks, scalings, y, ldy, plan, workspace,
                   workspace_bytes, stream) -> None:
    st = lib().lora_expand_ex(dtype, T, S, R, L, G, N, _p(h), ldh, _p(w_b), ldb, _p(slice_offsets),
                              _p(seg_indptr), _p(weight_indices), _p(permutation), _p(lora_ranks),
                              _p(scalings), _p(y), ldy, _plan(plan), _p(workspace),
                              workspace_bytes, stream)
    _check("lora_expand_ex", st)


def lora_expand(dtype, T, S, R, L, G, N, h, ldh, w_b, ldb, slice_offsets, seg_indptr,
                weight_indices, permutation, lora_ranks, scalings, y, ldy, workspace,
                workspace_bytes, stream) -> None:
    st = lib().lora_expand(dtype, T, S, R, L, G, N, _p(h), ldh, _p(w_b), ldb, _p(slice_offsets),
                           _p(seg_indptr), _p(weight_indices), _p(permutation), _p(lora_ranks),
                           _p(scalings), _p(y), ldy, _p(workspace), workspace_bytes, stream)
    _check("lora_expand", st)


def lora_expand_workspace_size(dtype, T, S, R, G, N) -> int:
    return int(lib().lora_expand_workspace_size(dtype, T, S, R, G, N))


def lora_shrink_expand(dtype, T, K, S, R, L, G, N, x, ldx, w_a, lda, w_b, ldb, slice_offsets,
                       seg_indptr, weight_indices, permutation, lora_ranks, scalings, h, ldh, y,
                       ldy, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_shrink_expand(dtype, T, K, S, R, L, G, N, _p(x), ldx, _p(w_a), lda, _p(w_b),
                                  ldb, _p(slice_offsets), _p(seg_indptr), _p(weight_indices),
                                  _p(permutation), _p(lora_ranks), _p(scalings), _p(h), ldh,
                                  _p(y), ldy, _p(workspace), workspace_bytes, stream)
    _check("lora_shrink_expand", st)


def lora_shrink_expand_workspace_size(dtype, T, K, S, R, G, N) -> int:
    return int(lib().lora_shrink_expand_workspace_size(dtype, T, K, S, R, G, N))


def lora_linear_prepare_backward(dtype, K, N, w, w_t, stream) -> None:
    _check("lora_linear_prepare_backward",
           lib().lora_linear_prepare_backward(dtype, K, N, _p(w), _p(w_t), stream))


def lora_linear_backward(dtype, M, K, N, r, scale, x, ldx, dout, lddo, w_t, a, b, dx, lddx, da,
                         db, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_linear_backward(dtype, M, K, N, r, scale, _p(x), ldx, _p(dout), lddo, _p(w_t),
                                    _p(a), _p(b), _p(dx), lddx, _p(da), _p(db), _p(workspace),
                                    workspace_bytes, stream)
    _check("lora_linear_backward", st)


def lora_linear_backward_workspace_size(dtype, M, K, N, r) -> int:
    return int(lib().lora_linear_backward_workspace_size(dtype, M, K, N, r))


def lora_qkv_prepare_backward(dtype, K, Nq, Nkv, w_q, w_k, w_v, w_qkv_t, stream) -> None:
    _check("lora_qkv_prepare_backward",
           lib().lora_qkv_prepare_backward(dtype, K, Nq, Nkv, _p(w_q), _p(w_k), _p(w_v),
                                           _p(w_qkv_t), stream))


def lora_qkv_backward(dtype, M, K, Nq, Nkv, r, scale, x, ldx, dq, lddq, dk, lddk, dv, lddv,
                      w_qkv_t, a_q, b_q, a_k, b_k, a_v, b_v, dx, lddx, da_q, db_q, da_k, db_k,
                      da_v, db_v, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_qkv_backward(dtype, M, K, Nq, Nkv, r, scale, _p(x), ldx, _p(dq), lddq, _p(dk),
                                 lddk, _p(dv), lddv, _p(w_qkv_t), _p(a_q), _p(b_q), _p(a_k),
                                 _p(b_k), _p(a_v), _p(b_v), _p(dx), lddx, _p(da_q), _p(db_q),
                                 _p(da_k), _p(db_k), _p(da_v), _p(db_v), _p(workspace),
                                 workspace_bytes, stream)
    _check("lora_qkv_backward", st)


def lora_qkv_backward_workspace_size(dtype, M, K, Nq, Nkv, r) -> int:
    return int(lib().lora_qkv_backward_workspace_size(dtype, M, K, Nq, Nkv, r))


LORA_SHRINK_EXPAND_FLAG_OFFSET = 32764  # byte offset of the wait-bound flag in the workspace


def lora_schedule_tiles(T, G, BM, method, seg_indptr, weight_indices, lora_ranks, tiles,
                        max_tiles, count, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_schedule_tiles(T, G, BM, method, _p(seg_indptr), _p(weight_indices),
                                   _p(lora_ranks), _p(tiles), max_tiles, _p(count), _p(workspace),
                                   workspace_bytes, stream)
    _check("lora_schedule_tiles", st)


def lora_mlp_fused(dtype, M, H, I, r, scale, x, ldx, w_gate, w_up, w_down, a_gate, b_gate, a_up,
                   b_up, a_down, b_down, out, ldo, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_mlp_fused(dtype, M, H, I, r, scale, _p(x), ldx, _p(w_gate), _p(w_up),
                              _p(w_down), _p(a_gate), _p(b_gate), _p(a_up), _p(b_up), _p(a_down),
                              _p(b_down), _p(out), ldo, _p(workspace), workspace_bytes, stream)
    _check("lora_mlp_fused", st)


def lora_mlp_workspace_size(dtype, M, H, I, r) -> int:
    return int(lib().lora_mlp_workspace_size(dtype, M, H, I, r))


def lora_mlp_fused_train(dtype, M, H, I, r, scale, x, ldx, w_gate, w_up, w_down, a_gate, b_gate,
                         a_up, b_up, a_down, b_down, out, ldo, e, v, lde, workspace,
                         workspace_bytes, stream) -> None:
    st = lib().lora_mlp_fused_train(dtype, M, H, I, r, scale, _p(x), ldx, _p(w_gate), _p(w_up),
                                    _p(w_down), _p(a_gate), _p(b_gate), _p(a_up), _p(b_up),
                                    _p(a_down), _p(b_down), _p(out), ldo, _p(e), _p(v), lde,
                                    _p(workspace), workspace_bytes, stream)
    _check("lora_mlp_fused_train", st)


def lora_mlp_prepare_backward(dtype, H, I, w_gate, w_up, w_down, w_gu_t, w_down_t, stream) -> None:
    st = lib().lora_mlp_prepare_backward(dtype, H, I, _p(w_gate), _p(w_up), _p(w_down), _p(w_gu_t),
                                         _p(w_down_t), stream)
    _check("lora_mlp_prepare_backward", st)


def lora_mlp_backward(dtype, M, H, I, r, scale, x, ldx, e, v, lde, dout, lddo, w_gu_t, w_down_t,
                      a_gate, b_gate, a_up, b_up, a_down, b_down, dx, lddx, da_gate, db_gate,
                      da_up, db_up, da_down, db_down, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_mlp_backward(dtype, M, H, I, r, scale, _p(x), ldx, _p(e), _p(v), lde, _p(dout),
                                 lddo, _p(w_gu_t), _p(w_down_t), _p(a_gate), _p(b_gate), _p(a_up),
                                 _p(b_up), _p(a_down), _p(b_down), _p(dx), lddx, _p(da_gate),
                                 _p(db_gate), _p(da_up), _p(db_up), _p(da_down), _p(db_down),
                                 _p(workspace), workspace_bytes, stream)
    _check("lora_mlp_backward", st)


def lora_mlp_backward_workspace_size(dtype, M, H, I, r) -> int:
    return int(lib().lora_mlp_backward_workspace_size(dtype, M, H, I, r))


def lora_linear_fused(dtype, M, K, N, r, scale, x, ldx, w, a, b, out, ldo, workspace,
                      workspace_bytes, stream) -> None:
    st = lib().lora_linear_fused(dtype, M, K, N, r, scale, _p(x), ldx, _p(w), _p(a), _p(b),
                                 _p(out), ldo, _p(workspace), workspace_bytes, stream)
    _check("lora_linear_fused", st)


def lora_linear_workspace_size(dtype, M, K, N, r) -> int:
    return int(lib().lora_linear_workspace_size(dtype, M, K, N, r))


def lora_qkv_fused(dtype, M, K, Nq, Nkv, r, scale, x, ldx, w_q, w_k, w_v, a_q, b_q, a_k, b_k, a_v,
                   b_v, q, ldq, k, ldk, v, ldv, workspace, workspace_bytes, stream) -> None:
    st = lib().lora_qkv_fused(dtype, M, K, Nq, Nkv, r, scale, _p(x), ldx, _p(w_q), _p(w_k),
                              _p(w_v), _p(a_q), _p(b_q), _p(a_k), _p(b_k), _p(a_v), _p(b_v),
                              _p(q), ldq, _p(k), ldk, _p(v), ldv, _p(workspace), workspace_bytes,
                              stream)
    _check("lora_qkv_fused", st)


def lora_qkv_workspace_size(dtype, M, K, Nq, Nkv, r) -> int:
    return int(lib().lora_qkv_workspace_size(dtype, M, K, Nq, Nkv, r))


def lora_embedding_a(dtype, T, V, R, L, G, input_ids, w_a, stride_l, stride_r, stride_v,
                     seg_indptr, weight_indices, permutation, lora_ranks, h, ldh, stream) -> None:
    st = lib().lora_embedding_a(dtype, T, V, R, L, G, _p(input_ids), _p(w_a), stride_l, stride_r,
                                stride_v, _p(seg_indptr), _p(weight_indices), _p(permutation),
                                _p(lora_ranks), _p(h), ldh, stream)
    _check("lora_embedding_a", st)


def lora_mlp_backward_intermediates(M, H, I, r) -> tuple[int, list[int]]:
    """(rp, byte offsets of hmid, [de|dv], [xa_g|xa_u], xa_d, dxa_d, [dxa_g|dxa_u])."""
    offs = (ctypes.c_size_t * 6)()
    rp = int(lib().lora_mlp_backward_intermediates(M, H, I, r, offs))
    return rp, [int(o) for o in offs]


def lora_check_metadata(T, G, L, R, S, N, seg_indptr, weight_indices, permutation, lora_ranks,
                        slice_offsets, workspace, workspace_bytes, stream) -> int:
    """Rule number broken (0 = valid); argument errors raise."""
    rule = ctypes.c_int32(0)
    st = lib().lora_check_metadata(T, G, L, R, S, N, _p(seg_indptr), _p(weight_indices),
                                   _p(permutation), _p(lora_ranks), _p(slice_offsets),
                                   ctypes.byref(rule), _p(workspace), workspace_bytes, stream)
    if st not in (LORA_OK, LORA_EVALUE):
        _check("lora_check_metadata", st)
    return int(rule.value)


def lora_check_metadata_workspace_size(T) -> int:
    return int(lib().lora_check_metadata_workspace_size(T))
