"""fp64 oracle of the chunked-SGMV LoRA shrink and expand, and of their segment schedule.

Test infrastructure only (see the package docstring).

Problem statement ("Decode LoRA kernels are optimized", Summary and Behaviour changes): tokens are
grouped into segments by ``seg_indptr``; segment ``g`` uses adapter ``weight_indices[g]``; a token
permutation maps sorted positions to token rows; the shrink is a gathered grouped GEMM with one
rank block per output slice, the expand a scattered grouped GEMM whose epilogue applies the
adapter scaling and writes each slice at its column offset. The weight operand is stored
``[N][K]`` row-major (the masked operand load printed in the review thread, element ``n*K + k``).

Readings (the pages do not state these):
* ``permutation[i]`` is the token row held by sorted position ``i`` (a gather index).
* ``h`` is stored in sorted (segment) order; shrink gathers rows of ``x``, expand scatters rows
  of ``y``.
* ``A`` is stacked ``[L][S*R][K]``: slice ``s`` of adapter ``a`` uses rows ``s*R .. s*R+r_a-1``.
  ``B`` is stacked ``[L][N][R]``: row ``n`` is output column ``n`` and uses ``B[a, n, :r_a]``.
* Entries of ``A`` and ``B`` at rank index ``j >= r_a`` are never read; ``h`` at those columns
  is exactly zero.
* The scaling multiplies the expand product only; expand is a read-modify-write of ``y``.
* Each stored tensor is rounded exactly once (``rho``) from the exact (fp64) value.
"""

from __future__ import annotations

import numpy as np

from .rounding import rho


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor
        import torch

        return a.detach().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy().astype(np.int64)
    return np.asarray(a, dtype=np.int64)


def shrink(x, A, seg_indptr, weight_indices, permutation, lora_ranks, S: int, R: int,
           out_dtype: str) -> np.ndarray:
    """Chunked-SGMV shrink.

    For segment ``g`` with adapter ``a = weight_indices[g]`` and rank ``r = lora_ranks[a]``, every
    sorted position ``i`` in it, slice ``s`` and ``j < R``::

        h[i, s*R + j] = rho( sum_k x[perm[i], k] * A[a, s*R + j, k] )   if j < r
        h[i, s*R + j] = 0                                               otherwise

    ``x`` is ``[T][K]``, ``A`` is ``[L][S*R][K]``. Returns fp64 ``[T][S*R]``; a row no segment
    covers stays NaN. Each segment's product is one fp64 matrix product (a library step).
    """
    x = _f64(x)
    A = _f64(A)
    indptr = _i64(seg_indptr)
    widx = _i64(weight_indices)
    perm = _i64(permutation)
    ranks = _i64(lora_ranks)
    T = x.shape[0]
    h = np.full((T, S * R), np.nan)
    for g in range(len(widx)):
        i0, i1 = int(indptr[g]), int(indptr[g + 1])
        if i1 <= i0:
            continue
        a = int(widx[g])
        r = int(ranks[a])
        rows = x[perm[i0:i1]]  # gathered activations, [len][K]
        for s in range(S):
            block = A[a, s * R: s * R + r]  # [r][K]
            h[i0:i1, s * R: s * R + r] = rho(rows @ block.T, out_dtype)
            h[i0:i1, s * R + r: (s + 1) * R] = 0.0
    return h


def expand(h, B, slice_offsets, seg_indptr, weight_indices, permutation, lora_ranks, scalings,
           y_in, R: int, out_dtype: str) -> np.ndarray:
    """Chunked-SGMV expand (scaled scatter-add).

    For segment ``g`` (adapter ``a``, rank ``r``, scaling ``sigma = scalings[a]``), sorted
    position ``i`` in it, slice ``s`` and column ``n`` in ``[slice_offsets[s], slice_offsets[s+1])``::

        y[perm[i], n] = rho( y_in[perm[i], n] + sigma * sum_{j<r} h[i, s*R + j] * B[a, n, j] )

    ``h`` is ``[T][S*R]`` in sorted order, ``B`` is ``[L][N][R]``, ``y_in`` is ``[T][W]`` with
    ``W >= N`` in token order. Entries the formula does not name keep their ``y_in`` value.
    """
    h = _f64(h)
    B = _f64(B)
    y_in = _f64(y_in)
    offs = _i64(slice_offsets)
    indptr = _i64(seg_indptr)
    widx = _i64(weight_indices)
    perm = _i64(permutation)
    ranks = _i64(lora_ranks)
    sig = _f64(scalings)
    y = y_in.copy()
    S = len(offs) - 1
    for g in range(len(widx)):
        i0, i1 = int(indptr[g]), int(indptr[g + 1])
        if i1 <= i0:
            continue
        a = int(widx[g])
        r = int(ranks[a])
        rows = perm[i0:i1]
        for s in range(S):
            n0, n1 = int(offs[s]), int(offs[s + 1])
            if n1 <= n0:
                continue
            delta = h[i0:i1, s * R: s * R + r] @ B[a, n0:n1, :r].T  # [len][n1-n0]
            y[rows, n0:n1] = rho(y_in[rows, n0:n1] + sig[a] * delta, out_dtype)
    return y


def tile_list(seg_indptr, weight_indices, lora_ranks, BM: int) -> np.ndarray:
    """The M-tiles a segment scheduler must produce, by enumeration.

    Each non-empty segment ``g`` is cut into row tiles of at most ``BM`` sorted positions,
    starting at ``seg_indptr[g]``; empty segments yield nothing. Rows are
    ``(g, m0, mlen, a, r)`` in segment-major order with ascending ``m0``; the list is unique.
    """
    indptr = _i64(seg_indptr)
    widx = _i64(weight_indices)
    ranks = _i64(lora_ranks)
    out = []
    for g in range(len(widx)):
        i0, i1 = int(indptr[g]), int(indptr[g + 1])
        a = int(widx[g])
        m0 = i0
        while m0 < i1:
            out.append((g, m0, min(BM, i1 - m0), a, int(ranks[a])))
            m0 += BM
    return np.asarray(out, dtype=np.int32).reshape(-1, 5)


def slice_blocks(slice_offsets, BN: int) -> np.ndarray:
    """Column blocks of at most ``BN`` columns that never straddle a slice boundary:
    rows ``(s, n0, nlen)`` with slices in order and ascending ``n0``."""
    offs = _i64(slice_offsets)
    out = []
    for s in range(len(offs) - 1):
        n0 = int(offs[s])
        while n0 < int(offs[s + 1]):
            out.append((s, n0, min(BN, int(offs[s + 1]) - n0)))
            n0 += BN
    return np.asarray(out, dtype=np.int32).reshape(-1, 3)


# Result codes of validate_metadata (first failing rule, in this order).
META_OK = 0
META_BAD_INDPTR = 1  # seg_indptr[0] != 0, decreasing, or seg_indptr[G] != T
META_BAD_INDEX = 2  # weight_indices outside [0, L)
META_BAD_RANK = 3  # lora_ranks outside [0, R]
META_BAD_PERM = 4  # permutation is not a bijection of [0, T)
META_BAD_SLICES = 5  # slice_offsets not nondecreasing from >= 0, or last != N


def validate_metadata(T: int, L: int, R: int, N: int, seg_indptr, weight_indices, permutation,
                      lora_ranks, slice_offsets=None) -> int:
    """Which validity rule the metadata breaks first (0 = valid).

    Invalid metadata is undefined behaviour on the fast path ("Decode LoRA kernels are optimized",
    Behaviour changes); this is the definition the optional value check enforces.
    """
    indptr = _i64(seg_indptr)
    widx = _i64(weight_indices)
    perm = _i64(permutation)
    ranks = _i64(lora_ranks)
    if len(indptr) != len(widx) + 1 or indptr[0] != 0 or indptr[-1] != T or np.any(np.diff(indptr) < 0):
        return META_BAD_INDPTR
    if np.any(widx < 0) or np.any(widx >= L):
        return META_BAD_INDEX
    if np.any(ranks < 0) or np.any(ranks > R):
        return META_BAD_RANK
    if len(perm) != T or np.any(perm < 0) or np.any(perm >= T) or len(np.unique(perm)) != T:
        return META_BAD_PERM
    if slice_offsets is not None:
        offs = _i64(slice_offsets)
        if offs[0] < 0 or np.any(np.diff(offs) < 0) or offs[-1] != N:
            return META_BAD_SLICES
    return META_OK
