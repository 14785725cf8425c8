"""fp64 oracle of the embedding LoRA-A product of the multi-adapter LoRA ops.

Test infrastructure only (see the package docstring).

Source: "Decode LoRA kernels are optimized" (sgl-kernel-xpu pull request 550), Summary and
Behaviour changes: the embedding LoRA-A forward is one of the LoRA ops driven by the same
segment metadata (seg_indptr, weight_indices), and takes an optional longest-segment launch bound
(max_len) so that no per-call device-to-host read is needed; its test runs 16,384 one-token
segments. The page does not print the arithmetic. Reading: for an embedding layer the LoRA-A
product of a token is the column of its adapter's A at the token's vocabulary id (the product of
a one-hot row with A^T), so

    h[i, j] = A[a, j, input_ids[perm[i]]]   for j < r_a,   0 for r_a <= j < R,

with a the adapter of the segment holding sorted position i. It copies values: no rounding.
A is [L][R][V] (one row per rank index, as the LoRA-A weight of an embedding is stored).
"""

from __future__ import annotations

import numpy as np


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy().astype(np.int64)
    return np.asarray(a, dtype=np.int64)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        import torch

        return a.detach().to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def embedding_lora_a(input_ids, A, seg_indptr, weight_indices, permutation, lora_ranks,
                     R: int) -> np.ndarray:
    """h [T][R] in sorted order (fp64 holding the exact stored values; rows no segment covers
    stay NaN). ``permutation`` None means the identity."""
    ids = _i64(input_ids)
    A = _f64(A)
    indptr = _i64(seg_indptr)
    widx = _i64(weight_indices)
    ranks = _i64(lora_ranks)
    T = ids.shape[0]
    perm = np.arange(T) if permutation is None else _i64(permutation)
    h = np.full((T, R), np.nan)
    for g in range(len(widx)):
        i0, i1 = int(indptr[g]), int(indptr[g + 1])
        if i1 <= i0:
            continue
        a = int(widx[g])
        r = int(ranks[a])
        cols = ids[perm[i0:i1]]                 # vocabulary ids of the segment's tokens
        h[i0:i1, :r] = A[a, :r][:, cols].T      # gather: column id of A[a] for each token
        h[i0:i1, r:] = 0.0
    return h
