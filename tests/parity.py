"""Parity helpers shared by the GPU tests: tolerances and case transfer.

Tolerances (stated by the workload definition and restated here):
* bf16 / fp16 outputs: |gpu - ref| <= 1e-2 + 1e-2 * |ref|, where ref is the oracle value rounded
  once to the storage type.
* fp32 outputs: |gpu - oracle| <= 1e-5 * M per element, where M is the magnitude the sum is
  conditioned on (sum of |terms|, plus |y_in| for expand), computed by the oracle on absolute
  values; this equals 1e-5 * |oracle| when nothing cancels.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle


def to_dev(c, device="cuda"):
    """Copy every tensor field of an SgmvCase to the GPU (returns a dict)."""
    out = {}
    for k in ("slice_offsets", "seg_indptr", "weight_indices", "permutation", "lora_ranks",
              "scalings", "x", "A", "B", "y_in"):
        out[k] = getattr(c, k).to(device).contiguous()
    return out


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close_lowp(got, ref, what=""):
    g = f64(got)
    r = f64(ref)
    bad = ~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))
    bad |= np.isnan(g) != np.isnan(r)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first "
                             f"{[(tuple(i), g[tuple(i)], r[tuple(i)]) for i in idx]}")


def assert_close_f32(got, ref, mag, what=""):
    g = f64(got)
    r = f64(ref)
    bad = ~(np.abs(g - r) <= 1e-5 * mag)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside 1e-5*M; first "
                             f"{[(tuple(i), g[tuple(i)], r[tuple(i)], mag[tuple(i)]) for i in idx]}")


def check_h(c, h_gpu, x=None, A=None):
    """Compare a GPU shrink output with the oracle, under the tolerance of the case dtype."""
    x = c.x if x is None else x
    A = c.A if A is None else A
    ref = oracle.shrink(x, A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R,
                        c.dtype)
    if c.dtype == "f32":
        mag = oracle.shrink(np.abs(f64(x)), np.nan_to_num(np.abs(f64(A))), c.seg_indptr,
                            c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "f64")
        assert_close_f32(h_gpu, ref, mag, "shrink")
    else:
        assert_close_lowp(h_gpu, ref, "shrink")
    return ref


def check_y(c, h_in, y_gpu, B=None, y_in=None):
    B = c.B if B is None else B
    y_in = c.y_in if y_in is None else y_in
    ref = oracle.expand(h_in, B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation,
                        c.lora_ranks, c.scalings, y_in, c.R, c.dtype)
    if c.dtype == "f32":
        mag = oracle.expand(np.abs(f64(h_in)), np.nan_to_num(np.abs(f64(B))), c.slice_offsets,
                            c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                            np.abs(f64(c.scalings)), np.abs(f64(y_in)), c.R, "f64")
        assert_close_f32(y_gpu, ref, mag, "expand")
    else:
        assert_close_lowp(y_gpu, ref, "expand")
    return ref
