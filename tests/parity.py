"""Parity helpers shared by the GPU tests: tolerances and case transfer.

Tolerances (stated by the workload definition and restated here):
* bf16 / fp16 outputs: |gpu - ref| <= 1e-2 + 1e-2 * |ref|, where ref is the oracle value rounded
  once to the storage type.
* fp32 outputs: |gpu - oracle| <= 1e-5 * |oracle| per element, relaxed to 1e-5 * M only where
  the sum cancels (|oracle| < M / 2), M being the magnitude the sum is conditioned on (sum of
  |terms|, plus |y_in| for expand), computed by the oracle on absolute values. Where |oracle| is
  small against M, the fp32 evaluation's own rounding (which scales with M, not with the result)
  can exceed 1e-5 * |oracle| for a correct kernel; everywhere else the plain relative bar holds.
* bf16 gradients of the MLP backward (sums whose terms carry bf16-stored factors, such as
  dA = dxa^T x over 4096 tokens): |gpu - ref| <= 1e-2 + 1e-2 |ref| + 2u * RSS, with u = 2^-8 the
  unit roundoff of bf16 and RSS the root-sum-square of the sum's terms, from the oracle's own
  values; and normwise ||gpu - ref|| <= 2u ||ref|| (the output's own rounding contributes up to
  u/sqrt(3), and a scale that is not a power of two, folded into a bf16 copy of B, about as much
  again through each rounded factor). Derivation of the per-entry bar: a stored bf16 factor (de, dv,
  hmid, the LoRA-A products) whose exact value lies within the accumulation error of a rounding
  boundary is rounded one way by an fp32 evaluation and the other way by the fp64 oracle. Such a
  one-unit disagreement moves its term by at most 2u of the term, so by at most 2u RSS: the
  allowance covers any single disagreement in full (one term can dominate a sum over a few
  tokens). Disagreements in a fraction p of the terms, with independent signs, move the sum by
  about 2u sqrt(p) RSS, so the allowance is 1/sqrt(p) standard deviations; an fp32 evaluation
  disagrees on fewer than 0.1% of the stored values. Near |ref| = 0 (cancellation over the
  tokens) the plain 1e-2 + 1e-2 |ref| bar is far below that noise: a correct fp32 evaluation
  fails it on 0.07-1.8% of the weight-gradient entries at the Qwen3-8B layer
  (tests/test_backward_tolerance.py shows it on the CPU).
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


BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand)


def assert_close_sum_lowp(got, ref, rss, what=""):
    """bf16 sum whose terms carry bf16-stored factors: |got - ref| <= 1e-2 + 1e-2 |ref| + 2u RSS
    per entry, and ||got - ref|| <= 2u ||ref|| over the whole tensor."""
    g = f64(got)
    r = f64(ref)
    q = f64(rss)
    nw = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    if not nw <= 2 * BF16_U:
        raise AssertionError(f"{what}: normwise error {nw:.3e} above 2u = {2 * BF16_U:.3e}")
    bad = ~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r) + 2 * BF16_U * q)
    bad |= np.isnan(g) != np.isnan(r)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside 1e-2+1e-2|ref|+2u*RSS; first "
                             f"{[(tuple(i), g[tuple(i)], r[tuple(i)], q[tuple(i)]) for i in idx]}")


def strict_fail_fraction(got, ref) -> float:
    """Fraction of entries outside the plain bar 1e-2 + 1e-2 |ref| (reported, not asserted)."""
    g = f64(got)
    r = f64(ref)
    return float(np.mean(~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))))


def backward_rss(x, dout, w, inter, scale, rows=None):
    """Root-sum-square of the terms of each MLP-backward gradient's sum, from the oracle's own
    fp64 values (``inter`` from oracle.lora_mlp_backward(..., return_intermediates=True); ``w``
    maps the weight names to tensors). ``rows``: dx on those token rows only.

    dx[m]      = de[m] W_g + dv[m] W_u + dxa_g[m] A_g + dxa_u[m] A_u
    dA_g[j][k] = sum_m dxa_g[m][j] x[m][k]       dB_g[i][j] = s sum_m de[m][i] xa_g[m][j]
    dA_d[j][i] = sum_m dxa_d[m][j] hmid[m][i]    dB_d[n][j] = s sum_m dout[m][n] xa_d[m][j]
    (up like gate)."""
    sq = lambda t: np.square(f64(t))
    s2 = float(scale) ** 2
    X, D = sq(x), sq(dout)
    sel = (lambda t: t) if rows is None else (lambda t: t[rows])
    de, dv = sq(inter["de"]), sq(inter["dv"])
    dx = (sel(de) @ sq(w["w_gate"]) + sel(dv) @ sq(w["w_up"]) + sel(sq(inter["dxa_g"])) @ sq(w["a_gate"])
          + sel(sq(inter["dxa_u"])) @ sq(w["a_up"]))
    out = {
        "dx": np.sqrt(dx),
        "da_gate": np.sqrt(sq(inter["dxa_g"]).T @ X), "db_gate": np.sqrt(s2 * (de.T @ sq(inter["xa_g"]))),
        "da_up": np.sqrt(sq(inter["dxa_u"]).T @ X), "db_up": np.sqrt(s2 * (dv.T @ sq(inter["xa_u"]))),
        "da_down": np.sqrt(sq(inter["dxa_d"]).T @ sq(inter["hmid"])),
        "db_down": np.sqrt(s2 * (D.T @ sq(inter["xa_d"]))),
    }
    return out


def assert_close_f32(got, ref, mag, what=""):
    g = f64(got)
    r = f64(ref)
    m = np.asarray(mag, dtype=np.float64)
    bar = 1e-5 * np.where(np.abs(r) >= 0.5 * m, np.abs(r), m)
    bad = ~(np.abs(g - r) <= bar)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside 1e-5*|ref| (1e-5*M "
                             f"where |ref| < M/2); first "
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
