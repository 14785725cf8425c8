"""Pins for the SGMV oracle (CPU only).

Each pin is independent of the oracle's own code path: pure-Python brute force on tiny inputs,
a hand-worked fixture, dense products in another library (torch fp64) and by another
association (merged B*A), and invariants (B = 0, linearity in the scaling, permutation
covariance, masking of rank padding).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import lora_inputs as li
from oracle import expand, rho, shrink, slice_blocks, tile_list, validate_metadata
from oracle.sgmv import (META_BAD_INDEX, META_BAD_INDPTR, META_BAD_PERM, META_BAD_RANK,
                         META_BAD_SLICES, META_OK)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sgmv_handworked.json")


def _load_golden():
    with open(GOLDEN) as f:
        d = json.load(f)

    d["x"] = np.array(d["x"], dtype=np.float64)
    d["A"] = np.array([[[float(e) for e in r] for r in blk] for blk in d["A"]])
    d["B"] = np.array([[[float(e) for e in r] for r in blk] for blk in d["B"]])
    d["y_in"] = np.array(d["y_in"], dtype=np.float64)
    return d


def _brute_shrink(x, A, indptr, widx, perm, ranks, S, R):
    """Pure-Python loops, exactly-rounded sums (math.fsum)."""
    T = len(x)
    K = len(x[0])
    h = [[float("nan")] * (S * R) for _ in range(T)]
    for g in range(len(widx)):
        a = int(widx[g])
        r = int(ranks[a])
        for i in range(int(indptr[g]), int(indptr[g + 1])):
            t = int(perm[i])
            for s in range(S):
                for j in range(R):
                    if j < r:
                        h[i][s * R + j] = math.fsum(float(x[t][k]) * float(A[a][s * R + j][k]) for k in range(K))
                    else:
                        h[i][s * R + j] = 0.0
    return np.array(h)


def _brute_expand(h, B, offs, indptr, widx, perm, ranks, sig, y_in, R):
    y = [list(map(float, row)) for row in y_in]
    for g in range(len(widx)):
        a = int(widx[g])
        r = int(ranks[a])
        for i in range(int(indptr[g]), int(indptr[g + 1])):
            t = int(perm[i])
            for s in range(len(offs) - 1):
                for n in range(int(offs[s]), int(offs[s + 1])):
                    acc = math.fsum(float(h[i][s * R + j]) * float(B[a][n][j]) for j in range(r))
                    y[t][n] = float(y_in[t][n]) + float(sig[a]) * acc
    return np.array(y)


def _tiny_case(seed, T=9, K=7, S=2, R=4, L=3, offs=(0, 5, 8), ranks=(4, 1, 3), dtype="bf16",
               lengths="uniform"):
    return li.make_sgmv(f"tiny{seed}", seed=seed, T=T, K=K, S=S, R=R, L=L, slice_offsets=list(offs),
                        dtype=dtype, ranks=list(ranks), lengths=lengths)


def _np(c):
    return dict(x=c.x.double().numpy(), A=c.A.double().numpy(), B=c.B.double().numpy(),
                y=c.y_in.double().numpy(), indptr=c.seg_indptr.numpy(), widx=c.weight_indices.numpy(),
                perm=c.permutation.numpy(), ranks=c.lora_ranks.numpy(), sig=c.scalings.double().numpy(),
                offs=c.slice_offsets.numpy())


# ---------------------------------------------------------------- hand-worked fixture

def test_handworked_fixture():
    d = _load_golden()
    S, R = d["S"], d["R"]
    for dt in ("f32", "bf16", "f16", "f64"):
        h = shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                   d["lora_ranks"], S, R, dt)
        assert np.array_equal(h, np.array(d["h_expected"], dtype=np.float64)), dt
        y = expand(h, d["B"], d["slice_offsets"], d["seg_indptr"], d["weight_indices"],
                   d["permutation"], d["lora_ranks"], d["scalings"], d["y_in"], R, dt)
        assert np.array_equal(y, np.array(d["y_expected"], dtype=np.float64)), dt
    assert np.array_equal(tile_list(d["seg_indptr"], d["weight_indices"], d["lora_ranks"], 1),
                          np.array(d["tiles_BM1_expected"]))
    assert np.array_equal(tile_list(d["seg_indptr"], d["weight_indices"], d["lora_ranks"], 16),
                          np.array(d["tiles_BM16_expected"]))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_shrink_brute_force(seed):
    c = _tiny_case(seed)
    n = _np(c)
    ref = _brute_shrink(n["x"], n["A"], n["indptr"], n["widx"], n["perm"], n["ranks"], c.S, c.R)
    got = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "f64")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    # bf16 inputs: every product and sum here is exact in fp64, so rounding must agree bitwise
    got_r = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    assert np.array_equal(got_r, rho(ref, "bf16"))


@pytest.mark.parametrize("seed", range(6))
def test_expand_brute_force(seed):
    c = _tiny_case(seed + 10)
    n = _np(c)
    h = li.random_h(seed, c.T, c.S * c.R, "bf16").double().numpy()
    ref = _brute_expand(h, n["B"], n["offs"], n["indptr"], n["widx"], n["perm"], n["ranks"], n["sig"],
                        n["y"], c.R)
    got = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                 c.scalings, c.y_in, c.R, "f64")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    got_r = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                   c.scalings, c.y_in, c.R, "bf16")
    assert np.array_equal(got_r, rho(ref, "bf16"))


@pytest.mark.parametrize("seed", range(4))
def test_chain_matches_brute_dense(seed):
    """Unrounded shrink->expand equals y_in + scale * x[perm] (B_s A_s)^T per segment, with the
    product associated the other way (merged weights) and computed in pure Python."""
    c = _tiny_case(seed + 20, T=7, K=5, S=2, R=3, L=2, offs=(0, 3, 6), ranks=(3, 2))
    n = _np(c)
    h = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "f64")
    y = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
               c.scalings, c.y_in, c.R, "f64")
    ref = [list(map(float, r)) for r in n["y"]]
    for g in range(c.G):
        a = int(n["widx"][g])
        r = int(n["ranks"][a])
        for i in range(int(n["indptr"][g]), int(n["indptr"][g + 1])):
            t = int(n["perm"][i])
            for s in range(c.S):
                for col in range(int(n["offs"][s]), int(n["offs"][s + 1])):
                    # merged weight W[col][k] = sum_j B[a, col, j] * A[a, s*R+j, k]
                    w = [math.fsum(n["B"][a][col][j] * n["A"][a][s * c.R + j][k] for j in range(r))
                         for k in range(c.K)]
                    ref[t][col] = n["y"][t][col] + n["sig"][a] * math.fsum(n["x"][t][k] * w[k] for k in range(c.K))
    assert np.allclose(y, np.array(ref), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_b_zero_leaves_y_unchanged():
    c = _tiny_case(30, T=40, K=33)
    h = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    y = expand(h, torch.zeros_like(c.B), c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation,
               c.lora_ranks, c.scalings, c.y_in, c.R, "bf16")
    assert np.array_equal(y, c.y_in.double().numpy())  # value compare: +0 == -0


def test_linear_in_scale():
    c = _tiny_case(31, T=40, K=33)
    h = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    z = np.zeros(c.y_in.shape)
    d1 = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                c.scalings, z, c.R, "f64")
    d2 = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                c.scalings * 2, z, c.R, "f64")
    assert np.array_equal(d2, 2 * d1)
    d3 = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                c.scalings * 0.375, z, c.R, "f64")
    assert np.allclose(d3, 0.375 * d1, rtol=1e-15, atol=0)


def test_token_relabelling_covariance():
    """Relabel tokens by a bijection pi: x'[pi[t]] = x[t], y_in'[pi[t]] = y_in[t], perm' = pi[perm].
    h must not change and y'[pi[t]] must equal y[t], bitwise."""
    c = _tiny_case(32, T=50, K=40)
    rng = np.random.default_rng(99)
    pi = rng.permutation(c.T)
    x2 = torch.empty_like(c.x)
    x2[torch.from_numpy(pi)] = c.x
    y2 = torch.empty_like(c.y_in)
    y2[torch.from_numpy(pi)] = c.y_in
    perm2 = torch.from_numpy(pi[c.permutation.numpy()].astype(np.int32))
    args = (c.seg_indptr, c.weight_indices)
    h1 = shrink(c.x, c.A, *args, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    h2 = shrink(x2, c.A, *args, perm2, c.lora_ranks, c.S, c.R, "bf16")
    assert np.array_equal(h1, h2)
    y1 = expand(h1, c.B, c.slice_offsets, *args, c.permutation, c.lora_ranks, c.scalings, c.y_in, c.R, "bf16")
    yb = expand(h2, c.B, c.slice_offsets, *args, perm2, c.lora_ranks, c.scalings, y2, c.R, "bf16")
    assert np.array_equal(yb[pi], y1)


def test_within_segment_reorder_invariance():
    """Reordering sorted positions inside each segment (perm and h rows together) leaves y,
    in token order, bitwise unchanged."""
    c = _tiny_case(33, T=60, K=40)
    rng = np.random.default_rng(7)
    indptr = c.seg_indptr.numpy()
    order = np.arange(c.T)
    for g in range(c.G):
        i0, i1 = indptr[g], indptr[g + 1]
        order[i0:i1] = i0 + rng.permutation(i1 - i0)
    perm2 = torch.from_numpy(c.permutation.numpy()[order].astype(np.int32))
    h1 = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    h2 = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, perm2, c.lora_ranks, c.S, c.R, "bf16")
    assert np.array_equal(h2, h1[order])
    y1 = expand(h1, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                c.scalings, c.y_in, c.R, "bf16")
    y2 = expand(h2, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, perm2, c.lora_ranks,
                c.scalings, c.y_in, c.R, "bf16")
    assert np.array_equal(y1, y2)


def test_single_segment_equals_dense_torch():
    """One segment, identity permutation: h = rho(x A^T) and y = rho(y_in + s h B^T), checked
    against torch fp64 dense products."""
    c = li.make_sgmv("one", seed=5, T=33, K=70, S=1, R=6, L=1, slice_offsets=[0, 45], dtype="bf16",
                     identity_perm=True, fixed_indptr=[0, 33], fixed_weight_indices=[0], scale=0.75)
    h = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, 1, 6, "bf16")
    href = torch.from_numpy(rho((c.x.double() @ c.A[0].double().T).numpy(), "bf16"))
    assert np.array_equal(h, href.numpy())
    y = expand(h, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
               c.scalings, c.y_in, 6, "bf16")
    yref = rho((c.y_in.double() + 0.75 * (href @ c.B[0].double().T)).numpy(), "bf16")
    assert np.array_equal(y, yref)


def test_rank_padding_never_read():
    """NaN in A rows / B columns beyond each adapter's rank, and in unused A blocks, never
    reaches the outputs; padded h columns are exactly zero."""
    c = _tiny_case(34, T=30, K=20, ranks=(4, 1, 0))
    A = c.A.clone()
    B = c.B.clone()
    for a in range(c.L):
        r = int(c.lora_ranks[a])
        A.view(c.L, c.S, c.R, c.K)[a, :, r:, :] = float("nan")
        B[a, :, r:] = float("nan")
    h = shrink(c.x, A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    assert np.isfinite(h).all()
    h0 = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, c.S, c.R, "bf16")
    assert np.array_equal(h, h0)
    widx = c.weight_indices.numpy()
    for g in range(c.G):
        r = int(c.lora_ranks[widx[g]])
        i0, i1 = c.seg_indptr[g].item(), c.seg_indptr[g + 1].item()
        for s in range(c.S):
            assert (h[i0:i1, s * c.R + r:(s + 1) * c.R] == 0).all()
    y = expand(h, B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
               c.scalings, c.y_in, c.R, "bf16")
    assert np.isfinite(y).all()


def test_empty_segments_and_uncovered_columns():
    """Empty segments contribute nothing; columns outside the slices keep y_in."""
    c = li.make_sgmv("emp", seed=6, T=20, K=9, S=2, R=2, L=4, slice_offsets=[2, 5, 7], dtype="f32",
                     fixed_indptr=[0, 0, 12, 12, 20], fixed_weight_indices=[3, 0, 1, 2])
    y_in = torch.randn(20, 9, generator=torch.Generator().manual_seed(0))
    h = shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, 2, 2, "f32")
    assert np.isfinite(h).all()
    B = torch.randn(4, 9, 2, generator=torch.Generator().manual_seed(1))
    y = expand(h, B, c.slice_offsets, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
               c.scalings, y_in, 2, "f32")
    yi = y_in.double().numpy()
    assert np.array_equal(y[:, :2], yi[:, :2]) and np.array_equal(y[:, 7:], yi[:, 7:])
    assert not np.array_equal(y[:, 2:7], yi[:, 2:7])
    assert len(tile_list(c.seg_indptr, c.weight_indices, c.lora_ranks, 4)) == 3 + 2


# ---------------------------------------------------------------- schedule

@pytest.mark.parametrize("BM", [1, 3, 16, 64])
def test_tile_list_properties(BM):
    c = li.config_irregular()
    tl = tile_list(c.seg_indptr, c.weight_indices, c.lora_ranks, BM)
    lens = np.diff(c.seg_indptr.numpy())
    assert len(tl) == int(sum((n + BM - 1) // BM for n in lens))
    # the tiles cover every sorted position exactly once, in order
    covered = np.concatenate([np.arange(m0, m0 + ml) for _, m0, ml, _, _ in tl])
    assert np.array_equal(covered, np.arange(c.T))
    assert (tl[:, 2] >= 1).all() and (tl[:, 2] <= BM).all()
    assert np.array_equal(tl[:, 3], c.weight_indices.numpy()[tl[:, 0]])
    assert np.array_equal(tl[:, 4], c.lora_ranks.numpy()[tl[:, 3]])
    assert (np.diff(tl[:, 0]) >= 0).all()


def test_slice_blocks():
    b = slice_blocks([0, 4096, 5117, 6138], 512)
    assert b.tolist()[:1] == [[0, 0, 512]]
    assert [r for r in b.tolist() if r[0] == 1] == [[1, 4096, 512], [1, 4608, 509]]
    assert [r for r in b.tolist() if r[0] == 2] == [[2, 5117, 512], [2, 5629, 509]]
    assert slice_blocks([0, 0, 5], 4).tolist() == [[1, 0, 4], [1, 4, 1]]


def test_validate_metadata_rules():
    T, L, R, N = 6, 2, 4, 8
    ok = dict(seg_indptr=[0, 2, 6], weight_indices=[1, 0], permutation=[5, 4, 3, 2, 1, 0], lora_ranks=[4, 0],
              slice_offsets=[0, 3, 8])
    assert validate_metadata(T, L, R, N, **ok) == META_OK
    assert validate_metadata(T, L, R, N, **{**ok, "seg_indptr": [0, 3, 2]}) == META_BAD_INDPTR
    assert validate_metadata(T, L, R, N, **{**ok, "seg_indptr": [1, 2, 6]}) == META_BAD_INDPTR
    assert validate_metadata(T, L, R, N, **{**ok, "seg_indptr": [0, 2, 5]}) == META_BAD_INDPTR
    assert validate_metadata(T, L, R, N, **{**ok, "weight_indices": [2, 0]}) == META_BAD_INDEX
    assert validate_metadata(T, L, R, N, **{**ok, "weight_indices": [-1, 0]}) == META_BAD_INDEX
    assert validate_metadata(T, L, R, N, **{**ok, "lora_ranks": [5, 0]}) == META_BAD_RANK
    assert validate_metadata(T, L, R, N, **{**ok, "permutation": [5, 4, 3, 2, 1, 1]}) == META_BAD_PERM
    assert validate_metadata(T, L, R, N, **{**ok, "permutation": [5, 4, 3, 2, 1, 6]}) == META_BAD_PERM
    assert validate_metadata(T, L, R, N, **{**ok, "slice_offsets": [0, 3, 7]}) == META_BAD_SLICES
    assert validate_metadata(T, L, R, N, **{**ok, "slice_offsets": [0, 4, 3, 8]}) == META_BAD_SLICES
