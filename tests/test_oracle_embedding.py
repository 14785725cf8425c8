"""Pins for the embedding LoRA-A oracle (CPU only): a hand-worked fixture, pure-Python brute
force, the shrink oracle applied to one-hot rows (the product reading of the gather), torch's
embedding lookup per segment (a library routine), the 16,384 one-token-segment case, empty
segments and NULL permutation."""

import json
import os

import numpy as np
import pytest
import torch

import lora_inputs as li
from oracle import embedding_lora_a, shrink

HERE = os.path.dirname(__file__)


def test_handworked_fixture():
    with open(os.path.join(HERE, "golden", "embedding_handworked.json")) as f:
        d = json.load(f)
    A = np.array([[[float(e) for e in r] for r in b] for b in d["A"]])
    h = embedding_lora_a(d["input_ids"], A, d["seg_indptr"], d["weight_indices"], d["permutation"],
                         d["lora_ranks"], d["R"])
    assert np.array_equal(h, np.array(d["h_expected"], dtype=float))


def _brute(c, perm):
    ids, A = c.input_ids.tolist(), c.A.double().tolist()
    indptr, widx, ranks = c.seg_indptr.tolist(), c.weight_indices.tolist(), c.lora_ranks.tolist()
    h = [[float("nan")] * c.R for _ in range(c.T)]
    for g in range(len(widx)):
        a = widx[g]
        for i in range(indptr[g], indptr[g + 1]):
            v = ids[perm[i]]
            for j in range(c.R):
                h[i][j] = A[a][j][v] if j < ranks[a] else 0.0
    return np.array(h)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force(seed):
    c = li.make_embedding("e", seed=seed, T=37, V=101, R=16, L=3, dtype="bf16", ranks=[16, 5, 0])
    h = embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices, c.permutation,
                         c.lora_ranks, c.R)
    assert np.array_equal(h, _brute(c, c.permutation.tolist()), equal_nan=True)


def test_is_shrink_of_one_hot_rows():
    c = li.make_embedding("e", seed=5, T=24, V=50, R=8, L=2, dtype="bf16", ranks=[8, 3])
    x = torch.nn.functional.one_hot(c.input_ids.long(), c.V).double()
    ref = shrink(x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks, 1, c.R, "f64")
    h = embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices, c.permutation,
                         c.lora_ranks, c.R)
    assert np.array_equal(h, ref, equal_nan=True)


def test_matches_torch_embedding_per_segment():
    c = li.make_embedding("e", seed=6, T=60, V=77, R=16, L=4, dtype="bf16")
    h = embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices, c.permutation,
                         c.lora_ranks, c.R)
    ptr, widx, perm = c.seg_indptr.tolist(), c.weight_indices.tolist(), c.permutation.long()
    for g in range(len(widx)):
        i0, i1 = ptr[g], ptr[g + 1]
        emb = torch.nn.functional.embedding(c.input_ids.long()[perm[i0:i1]], c.A[widx[g]].double().T)
        assert np.array_equal(h[i0:i1], emb.numpy())


def test_one_token_segments_and_identity():
    c = li.make_embedding("e", seed=7, T=16384, V=1000, R=16, L=8, dtype="bf16", lengths="ones",
                          identity_perm=True)
    h = embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices, None, c.lora_ranks, c.R)
    A = c.A.double().numpy()
    ids, w = c.input_ids.numpy(), c.weight_indices.numpy()
    assert np.array_equal(h, A[w, :, ids])


def test_empty_segments_leave_rows_untouched():
    c = li.make_embedding("e", seed=8, T=10, V=30, R=4, L=3, dtype="bf16",
                          fixed_indptr=[0, 0, 6, 6, 10], fixed_weight_indices=[2, 0, 1, 1])
    h = embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices, c.permutation,
                         c.lora_ranks, c.R)
    assert not np.isnan(h).any()
    c2 = li.make_embedding("e", seed=8, T=10, V=30, R=4, L=3, dtype="bf16",
                           fixed_indptr=[0, 0, 6, 6, 8], fixed_weight_indices=[2, 0, 1, 1])
    h2 = embedding_lora_a(c2.input_ids, c2.A, c2.seg_indptr, c2.weight_indices, c2.permutation,
                          c2.lora_ranks, c2.R)
    assert np.isnan(h2[8:]).all() and not np.isnan(h2[:8]).any()
