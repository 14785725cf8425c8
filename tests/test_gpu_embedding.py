"""GPU parity of lora_embedding_a (through the C ABI) against the CPU oracle: bit-exact, since the
product copies stored values.

Covers both A layouts ([L][R][V] storage and a transposed view of [L][V][R] storage), fp32 /
bf16 / fp16, rank padding (rows past an adapter's rank hold NaN, so a read of them would show),
rank 0, empty segments, rows no segment covers (left untouched), ids 0 and V - 1, ids outside
the vocabulary (zero rows), the identity permutation passed as NULL, 2000 segments of 0..8 tokens,
runs of 70 and 80 empty segments inside one wave's 64 positions (more than 63 segment ends: the
in-memory fallback search) and 16,384 one-token segments over a 151,936-entry vocabulary.
"""

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle

pytestmark = pytest.mark.gpu

_BITS = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}


def _poison_padding(c):
    """Rows of A past each adapter's rank become NaN: the op must never read them."""
    A = c.A.clone()
    for a in range(c.L):
        A[a, int(c.lora_ranks[a]):] = float("nan")
    return A


def _run(c, A, layout, null_perm=False, h=None, ids=None):
    alp = __import__("adapter_lora_projection_amd")
    g = lambda t: t.to("cuda").contiguous()
    if layout == "rv":
        wa = g(A)
    else:  # [L][V][R] storage, passed as its [L][R][V] view (unit rank stride)
        wa = g(A.permute(0, 2, 1)).permute(0, 2, 1)
        assert wa.stride(1) == 1
    perm = None if null_perm else g(c.permutation)
    out = alp.embedding_a(g(c.input_ids if ids is None else ids), wa, g(c.seg_indptr),
                          g(c.weight_indices), perm, g(c.lora_ranks), h=h)
    torch.cuda.synchronize()
    return out.cpu()


def _assert_bits(got, ref, rows, what):
    """got (stored dtype) equals the oracle's exact values bit for bit on the given rows."""
    exp = torch.from_numpy(ref[rows]).to(got.dtype)
    g = got[rows]
    bt = _BITS[got.dtype]
    bad = (g.view(bt) != exp.view(bt))
    if bad.any():
        i, j = [int(v) for v in bad.nonzero()[0]]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches; first at row {rows[i]} col {j}: "
                             f"{float(g[i, j])} vs {float(exp[i, j])}")


def _covered(c):
    ip = c.seg_indptr.numpy()
    return np.arange(int(ip[0]), int(ip[-1]))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("layout", ["rv", "vr"])
def test_small(dtype, layout):
    c = li.make_embedding(f"emb_small_{dtype}", seed=3, T=300, V=1000, R=16, L=4, dtype=dtype)
    print("case", c.name, layout, flush=True)
    A = _poison_padding(c)
    got = _run(c, A, layout)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), f"{c.name} {layout}")


@pytest.mark.parametrize("layout", ["rv", "vr"])
def test_rank_padding_and_rank_zero(layout):
    c = li.make_embedding("emb_ranks", seed=4, T=517, V=4099, R=64, L=4, dtype="bf16",
                          ranks=[64, 33, 1, 0])
    print("case", c.name, layout, flush=True)
    A = _poison_padding(c)
    got = _run(c, A, layout)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), c.name)
    # a rank-0 adapter contributes an all-zero row
    a0 = int(np.flatnonzero(c.lora_ranks.numpy() == 0)[0])
    g0 = np.flatnonzero(c.weight_indices.numpy() == a0)
    ip = c.seg_indptr.numpy()
    for g in g0:
        assert torch.all(got[ip[g]:ip[g + 1]] == 0)


def test_empty_segments_and_uncovered_rows():
    # segments 1 and 4 are empty; rows 0..2 and 47..49 belong to no segment and keep their values
    c = li.make_embedding("emb_empty", seed=6, T=50, V=777, R=32, L=3, dtype="bf16",
                          ranks=[32, 5, 17], fixed_indptr=[3, 10, 10, 30, 31, 31, 47],
                          fixed_weight_indices=[0, 1, 2, 1, 0, 2])
    print("case", c.name, flush=True)
    A = _poison_padding(c)
    sentinel = torch.full((c.T, c.R), 7.0, dtype=torch.bfloat16, device="cuda")
    got = _run(c, A, "vr", h=sentinel)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), c.name)
    assert torch.all(got[:3] == 7.0) and torch.all(got[47:] == 7.0)


@pytest.mark.parametrize("layout", ["rv", "vr"])
def test_null_permutation_is_identity(layout):
    c = li.make_embedding("emb_ident", seed=7, T=129, V=2048, R=16, L=2, dtype="f16",
                          identity_perm=True)
    print("case", c.name, layout, flush=True)
    A = _poison_padding(c)
    got_null = _run(c, A, layout, null_perm=True)
    got_perm = _run(c, A, layout)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, None,
                                  c.lora_ranks, c.R)
    _assert_bits(got_null, ref, _covered(c), c.name)
    assert torch.equal(got_null.view(torch.int16), got_perm.view(torch.int16))


def test_ids_outside_the_vocabulary_give_zero_rows():
    c = li.make_embedding("emb_badids", seed=8, T=64, V=500, R=16, L=2, dtype="f32")
    print("case", c.name, flush=True)
    ids = c.input_ids.clone()
    ids[5], ids[9], ids[40] = -1, 500, 1 << 30
    got = _run(c, c.A, "rv", ids=ids)
    ref = oracle.embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices,
                                  c.permutation, c.lora_ranks, c.R)
    inv = torch.argsort(c.permutation.long())  # sorted position of each token
    bad_pos = {int(inv[t]) for t in (5, 9, 40)}
    for p in bad_pos:
        assert torch.all(got[p] == 0), p
    good = np.array([p for p in range(c.T) if p not in bad_pos])
    _assert_bits(got, ref, good, c.name)


def test_many_short_and_empty_segments():
    # 2000 segments of 0..8 tokens
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 9, size=2000)
    ip = np.concatenate([[0], np.cumsum(lens)])
    c = li.make_embedding("emb_2000seg", seed=11, T=int(ip[-1]), V=3001, R=16, L=8, dtype="bf16",
                          ranks=[16, 8, 16, 3, 16, 16, 1, 12], fixed_indptr=ip,
                          fixed_weight_indices=rng.integers(0, 8, size=2000))
    print("case", c.name, c.T, flush=True)
    A = _poison_padding(c)
    got = _run(c, A, "vr")
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), c.name)


@pytest.mark.parametrize("layout", ["rv", "vr"])
def test_runs_of_empty_segments_past_63_ends(layout):
    # 80 empty segments at position 1 and 70 at position 30: 63 positions of the first wave see
    # more than 63 segment ends before them and take the fallback search
    ip = [0, 1] + [1] * 80 + [30] + [30] * 70 + [64, 100, 128, 128, 200]
    G = len(ip) - 1
    rng = np.random.default_rng(14)
    c = li.make_embedding("emb_empty_runs", seed=14, T=210, V=999, R=16, L=5, dtype="bf16",
                          ranks=[16, 9, 16, 2, 16], fixed_indptr=ip,
                          fixed_weight_indices=rng.integers(0, 5, size=G))
    print("case", c.name, layout, flush=True)
    A = _poison_padding(c)
    sentinel = torch.full((c.T, c.R), 3.0, dtype=torch.bfloat16, device="cuda")
    got = _run(c, A, layout, h=sentinel)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), f"{c.name} {layout}")
    assert torch.all(got[200:] == 3.0)


@pytest.mark.parametrize("layout", ["rv", "vr"])
def test_16384_one_token_segments(layout):
    c = li.make_embedding("emb_16384x1", seed=12, T=16384, V=151936, R=16, L=8, dtype="bf16",
                          lengths="ones", ranks=[16, 16, 8, 16, 4, 16, 16, 1])
    print("case", c.name, layout, flush=True)
    assert c.G == 16384
    A = _poison_padding(c)
    got = _run(c, A, layout)
    ref = oracle.embedding_lora_a(c.input_ids, A, c.seg_indptr, c.weight_indices, c.permutation,
                                  c.lora_ranks, c.R)
    _assert_bits(got, ref, _covered(c), f"{c.name} {layout}")


def test_single_token_and_empty_batch():
    alp = __import__("adapter_lora_projection_amd")
    c = li.make_embedding("emb_one", seed=13, T=1, V=10, R=16, L=1, dtype="bf16")
    print("case", c.name, flush=True)
    got = _run(c, c.A, "rv")
    ref = oracle.embedding_lora_a(c.input_ids, c.A, c.seg_indptr, c.weight_indices,
                                  c.permutation, c.lora_ranks, c.R)
    _assert_bits(got, ref, np.arange(1), c.name)
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    h = alp.embedding_a(z, c.A.to("cuda"), torch.zeros(1, dtype=torch.int32, device="cuda"), z,
                        None, c.lora_ranks.to("cuda"))
    assert h.shape == (0, 16)
