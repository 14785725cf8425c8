"""The seeded input generators: determinism and the structure each workload states (CPU only)."""

import numpy as np
import torch

import lora_inputs as li


def test_deterministic():
    a = li.config_decode_qkv()
    b = li.config_decode_qkv()
    for f in ("seg_indptr", "weight_indices", "permutation", "x", "A", "B", "y_in"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_tiny_f32():
    c = li.config_tiny_f32()
    assert c.dtype == "f32" and c.x.dtype == torch.float32
    assert c.seg_indptr.tolist() == [0, 40, 64]
    assert c.weight_indices.tolist() == [0, 1]
    assert c.permutation.tolist() == list(range(64))
    assert (c.T, c.K, c.S, c.R, c.L, c.N) == (64, 256, 1, 8, 2, 256)
    assert c.scalings.tolist() == [2.0, 2.0]


def test_decode_qkv():
    c = li.config_decode_qkv()
    assert (c.T, c.K, c.S, c.R, c.L, c.N, c.G) == (50, 4096, 3, 16, 4, 6144, 4)
    assert c.slice_offsets.tolist() == [0, 4096, 5120, 6144]
    assert c.seg_indptr[-1].item() == 50 and (np.diff(c.seg_indptr.numpy()) >= 0).all()
    assert sorted(c.weight_indices.tolist()) == [0, 1, 2, 3]
    assert sorted(c.permutation.tolist()) == list(range(50))
    assert c.x.dtype == torch.bfloat16
    # value distributions: x ~ N(0,1), A,B ~ N(0,0.02)
    assert abs(c.x.float().std().item() - 1.0) < 0.02
    assert abs(c.A.float().std().item() - 0.02) < 0.001


def test_prefill_pair():
    gu, down = li.config_prefill()
    assert (gu.T, gu.K, gu.S, gu.R, gu.L, gu.N) == (2048, 4096, 2, 64, 8, 24576)
    assert (down.T, down.K, down.S, down.R, down.L, down.N) == (2048, 12288, 1, 64, 8, 4096)
    assert torch.equal(gu.seg_indptr, down.seg_indptr) and torch.equal(gu.permutation, down.permutation)
    assert not torch.equal(gu.x[:, :10], down.x[:, :10])


def test_irregular():
    c = li.config_irregular()
    lens = np.diff(c.seg_indptr.numpy())
    assert c.seg_indptr[-1].item() == 8192 and (lens >= 0).all()
    assert int((lens == 0).sum()) == 4
    assert c.lora_ranks.tolist() == [li.IRREGULAR_RANKS[a % 5] for a in range(32)]
    assert sum(c.lora_ranks.tolist()) == 755
    assert c.slice_offsets.tolist() == [0, 4096, 5117, 6138]
    assert c.K == 4093 and c.x.dtype == torch.float16
    # padding beyond each rank is zero in generated weights
    A = c.A.view(32, 3, 64, 4093)
    for a in range(32):
        r = c.lora_ranks[a].item()
        assert (A[a, :, r:, :] == 0).all() and (c.B[a, :, r:] == 0).all()
        assert (A[a, :, :r, :] != 0).any()


def test_sweep_points():
    assert li.SWEEP_TOKENS[0] == 50 and li.SWEEP_TOKENS[-1] == 8192 and len(li.SWEEP_TOKENS) == 9
    c = li.sweep_case(128)
    assert c.T == 128 and c.seg_indptr[-1].item() == 128
    assert torch.equal(li.sweep_case(50).x, li.config_decode_qkv().x)


def test_mlp_small_shapes():
    c = li.config_mlp(M=8, H=16, I=24, r=4)
    assert c.x.shape == (8, 16) and c.w_gate.shape == (24, 16) and c.w_down.shape == (16, 24)
    assert c.a_gate.shape == (4, 16) and c.b_gate.shape == (24, 4)
    assert c.a_down.shape == (4, 24) and c.b_down.shape == (16, 4)
    assert c.scale == 4.0
