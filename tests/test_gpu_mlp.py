"""GPU parity of lora_mlp_fused (bf16) against the fp64 CPU oracle, through the C ABI.

Small layers are compared element by element (ragged M against the 256-row tiles, an
intermediate size that leaves a partial 128-column gate/up block, odd ranks, ranks above 16,
power-of-two and other scales); the Qwen3-8B-shaped layer of the fused-MLP workload
(M = H = 4096, I = 12288, r = 16, scale 4) is compared on sampled rows, each of which the oracle
computes on its own.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import lora_inputs as li
import oracle
from tests.parity import assert_close_lowp

pytestmark = pytest.mark.gpu


def _run(c, scale=None):
    import adapter_lora_projection_amd as alp

    g = lambda t: t.to("cuda").contiguous()
    out = alp.mlp_fused(g(c.x), g(c.w_gate), g(c.w_up), g(c.w_down), g(c.a_gate), g(c.b_gate),
                        g(c.a_up), g(c.b_up), g(c.a_down), g(c.b_down), c.scale if scale is None else scale)
    torch.cuda.synchronize()
    return out.cpu()


def _args(c):
    return (c.x, c.w_gate, c.w_up, c.w_down, c.a_gate, c.b_gate, c.a_up, c.b_up, c.a_down, c.b_down)


@pytest.mark.parametrize("M,H,I,r,scale", [
    (96, 128, 192, 16, 4.0),     # ragged M, partial gate/up column block
    (300, 256, 320, 7, 2.0),     # odd rank
    (64, 64, 96, 33, 0.5),       # rank above 16 (two K=16 LoRA steps, padded to 64)
    (512, 512, 1024, 16, 1.5),   # non-power-of-two scale (one extra rounding of s*B)
    (1, 32, 32, 1, 4.0),         # single token, rank 1, smallest sizes
])
def test_mlp_small(M, H, I, r, scale):
    c = li.config_mlp(seed=M + H + r, M=M, H=H, I=I, r=r, scale=scale)
    print("case", c.name, flush=True)
    got = _run(c)
    ref = oracle.lora_mlp(*_args(c), c.scale, "bf16")
    assert_close_lowp(got, ref, f"mlp {c.name}")


def test_mlp_b_zero_is_plain_mlp():
    c = li.config_mlp(seed=9, M=128, H=128, I=256, r=16)
    for t in (c.b_gate, c.b_up, c.b_down):
        t.zero_()
    got = _run(c)
    ref = oracle.lora_mlp(*_args(c), c.scale, "bf16")
    assert_close_lowp(got, ref, "mlp B=0")


def test_mlp_full_size_sampled_rows():
    """The fused-MLP workload at full size; 48 sampled rows checked against the oracle."""
    c = li.config_mlp()
    print("case", c.name, flush=True)
    got = _run(c)
    assert torch.isfinite(got.float()).all()
    rows = np.random.default_rng(0).choice(c.M, size=48, replace=False)
    ref = oracle.lora_mlp_rows(rows, *_args(c), c.scale, "bf16")
    assert_close_lowp(got[torch.from_numpy(rows)], ref, "mlp full size")


def test_mlp_rejects_unsupported():
    from adapter_lora_projection_amd import _lib

    c = li.config_mlp(seed=3, M=16, H=48, I=64, r=4)  # H not a multiple of 32
    with pytest.raises(_lib.LoraError) as e:
        _run(c)
    assert e.value.status == _lib.LORA_EUNSUPPORTED
