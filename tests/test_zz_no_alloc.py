"""lora_shrink_noalloc (the allocation-free shrink: scratch in a fixed device array of the
library) against lora_shrink with a caller workspace, through the C ABI: two calls in a row on
the same array, the second with a smaller input, each bit-identical to lora_shrink and within
the bf16 bar of the oracle."""

import pytest
import torch

import lora_inputs as li
from adapter_lora_projection_amd import _lib
from tests.parity import check_h, to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1, "f16": 2}


def _call(c, d, noalloc):
    h = torch.full((c.T, c.S * c.R), float("nan"), dtype=d["x"].dtype, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    args = (DT[c.dtype], c.T, c.K, c.S, c.R, c.L, c.G, d["x"], c.K, d["A"], c.K, d["seg_indptr"],
            d["weight_indices"], d["permutation"], d["lora_ranks"], h, c.S * c.R)
    if noalloc:
        _lib.lora_shrink_noalloc(*args, st)
    else:
        n = _lib.lora_shrink_workspace_size(DT[c.dtype], c.T, c.K, c.S, c.R, c.G)
        ws = torch.zeros(max(n, 1), dtype=torch.uint8, device="cuda")
        _lib.lora_shrink(*args, ws, n, st)
    torch.cuda.synchronize()
    return h.cpu()


@pytest.mark.parametrize("pair", [
    ("decode 128 then 50 tokens (pieces added in the launch)", lambda: (li.sweep_case(128), li.sweep_case(50))),
    ("3000 then 1500 one-token segments (tile list in the array)", lambda: (
        li.make_sgmv("ones3000", seed=47, T=3000, K=256, S=1, R=16, L=8, slice_offsets=[0, 16],
                     dtype="bf16", lengths="ones"),
        li.make_sgmv("ones1500", seed=48, T=1500, K=256, S=1, R=16, L=8, slice_offsets=[0, 16],
                     dtype="bf16", lengths="ones"))),
    ("irregular fp16 then decode 50", lambda: (li.config_irregular(), li.sweep_case(50))),
])
def test_noalloc_matches_the_workspace_entry_point(pair):
    name, make = pair
    print("case", name, flush=True)
    for c in make():
        d = to_dev(c)
        ref = _call(c, d, noalloc=False)
        got = _call(c, d, noalloc=True)
        assert torch.equal(got, ref), c.name
        check_h(c, got)


def test_noalloc_refuses_problems_beyond_its_scratch():
    # 2^20 one-token segments need a 32 MiB tile list: more than the 16 MiB array
    assert _lib.lora_shrink_noalloc_max_workspace() == 16 << 20
    L = _lib.lib()
    st = L.lora_shrink_noalloc(1, 1 << 20, 256, 1, 16, 8, 1 << 20, 1, 256, 1, 256, 1, 1, 1, 1, 1,
                               16, None)
    assert st == _lib.LORA_EWORKSPACE
