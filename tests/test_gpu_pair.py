"""GPU parity of lora_shrink_expand (shrink then expand in one call; one launch at decode sizes).

Through the C ABI (ctypes binding):
- h and y equal those of lora_shrink followed by lora_expand bit for bit, on the single-launch
  path (bf16 and fp16, rank-0 and odd-rank adapters, empty segments, the identity permutation, y
  rows and slice starts off the 16-byte grid, K not a multiple of the MFMA step, padded rank 32,
  one token) and on sizes that take the two-launch path (one workgroup per tile at 1000 and 1024
  tokens, fp32, rows off the 16-byte grid);
- y against the oracle's whole chain from x (nothing computed on the GPU is fed to the oracle);
- one workspace reused across calls of different sizes and across graph replays, with the
  counters left zero and the wait-bound flag never set.
"""

from __future__ import annotations

import pytest
import torch

import lora_inputs as li
import oracle
from tests.parity import assert_close_lowp, check_h, to_dev

pytestmark = pytest.mark.gpu

FLAG = 32764  # LORA_SHRINK_EXPAND_FLAG_OFFSET


def _alp():
    import adapter_lora_projection_amd as alp

    return alp


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _separate(c, d, y0):
    alp = _alp()
    h = alp.shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                   d["lora_ranks"], c.S, c.R)
    y = y0.clone()
    alp.expand(h, d["B"], d["slice_offsets"], d["seg_indptr"], d["weight_indices"],
               d["permutation"], d["lora_ranks"], d["scalings"], y, c.S, c.R)
    return h, y


def _pair(c, d, y0, ws=None, h=None):
    alp = _alp()
    y = y0.clone()
    h, _ = alp.shrink_expand(d["x"], d["A"], d["B"], d["slice_offsets"], d["seg_indptr"],
                             d["weight_indices"], d["permutation"], d["lora_ranks"],
                             d["scalings"], y, c.S, c.R, h=h, workspace=ws)
    return h, y


def _case(kind: str):
    if kind.startswith("sweep"):
        return li.sweep_case(int(kind[5:]))
    if kind == "direct1000":  # one workgroup per tile (no split): the two launches
        return li.sweep_case(1000)
    if kind == "f16":
        return li.make_sgmv("pair_f16", seed=21, T=200, K=4096, S=3, R=16, L=4,
                            slice_offsets=[0, 4096, 5120, 6144], dtype="f16")
    if kind == "ranks":  # rank-0 and odd-rank adapters, more segments than adapters
        return li.make_sgmv("pair_ranks", seed=22, T=300, K=2048, S=3, R=16, L=4,
                            slice_offsets=[0, 2048, 2560, 3072], dtype="bf16",
                            ranks=[16, 0, 7, 13], fixed_indptr=[0, 40, 40, 97, 150, 150, 211, 300],
                            fixed_weight_indices=[0, 1, 2, 3, 1, 0, 2])
    if kind == "identity":
        return li.make_sgmv("pair_identity", seed=23, T=77, K=1024, S=3, R=16, L=3,
                            slice_offsets=[0, 1024, 1280, 1536], dtype="bf16", identity_perm=True)
    if kind == "offsets":  # slice starts off the 8- and 16-byte grid
        return li.make_sgmv("pair_offsets", seed=24, T=150, K=4096, S=3, R=16, L=4,
                            slice_offsets=[0, 4096, 5117, 6138], dtype="bf16")
    if kind == "kpartial":  # K % 32 != 0 (partial last MFMA step)
        return li.make_sgmv("pair_kpartial", seed=25, T=90, K=4040, S=3, R=16, L=4,
                            slice_offsets=[0, 4096, 5120, 6144], dtype="bf16")
    if kind == "rank32":
        return li.make_sgmv("pair_rank32", seed=26, T=64, K=2048, S=3, R=32, L=2,
                            slice_offsets=[0, 2048, 2560, 3072], dtype="bf16", ranks=[32, 19])
    if kind == "allrank0":  # every adapter of rank 0: no pieces, no waits, y untouched
        return li.make_sgmv("pair_rank0", seed=28, T=100, K=1024, S=3, R=16, L=3,
                            slice_offsets=[0, 1024, 1280, 1536], dtype="bf16", ranks=[0, 0, 0])
    if kind == "manysegs":  # 30 segments (a run of empty ones) over 300 tokens, split shrink
        import numpy as np

        rng = np.random.default_rng(29)
        cuts = np.sort(rng.integers(0, 301, size=29))
        cuts[5:12] = cuts[5]  # a run of empty segments
        indptr = [0] + [int(v) for v in cuts] + [300]
        return li.make_sgmv("pair_manysegs", seed=29, T=300, K=1024, S=3, R=16, L=8,
                            slice_offsets=[0, 1024, 1280, 1536], dtype="bf16",
                            ranks=[16, 9, 0, 16, 5, 16, 12, 16], fixed_indptr=indptr,
                            fixed_weight_indices=[int(v) for v in rng.integers(0, 8, size=30)])
    if kind == "onetoken":
        return li.make_sgmv("pair_onetoken", seed=30, T=1, K=4096, S=3, R=16, L=2,
                            slice_offsets=[0, 4096, 5120, 6144], dtype="bf16")
    # sizes that take the two launches
    if kind == "two_T1024":
        return li.sweep_case(1024)
    if kind == "two_f32":
        return li.config_tiny_f32()
    if kind == "two_irregular":  # K = 4093: rows off the 16-byte grid
        return li.make_sgmv("pair_irr", seed=27, T=300, K=4093, S=3, R=64, L=8,
                            slice_offsets=[0, 4096, 5117, 6138], dtype="f16", lengths="zipf",
                            ranks=[4, 7, 16, 33, 64, 4, 7, 16])
    raise ValueError(kind)


KINDS = ["sweep50", "sweep128", "sweep256", "sweep512", "direct1000", "f16", "ranks", "identity",
         "offsets", "kpartial", "rank32", "allrank0", "manysegs", "onetoken", "two_T1024",
         "two_f32", "two_irregular"]


@pytest.mark.parametrize("kind", KINDS)
def test_pair_equals_separate_calls(kind):
    c = _case(kind)
    print("case", kind, c.name, flush=True)
    d = to_dev(c)
    y0 = d["y_in"]
    if kind == "identity":
        d["permutation"] = None
    if kind == "offsets":  # y rows of 6141 elements: off the 16-byte grid
        wide = torch.randn(c.T, 6141, device="cuda").to(y0.dtype)
        wide[:, :y0.shape[1]] = y0
        y0 = wide
    h_ref, y_ref = _separate(c, d, y0)
    h, y = _pair(c, d, y0)
    torch.cuda.synchronize()
    assert torch.equal(_bits(h), _bits(h_ref)), "h differs from lora_shrink"
    assert torch.equal(_bits(y), _bits(y_ref)), "y differs from lora_shrink + lora_expand"
    if kind == "allrank0":
        assert torch.equal(_bits(y), _bits(y0)) and int(h.count_nonzero()) == 0


@pytest.mark.parametrize("kind", ["sweep50", "sweep512", "ranks", "direct1000", "manysegs"])
def test_pair_chain_from_x(kind):
    """h against the oracle's shrink and y against the oracle's whole chain from x."""
    c = _case(kind)
    print("case", kind, c.name, "chain", flush=True)
    d = to_dev(c)
    h, y = _pair(c, d, d["y_in"])
    torch.cuda.synchronize()
    check_h(c, h.cpu())
    h_ref = oracle.shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                          c.S, c.R, c.dtype)
    y_ref = oracle.expand(h_ref, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices,
                          c.permutation, c.lora_ranks, c.scalings, c.y_in, c.R, c.dtype)
    assert_close_lowp(y.cpu(), y_ref, f"pair chain {c.name}")


def _ws_for(cases):
    from adapter_lora_projection_amd import _lib

    n = max(_lib.lora_shrink_expand_workspace_size(_lib.LORA_BF16, c.T, c.K, c.S, c.R, c.G,
                                                   int(c.slice_offsets[-1])) for c in cases)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def test_pair_workspace_reuse():
    """One workspace across calls of different sizes (single launches and, at 1000 tokens, the two
    launches): every call equals the separate calls bit for bit, the flag stays 0 and the counters
    end zero."""
    cases = [li.sweep_case(t) for t in (128, 50, 512, 1000, 256, 128)]
    ws = _ws_for(cases)
    for c in cases:
        print("case reuse", c.name, flush=True)
        d = to_dev(c)
        h_ref, y_ref = _separate(c, d, d["y_in"])
        # h starts as NaN: an expand wave that did not wait for its tile would read it
        hn = torch.full((c.T, c.S * c.R), float("nan"), dtype=torch.bfloat16, device="cuda")
        h, y = _pair(c, d, d["y_in"], ws=ws, h=hn)
        torch.cuda.synchronize()
        assert torch.equal(_bits(h), _bits(h_ref)) and torch.equal(_bits(y), _bits(y_ref)), c.name
        assert int(ws[FLAG:FLAG + 4].view(torch.int32)[0]) == 0
        assert int(ws[:FLAG].count_nonzero()) == 0


def test_pair_graph_replay():
    """The call captured in a HIP graph: every replay (eager work and synchronisations between
    them) equals the eager result bit for bit."""
    c = li.sweep_case(256)
    d = to_dev(c)
    ws = _ws_for([c])
    h = torch.empty((c.T, c.S * c.R), dtype=torch.bfloat16, device="cuda")
    y = d["y_in"].clone()

    def run():
        _alp().shrink_expand(d["x"], d["A"], d["B"], d["slice_offsets"], d["seg_indptr"],
                             d["weight_indices"], d["permutation"], d["lora_ranks"],
                             d["scalings"], y, c.S, c.R, h=h, workspace=ws)

    run()
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), y.clone()
    h_sep, y_sep = _separate(c, d, d["y_in"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(h_ref), _bits(h_sep)) and torch.equal(_bits(y_ref), _bits(y_sep))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    y.copy_(d["y_in"])
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        run()
    for rep in range(4):
        y.copy_(d["y_in"])
        h.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(h), _bits(h_ref)) and torch.equal(_bits(y), _bits(y_ref)), rep
        assert int(ws[FLAG:FLAG + 4].view(torch.int32)[0]) == 0
        del junk


def test_pair_no_op_and_errors():
    from adapter_lora_projection_amd import _lib

    c = li.sweep_case(50)
    d = to_dev(c)
    # T = 0 and G = 0 are no-ops that need no workspace
    st = _lib.lib().lora_shrink_expand(_lib.LORA_BF16, 0, c.K, c.S, c.R, c.L, c.G, 6144, None,
                                       c.K, None, c.K, None, c.R, None, None, None, None, None,
                                       None, None, c.S * c.R, None, 6144, None, 0, None)
    assert st == 0
    # a short workspace is refused before anything is launched
    n = _lib.lora_shrink_expand_workspace_size(_lib.LORA_BF16, c.T, c.K, c.S, c.R, c.G, 6144)
    assert n >= 32768
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    h = torch.empty((c.T, c.S * c.R), dtype=torch.bfloat16, device="cuda")
    y = d["y_in"].clone()
    args = (_lib.LORA_BF16, c.T, c.K, c.S, c.R, c.L, c.G, 6144, d["x"], c.K, d["A"], c.K, d["B"],
            c.R, d["slice_offsets"], d["seg_indptr"], d["weight_indices"], d["permutation"],
            d["lora_ranks"], d["scalings"], h, c.S * c.R, y, 6144)
    stream = torch.cuda.current_stream().cuda_stream
    with pytest.raises(_lib.LoraError):
        _lib.lora_shrink_expand(*args, ws, n - 256, stream)
    with pytest.raises(_lib.LoraError):
        _lib.lora_shrink_expand(*args, None, 0, stream)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(d["y_in"]))  # nothing ran
    _lib.lora_shrink_expand(*args, ws, n, stream)
    torch.cuda.synchronize()
    h_ref, y_ref = _separate(c, d, d["y_in"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(h), _bits(h_ref)) and torch.equal(_bits(y), _bits(y_ref))
