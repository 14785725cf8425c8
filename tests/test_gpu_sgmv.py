"""GPU parity of lora_shrink / lora_expand / lora_schedule_tiles against the CPU oracle.

Every call goes through the C ABI (ctypes binding). Cases: the four SGMV workloads at full size
(every output element compared), small cases spanning several tiles with ragged tails, the token
sweep, every kernel shape, and the edge cases: empty segments, 16,384 one-token segments, rank-0
and odd-rank adapters, NaN in rank padding and in row-stride gaps, misaligned base pointers and
strides, B = 0, T = 0 / G = 0, permutation covariance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import lora_inputs as li
from adapter_lora_projection_amd import _lib
import oracle
from tests.parity import assert_close_lowp, check_h, check_y, f64, to_dev

pytestmark = pytest.mark.gpu


def _alp():
    import adapter_lora_projection_amd as alp

    return alp


def _plan(variant=(None, None), ksplit=None, lds=None, bn=None, finish=None):
    from adapter_lora_projection_amd import _lib

    v = lambda q: -1 if q is None else q
    return _lib.Plan(shrink_kernel=v(lds), shrink_shape=v(variant[0]), shrink_split=v(ksplit),
                     shrink_finish=v(finish), expand_shape=v(variant[1]), expand_block_n=v(bn))


def _run_pair(c, d=None, variant=(None, None), ksplit=None, lds=None, bn=None, finish=None):
    alp = _alp()
    d = d or to_dev(c)
    plan = _plan(variant, ksplit, lds, bn, finish)
    h = alp.shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                   d["lora_ranks"], c.S, c.R, plan=plan)
    y = d["y_in"].clone()
    alp.expand(h, d["B"], d["slice_offsets"], d["seg_indptr"], d["weight_indices"],
               d["permutation"], d["lora_ranks"], d["scalings"], y, c.S, c.R, plan=plan)
    torch.cuda.synchronize()
    return h.cpu(), y.cpu()


def _check_pair(c, h, y):
    check_h(c, h)
    # expand is checked on the GPU's own h (its input), so the two checks are independent
    check_y(c, h, y)


# ------------------------------------------------------------------ the workloads at full size

def test_tiny_f32():
    c = li.config_tiny_f32()
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


def test_decode_qkv_bf16():
    c = li.config_decode_qkv()
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


@pytest.mark.parametrize("part", [0, 1])
def test_prefill_bf16(part):
    c = li.config_prefill()[part]
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


def test_irregular_f16():
    c = li.config_irregular()
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


@pytest.mark.parametrize("T", li.SWEEP_TOKENS)
def test_sweep(T):
    c = li.sweep_case(T)
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


# ------------------------------------------------------------------ every kernel shape

@pytest.mark.parametrize("direct", [False, True])
@pytest.mark.parametrize("sv", range(5))
@pytest.mark.parametrize("ev", range(10))  # every expand kernel shape
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_variants_small(sv, ev, dtype, direct):
    """Several tiles per segment plus ragged tails, odd ranks, K tail, unaligned slices; every
    shrink shape both with the shared (tile, step) work and with one workgroup per tile."""
    c = li.make_sgmv(f"var_{dtype}", seed=40, T=301, K=517, S=3, R=32, L=5,
                     slice_offsets=[0, 130, 131, 333], dtype=dtype, ranks=[32, 7, 1, 0, 17])
    print("case", c.name, sv, ev, direct, flush=True)
    h, y = _run_pair(c, variant=(sv, ev), ksplit=0 if direct else None)
    _check_pair(c, h, y)


@pytest.mark.parametrize("R", [32, 16])
@pytest.mark.parametrize("ev", [5, 6, 7])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("offs", [[0, 128, 256, 520], [0, 132, 264, 520], [0, 1024, 1032, 2064]])
def test_wide_expand_shapes(ev, dtype, offs, R):
    """The 128-column chunks with 16-byte y pieces (16-byte aligned y rows): slices starting on a
    16-byte boundary take them, others (132, 264 elements) the 8-byte form in the same launch;
    tail chunks of 8 and fewer than 8 columns; padded rank 32 (16x16x32 MFMA) and 16 (16x16x16
    MFMA, 4 ranks per lane); adapter ranks 0, 1, 7 and 12..32, NaN in the padding."""
    c = li.make_sgmv(f"wide_{dtype}_R{R}", seed=44, T=157, K=256, S=3, R=R, L=5,
                     slice_offsets=offs, dtype=dtype, ranks=[R, 7, 1, 0, min(17, R) - (R == 16) * 5])
    for a in range(c.L):  # rank padding of A and B holds NaN: it must never be read
        r = int(c.lora_ranks[a])
        c.A.view(c.L, c.S, c.R, c.K)[a, :, r:, :] = float("nan")
        c.B[a, :, r:] = float("nan")
    print("case", c.name, ev, offs, flush=True)
    h, y = _run_pair(c, variant=(0, ev))
    _check_pair(c, h, y)


@pytest.mark.parametrize("null_perm", [False, True])
@pytest.mark.parametrize("bn", [None, 128, 256])
@pytest.mark.parametrize("ev", [8, 9])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("offs", [[0, 128, 256, 520], [0, 132, 264, 520], [0, 1024, 1032, 2064]])
def test_shared_b_expand(ev, dtype, offs, bn, null_perm):
    """The rank-16 expand with B chunks shared through LDS (64-token tiles, 16 per wave), one or
    two y chunks in flight: segments of 0, 5, 17, 37, 49, 64, 130 and 200 tokens, so tiles of
    64 positions end inside a wave's 16 or leave whole waves idle; adapter ranks 16, 12, 7, 1
    and 0 with NaN in the rank padding; slices on and off the 16-byte grid (the latter run the
    8-byte form per wave); column blocks of one and two chunks and whole slices; tail chunks
    of 8 columns; random permutation or NULL (identity)."""
    lens = [37, 0, 5, 130, 64, 17, 200, 49]
    indptr = np.concatenate(([0], np.cumsum(lens)))
    c = li.make_sgmv(f"sharedb_{dtype}", seed=46, T=int(indptr[-1]), K=256, S=3, R=16, L=5,
                     slice_offsets=offs, dtype=dtype, ranks=[16, 7, 1, 0, 12],
                     fixed_indptr=indptr, fixed_weight_indices=[0, 1, 2, 3, 4, 0, 4, 1],
                     identity_perm=null_perm)
    for a in range(c.L):
        r = int(c.lora_ranks[a])
        c.A.view(c.L, c.S, c.R, c.K)[a, :, r:, :] = float("nan")
        c.B[a, :, r:] = float("nan")
    d = to_dev(c)
    if null_perm:
        d["permutation"] = None
    print("case", c.name, ev, offs, bn, null_perm, flush=True)
    h, y = _run_pair(c, d=d, variant=(0, ev), bn=bn)
    _check_pair(c, h, y)


@pytest.mark.parametrize("finish", [0, 1])
@pytest.mark.parametrize("wgs", [0, 1, 7, 64, 1000])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_shared_work_split(wgs, dtype, finish):
    """The (tile, K step) work shared over `wgs` workgroups (0 = one per tile): a single
    workgroup walking every tile, ranges that start and end inside tiles, and one step per
    workgroup (up to 18 pieces per tile), the pieces summed by a second launch (finish 0) or by
    each tile's last workgroup in the same launch (finish 1, arrival counters)."""
    c = li.make_sgmv(f"sk_{dtype}", seed=43, T=203, K=517, S=3, R=32, L=5,
                     slice_offsets=[0, 130, 131, 333], dtype=dtype, ranks=[32, 7, 1, 0, 17])
    print("case", c.name, wgs, finish, flush=True)
    h, y = _run_pair(c, ksplit=wgs, finish=finish)
    _check_pair(c, h, y)


@pytest.mark.parametrize("finish", [0, 1])
@pytest.mark.parametrize("wgs", [0, 5, 300])
@pytest.mark.parametrize("sv", range(_lib.LORA_SHRINK_LDS_SHAPES))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_lds_shrink_shapes(sv, wgs, dtype, finish):
    """The LDS-staged shrink in every shape (2..12 column blocks per workgroup, so the 6 blocks
    here are split over 3, 2, 2, 1 and 1 workgroups; tiles of 128, 64, 48 or 32 positions; 3 to 6
    stages; 2 to 4 waves), one workgroup per tile or the work shared over 5 or 300 workgroups
    (pieces added by a second launch or in the same launch); K = 1032 ends in a stage with one
    valid 8-element chunk; ragged tile ends; rank 0, 1, 7, 17 and 32 adapters."""
    c = li.make_sgmv(f"lds_{dtype}", seed=44, T=301, K=1032, S=3, R=32, L=5,
                     slice_offsets=[0, 130, 131, 333], dtype=dtype, ranks=[32, 7, 1, 0, 17])
    print("case", c.name, sv, wgs, finish, flush=True)
    h, y = _run_pair(c, variant=(sv, None), ksplit=wgs, lds=1, finish=finish)
    _check_pair(c, h, y)


@pytest.mark.parametrize("case", ["var", "decode50", "decode1024", "ones"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gemv_shrink(case, dtype):
    """The wave-reduction (GEMV) shrink: tiles of up to 16 positions with ragged ends, odd ranks
    and rank 0 with NaN in the rank padding, unaligned slices, 16,384-segment schedule, K with a
    partial 512-element sweep (K = 520), and the decode workloads."""
    if case == "var":
        c = li.make_sgmv(f"gemv_{dtype}", seed=49, T=301, K=520, S=3, R=32, L=5,
                         slice_offsets=[0, 130, 131, 333], dtype=dtype, ranks=[32, 7, 1, 0, 17])
        for a in range(c.L):
            c.A.view(c.L, c.S, c.R, c.K)[a, :, int(c.lora_ranks[a]):, :] = float("nan")
    elif case == "ones":
        c = li.make_sgmv(f"gemv_ones_{dtype}", seed=50, T=3000, K=256, S=1, R=16, L=8,
                         slice_offsets=[0, 16], dtype=dtype, lengths="ones")
    else:
        c = li.sweep_case(50 if case == "decode50" else 1024)
        if dtype == "f16":
            c = li.make_sgmv(f"gemv_dec_{dtype}", seed=1, T=c.T, K=4096, S=3, R=16, L=4,
                             slice_offsets=[0, 4096, 5120, 6144], dtype=dtype)
    print("case", c.name, "gemv", flush=True)
    h, y = _run_pair(c, lds=2)
    _check_pair(c, h, y)


@pytest.mark.parametrize("wgs", [16, 96, 256, 512, 2048])
@pytest.mark.parametrize("sv", range(5))
@pytest.mark.parametrize("T", [50, 128, 1024])
def test_in_launch_split_decode_shapes(T, sv, wgs):
    """The decode-QKV workload (4 adapters r16, K = 4096, empty segments possible) with every
    register-ring shape and the work shared over 16 .. 2048 workgroups, pieces added in the
    same launch: up to 129 pieces per tile."""
    c = li.sweep_case(T)
    print("case", c.name, sv, wgs, flush=True)
    h, y = _run_pair(c, variant=(sv, None), ksplit=wgs, lds=0, finish=1)
    _check_pair(c, h, y)


def test_workspace_counters_left_zero_and_reused():
    """One workspace for many calls: its arrival counters are zero after every call, and
    repeated calls (also of other shapes) give bit-identical results."""
    alp = _alp()
    from adapter_lora_projection_amd import _lib

    cases = [li.sweep_case(50), li.sweep_case(1024), li.config_irregular()]
    nbytes = max(_lib.lora_shrink_workspace_size(li_dt(c), c.T, c.K, c.S, c.R, c.G) for c in cases)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    first = {}
    for rep in range(3):
        for c in cases:
            d = to_dev(c)
            h = alp.shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                           d["lora_ranks"], c.S, c.R, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:32768].count_nonzero()) == 0, (c.name, rep)
            if rep == 0:
                check_h(c, h.cpu())
                first[c.name] = h.cpu()
            else:
                assert torch.equal(h.cpu(), first[c.name]), (c.name, rep)


def li_dt(c):
    return {"f32": 0, "bf16": 1, "f16": 2}[c.dtype]


def test_graph_capture_replays():
    """shrink + expand captured in a HIP graph over one workspace: every replay (with eager work
    and synchronisations between them) equals the eager result bit for bit."""
    alp = _alp()
    from adapter_lora_projection_amd import _lib

    c = li.sweep_case(128)
    d = to_dev(c)
    nbytes = _lib.lora_shrink_workspace_size(li_dt(c), c.T, c.K, c.S, c.R, c.G)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    h = torch.empty((c.T, c.S * c.R), dtype=torch.bfloat16, device="cuda")
    y = d["y_in"].clone()

    def run():
        alp.shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], d["permutation"],
                   d["lora_ranks"], c.S, c.R, h=h, workspace=ws)
        alp.expand(h, d["B"], d["slice_offsets"], d["seg_indptr"], d["weight_indices"],
                   d["permutation"], d["lora_ranks"], d["scalings"], y, c.S, c.R)

    run()
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), y.clone()
    check_h(c, h_ref.cpu())
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
        assert torch.equal(h, h_ref) and torch.equal(y, y_ref), rep
        assert int(ws[:32768].count_nonzero()) == 0
        del junk


# ------------------------------------------------------------------ the whole chain from x

@pytest.mark.parametrize("which", ["decode", "prefill0", "prefill1", "irregular"])
def test_chain_from_x(which):
    """y from the GPU's shrink and expand compared with oracle.expand(oracle.shrink(x)), the
    oracle's own h: nothing computed on the GPU is fed to the oracle."""
    c = {"decode": li.config_decode_qkv, "irregular": li.config_irregular,
         "prefill0": lambda: li.config_prefill()[0], "prefill1": lambda: li.config_prefill()[1]}[which]()
    print("case", c.name, "chain", flush=True)
    _, y = _run_pair(c)
    h_ref = oracle.shrink(c.x, c.A, c.seg_indptr, c.weight_indices, c.permutation, c.lora_ranks,
                          c.S, c.R, c.dtype)
    y_ref = oracle.expand(h_ref, c.B, c.slice_offsets, c.seg_indptr, c.weight_indices,
                          c.permutation, c.lora_ranks, c.scalings, c.y_in, c.R, c.dtype)
    assert_close_lowp(y, y_ref, f"chain {c.name}")


@pytest.mark.parametrize("lds", [0, 1])
def test_shrink_families_agree_on_prefill(lds):
    """Both shrink kernel families on the prefill gate_up workload (8 column blocks, K = 4096)."""
    c = li.config_prefill()[0]
    print("case", c.name, lds, flush=True)
    h, y = _run_pair(c, lds=lds)
    _check_pair(c, h, y)


@pytest.mark.parametrize("lds", [0, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_identity_permutation_null(dtype, lds):
    """The non-chunked ops: permutation NULL means the identity. Checked against the oracle
    with an identity permutation (tokens already grouped by segment)."""
    c = li.make_sgmv(f"nochunk_{dtype}", seed=45, T=333, K=520, S=2, R=16, L=4,
                     slice_offsets=[0, 200, 264], dtype=dtype, identity_perm=True)
    assert torch.equal(c.permutation, torch.arange(c.T, dtype=torch.int32))
    d = to_dev(c)
    alp = _alp()
    plan = _plan(lds=lds)
    h = alp.shrink(d["x"], d["A"], d["seg_indptr"], d["weight_indices"], None,
                   d["lora_ranks"], c.S, c.R, plan=plan)
    y = d["y_in"].clone()
    alp.expand(h, d["B"], d["slice_offsets"], d["seg_indptr"], d["weight_indices"], None,
               d["lora_ranks"], d["scalings"], y, c.S, c.R, plan=plan)
    torch.cuda.synchronize()
    _check_pair(c, h.cpu(), y.cpu())


# ------------------------------------------------------------------ edge cases

def test_empty_and_zero_sizes():
    alp = _alp()
    c = li.make_sgmv("empties", seed=41, T=64, K=96, S=2, R=16, L=6, slice_offsets=[0, 40, 72],
                     dtype="bf16", fixed_indptr=[0, 0, 30, 30, 30, 64, 64],
                     fixed_weight_indices=[5, 0, 1, 2, 3, 4])
    h, y = _run_pair(c)
    _check_pair(c, h, y)
    # T == 0 and G == 0 are no-ops that touch nothing
    d = to_dev(c)
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    hh = torch.full((64, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    alp.shrink(d["x"][:0], d["A"], torch.zeros(1, dtype=torch.int32, device="cuda"), z, z,
               d["lora_ranks"], 2, 16, h=hh[:0])
    assert (hh == 7).all()


def test_one_token_segments_16384():
    """16,384 segments of one token each (the standalone scheduler path)."""
    T = 16384
    c = li.make_sgmv("ones", seed=42, T=T, K=256, S=3, R=16, L=8, slice_offsets=[0, 128, 160, 192],
                     dtype="bf16", lengths="ones")
    print("case", c.name, flush=True)
    h, y = _run_pair(c)
    _check_pair(c, h, y)


def test_nan_padding_and_stride_gaps_misaligned():
    """NaN in A rows / B columns beyond each rank and in the row-stride gaps of x, A, B, h and y
    must never reach an output; base pointers offset by one element exercise unaligned loads."""
    alp = _alp()
    c = li.make_sgmv("nanpad", seed=43, T=200, K=301, S=2, R=16, L=4, slice_offsets=[0, 77, 141],
                     dtype="f16", ranks=[16, 3, 9, 1])
    d = to_dev(c)
    nan = float("nan")
    T, K, S, R, L, N = c.T, c.K, c.S, c.R, c.L, c.N
    xb = torch.full((T, K + 13), nan, dtype=torch.float16, device="cuda")
    x = xb[:, 1:K + 1]
    x.copy_(d["x"])
    Ab = torch.full((L * S * R * (K + 7) + 1,), nan, dtype=torch.float16, device="cuda")
    A = Ab[1:].view(L, S * R, K + 7)[:, :, :K]
    A.copy_(d["A"])
    for a in range(L):
        r = c.lora_ranks[a].item()
        A.unflatten(1, (S, R))[a, :, r:, :] = nan
    Bb = torch.full((L * N * (R + 3) + 1,), nan, dtype=torch.float16, device="cuda")
    B = Bb[1:].view(L, N, R + 3)[:, :, :R]
    B.copy_(d["B"])
    for a in range(L):
        B[a, :, c.lora_ranks[a].item():] = nan
    hb = torch.full((T, S * R + 5), nan, dtype=torch.float16, device="cuda")
    h = hb[:, :S * R]
    alp.shrink(x, A, d["seg_indptr"], d["weight_indices"], d["permutation"], d["lora_ranks"], S, R, h=h)
    yb = torch.full((T, N + 9), nan, dtype=torch.float16, device="cuda")
    yb[:, 1:N + 1] = d["y_in"]
    y = yb[:, 1:N + 1]
    alp.expand(h, B, d["slice_offsets"], d["seg_indptr"], d["weight_indices"], d["permutation"],
               d["lora_ranks"], d["scalings"], y, S, R)
    torch.cuda.synchronize()
    hc, ybc = h.cpu(), yb.cpu()
    assert torch.isfinite(hc).all()
    assert torch.isnan(hb[:, S * R:]).all()
    check_h(c, hc)
    check_y(c, hc, ybc[:, 1:N + 1])
    assert torch.isnan(ybc[:, 0]).all() and torch.isnan(ybc[:, N + 1:]).all()


def test_b_zero_exact():
    c = li.make_sgmv("bzero", seed=44, T=333, K=128, S=3, R=16, L=4, slice_offsets=[0, 64, 96, 128],
                     dtype="bf16")
    c.B.zero_()
    h, y = _run_pair(c)
    assert torch.equal(y.float(), c.y_in.float())  # value compare: +0 == -0


def test_permutation_covariance_bitwise():
    """Relabelling tokens permutes y rows and leaves h unchanged, bitwise."""
    c = li.make_sgmv("cov", seed=45, T=500, K=256, S=3, R=16, L=4, slice_offsets=[0, 256, 320, 384],
                     dtype="bf16")
    h1, y1 = _run_pair(c)
    pi = torch.from_numpy(np.random.default_rng(5).permutation(c.T))
    c2 = li.make_sgmv("cov", seed=45, T=500, K=256, S=3, R=16, L=4, slice_offsets=[0, 256, 320, 384],
                      dtype="bf16")
    c2.x = torch.empty_like(c.x); c2.x[pi] = c.x
    c2.y_in = torch.empty_like(c.y_in); c2.y_in[pi] = c.y_in
    c2.permutation = pi[c.permutation.long()].to(torch.int32)
    h2, y2 = _run_pair(c2)
    assert torch.equal(h1, h2)
    assert torch.equal(y2[pi], y1)


def test_deterministic_repeat():
    c = li.config_irregular()
    d = to_dev(c)
    h1, y1 = _run_pair(c, d)
    h2, y2 = _run_pair(c, d)
    assert torch.equal(h1, h2) and torch.equal(y1, y2)


# ------------------------------------------------------------------ the schedule (bit-exact)

@pytest.mark.parametrize("method", [0, 1])
@pytest.mark.parametrize("BM", [1, 16, 64, 100])
def test_schedule_bit_exact(method, BM):
    alp = _alp()
    for c in (li.config_irregular(), li.config_decode_qkv(),
              li.make_sgmv("ones", seed=46, T=3000, K=8, S=1, R=16, L=8, slice_offsets=[0, 16],
                           dtype="bf16", lengths="ones")):
        got = alp.schedule_tiles(c.T, c.seg_indptr.cuda(), c.weight_indices.cuda(),
                                 c.lora_ranks.cuda(), BM, method).cpu().numpy()
        ref = oracle.tile_list(c.seg_indptr, c.weight_indices, c.lora_ranks, BM)
        assert np.array_equal(got, ref), (c.name, method, BM)
