"""Host-side argument checks of the tensor wrappers (CPU only). Every case carries exactly one
wrong argument that the wrapper must reject with ValueError before anything reaches the
library; the device check is bypassed so that CPU tensors can stand in for device ones."""

import pytest
import torch

from adapter_lora_projection_amd import ops

bf = torch.bfloat16


@pytest.fixture
def no_device_check(monkeypatch):
    monkeypatch.setattr(ops, "_dev", lambda *ts: None)


def _mlp(M=8, H=32, I=64, r=4, xdtype=bf):
    z = lambda *s: torch.zeros(*s, dtype=bf)
    return dict(x=torch.zeros(M, H, dtype=xdtype), w_gate=z(I, H), w_up=z(I, H), w_down=z(H, I),
                a_gate=z(r, H), b_gate=z(I, r), a_up=z(r, H), b_up=z(I, r), a_down=z(r, I),
                b_down=z(H, r))


def test_cpu_tensors_are_refused():
    with pytest.raises(ValueError, match="GPU"):
        ops.mlp_fused(**_mlp(), scale=2.0)


@pytest.mark.parametrize("out", [torch.zeros(7, 32, dtype=bf),        # too few rows
                                 torch.zeros(8, 16, dtype=bf),        # too few columns
                                 torch.zeros(8, 32, dtype=torch.float32)])
def test_mlp_fused_output_checked(no_device_check, out):
    with pytest.raises(ValueError, match="out"):
        ops.mlp_fused(**_mlp(), scale=2.0, out=out)


@pytest.mark.parametrize("fn", ["mlp_fused", "mlp_fused_train"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_mlp_x_must_be_bf16(no_device_check, fn, dtype):
    with pytest.raises(ValueError, match="bf16"):
        getattr(ops, fn)(**_mlp(xdtype=dtype), scale=2.0)


def test_mlp_weight_shape_checked(no_device_check):
    args = _mlp()
    args["b_down"] = torch.zeros(31, 4, dtype=bf)
    with pytest.raises(ValueError, match="b_down"):
        ops.mlp_fused(**args, scale=2.0)


def test_mlp_backward_checks(no_device_check):
    M, H, I, r = 8, 32, 64, 4
    z = lambda *s: torch.zeros(*s, dtype=bf)
    good = dict(x=z(M, H), e=z(M, I), v=z(M, I), dout=z(M, H), w_gu_t=z(H, 2 * I), w_down_t=z(I, H),
                a_gate=z(r, H), b_gate=z(I, r), a_up=z(r, H), b_up=z(I, r), a_down=z(r, I),
                b_down=z(H, r))
    for name, bad in (("x", torch.zeros(M, H)), ("e", z(M, I - 1)), ("dout", z(M + 1, H)),
                      ("w_gu_t", z(H, I))):
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError):
            ops.mlp_backward(**args, scale=2.0)


@pytest.mark.parametrize("out", [torch.zeros(5, 48, dtype=bf), torch.zeros(6, 48, dtype=torch.float16)])
def test_linear_output_checked(no_device_check, out):
    with pytest.raises(ValueError, match="out"):
        ops.linear_fused(torch.zeros(6, 32, dtype=bf), torch.zeros(48, 32, dtype=bf),
                         torch.zeros(4, 32, dtype=bf), torch.zeros(48, 4, dtype=bf), 2.0, out=out)


@pytest.mark.parametrize("fn", ["linear", "qkv"])
def test_linear_x_must_be_bf16(no_device_check, fn):
    x = torch.zeros(6, 32, dtype=torch.float32)
    w, a, b = torch.zeros(48, 32, dtype=bf), torch.zeros(4, 32, dtype=bf), torch.zeros(48, 4, dtype=bf)
    with pytest.raises(ValueError, match="bf16"):
        if fn == "linear":
            ops.linear_fused(x, w, a, b, 2.0)
        else:
            ops.qkv_fused(x, w, w, w, a, b, a, b, a, b, 2.0)


def _sgmv_meta(T=10, G=2, L=3):
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32)
    return dict(seg_indptr=i32(0, 4, T), weight_indices=i32(0, 2), permutation=torch.arange(T, dtype=torch.int32),
                lora_ranks=i32(*([4] * L)))


@pytest.mark.parametrize("h", [torch.zeros(9, 6, dtype=bf),           # too few rows
                               torch.zeros(10, 5, dtype=bf),          # too few columns
                               torch.zeros(10, 6, dtype=torch.float16)])
def test_shrink_output_checked(no_device_check, h):
    m = _sgmv_meta()
    x = torch.zeros(10, 64, dtype=bf)
    w_a = torch.zeros(3, 6, 64, dtype=bf)  # S = 3 slices of R = 2
    with pytest.raises(ValueError, match="h"):
        ops.shrink(x, w_a, m["seg_indptr"], m["weight_indices"], m["permutation"], m["lora_ranks"],
                   S=3, R=2, h=h)


@pytest.mark.parametrize("h", [torch.zeros(9, 8, dtype=bf), torch.zeros(10, 8, dtype=torch.float32)])
def test_embedding_output_checked(no_device_check, h):
    m = _sgmv_meta()
    ids = torch.zeros(10, dtype=torch.int32)
    w_a = torch.zeros(3, 8, 100, dtype=bf)
    with pytest.raises(ValueError, match="h"):
        ops.embedding_a(ids, w_a, m["seg_indptr"], m["weight_indices"], m["permutation"],
                        m["lora_ranks"], h=h)


def test_expand_shapes_checked(no_device_check):
    m = _sgmv_meta()
    h = torch.zeros(10, 6, dtype=bf)
    w_b = torch.zeros(3, 48, 2, dtype=bf)
    sl = torch.tensor([0, 16, 32, 48], dtype=torch.int32)
    sc = torch.ones(3, dtype=torch.float32)
    with pytest.raises(ValueError, match="y"):
        ops.expand(h, w_b, sl, m["seg_indptr"], m["weight_indices"], m["permutation"],
                   m["lora_ranks"], sc, torch.zeros(9, 48, dtype=bf), S=3, R=2)
    with pytest.raises(ValueError, match="scalings"):
        ops.expand(h, w_b, sl, m["seg_indptr"], m["weight_indices"], m["permutation"],
                   m["lora_ranks"], sc[:2], torch.zeros(10, 48, dtype=bf), S=3, R=2)


def test_linear_backward_checks(no_device_check):
    z = lambda *s: torch.zeros(*s, dtype=bf)
    good = dict(x=z(8, 64), dout=z(8, 32), w_t=z(64, 32), a=z(4, 64), b=z(32, 4))
    for name, bad in (("w_t", z(32, 64)), ("a", z(4, 32)), ("dout", z(8, 16)),
                      ("x", torch.zeros(8, 64, dtype=torch.float32))):
        kw = dict(good, **{name: bad})
        with pytest.raises(ValueError):
            ops.linear_backward(**kw, scale=2.0)
    with pytest.raises(ValueError, match="w"):
        ops.linear_prepare_backward(torch.zeros(32, 64, dtype=torch.float16))


def test_qkv_backward_checks(no_device_check):
    z = lambda *s: torch.zeros(*s, dtype=bf)
    good = dict(x=z(8, 64), dq=z(8, 64), dk=z(8, 32), dv=z(8, 32), w_qkv_t=z(64, 128), a_q=z(4, 64),
                b_q=z(64, 4), a_k=z(4, 64), b_k=z(32, 4), a_v=z(4, 64), b_v=z(32, 4))
    for name, bad in (("w_qkv_t", z(64, 96)), ("dv", z(8, 64)), ("a_v", z(4, 32)),
                      ("x", torch.zeros(8, 64, dtype=torch.float16))):
        kw = dict(good, **{name: bad})
        with pytest.raises(ValueError):
            ops.qkv_backward(**kw, scale=2.0)


def test_shrink_expand_checks(no_device_check):
    z = lambda *s: torch.zeros(*s, dtype=bf)
    i32 = lambda *v: torch.tensor(v, dtype=torch.int32)
    good = dict(x=z(10, 64), w_a=z(2, 48, 64), w_b=z(2, 96, 16), slice_offsets=i32(0, 32, 64, 96),
                seg_indptr=i32(0, 4, 10), weight_indices=i32(0, 1), permutation=None,
                lora_ranks=i32(16, 8), scalings=torch.ones(2), y=z(10, 96))
    for name, bad in (("w_a", z(2, 32, 64)), ("w_b", z(2, 96, 8)), ("y", z(9, 96)),
                      ("scalings", torch.ones(2, dtype=torch.float64)), ("seg_indptr", i32(0, 10))):
        kw = dict(good, **{name: bad})
        with pytest.raises((ValueError, TypeError)):
            ops.shrink_expand(**kw, S=3, R=16)
    with pytest.raises(ValueError, match="h"):
        ops.shrink_expand(**good, S=3, R=16, h=z(10, 40))
