"""The C-ABI library loads, exports every symbol the public headers declare, and rejects bad
arguments on the host (no GPU needed: only argument-error paths and size queries are called)."""

import ctypes
import glob
import os
import re

import pytest

from adapter_lora_projection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(hdr).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(lora_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = _declared()
    assert {"lora_shrink", "lora_expand", "lora_schedule_tiles"} <= names
    for n in names:
        assert hasattr(L, n), n
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)


def test_status_strings_and_version():
    assert _lib.status_str(0) == "LORA_OK"
    assert "EINVAL" in _lib.status_str(1)
    assert "unknown" in _lib.status_str(99)
    assert "gfx950" in _lib.lora_version()


def _shrink(**kw):
    args = dict(dtype=1, T=8, K=16, S=1, R=16, L=1, G=1, x=0x1000, ldx=16, w_a=0x2000, lda=16,
                seg_indptr=0x3000, weight_indices=0x4000, permutation=0x5000, lora_ranks=0x6000,
                h=0x7000, ldh=16, workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return _lib.lib().lora_shrink(*args.values())


def _expand(**kw):
    args = dict(dtype=1, T=8, S=1, R=16, L=1, G=1, N=32, h=0x1000, ldh=16, w_b=0x2000, ldb=16,
                slice_offsets=0x3000, seg_indptr=0x4000, weight_indices=0x5000, permutation=0x6000,
                lora_ranks=0x7000, scalings=0x8000, y=0x9000, ldy=32, workspace=None,
                workspace_bytes=0, stream=None)
    args.update(kw)
    return _lib.lib().lora_expand(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.LORA_EUNSUPPORTED),
    (dict(T=-1), _lib.LORA_EINVAL),
    (dict(S=0), _lib.LORA_EINVAL),
    (dict(R=0), _lib.LORA_EINVAL),
    (dict(R=2048), _lib.LORA_EUNSUPPORTED),
    (dict(K=0), _lib.LORA_EINVAL),
    (dict(x=None), _lib.LORA_EINVAL),
    (dict(h=None), _lib.LORA_EINVAL),
    (dict(ldx=15), _lib.LORA_EINVAL),
    (dict(lda=8), _lib.LORA_EINVAL),
    (dict(ldh=15), _lib.LORA_EINVAL),
    (dict(T=5000, G=5000), _lib.LORA_EWORKSPACE),
    (dict(T=0, x=None, h=None), _lib.LORA_OK),
    (dict(G=0, x=None), _lib.LORA_OK),
])
def test_shrink_host_validation(kw, code):
    assert _shrink(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=-1), _lib.LORA_EUNSUPPORTED),
    (dict(N=-1), _lib.LORA_EINVAL),
    (dict(scalings=None), _lib.LORA_EINVAL),
    (dict(slice_offsets=None), _lib.LORA_EINVAL),
    (dict(ldb=15), _lib.LORA_EINVAL),
    (dict(ldy=31), _lib.LORA_EINVAL),
    (dict(ldh=8), _lib.LORA_EINVAL),
    (dict(S=65), _lib.LORA_EUNSUPPORTED),
    (dict(T=5000, G=5000), _lib.LORA_EWORKSPACE),
    (dict(N=0, y=None), _lib.LORA_OK),
    (dict(T=0, h=None, y=None), _lib.LORA_OK),
])
def test_expand_host_validation(kw, code):
    assert _expand(**kw) == code


def test_workspace_sizes():
    assert _lib.lora_expand_workspace_size(1, 50, 3, 16, 4, 6144) == 0
    P = _lib.Plan
    # one workgroup per tile over all of K: nothing needed for few segments
    assert _lib.lora_shrink_workspace_size_ex(1, 50, 4096, 3, 16, 4, P(shrink_split=0)) == 0
    # shared work over 256 workgroups, register-ring shape 2 (16-token tiles, one 16-column block
    # per workgroup: 3 grid rows): 50 tokens give a bound of 4 + 4 segments = 8 tiles of 128
    # steps, 4 steps per workgroup, at most 127 // 4 + 2 = 33 pieces per tile, each an fp32 plane
    # of [T][S*R], after the 32 KiB counter region
    plan = P(shrink_kernel=0, shrink_shape=2, shrink_split=256)
    for dt in (1, 2):
        assert _lib.lora_shrink_workspace_size_ex(dt, 50, 4096, 3, 16, 4, plan) == 32768 + 33 * 50 * 48 * 4
    # a plan outside its ranges is refused
    assert _lib.lora_shrink_workspace_size_ex(1, 50, 4096, 3, 16, 4, P(shrink_shape=13)) == 0
    assert _lib.lora_shrink_workspace_size_ex(1, 50, 4096, 3, 16, 4, P(shrink_kernel=0, shrink_shape=5)) == 0
    assert _lib.lora_shrink_workspace_size_ex(1, 50, 4096, 3, 16, 4, P(shrink_finish=2)) == 0
    assert _lib.lora_shrink_workspace_size_ex(1, 50, 4096, 3, 16, 4, None) == \
        _lib.lora_shrink_workspace_size(1, 50, 4096, 3, 16, 4)
    assert _lib.lora_shrink_workspace_size(1, 50, 4096, 3, 16, 4) % 4 == 0
    n = _lib.lora_shrink_workspace_size(1, 16384, 256, 3, 16, 16384)
    assert n >= 32768 + 16 * 16384
    assert _lib.lora_shrink_workspace_size(1, 0, 256, 3, 16, 4) == 0


def test_queries_are_pure():
    """The same query gives the same answer whatever plans other calls used (no hidden state)."""
    a = _lib.lora_shrink_workspace_size(1, 300, 4096, 3, 16, 4)
    _lib.lora_shrink_workspace_size_ex(1, 300, 4096, 3, 16, 4, _lib.Plan(shrink_split=7))
    _lib.lora_shrink_workspace_size_ex(1, 300, 4096, 3, 16, 4, _lib.Plan(shrink_kernel=1))
    assert _lib.lora_shrink_workspace_size(1, 300, 4096, 3, 16, 4) == a


def test_schedule_host_validation():
    L = _lib.lib()
    assert L.lora_schedule_tiles(10, 2, 0, 0, 1, 1, 1, 1, 100, 1, None, 0, None) == _lib.LORA_EINVAL
    assert L.lora_schedule_tiles(10, 2, 4, 2, 1, 1, 1, 1, 100, 1, None, 0, None) == _lib.LORA_EINVAL
    assert L.lora_schedule_tiles(10, 2, 4, 0, 1, 1, 1, 1, 4, 1, None, 0, None) == _lib.LORA_EINVAL
    assert L.lora_schedule_tiles(10, 2, 4, 1, 1, 1, 1, 1, 100, 1, None, 0, None) == _lib.LORA_EWORKSPACE


def _mlp(**kw):
    args = dict(dtype=1, M=8, H=64, I=96, r=16, scale=2.0, x=0x1000, ldx=64, w_gate=0x2000, w_up=0x3000,
                w_down=0x4000, a_gate=0x5000, b_gate=0x6000, a_up=0x7000, b_up=0x8000, a_down=0x9000,
                b_down=0xA000, out=0xB000, ldo=64, workspace=0x100000, workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return _lib.lib().lora_mlp_fused(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), _lib.LORA_EUNSUPPORTED),
    (dict(dtype=2), _lib.LORA_EUNSUPPORTED),
    (dict(H=48, ldx=48, ldo=48), _lib.LORA_EUNSUPPORTED),
    (dict(I=100), _lib.LORA_EUNSUPPORTED),
    (dict(r=65), _lib.LORA_EUNSUPPORTED),
    (dict(r=0), _lib.LORA_EINVAL),
    (dict(M=-1), _lib.LORA_EINVAL),
    (dict(x=None), _lib.LORA_EINVAL),
    (dict(b_down=None), _lib.LORA_EINVAL),
    (dict(ldx=32), _lib.LORA_EINVAL),
    (dict(x=0x1002), _lib.LORA_EUNSUPPORTED),
    (dict(workspace=None), _lib.LORA_EWORKSPACE),
    (dict(workspace_bytes=1024), _lib.LORA_EWORKSPACE),
    (dict(M=0, x=None, out=None), _lib.LORA_OK),
])
def test_mlp_host_validation(kw, code):
    assert _mlp(**kw) == code


def test_mlp_workspace_size_covers_hmid():
    M, H, I = 4096, 4096, 12288
    n = _lib.lora_mlp_workspace_size(1, M, H, I, 16)
    assert n >= M * I * 2 and n < M * I * 2 + 64 * (1 << 20)


def _linear(**kw):
    args = dict(dtype=1, M=8, K=64, N=32, r=16, scale=2.0, x=0x1000, ldx=64, w=0x2000, a=0x3000,
                b=0x4000, out=0x5000, ldo=32, workspace=0x100000, workspace_bytes=1 << 30,
                stream=None)
    args.update(kw)
    return _lib.lib().lora_linear_fused(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), _lib.LORA_EUNSUPPORTED),
    (dict(K=48, ldx=48), _lib.LORA_EUNSUPPORTED),   # K % 32 != 0
    (dict(r=65), _lib.LORA_EUNSUPPORTED),
    (dict(r=0), _lib.LORA_EINVAL),
    (dict(N=0), _lib.LORA_EINVAL),
    (dict(x=None), _lib.LORA_EINVAL),
    (dict(b=None), _lib.LORA_EINVAL),
    (dict(ldx=32), _lib.LORA_EINVAL),
    (dict(ldo=31), _lib.LORA_EINVAL),
    (dict(x=0x1002), _lib.LORA_EUNSUPPORTED),       # unaligned rows
    (dict(workspace_bytes=16), _lib.LORA_EWORKSPACE),
    (dict(M=0, x=None), _lib.LORA_OK),
])
def test_linear_host_validation(kw, code):
    assert _linear(**kw) == code


def test_qkv_host_validation():
    # every call below is rejected on the host before anything is enqueued (the addresses are
    # placeholders, never dereferenced)
    L = _lib.lib()
    base = [1, 8, 64, 32, 16, 8, 2.0, 0x1000, 64, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000,
            0x8000, 0x9000, 0xA000, 0xB000, 32, 0xC000, 16, 0xD000, 16, 0x100000, 1 << 30, None]
    bad = list(base); bad[11] = None  # w_v
    assert L.lora_qkv_fused(*bad) == _lib.LORA_EINVAL
    bad = list(base); bad[23] = 15  # ldv < Nkv
    assert L.lora_qkv_fused(*bad) == _lib.LORA_EINVAL
    bad = list(base); bad[25] = 64  # workspace too small
    assert L.lora_qkv_fused(*bad) == _lib.LORA_EWORKSPACE
    assert _lib.lora_qkv_workspace_size(1, 8, 64, 32, 16, 8) > 0
    assert _lib.lora_linear_workspace_size(1, 0, 64, 32, 16) == 0


def _emb(**kw):
    args = dict(dtype=1, T=8, V=100, R=16, L=2, G=2, input_ids=0x1000, w_a=0x2000,
                stride_l=1600, stride_r=100, stride_v=1, seg_indptr=0x3000, weight_indices=0x4000, permutation=0x5000, lora_ranks=0x6000,
                h=0x7000, ldh=16, stream=None)
    args.update(kw)
    return _lib.lib().lora_embedding_a(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), _lib.LORA_EUNSUPPORTED),
    (dict(T=-1), _lib.LORA_EINVAL),
    (dict(R=0), _lib.LORA_EINVAL),
    (dict(R=2048), _lib.LORA_EUNSUPPORTED),
    (dict(V=0), _lib.LORA_EINVAL),
    (dict(L=0), _lib.LORA_EINVAL),
    (dict(input_ids=None), _lib.LORA_EINVAL),
    (dict(w_a=None), _lib.LORA_EINVAL),
    (dict(h=None), _lib.LORA_EINVAL),
    (dict(stride_l=-1), _lib.LORA_EINVAL),
    (dict(stride_r=0), _lib.LORA_EINVAL),
    (dict(stride_v=0), _lib.LORA_EINVAL),
    (dict(ldh=15), _lib.LORA_EINVAL),
    (dict(T=(1 << 31) - 100), _lib.LORA_EUNSUPPORTED),
])
def test_embedding_host_validation(kw, code):
    # rejected on the host before anything is enqueued (the addresses are placeholders)
    assert _emb(**kw) == code


def test_embedding_empty_calls_are_no_ops():
    # nothing to do: returns before touching any pointer
    assert _emb(T=0) == _lib.LORA_OK
    assert _emb(G=0) == _lib.LORA_OK


def _mlp_bwd(**kw):
    args = dict(dtype=1, M=8, H=64, I=96, r=16, scale=2.0, x=0x1000, ldx=64, e=0x2000, v=0x3000,
                lde=96, dout=0x4000, lddo=64, w_gu_t=0x5000, w_down_t=0x6000, a_gate=0x7000,
                b_gate=0x8000, a_up=0x9000, b_up=0xA000, a_down=0xB000, b_down=0xC000, dx=0xD000,
                lddx=64, da_gate=0xE000, db_gate=0xF000, da_up=0x10000, db_up=0x11000,
                da_down=0x12000, db_down=0x13000, workspace=0x100000, workspace_bytes=16,
                stream=None)
    args.update(kw)
    return _lib.lib().lora_mlp_backward(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), _lib.LORA_EUNSUPPORTED),
    (dict(dtype=2), _lib.LORA_EUNSUPPORTED),
    (dict(M=-1), _lib.LORA_EINVAL),
    (dict(r=0), _lib.LORA_EINVAL),
    (dict(r=65), _lib.LORA_EUNSUPPORTED),
    (dict(H=48, ldx=48, lddo=48, lddx=48), _lib.LORA_EUNSUPPORTED),
    (dict(I=100, lde=100), _lib.LORA_EUNSUPPORTED),
    (dict(e=None), _lib.LORA_EINVAL),
    (dict(db_down=None), _lib.LORA_EINVAL),
    (dict(w_gu_t=None), _lib.LORA_EINVAL),
    (dict(lde=95), _lib.LORA_EINVAL),
    (dict(lddo=32), _lib.LORA_EINVAL),
    (dict(dx=0x1000), _lib.LORA_EINVAL),             # dx would overwrite the saved x
    (dict(dx=0x4000), _lib.LORA_EINVAL),             # ... or dout
    (dict(x=0x1002), _lib.LORA_EUNSUPPORTED),        # unaligned rows
    (dict(e=0x2002), _lib.LORA_EUNSUPPORTED),
    (dict(lde=100), _lib.LORA_EUNSUPPORTED),         # 200-byte rows: not 16-byte aligned
    (dict(workspace=None), _lib.LORA_EWORKSPACE),
    (dict(workspace_bytes=16), _lib.LORA_EWORKSPACE),
])
def test_mlp_backward_host_validation(kw, code):
    # every call is rejected on the host before anything is enqueued (placeholder addresses)
    assert _mlp_bwd(**kw) == code


def test_mlp_backward_empty_and_workspace_size():
    assert _mlp_bwd(M=0) == _lib.LORA_OK
    n = _lib.lora_mlp_backward_workspace_size(1, 4096, 4096, 12288, 16)
    # at least hmid [M][I] and [de | dv] [M][2I] in bf16
    assert n >= 3 * 4096 * 12288 * 2
    assert _lib.lora_mlp_backward_workspace_size(1, 0, 64, 96, 16) == 0
    assert _lib.lora_mlp_backward_workspace_size(1, 8, 64, 96, 65) == 0


def test_mlp_train_and_prepare_host_validation():
    L = _lib.lib()
    base = [1, 8, 64, 96, 16, 2.0, 0x1000, 64, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000,
            0x8000, 0x9000, 0xA000, 0xB000, 64, 0xC000, 0xD000, 96, 0x100000, 16, None]
    bad = list(base); bad[19] = None  # e
    assert L.lora_mlp_fused_train(*bad) == _lib.LORA_EINVAL
    bad = list(base); bad[21] = 95  # lde < I
    assert L.lora_mlp_fused_train(*bad) == _lib.LORA_EINVAL
    bad = list(base); bad[23] = 16  # workspace too small
    assert L.lora_mlp_fused_train(*bad) == _lib.LORA_EWORKSPACE
    assert L.lora_mlp_prepare_backward(0, 64, 96, 0x1, 0x2, 0x3, 0x4, 0x5, None) == _lib.LORA_EUNSUPPORTED
    assert L.lora_mlp_prepare_backward(1, 0, 96, 0x1, 0x2, 0x3, 0x4, 0x5, None) == _lib.LORA_EINVAL
    assert L.lora_mlp_prepare_backward(1, 64, 96, 0x1, None, 0x3, 0x4, 0x5, None) == _lib.LORA_EINVAL


def test_check_metadata_host_validation():
    # rejected before anything is enqueued (placeholder addresses)
    L = _lib.lib()
    args = [8, 2, 2, 16, 1, 32, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None, 0x100000, 1 << 20, None]
    bad = list(args); bad[0] = -1
    assert L.lora_check_metadata(*bad) == _lib.LORA_EINVAL
    bad = list(args); bad[6] = None  # seg_indptr
    assert L.lora_check_metadata(*bad) == _lib.LORA_EINVAL
    bad = list(args); bad[7] = None  # weight_indices with G > 0
    assert L.lora_check_metadata(*bad) == _lib.LORA_EINVAL
    bad = list(args); bad[13] = 16  # workspace too small for T = 8
    assert L.lora_check_metadata(*bad) == _lib.LORA_EWORKSPACE
    bad = list(args); bad[12] = None
    assert L.lora_check_metadata(*bad) == _lib.LORA_EWORKSPACE
    assert _lib.lora_check_metadata_workspace_size(8) == 256 + 32


def test_shrink_expand_workspace_size():
    """lora_shrink_expand's workspace covers the two-launch path (the shrink's workspace, then the
    expand's) and always holds the 32 KiB counter region; T = 0 or G = 0 needs none."""
    for T, G in ((50, 4), (512, 4), (1024, 4), (8192, 4), (300, 2000)):
        n = _lib.lora_shrink_expand_workspace_size(1, T, 4096, 3, 16, G, 6144)
        s = _lib.lora_shrink_workspace_size(1, T, 4096, 3, 16, G)
        e = _lib.lora_expand_workspace_size(1, T, 3, 16, G, 6144)
        assert n >= 32768 and n >= ((s + 255) // 256) * 256 + e, (T, G, n, s, e)
    assert _lib.lora_shrink_expand_workspace_size(1, 0, 4096, 3, 16, 4, 6144) == 0
    assert _lib.lora_shrink_expand_workspace_size(1, 50, 4096, 3, 16, 0, 6144) == 0
    assert _lib.lora_shrink_expand_workspace_size(7, 50, 4096, 3, 16, 4, 6144) == 0
    assert _lib.LORA_SHRINK_EXPAND_FLAG_OFFSET == 32764


def test_projection_backward_workspace_sizes():
    """The projection-backward queries: positive and growing with M for valid sizes; 0 for an
    unsupported dtype, a rank above 64 or an empty size. The q/k/v workspace holds at least the
    side-by-side copy of the three gradients."""
    lin = lambda M, K, N, r, dt=1: _lib.lora_linear_backward_workspace_size(dt, M, K, N, r)
    qkv = lambda M, K, Nq, Nkv, r, dt=1: _lib.lora_qkv_backward_workspace_size(dt, M, K, Nq, Nkv, r)
    assert 0 < lin(128, 256, 192, 16) < lin(4096, 256, 192, 16)
    assert 0 < qkv(128, 256, 192, 64, 16) < qkv(4096, 256, 192, 64, 16)
    assert qkv(4096, 4096, 4096, 1024, 16) >= 4096 * 6144 * 2
    assert lin(128, 256, 192, 16, dt=0) == 0 and qkv(128, 256, 192, 64, 16, dt=2) == 0
    assert lin(128, 256, 192, 65) == 0 and qkv(128, 256, 192, 64, 0) == 0
    assert lin(0, 256, 192, 16) == 0 and qkv(128, 0, 192, 64, 16) == 0
