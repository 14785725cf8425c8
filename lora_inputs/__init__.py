"""Seeded synthetic inputs for the multi-adapter LoRA projection and the fused LoRA+SwiGLU MLP.

This module only draws random numbers and lays them out: segment lengths, adapter assignment,
token permutation, activations, adapter weights and the base output ``y_in``. It contains none
of the method's arithmetic, so both the CPU oracle and the HIP path may use it.

Conventions (shared by every generator):

* ``numpy.random.default_rng(seed)`` (PCG64). Draw order: segment lengths, ``weight_indices``,
  ``permutation``, then ``x``, ``A``, ``B``, ``y_in`` (and the second problem's tensors after the
  first problem's, where a case has two).
* ``N(0, s)`` means mean 0 and standard deviation ``s``. Values are drawn in float32 and cast to
  the case dtype by torch (round to nearest even).
* ``permutation[i]`` is the original token row held by sorted position ``i``; segment ``g`` owns
  sorted positions ``seg_indptr[g] .. seg_indptr[g+1]-1`` and uses adapter ``weight_indices[g]``.
* Stacked adapter weights: ``A[L][S*R][K]`` (slice ``s`` owns rows ``s*R .. s*R+R-1``) and
  ``B[L][N][R]`` (row ``n`` is output column ``n``). Entries beyond an adapter's rank are zero
  here; tests that want to prove masking overwrite them with NaN.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# The nine-point token sweep on the decode-QKV shape (4 adapters, rank 16, K=4096,
# slices 4096/1024/1024), standing in for the nine unpublished cases tok = 50 .. 8192.
SWEEP_TOKENS = (50, 128, 256, 512, 1024, 2048, 4096, 6144, 8192)


@dataclass
class SgmvCase:
    """One shrink+expand problem. Tensors are CPU tensors; metadata is int32."""

    name: str
    dtype: str
    T: int
    K: int
    S: int
    R: int
    L: int
    slice_offsets: torch.Tensor  # int32 [S+1]
    seg_indptr: torch.Tensor  # int32 [G+1]
    weight_indices: torch.Tensor  # int32 [G]
    permutation: torch.Tensor  # int32 [T]
    lora_ranks: torch.Tensor  # int32 [L]
    scalings: torch.Tensor  # float32 [L]
    x: torch.Tensor  # dtype [T][K]
    A: torch.Tensor  # dtype [L][S*R][K]
    B: torch.Tensor  # dtype [L][N][R]
    y_in: torch.Tensor  # dtype [T][N]
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return int(self.weight_indices.numel())

    @property
    def N(self) -> int:
        return int(self.slice_offsets[-1])


@dataclass
class MlpCase:
    """One single-adapter LoRA+SwiGLU MLP problem (nn.Linear [out][in] layouts)."""

    name: str
    dtype: str
    M: int
    H: int
    I: int
    r: int
    scale: float
    x: torch.Tensor  # [M][H]
    w_gate: torch.Tensor  # [I][H]
    w_up: torch.Tensor  # [I][H]
    w_down: torch.Tensor  # [H][I]
    a_gate: torch.Tensor  # [r][H]
    b_gate: torch.Tensor  # [I][r]
    a_up: torch.Tensor  # [r][H]
    b_up: torch.Tensor  # [I][r]
    a_down: torch.Tensor  # [r][I]
    b_down: torch.Tensor  # [H][r]


def _i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32)))


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return torch.from_numpy(v).to(DTYPES[dtype])


def uniform_composition(rng: np.random.Generator, total: int, parts: int) -> np.ndarray:
    """Split ``total`` into ``parts`` nonnegative lengths at sorted uniform cut points."""
    cuts = np.sort(rng.integers(0, total + 1, size=parts - 1))
    return np.diff(np.concatenate(([0], cuts, [total]))).astype(np.int64)


def zipf_lengths(rng: np.random.Generator, total: int, parts: int, a: float, n_empty: int) -> np.ndarray:
    """Multinomial lengths with p_i proportional to i**-a in a seeded order; ``n_empty`` seeded
    segments are then emptied and their tokens moved to the largest segment."""
    p = np.arange(1, parts + 1, dtype=np.float64) ** (-a)
    p = p[rng.permutation(parts)]
    p /= p.sum()
    lens = rng.multinomial(total, p).astype(np.int64)
    empties = rng.choice(parts, size=n_empty, replace=False)
    moved = int(lens[empties].sum())
    lens[empties] = 0
    biggest = int(np.argmax(lens))
    lens[biggest] += moved
    return lens


def _indptr(lens: np.ndarray) -> np.ndarray:
    return np.concatenate(([0], np.cumsum(lens))).astype(np.int32)


def _weights(rng, T, K, S, R, L, N, ranks, dtype, x_std=1.0, w_std=0.02):
    x = _normal(rng, (T, K), x_std, dtype)
    A = _normal(rng, (L, S * R, K), w_std, dtype)
    B = _normal(rng, (L, N, R), w_std, dtype)
    y_in = _normal(rng, (T, N), 1.0, dtype)
    for a in range(L):
        r = int(ranks[a])
        A.view(L, S, R, K)[a, :, r:, :] = 0
        B[a, :, r:] = 0
    return x, A, B, y_in


def make_sgmv(
    name: str,
    *,
    seed: int,
    T: int,
    K: int,
    S: int,
    R: int,
    L: int,
    slice_offsets,
    dtype: str,
    lengths: str = "uniform",
    ranks=None,
    scale: float = 2.0,
    identity_perm: bool = False,
    fixed_indptr=None,
    fixed_weight_indices=None,
) -> SgmvCase:
    """General seeded SGMV case; ``lengths`` is 'uniform' (composition) or 'zipf'."""
    rng = np.random.default_rng(seed)
    if fixed_indptr is not None:
        indptr = np.asarray(fixed_indptr, dtype=np.int32)
    elif lengths == "uniform":
        indptr = _indptr(uniform_composition(rng, T, L))
    elif lengths == "zipf":
        indptr = _indptr(zipf_lengths(rng, T, L, 1.1, 4))
    elif lengths == "ones":
        indptr = np.arange(T + 1, dtype=np.int32)
    else:
        raise ValueError(lengths)
    G = len(indptr) - 1
    if fixed_weight_indices is not None:
        widx = np.asarray(fixed_weight_indices, dtype=np.int32)
    elif G == L:
        widx = rng.permutation(L).astype(np.int32)
    else:
        widx = rng.integers(0, L, size=G).astype(np.int32)
    perm = np.arange(T, dtype=np.int32) if identity_perm else rng.permutation(T).astype(np.int32)
    offs = np.asarray(slice_offsets, dtype=np.int32)
    N = int(offs[-1])
    if ranks is None:
        ranks = np.full(L, R, dtype=np.int32)
    ranks = np.asarray(ranks, dtype=np.int32)
    x, A, B, y_in = _weights(rng, T, K, S, R, L, N, ranks, dtype)
    return SgmvCase(
        name=name, dtype=dtype, T=T, K=K, S=S, R=R, L=L,
        slice_offsets=_i32(offs), seg_indptr=_i32(indptr), weight_indices=_i32(widx),
        permutation=_i32(perm), lora_ranks=_i32(ranks),
        scalings=torch.full((L,), float(scale), dtype=torch.float32),
        x=x, A=A, B=B, y_in=y_in,
    )


def config_tiny_f32() -> SgmvCase:
    """Tiny fp32 SGMV: 64 tokens, 2 adapters, K=256, rank 8, one slice N=256, segments 40+24,
    identity permutation, scale 2.0, seed 0."""
    return make_sgmv("tiny_f32", seed=0, T=64, K=256, S=1, R=8, L=2, slice_offsets=[0, 256],
                     dtype="f32", identity_perm=True, fixed_indptr=[0, 40, 64],
                     fixed_weight_indices=[0, 1], scale=2.0)


def config_decode_qkv(T: int = 50, seed: int = 1) -> SgmvCase:
    """Decode QKV bf16: 4 adapters rank 16, K=4096, slices N=(4096,1024,1024), uniform-random
    segment lengths, random adapter order and permutation, scale 2."""
    return make_sgmv(f"decode_qkv_bf16_tok{T}", seed=seed, T=T, K=4096, S=3, R=16, L=4,
                     slice_offsets=[0, 4096, 5120, 6144], dtype="bf16")


def config_prefill(seed: int = 2) -> tuple[SgmvCase, SgmvCase]:
    """Prefill bf16: tok=2048, 8 adapters rank 64. gate_up: K=4096, 2 slices of 12288;
    down: K=12288, one slice of 4096. Same segment metadata, fresh down-projection input."""
    gu = make_sgmv("prefill_gate_up_bf16", seed=seed, T=2048, K=4096, S=2, R=64, L=8,
                   slice_offsets=[0, 12288, 24576], dtype="bf16")
    # The down problem continues the same stream: reuse the metadata, draw fresh tensors.
    rng = np.random.default_rng([seed, 1])
    ranks = gu.lora_ranks.numpy()
    x, A, B, y_in = _weights(rng, 2048, 12288, 1, 64, 8, 4096, ranks, "bf16")
    down = SgmvCase(
        name="prefill_down_bf16", dtype="bf16", T=2048, K=12288, S=1, R=64, L=8,
        slice_offsets=_i32([0, 4096]), seg_indptr=gu.seg_indptr.clone(),
        weight_indices=gu.weight_indices.clone(), permutation=gu.permutation.clone(),
        lora_ranks=gu.lora_ranks.clone(), scalings=gu.scalings.clone(),
        x=x, A=A, B=B, y_in=y_in,
    )
    return gu, down


IRREGULAR_RANKS = (4, 7, 16, 33, 64)


def config_irregular(seed: int = 3) -> SgmvCase:
    """Irregular fp16: tok=8192, 32 adapters with ranks (4,7,16,33,64)[a mod 5] padded to 64,
    Zipf(1.1) segment lengths with 4 forced-empty segments, K=4093, slices N=(4096,1021,1021)
    at offsets 0/4096/5117 (row starts not 16-byte aligned), scale 2."""
    ranks = [IRREGULAR_RANKS[a % 5] for a in range(32)]
    return make_sgmv("irregular_f16", seed=seed, T=8192, K=4093, S=3, R=64, L=32,
                     slice_offsets=[0, 4096, 5117, 6138], dtype="f16", lengths="zipf",
                     ranks=ranks)


def config_mlp(seed: int = 4, M: int = 4096, H: int = 4096, I: int = 12288, r: int = 16,
               scale: float = 4.0, dtype: str = "bf16") -> MlpCase:
    """Single-adapter fused LoRA+SwiGLU MLP (Qwen3-8B-shaped layer by default):
    x~N(0,1) [M][H]; frozen W and LoRA A/B ~N(0,0.02); scale alpha/r = 4; dropout 0."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, H), 1.0, dtype)
    w_gate = _normal(rng, (I, H), 0.02, dtype)
    w_up = _normal(rng, (I, H), 0.02, dtype)
    w_down = _normal(rng, (H, I), 0.02, dtype)
    a_gate = _normal(rng, (r, H), 0.02, dtype)
    b_gate = _normal(rng, (I, r), 0.02, dtype)
    a_up = _normal(rng, (r, H), 0.02, dtype)
    b_up = _normal(rng, (I, r), 0.02, dtype)
    a_down = _normal(rng, (r, I), 0.02, dtype)
    b_down = _normal(rng, (H, r), 0.02, dtype)
    return MlpCase(name=f"mlp_{dtype}_M{M}_H{H}_I{I}_r{r}", dtype=dtype, M=M, H=H, I=I, r=r,
                   scale=scale, x=x, w_gate=w_gate, w_up=w_up, w_down=w_down,
                   a_gate=a_gate, b_gate=b_gate, a_up=a_up, b_up=b_up,
                   a_down=a_down, b_down=b_down)


def mlp_dout(seed: int = 4, M: int = 4096, H: int = 4096, dtype: str = "bf16") -> torch.Tensor:
    """Seeded upstream gradient of the MLP output for the backward, dout ~ N(0,1) [M][H], drawn
    from its own stream (seed, 1) so the forward inputs of the same seed are unchanged."""
    rng = np.random.default_rng([seed, 1])
    return _normal(rng, (M, H), 1.0, dtype)


def projection_douts(seed: int = 5, M: int = 4096, widths=(4096, 1024, 1024, 4096),
                     dtype: str = "bf16") -> list:
    """Seeded upstream gradients of projection outputs for the backward, each dout ~ N(0,1)
    [M][N] for N in ``widths`` (query, key, value and output projections by default), drawn in
    that order from their own stream (seed, 1) so the forward inputs of the same seed are
    unchanged."""
    rng = np.random.default_rng([seed, 1])
    return [_normal(rng, (M, n), 1.0, dtype) for n in widths]


@dataclass
class QkvCase:
    """Single-adapter LoRA attention projections of one x (nn.Linear [out][in] layouts)."""

    name: str
    dtype: str
    M: int
    H: int
    Nq: int
    Nkv: int
    r: int
    scale: float
    x: torch.Tensor  # [M][H]
    w_q: torch.Tensor  # [Nq][H]
    w_k: torch.Tensor  # [Nkv][H]
    w_v: torch.Tensor  # [Nkv][H]
    a_q: torch.Tensor  # [r][H]
    b_q: torch.Tensor  # [Nq][r]
    a_k: torch.Tensor
    b_k: torch.Tensor  # [Nkv][r]
    a_v: torch.Tensor
    b_v: torch.Tensor
    w_o: torch.Tensor  # [H][Nq] (output projection, reads the attention output)
    a_o: torch.Tensor  # [r][Nq]
    b_o: torch.Tensor  # [H][r]


def config_qkv(seed: int = 5, M: int = 4096, H: int = 4096, Nq: int = 4096, Nkv: int = 1024,
               r: int = 16, scale: float = 4.0, dtype: str = "bf16") -> QkvCase:
    """Single-adapter LoRA Q/K/V and O projections (Qwen3-8B-shaped attention by default:
    32 query heads and 8 key/value heads of 128): x~N(0,1) [M][H]; frozen W and LoRA A/B
    ~N(0,0.02); scale alpha/r = 4; dropout 0."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, H), 1.0, dtype)
    w_q = _normal(rng, (Nq, H), 0.02, dtype)
    w_k = _normal(rng, (Nkv, H), 0.02, dtype)
    w_v = _normal(rng, (Nkv, H), 0.02, dtype)
    a_q = _normal(rng, (r, H), 0.02, dtype)
    b_q = _normal(rng, (Nq, r), 0.02, dtype)
    a_k = _normal(rng, (r, H), 0.02, dtype)
    b_k = _normal(rng, (Nkv, r), 0.02, dtype)
    a_v = _normal(rng, (r, H), 0.02, dtype)
    b_v = _normal(rng, (Nkv, r), 0.02, dtype)
    w_o = _normal(rng, (H, Nq), 0.02, dtype)
    a_o = _normal(rng, (r, Nq), 0.02, dtype)
    b_o = _normal(rng, (H, r), 0.02, dtype)
    return QkvCase(name=f"qkv_{dtype}_M{M}_H{H}_Nq{Nq}_Nkv{Nkv}_r{r}", dtype=dtype, M=M, H=H,
                   Nq=Nq, Nkv=Nkv, r=r, scale=scale, x=x, w_q=w_q, w_k=w_k, w_v=w_v, a_q=a_q,
                   b_q=b_q, a_k=a_k, b_k=b_k, a_v=a_v, b_v=b_v, w_o=w_o, a_o=a_o, b_o=b_o)


@dataclass
class EmbeddingCase:
    """Multi-adapter embedding LoRA-A problem: token ids, stacked A [L][R][V], segments."""

    name: str
    dtype: str
    T: int
    V: int
    R: int
    L: int
    input_ids: torch.Tensor  # int32 [T] (token order)
    A: torch.Tensor  # [L][R][V]
    seg_indptr: torch.Tensor
    weight_indices: torch.Tensor
    permutation: torch.Tensor
    lora_ranks: torch.Tensor

    @property
    def G(self) -> int:
        return int(self.weight_indices.numel())


def make_embedding(name: str, *, seed: int, T: int, V: int, R: int, L: int, dtype: str,
                   lengths: str = "uniform", ranks=None, identity_perm: bool = False,
                   fixed_indptr=None, fixed_weight_indices=None) -> EmbeddingCase:
    """Seeded embedding LoRA-A inputs: segment lengths, weight_indices and permutation as for
    make_sgmv, then token ids uniform over the vocabulary (with ids 0 and V-1 forced in), then
    A ~ N(0, 0.02) with the rows past each adapter's rank zeroed."""
    rng = np.random.default_rng(seed)
    if fixed_indptr is not None:
        indptr = np.asarray(fixed_indptr, dtype=np.int64)
        widx = np.asarray(fixed_weight_indices, dtype=np.int64)
    else:
        G = T if lengths == "ones" else L
        if lengths == "ones":
            lens = np.ones(T, dtype=np.int64)
            widx = rng.integers(0, L, size=G)
        else:
            cuts = np.sort(rng.integers(0, T + 1, size=G - 1))
            lens = np.diff(np.concatenate([[0], cuts, [T]]))
            widx = rng.permutation(L)[:G]
        indptr = np.concatenate([[0], np.cumsum(lens)])
    perm = np.arange(T) if identity_perm else rng.permutation(T)
    ids = rng.integers(0, V, size=T)
    if T >= 2:
        ids[0], ids[-1] = 0, V - 1
    ranks = np.full(L, R, dtype=np.int64) if ranks is None else np.asarray(ranks, dtype=np.int64)
    A = _normal(rng, (L, R, V), 0.02, dtype)
    for a in range(L):
        A[a, int(ranks[a]):] = 0
    i32 = lambda v: torch.from_numpy(np.asarray(v, dtype=np.int32))
    return EmbeddingCase(name=name, dtype=dtype, T=T, V=V, R=R, L=L, input_ids=i32(ids), A=A,
                         seg_indptr=i32(indptr), weight_indices=i32(widx), permutation=i32(perm),
                         lora_ranks=i32(ranks))


def sweep_case(T: int) -> SgmvCase:
    """One point of the decode-QKV token sweep (same generator and seed as the tok=50 case)."""
    return config_decode_qkv(T=T, seed=1)


def random_h(rng_seed: int, T: int, width: int, dtype: str) -> torch.Tensor:
    """Seeded stand-in for a shrink output, used to drive expand on its own."""
    rng = np.random.default_rng(rng_seed)
    return _normal(rng, (T, width), 1.0, dtype)
