"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and slices them into rank shards; it holds none of
the MLP's arithmetic, so both the GPU path and the CPU oracle can be fed from it.

Random numbers come from torch's CPU generator (``torch.Generator().manual_seed``):
values are drawn N(0, 1) in float32, scaled by the standard deviation in float32,
then rounded to the storage dtype (round-to-nearest-even for bfloat16).

The 70B-class model (d_model 8192, ffn 28672) is drawn as eight column pieces of
the gate and up weights and eight row pieces of the down weight, each from its own
seed.  A rank shard at tensor-parallel degree k in {1, 2, 4, 8} is the
concatenation of ``8 // k`` consecutive pieces, so every degree slices the same
model, and a single rank's shard can be drawn without drawing the whole model.

Shard layout (the split of the page "大模型推理系统揭秘（07）Multi-GPU",
sections 1.2.2-1.2.4: contiguous, equal column blocks of the first weight and the
matching row blocks of the second):

* tanh / identity: first weight ``A_i`` [d, F_i], second weight ``B_i`` [F_i, d];
* silu_gate: ``A_i`` [d, 2 F_i] holds the rank's F_i gate columns, then its F_i up
  columns over the same hidden indices; ``B_i`` [F_i, d] are the matching rows of
  the down weight.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

D_MODEL = 8192
FFN = 28672
PIECES = 8
WEIGHT_STD = 0.02
TOKEN_STD = 1.0

# seed layout: branch base + piece index; tokens use their own range
_SEED_GATE = 1000
_SEED_UP = 2000
_SEED_DOWN = 3000
_SEED_TOKENS = 50000


def randn(shape, seed: int, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) values on the CPU from a fresh generator seeded with ``seed``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    v = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        v = v * torch.tensor(std, dtype=torch.float32)
    return v.to(dtype)


def randn_device(shape, seed: int, device, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) values drawn on ``device`` by torch's generator for that device,
    seeded with ``seed``: for inputs of gigabytes, which the CPU generator would take
    minutes to draw.  Values differ from ``randn`` with the same seed; a test reads
    back whatever part of them its reference needs."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    v = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        v.mul_(torch.tensor(std, dtype=torch.float32, device=device))
    return v.to(dtype)


def split_columns(a: torch.Tensor, k: int):
    """k contiguous, equal column blocks of ``a``."""
    n = a.shape[1]
    if n % k:
        raise ValueError("%d columns do not split into %d equal blocks" % (n, k))
    w = n // k
    return [a[:, r * w:(r + 1) * w].contiguous() for r in range(k)]


def split_rows(b: torch.Tensor, k: int):
    """k contiguous, equal row blocks of ``b``."""
    n = b.shape[0]
    if n % k:
        raise ValueError("%d rows do not split into %d equal blocks" % (n, k))
    w = n // k
    return [b[r * w:(r + 1) * w].contiguous() for r in range(k)]


# --------------------------------------------------------------------------
# Toy two-projection MLP (fp32, tanh): X [4, 64], A [64, 256], B [256, 64],
# N(0, 0.1), split into TP=2 shards.
# --------------------------------------------------------------------------
TOY_M, TOY_D, TOY_F = 4, 64, 256
TOY_STD = 0.1


def toy_case():
    """(X, A, B) fp32 of the toy MLP."""
    X = randn((TOY_M, TOY_D), seed=13, std=TOY_STD)
    A = randn((TOY_D, TOY_F), seed=11, std=TOY_STD)
    B = randn((TOY_F, TOY_D), seed=12, std=TOY_STD)
    return X, A, B


def toy_shards(k: int = 2):
    """(X, a_shards, b_shards) for the toy MLP at tensor-parallel degree k."""
    X, A, B = toy_case()
    return X, split_columns(A, k), split_rows(B, k)


# --------------------------------------------------------------------------
# Piecewise-seeded gated MLP (the 70B-class shapes by default)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelSpec:
    d_model: int = D_MODEL
    ffn: int = FFN
    pieces: int = PIECES
    std: float = WEIGHT_STD
    dtype: torch.dtype = torch.bfloat16
    seed_offset: int = 0  # shifts every weight seed: a second, distinct model

    @property
    def piece_width(self) -> int:
        if self.ffn % self.pieces:
            raise ValueError("ffn must be a multiple of the piece count")
        return self.ffn // self.pieces

    def _piece(self, base: int, p: int, rows_are_ffn: bool) -> torch.Tensor:
        if not 0 <= p < self.pieces:
            raise IndexError(p)
        w = self.piece_width
        shape = (w, self.d_model) if rows_are_ffn else (self.d_model, w)
        return randn(shape, seed=base + self.seed_offset + p, std=self.std, dtype=self.dtype)

    def gate_piece(self, p: int) -> torch.Tensor:
        return self._piece(_SEED_GATE, p, rows_are_ffn=False)

    def up_piece(self, p: int) -> torch.Tensor:
        return self._piece(_SEED_UP, p, rows_are_ffn=False)

    def down_piece(self, p: int) -> torch.Tensor:
        return self._piece(_SEED_DOWN, p, rows_are_ffn=True)

    def _pieces_of(self, rank: int, tp: int):
        if tp < 1 or self.pieces % tp:
            raise ValueError("tensor-parallel degree %d must divide %d pieces" % (tp, self.pieces))
        if not 0 <= rank < tp:
            raise IndexError(rank)
        per = self.pieces // tp
        return range(rank * per, (rank + 1) * per)

    def shard(self, rank: int, tp: int, activation: str = "silu_gate"):
        """(A_i, B_i) of rank ``rank`` at degree ``tp`` (layouts in the module docstring).

        For tanh / identity the first weight is the gate weight alone."""
        ps = self._pieces_of(rank, tp)
        gate = torch.cat([self.gate_piece(p) for p in ps], dim=1)
        down = torch.cat([self.down_piece(p) for p in ps], dim=0)
        if activation == "silu_gate":
            up = torch.cat([self.up_piece(p) for p in ps], dim=1)
            a = torch.cat([gate, up], dim=1)
        elif activation in ("tanh", "identity"):
            a = gate
        else:
            raise ValueError(activation)
        return a.contiguous(), down.contiguous()

    def shards(self, tp: int, activation: str = "silu_gate"):
        pairs = [self.shard(r, tp, activation) for r in range(tp)]
        return [p[0] for p in pairs], [p[1] for p in pairs]


# --------------------------------------------------------------------------
# Attention-block projections of the same 70B-class model (page "7.4 推理侧并行",
# section 7.4.1: 64 query heads of width 128 over d_model 8192, 8 KV heads with
# GQA).  Each head's Q, K, V columns and Wo rows are drawn from their own seed, so
# a rank shard at any degree dividing 8 slices one model: rank r of tp holds query
# heads [r 64/tp, (r+1) 64/tp) and KV heads [r 8/tp, (r+1) 8/tp).
# --------------------------------------------------------------------------
_SEED_Q, _SEED_K, _SEED_V, _SEED_O = 4000, 5000, 6000, 7000


@dataclass(frozen=True)
class AttentionSpec:
    d_model: int = D_MODEL
    q_heads: int = 64
    kv_heads: int = 8
    head_dim: int = 128
    std: float = WEIGHT_STD
    dtype: torch.dtype = torch.bfloat16

    def _head(self, base: int, h: int, rows_are_heads: bool) -> torch.Tensor:
        shape = (self.head_dim, self.d_model) if rows_are_heads else (self.d_model, self.head_dim)
        return randn(shape, seed=base + h, std=self.std, dtype=self.dtype)

    def shard(self, rank: int, tp: int):
        """(W_qkv [d, (q + 2 kv) head_dim], W_o [q head_dim, d]) of rank ``rank`` at
        degree ``tp``: the rank's query-head columns, then its K and its V columns; and
        the rows of the output projection that meet its query heads."""
        if tp < 1 or self.q_heads % tp or self.kv_heads % tp:
            raise ValueError("tensor-parallel degree %d must divide the head counts" % tp)
        if not 0 <= rank < tp:
            raise IndexError(rank)
        qh = range(rank * self.q_heads // tp, (rank + 1) * self.q_heads // tp)
        kh = range(rank * self.kv_heads // tp, (rank + 1) * self.kv_heads // tp)
        cols = ([self._head(_SEED_Q, h, False) for h in qh] +
                [self._head(_SEED_K, h, False) for h in kh] +
                [self._head(_SEED_V, h, False) for h in kh])
        w_qkv = torch.cat(cols, dim=1).contiguous()
        w_o = torch.cat([self._head(_SEED_O, h, True) for h in qh], dim=0).contiguous()
        return w_qkv, w_o

    def q_width(self, tp: int) -> int:
        return self.q_heads // tp * self.head_dim


# --------------------------------------------------------------------------
# Experts of one GPU for the grouped expert MLP (page "大模型推理系统揭秘（07）
# Multi-GPU", MoE section: 64 experts with top-2 routing over EP = 4 GPUs, so 16
# experts per GPU; its grouped-GEMM example gives one GPU's experts 128, 64 and 96
# tokens).  The expert width is not given there; 2048 is used.  Each expert's
# weights come from their own seeds; token counts per expert are drawn around the
# example's 64-128.
# --------------------------------------------------------------------------
_SEED_EXPERT = 9000


@dataclass(frozen=True)
class ExpertSpec:
    d_model: int = D_MODEL
    ffn_expert: int = 2048
    n_experts: int = 16
    std: float = WEIGHT_STD
    dtype: torch.dtype = torch.bfloat16

    def weights(self, activation: str = "silu_gate"):
        """(W1 [E, d, 2F or F], W2 [E, F, d]) of the GPU's experts."""
        cols = 2 * self.ffn_expert if activation == "silu_gate" else self.ffn_expert
        w1 = torch.stack([randn((self.d_model, cols), _SEED_EXPERT + 2 * e, self.std, self.dtype)
                          for e in range(self.n_experts)])
        w2 = torch.stack([randn((self.ffn_expert, self.d_model), _SEED_EXPERT + 2 * e + 1,
                                self.std, self.dtype) for e in range(self.n_experts)])
        return w1, w2


def expert_counts(n_experts: int, lo: int = 64, hi: int = 128, seed: int = 77) -> list[int]:
    """Tokens per expert, uniform on [lo, hi], seeded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, (n_experts,), generator=g).tolist()


def tokens(M: int, d: int = D_MODEL, std: float = TOKEN_STD, dtype=torch.bfloat16,
           seed: int | None = None) -> torch.Tensor:
    """Token activations X [M, d], N(0, std^2); the seed defaults to one per M."""
    s = _SEED_TOKENS + M if seed is None else seed
    return randn((M, d), seed=s, std=std, dtype=dtype)


def sample_rows(M: int, n: int, seed: int = 7) -> list[int]:
    """A seeded subset of n distinct rows of [0, M) that always holds 0 and M-1."""
    if M <= n:
        return list(range(M))
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + M)
    perm = torch.randperm(M - 2, generator=g)[: max(n - 2, 0)] + 1
    rows = sorted(set([0, M - 1] + perm.tolist()))
    return rows


def attn_partials(rows: int, dim: int, k: int, keys_per_rank: int = 1024, seed: int = 8100,
                  dtype=torch.float32):
    """Synthetic attention partials of k ranks for `rows` query rows (tokens x heads)
    with value width `dim`, shaped like a split KV history of `keys_per_rank` keys per
    rank: per rank and row a local maximum m ~ N(3, 1), a sum of exponentials
    s ~ U(1, keys_per_rank) (the key at the maximum contributes exactly 1), and a
    weighted value sum v = sqrt(s) * N(0, 1) in `dtype`.  Returns lists
    (values [rows, dim], maxima [rows], expsums [rows]); statistics are float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    vals, maxs, sums = [], [], []
    for _ in range(k):
        m = torch.randn(rows, generator=g, dtype=torch.float32) + 3.0
        e = 1.0 + torch.rand(rows, generator=g, dtype=torch.float32) * (keys_per_rank - 1)
        v = torch.randn(rows, dim, generator=g, dtype=torch.float32) * e.sqrt()[:, None]
        vals.append(v.to(dtype))
        maxs.append(m)
        sums.append(e)
    return vals, maxs, sums
