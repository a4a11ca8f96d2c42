"""Seeded synthetic inputs for the attention workloads.

This module is shared by the fp64 oracle's tests and by the HIP path's tests
and benchmark. It only draws random numbers and describes shapes; it holds
none of the attention arithmetic (no norm, no mask, no softmax).

Workloads (shapes and per-layer windows as the workload descriptions state
them; window -1 means full causal):

  1  single full-causal layer, forward only:   B=1,  T=128,  Hq=4, Hkv=2, D=64
  2  single sliding-window layer, fwd+bwd:     B=16, T=2048, Hq=6, Hkv=3, D=128, W=1024
  3  single full-causal layer, fwd+bwd:        B=16, T=2048, Hq=6, Hkv=3, D=128
  4  8-layer SSSL stack, fwd+bwd:              B=16, T=2048, Hq=6, Hkv=3, D=128
  5  long-context 8-layer SSSL stack, fwd+bwd: B=4,  T=8192, Hq=6, Hkv=3, D=128,
     with a seeded 10 % of head rows scaled by 8 in q, k, v and dO

The model shape behind workloads 2-5 (n_embd 768 = 6 heads x 128, 8 layers,
T = 2048, SSSL windows) is the default GPT of the autoresearch trainer
("autoresearch Administrator & Developer Guide", sections 3.4 and 6.3).
Real activations are unavailable (weights are never persisted and the
dataset is not here), so N(0, 1) draws stand in for post-projection q/k/v
and for the upstream gradient.

Seeding: torch.Generator().manual_seed(42 + 1000*cfg + 10*layer + t) with
t = 0, 1, 2, 3 for q, k, v, dO and t = 4..7 for the row masks of workload 5.
Values are drawn in fp32 and rounded to bf16 (round-to-nearest-even) on the
CPU, so every consumer sees identical bits.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SEED_BASE = 42
EPS = 1e-6


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    windows: tuple  # per layer, -1 = full causal
    backward: bool
    scaled_row_frac: float = 0.0  # fraction of head rows multiplied by scaled_row_factor
    scaled_row_factor: float = 1.0
    eps: float = EPS
    chunked: bool = False  # draw each tensor one batch row at a time (same generator, in order)
    notes: str = field(default="", compare=False)

    @property
    def n_layer(self) -> int:
        return len(self.windows)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    1: Workload(1, "full_causal_fwd_B1_T128_Hq4_Hkv2_D64", 1, 128, 4, 2, 64, (-1,), False),
    2: Workload(2, "sliding_W1024_fwdbwd_B16_T2048_Hq6_Hkv3_D128", 16, 2048, 6, 3, 128, (1024,), True),
    3: Workload(3, "full_causal_fwdbwd_B16_T2048_Hq6_Hkv3_D128", 16, 2048, 6, 3, 128, (-1,), True),
    4: Workload(4, "sssl8_fwdbwd_B16_T2048_Hq6_Hkv3_D128", 16, 2048, 6, 3, 128,
                (1024, 1024, 1024, -1, 1024, 1024, 1024, -1), True),
    5: Workload(5, "sssl8_long_fwdbwd_B4_T8192_Hq6_Hkv3_D128_rows10pct_x8", 4, 8192, 6, 3, 128,
                (4096, 4096, 4096, -1, 4096, 4096, 4096, -1), True, 0.10, 8.0),
    # the pages' own model shape: multi-head attention (n_kv_head = n_head = 6,
    # head_dim 128) at device batch 128, sequence 2048, SSSL pattern
    6: Workload(6, "sssl8_mha_fwdbwd_B128_T2048_Hq6_Hkv6_D128", 128, 2048, 6, 6, 128,
                (1024, 1024, 1024, -1, 1024, 1024, 1024, -1), True, chunked=True),
}


def seed_for(cfg: int, layer: int, t: int) -> int:
    return SEED_BASE + 1000 * cfg + 10 * layer + t


def _randn_bf16(shape, seed: int, chunked: bool = False) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    if not chunked:
        return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    # one leading index at a time from the same generator: no full-size fp32 temporary
    out = torch.empty(shape, dtype=torch.bfloat16)
    for i in range(shape[0]):
        out[i] = torch.randn(shape[1:], generator=g, dtype=torch.float32)
    return out


def _row_mask(shape_rows, frac: float, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.rand(shape_rows, generator=g, dtype=torch.float32) < frac


def random_qkvdo(B, T, Hq, Hkv, D, seed_q, seed_k, seed_v, seed_do, with_do=True, chunked=False):
    """bf16 CPU tensors q [B,T,Hq,D], k/v [B,T,Hkv,D], dO [B,T,Hq,D] (or None)."""
    q = _randn_bf16((B, T, Hq, D), seed_q, chunked)
    k = _randn_bf16((B, T, Hkv, D), seed_k, chunked)
    v = _randn_bf16((B, T, Hkv, D), seed_v, chunked)
    do = _randn_bf16((B, T, Hq, D), seed_do, chunked) if with_do else None
    return q, k, v, do


def layer_inputs(w: Workload, layer: int, qk_rows_only: bool = False):
    """Seeded bf16 CPU inputs (q, k, v, dO) for one layer of workload ``w``.

    For workload 5 a Bernoulli(scaled_row_frac) mask over head rows (b, t, h)
    is drawn per tensor and those rows are multiplied by scaled_row_factor
    (exact in bf16, a power of two). ``qk_rows_only`` applies the scaling to
    q and k only (a variant used beside the literal reading).
    """
    s = [seed_for(w.cfg, layer, t) for t in range(8)]
    q, k, v, do = random_qkvdo(w.B, w.T, w.Hq, w.Hkv, w.D, s[0], s[1], s[2], s[3], with_do=w.backward,
                               chunked=w.chunked)
    if w.scaled_row_frac > 0:
        f = w.scaled_row_factor
        tensors = [q, k] if qk_rows_only else [q, k, v, do]
        for idx, x in enumerate(tensors):
            if x is None:
                continue
            m = _row_mask(x.shape[:3], w.scaled_row_frac, s[4 + idx])
            x[m] = (x[m].float() * f).to(torch.bfloat16)
    return q, k, v, do


VE_VOCAB = 8192  # the trainer's VOCAB_SIZE (the guide's constants table)
VE_CHANNELS = 768  # n_embd: the rows the gate reads the first 32 channels of


def ve_inputs(w: Workload, layer: int):
    """Seeded value-embedding inputs of one layer: x [B, T, 768] bf16 (the
    attention's input rows), gate weights [Hkv, 32] bf16 ~ N(0, 0.2^2) (zero at
    the trainer's start; a spread here so the gate varies), token ids [B, T]
    int32 uniform over the vocabulary, embedding table [8192, Hkv*D] bf16."""
    s = [seed_for(w.cfg, layer, t) for t in range(8, 12)]
    x = _randn_bf16((w.B, w.T, VE_CHANNELS), s[0], w.chunked)
    gw = (0.2 * torch.randn((w.Hkv, 32), generator=torch.Generator().manual_seed(s[1]))).to(torch.bfloat16)
    ids = torch.randint(0, VE_VOCAB, (w.B, w.T), generator=torch.Generator().manual_seed(s[2]), dtype=torch.int32)
    table = _randn_bf16((VE_VOCAB, w.Hkv * w.D), s[3])
    return x, gw, ids, table


def small_case(B, T, Hq, Hkv, D, seed=7, with_do=True, dtype=torch.bfloat16):
    """Small seeded case for parity tests at sizes the oracle finishes in seconds."""
    q, k, v, do = random_qkvdo(B, T, Hq, Hkv, D, seed, seed + 1, seed + 2, seed + 3, with_do)
    if dtype != torch.bfloat16:
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
        do = do.to(dtype) if do is not None else None
    return q, k, v, do
