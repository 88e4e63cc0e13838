"""Seeded synthetic inputs for the attention-backward workloads.

This module holds no attention arithmetic: it only names the workload shapes
and draws the random tensors (and, for packed batches, the sequence lengths)
that both the GPU path and the CPU oracle consume.

Recipe (same for every workload): one CPU ``torch.Generator`` seeded with
``seed``; draw order is [sequence lengths], then Q, K, V, dO, each
``torch.randn`` in fp32 and rounded to bf16 (round-to-nearest-even; fp16 for
the fp16 cases, ``dtype=torch.float16``).
Dense workloads are laid out (batch, seq, heads, dim); packed variable-length
workloads are (total_tokens, heads, dim) with int32 ``cu_seqlens`` prefix sums
and equal query/key lengths per sequence.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

SEED_BASE = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int                 # dense: B; packed: number of sequences
    heads: int                 # H (query heads)
    heads_k: int               # Hk (key/value heads)
    seqlen_q: int              # dense Sq; packed: unused (lengths are drawn)
    seqlen_k: int
    head_dim: int
    causal: bool
    varlen: bool = False
    len_lo: int = 0            # packed: lengths uniform in [len_lo, len_hi]
    len_hi: int = 0
    seed: int = SEED_BASE
    # local window (left, right), negative = unbounded; None: no window
    window: Optional[Tuple[int, int]] = None
    # soft cap c > 0 of the scaled scores (c * tanh(x / c)); 0: none
    softcap: float = 0.0
    # dropout (p, philox seed, philox offset); None: none
    dropout: Optional[Tuple[float, int, int]] = None

    @property
    def dropout_f32(self):
        """dropout with p rounded to fp32, the precision of the C ABI field
        (so that both sides draw the same keep threshold)."""
        if self.dropout is None:
            return None
        import numpy as np
        p, seed, offset = self.dropout
        return (float(np.float32(p)), seed, offset)

    @property
    def window_sizes(self) -> Tuple[int, int]:
        return (-1, -1) if self.window is None else tuple(self.window)

    @property
    def scale(self) -> float:
        """1/sqrt(head_dim) of the unpadded head dimension."""
        return self.head_dim ** -0.5


# The five reference workloads (bf16, N(0,1) inputs).
WORKLOADS = {
    1: Workload("mha_b1_h2_s128_d64_noncausal", 1, 2, 2, 128, 128, 64, False,
                seed=SEED_BASE + 1),
    2: Workload("mha_b4_h16_s1024_d64_causal", 4, 16, 16, 1024, 1024, 64, True,
                seed=SEED_BASE + 2),
    3: Workload("gqa_b2_h32_hk8_s4096_d128_causal", 2, 32, 8, 4096, 4096, 128, True,
                seed=SEED_BASE + 3),
    4: Workload("gqa_b1_h32_hk4_sq2048_sk8192_d128_causal_br", 1, 32, 4, 2048, 8192,
                128, True, seed=SEED_BASE + 4),
    5: Workload("varlen_16seq_l256_8192_h16_d96_causal", 16, 16, 16, 0, 0, 96, True,
                varlen=True, len_lo=256, len_hi=8192, seed=SEED_BASE + 5),
}


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor            # bf16 / fp16, (B,Sq,H,D) dense or (Tq,H,D) packed
    k: torch.Tensor
    v: torch.Tensor
    dout: torch.Tensor
    lens_q: List[int] = field(default_factory=list)
    lens_k: List[int] = field(default_factory=list)

    @property
    def cu_q(self) -> torch.Tensor:
        return _prefix(self.lens_q)

    @property
    def cu_k(self) -> torch.Tensor:
        return _prefix(self.lens_k)

    def packed(self, t: torch.Tensor) -> torch.Tensor:
        """(total, heads, dim) view of a dense or packed tensor."""
        return t.reshape(-1, t.shape[-2], t.shape[-1])


def _prefix(lens: List[int]) -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def _randn(gen: torch.Generator, shape, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


def draw_lengths(gen: torch.Generator, n: int, lo: int, hi: int) -> List[int]:
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=gen)]


def make_inputs(wl: Workload, lengths: Optional[List[int]] = None,
                dtype=torch.bfloat16) -> Inputs:
    """Draw Q, K, V, dO for a workload.  ``lengths`` overrides the drawn
    packed-sequence lengths (it still consumes no random numbers)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(wl.seed)
    H, Hk, D = wl.heads, wl.heads_k, wl.head_dim
    if wl.varlen:
        lens = list(lengths) if lengths is not None else draw_lengths(
            gen, wl.batch, wl.len_lo, wl.len_hi)
        T = sum(lens)
        q = _randn(gen, (T, H, D), dtype)
        k = _randn(gen, (T, Hk, D), dtype)
        v = _randn(gen, (T, Hk, D), dtype)
        do = _randn(gen, (T, H, D), dtype)
        return Inputs(wl, q, k, v, do, list(lens), list(lens))
    B, Sq, Sk = wl.batch, wl.seqlen_q, wl.seqlen_k
    q = _randn(gen, (B, Sq, H, D), dtype)
    k = _randn(gen, (B, Sk, Hk, D), dtype)
    v = _randn(gen, (B, Sk, Hk, D), dtype)
    do = _randn(gen, (B, Sq, H, D), dtype)
    return Inputs(wl, q, k, v, do, [Sq] * B, [Sk] * B)


def custom(name: str, batch: int, heads: int, heads_k: int, seqlen_q: int,
           seqlen_k: int, head_dim: int, causal: bool, seed: int,
           window: Optional[Tuple[int, int]] = None, softcap: float = 0.0,
           dropout: Optional[Tuple[float, int, int]] = None) -> Workload:
    """A dense workload of any shape (used for ragged / edge-case tests)."""
    return Workload(name, batch, heads, heads_k, seqlen_q, seqlen_k, head_dim,
                    causal, seed=seed, window=window, softcap=softcap, dropout=dropout)


def custom_varlen(name: str, lens_q: List[int], lens_k: List[int], heads: int,
                  heads_k: int, head_dim: int, causal: bool, seed: int,
                  dtype=torch.bfloat16, window: Optional[Tuple[int, int]] = None,
                  softcap: float = 0.0,
                  dropout: Optional[Tuple[float, int, int]] = None) -> Inputs:
    """Packed inputs with explicit (possibly unequal or zero) q/k lengths."""
    wl = Workload(name, len(lens_q), heads, heads_k, 0, 0, head_dim, causal,
                  varlen=True, seed=seed, window=window, softcap=softcap, dropout=dropout)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    Tq, Tk = sum(lens_q), sum(lens_k)
    q = _randn(gen, (Tq, heads, head_dim), dtype)
    k = _randn(gen, (Tk, heads_k, head_dim), dtype)
    v = _randn(gen, (Tk, heads_k, head_dim), dtype)
    do = _randn(gen, (Tq, heads, head_dim), dtype)
    return Inputs(wl, q, k, v, do, list(lens_q), list(lens_k))
