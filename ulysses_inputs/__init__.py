"""Seeded synthetic inputs for the per-rank Ulysses attention path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no attention, no permutation formula, no segment scan).
Both the CPU oracle tests and the HIP path take their inputs from here, so the
two sides see the very same bf16 bits.

Recipe (the pages run random bf16 tensors of shape [batch, seq, heads, dim],
see the long-context-attention issue "usage with pytorch FSDP", its test
script; the workloads below are the five simulated Ulysses configurations):

* one CPU ``torch.Generator().manual_seed(seed)`` per case, drawn in the fixed
  order: document lengths (packed varlen only), q, k, v, dout (fp32 ``randn``
  rounded once to bf16, round-to-nearest-even), then the sink logits (fp32
  ``randn``, only when the case has sinks);
* tensors are the full, unsharded ``[B, S, H, D]`` ones; the P sequence shards
  are contiguous slices in rank order (rank r holds tokens
  ``[r*S/P, (r+1)*S/P)``), as the accelerate PR "Add an FSDP2-native Ulysses
  sequence parallelism backend" numbers shards by where they sit;
* position_ids are ``arange(S)`` per batch row, or restart at 0 at every
  document start for packed inputs (the padding-free collator convention of
  the transformers issue "Add support for context parallelism", example 2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import torch

__all__ = ["Case", "WORKLOADS", "config_case", "make_inputs", "doc_lengths_uniform", "MlpInputs",
           "make_mlp_inputs",
           "positions_from_doc_lengths", "seq_shards"]


@dataclasses.dataclass(frozen=True)
class Variant:
    """One attention layer type run over the same inputs."""
    name: str
    causal: bool
    window_left: int = -1
    window_right: int = -1


@dataclasses.dataclass(frozen=True)
class Case:
    """Shape and mask description of one simulated Ulysses workload."""
    name: str
    seed: int
    P: int
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    variants: Tuple[Variant, ...]
    sink: bool = False
    doc_len_range: Optional[Tuple[int, int]] = None  # packed varlen: uniform [lo, hi]

    @property
    def hq(self) -> int:
        return self.Hq // self.P

    @property
    def hkv(self) -> int:
        """KV heads a rank holds (one, replicated, when there are fewer KV heads than ranks)."""
        return max(1, self.Hkv // self.P)

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)


CAUSAL = Variant("causal", True)
FULL = Variant("full", False)

# The five workloads: shapes, head counts, masks and sinks as listed for the
# simulated configurations (sequence lengths 512 .. 131072).
WORKLOADS = {
    1: Case("s512_h8_d64_causal", 1, P=2, B=1, S=512, Hq=8, Hkv=8, D=64, variants=(CAUSAL,)),
    2: Case("s4096_h12_d128", 2, P=2, B=1, S=4096, Hq=12, Hkv=12, D=128, variants=(FULL, CAUSAL)),
    3: Case("s32768_varlen_gqa32x8_d128", 3, P=4, B=1, S=32768, Hq=32, Hkv=8, D=128,
            variants=(CAUSAL,), doc_len_range=(512, 8192)),
    4: Case("s65536_gqa64x8_d64_swa128_sink", 4, P=8, B=1, S=65536, Hq=64, Hkv=8, D=64,
            variants=(Variant("swa128", True, 127, -1), CAUSAL), sink=True),
    5: Case("s131072_gqa28x4_d128_causal", 5, P=4, B=1, S=131072, Hq=28, Hkv=4, D=128,
            variants=(CAUSAL,)),
    # the packed workload over 16 ranks: 8 KV heads for 16 ranks, so each KV
    # head is replicated to 2 ranks (same seed, documents and tensors as 3)
    6: Case("s32768_varlen_gqa32x8_d128_p16_kvrep", 3, P=16, B=1, S=32768, Hq=32, Hkv=8, D=128,
            variants=(CAUSAL,), doc_len_range=(512, 8192)),
}


def config_case(cfg_id: int) -> Case:
    return WORKLOADS[cfg_id]


def doc_lengths_uniform(g: torch.Generator, total: int, lo: int, hi: int) -> List[int]:
    """Draw document lengths uniform in [lo, hi] until they cover ``total`` tokens.

    64 draws are taken in one call; the prefix whose running sum first reaches
    ``total`` is kept and the last document is cut to fit.
    """
    lens = torch.randint(lo, hi + 1, (64,), generator=g)
    out: List[int] = []
    acc = 0
    for x in lens.tolist():
        take = min(int(x), total - acc)
        out.append(take)
        acc += take
        if acc == total:
            return out
    raise ValueError("64 draws did not cover the sequence")


def positions_from_doc_lengths(lengths: Sequence[int]) -> torch.Tensor:
    """position_ids restarting at 0 at every document start (int64)."""
    return torch.cat([torch.arange(n, dtype=torch.int64) for n in lengths])


def seq_shards(full: torch.Tensor, P: int) -> torch.Tensor:
    """Split a ``[B, S, ...]`` tensor into ``[P, B, S/P, ...]`` contiguous rank shards."""
    B, S = full.shape[0], full.shape[1]
    assert S % P == 0
    return full.reshape(B, P, S // P, *full.shape[2:]).transpose(0, 1).contiguous()


@dataclasses.dataclass
class Inputs:
    case: Case
    q: torch.Tensor          # bf16 [B, S, Hq, D]
    k: torch.Tensor          # bf16 [B, S, Hkv, D]
    v: torch.Tensor          # bf16 [B, S, Hkv, D]
    dout: torch.Tensor       # bf16 [B, S, Hq, D]
    sink: Optional[torch.Tensor]   # fp32 [Hq]
    positions: torch.Tensor  # int64 [B, S]
    doc_lengths: Optional[List[int]]


def _randn_bf16(g: torch.Generator, shape, device=None) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_inputs(case: Case, *, with_dout: bool = True) -> Inputs:
    """Draw every input of ``case`` from its seed, in the fixed order."""
    g = torch.Generator().manual_seed(case.seed)
    doc_lengths = None
    if case.doc_len_range is not None:
        assert case.B == 1, "packed varlen inputs are drawn for one batch row"
        doc_lengths = doc_lengths_uniform(g, case.S, *case.doc_len_range)
    B, S, D = case.B, case.S, case.D
    q = _randn_bf16(g, (B, S, case.Hq, D))
    k = _randn_bf16(g, (B, S, case.Hkv, D))
    v = _randn_bf16(g, (B, S, case.Hkv, D))
    dout = _randn_bf16(g, (B, S, case.Hq, D)) if with_dout else None
    sink = torch.randn(case.Hq, generator=g, dtype=torch.float32) if case.sink else None
    if doc_lengths is not None:
        pos = positions_from_doc_lengths(doc_lengths).reshape(1, S)
    else:
        pos = torch.arange(S, dtype=torch.int64).repeat(B, 1)
    return Inputs(case, q, k, v, dout, sink, pos, doc_lengths)


def small_case(seed: int, *, P: int, B: int, S: int, Hq: int, Hkv: int, D: int,
               variants=(CAUSAL,), sink: bool = False,
               doc_lengths: Optional[Sequence[Sequence[int]]] = None) -> Inputs:
    """Inputs for an arbitrary test shape, drawn in the same order as the configs.

    ``doc_lengths`` gives, per batch row, fixed document lengths (no draw).
    """
    case = Case(f"test{seed}", seed, P, B, S, Hq, Hkv, D, tuple(variants), sink)
    g = torch.Generator().manual_seed(seed)
    q = _randn_bf16(g, (B, S, Hq, D))
    k = _randn_bf16(g, (B, S, Hkv, D))
    v = _randn_bf16(g, (B, S, Hkv, D))
    dout = _randn_bf16(g, (B, S, Hq, D))
    sk = torch.randn(Hq, generator=g, dtype=torch.float32) if sink else None
    if doc_lengths is not None:
        pos = torch.stack([positions_from_doc_lengths(r) for r in doc_lengths])
        flat = [x for r in doc_lengths for x in r]
    else:
        pos = torch.arange(S, dtype=torch.int64).repeat(B, 1)
        flat = None
    return Inputs(case, q, k, v, dout, sk, pos, flat)


# ------------------------------------------------------------ tiled MLP inputs
#
# The gated MLP of one rank's tokens: x [T][H], gate and up weights [I][H],
# down weight [H][I], output gradient dy [T][H], all bf16 (fp32 normal draws
# rounded to nearest even).  The weights are drawn with standard deviation
# 1/sqrt(fan-in) (gate, up: H; down: I), so the projections have unit scale.
@dataclasses.dataclass
class MlpInputs:
    x: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    dy: torch.Tensor


def make_mlp_inputs(seed: int, T: int, H: int, I: int, device=None) -> MlpInputs:
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g)
    wg = torch.randn(I, H, generator=g) / math.sqrt(H)
    wu = torch.randn(I, H, generator=g) / math.sqrt(H)
    wd = torch.randn(H, I, generator=g) / math.sqrt(I)
    dy = torch.randn(T, H, generator=g)
    def cvt(t):
        t = t.to(torch.bfloat16)
        return t.to(device) if device is not None else t
    return MlpInputs(cvt(x), cvt(wg), cvt(wu), cvt(wd), cvt(dy))
