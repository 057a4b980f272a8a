"""One simulated Ulysses step on one GPU: P ranks held in memory.

The step follows the accelerate PR "Add an FSDP2-native Ulysses sequence
parallelism backend": the position_ids are gathered once and cu_seqlens /
max_len rebuilt from them; Q, K, V go from sequence shards to head shards
(the sequence-to-head all-to-all); every rank runs attention over the whole
sequence for its heads with its slice of the sink logits; the output goes
back to sequence shards.  Backward mirrors it: dO is packed, each rank runs
the attention backward, dQ/dK/dV are unpacked (the all-to-all's backward is
the same exchange with its directions exchanged).
The exchange itself is a permutation here (one GPU); every step is a call
into the HIP library.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

from . import (a2a_pack_into, a2a_pack_multi_into, a2a_pack_replicated_into,
               a2a_reduce_replicated_into, a2a_unpack_into, a2a_unpack_multi_into, attn_bwd,
               attn_bwd_workspace_bytes, attn_fwd, attn_fwd_workspace_bytes, cu_seqlens_capacity,
               cu_seqlens_from_positions)


@dataclasses.dataclass
class StepBuffers:
    """Device buffers of one step; allocated once, reused by every call."""
    P: int
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    q_seq: torch.Tensor
    k_seq: torch.Tensor
    v_seq: torch.Tensor
    dout_seq: torch.Tensor
    pos_seq: torch.Tensor
    sink: Optional[torch.Tensor]
    # head-sharded (per rank) tensors
    q_head: torch.Tensor = None
    k_head: torch.Tensor = None
    v_head: torch.Tensor = None
    o_head: torch.Tensor = None
    do_head: torch.Tensor = None
    dq_head: torch.Tensor = None
    dk_head: torch.Tensor = None
    dv_head: torch.Tensor = None
    lse: torch.Tensor = None
    dsink: Optional[torch.Tensor] = None
    o_seq: torch.Tensor = None
    dq_seq: torch.Tensor = None
    dk_seq: torch.Tensor = None
    dv_seq: torch.Tensor = None
    cu: torch.Tensor = None
    n_seqs: torch.Tensor = None
    max_len: torch.Tensor = None
    workspace: torch.Tensor = None

    @property
    def hq(self):
        return self.Hq // self.P

    @property
    def hkv(self):
        return max(1, self.Hkv // self.P)

    @property
    def replicated(self):
        """Fewer KV heads than ranks: each KV head is sent to P // Hkv ranks."""
        return self.Hkv < self.P


def allocate(q_seq, k_seq, v_seq, dout_seq, pos_seq, sink) -> StepBuffers:
    """Wrap device sequence shards ``[P, B, S/P, H, D]`` and allocate the rest."""
    P, B, Sl, Hq, D = q_seq.shape
    Hkv = k_seq.shape[3]
    S = P * Sl
    dev = q_seq.device
    bf = torch.bfloat16
    b = StepBuffers(P, B, S, Hq, Hkv, D, q_seq, k_seq, v_seq, dout_seq, pos_seq, sink)
    hq, hkv = Hq // P, max(1, Hkv // P)
    if Hkv < P and P % Hkv:
        raise ValueError(f"Hkv={Hkv} KV heads neither divisible by nor dividing P={P}")
    b.q_head = torch.empty((P, B, S, hq, D), dtype=bf, device=dev)
    b.k_head = torch.empty((P, B, S, hkv, D), dtype=bf, device=dev)
    b.v_head = torch.empty_like(b.k_head)
    b.o_head = torch.empty_like(b.q_head)
    b.do_head = torch.empty_like(b.q_head)
    b.dq_head = torch.empty_like(b.q_head)
    # replicated KV heads: each replica's dK/dV stays fp32 until their sum is rounded
    kv_grad = torch.float32 if Hkv < P else bf
    b.dk_head = torch.empty(b.k_head.shape, dtype=kv_grad, device=dev)
    b.dv_head = torch.empty(b.k_head.shape, dtype=kv_grad, device=dev)
    b.lse = torch.empty((P, B, hq, S), dtype=torch.float32, device=dev)
    b.dsink = torch.empty(Hq, dtype=torch.float32, device=dev) if sink is not None else None
    b.o_seq = torch.empty_like(q_seq)
    b.dq_seq = torch.empty_like(q_seq)
    b.dk_seq = torch.empty_like(k_seq)
    b.dv_seq = torch.empty_like(v_seq)
    b.cu = torch.empty(cu_seqlens_capacity(B, S), dtype=torch.int32, device=dev)
    b.n_seqs = torch.empty(1, dtype=torch.int32, device=dev)
    b.max_len = torch.empty(1, dtype=torch.int32, device=dev)
    # the forward and backward run one after the other on one stream: one workspace
    ws = max(attn_bwd_workspace_bytes(B, S, hq, hkv, D), attn_fwd_workspace_bytes(B, S, hq, hkv, D))
    b.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    return b


def _views(b: StepBuffers, r: int, fused: bool):
    """Rank r's attention operands: its slices of the head-shard buffers, or
    (fused) strided views of its heads in the sequence shards themselves."""
    hq, hkv = b.hq, b.hkv
    if not fused:
        return dict(q=b.q_head[r], k=b.k_head[r], v=b.v_head[r], o=b.o_head[r], do=b.do_head[r],
                    dq=b.dq_head[r], dk=b.dk_head[r], dv=b.dv_head[r])
    qs, ks = slice(r * hq, (r + 1) * hq), slice(r * hkv, (r + 1) * hkv)
    return dict(q=b.q_seq[:, :, :, qs], k=b.k_seq[:, :, :, ks], v=b.v_seq[:, :, :, ks],
                o=b.o_seq[:, :, :, qs], do=b.dout_seq[:, :, :, qs], dq=b.dq_seq[:, :, :, qs],
                dk=b.dk_seq[:, :, :, ks], dv=b.dv_seq[:, :, :, ks])


def forward(b: StepBuffers, *, causal: bool, window_left: int = -1, window_right: int = -1,
            ranks: Optional[Sequence[int]] = None, softmax_scale: Optional[float] = None,
            fused: bool = False):
    """Gather positions -> cu_seqlens, pack Q/K/V, attention per rank, unpack O.
    ``fused``: attention reads Q/K/V and writes O in the sequence shards
    directly (the permutation folded into its addressing), no pack/unpack."""
    ranks = range(b.P) if ranks is None else ranks
    fused = fused and not b.replicated  # replicas' dK/dV must be summed: head buffers
    cu_seqlens_from_positions(b.pos_seq, b.cu, b.n_seqs, b.max_len)
    if b.replicated:
        a2a_pack_into(b.q_seq, b.q_head, b.P)
        a2a_pack_replicated_into(b.k_seq, b.k_head, b.P)
        a2a_pack_replicated_into(b.v_seq, b.v_head, b.P)
    elif not fused:
        a2a_pack_multi_into((b.q_seq, b.k_seq, b.v_seq), (b.q_head, b.k_head, b.v_head), b.P)
    hq = b.hq
    for r in ranks:
        t = _views(b, r, fused)
        sk = None if b.sink is None else b.sink[r * hq:(r + 1) * hq]
        attn_fwd(t["q"], t["k"], t["v"], sink=sk, cu_seqlens=b.cu, n_seqs=b.n_seqs, causal=causal,
                 window_left=window_left, window_right=window_right, softmax_scale=softmax_scale,
                 out=t["o"], lse=b.lse[r], workspace=b.workspace)
    if not fused:
        a2a_unpack_into(b.o_head, b.o_seq, b.P)


def backward(b: StepBuffers, *, causal: bool, window_left: int = -1, window_right: int = -1,
             ranks: Optional[Sequence[int]] = None, softmax_scale: Optional[float] = None,
             fused: bool = False):
    """Pack dO, attention backward per rank, unpack dQ/dK/dV (``fused``: in
    place on the sequence shards, as in ``forward``)."""
    ranks = range(b.P) if ranks is None else ranks
    fused = fused and not b.replicated
    if not fused:
        a2a_pack_into(b.dout_seq, b.do_head, b.P)
    hq = b.hq
    for r in ranks:
        t = _views(b, r, fused)
        sk = None if b.sink is None else b.sink[r * hq:(r + 1) * hq]
        ds = None if b.dsink is None else b.dsink[r * hq:(r + 1) * hq]
        attn_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], b.lse[r], sink=sk, cu_seqlens=b.cu,
                 n_seqs=b.n_seqs, causal=causal, window_left=window_left,
                 window_right=window_right, softmax_scale=softmax_scale, dq=t["dq"], dk=t["dk"],
                 dv=t["dv"], dsink=ds, workspace=b.workspace, kv_grad_fp32=b.replicated)
    if b.replicated:
        a2a_unpack_into(b.dq_head, b.dq_seq, b.P)
        a2a_reduce_replicated_into(b.dk_head, b.dk_seq, b.P)
        a2a_reduce_replicated_into(b.dv_head, b.dv_seq, b.P)
    elif not fused:
        a2a_unpack_multi_into((b.dq_head, b.dk_head, b.dv_head), (b.dq_seq, b.dk_seq, b.dv_seq),
                              b.P)


def step(b: StepBuffers, *, causal: bool, window_left: int = -1, window_right: int = -1,
         ranks: Optional[Sequence[int]] = None, softmax_scale: Optional[float] = None,
         fused: bool = False):
    forward(b, causal=causal, window_left=window_left, window_right=window_right, ranks=ranks,
            softmax_scale=softmax_scale, fused=fused)
    backward(b, causal=causal, window_left=window_left, window_right=window_right, ranks=ranks,
             softmax_scale=softmax_scale, fused=fused)
