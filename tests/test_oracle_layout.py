"""Pins of the oracle's layout permutation and segment scan (CPU only).

The permutation is the sequence-to-head all-to-all of the accelerate PR "Add
an FSDP2-native Ulysses sequence parallelism backend" (reply on the four
all-to-all call sites); the scan rebuilds cu_seqlens / max_len from the
gathered position_ids (same PR, comment on the flash-attention kwargs).
"""
import pytest
import torch

import oracle
from ulysses_inputs import (WORKLOADS, doc_lengths_uniform, make_inputs,
                            positions_from_doc_lengths, seq_shards)


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _full(B, S, H, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    if dtype.is_floating_point:
        return torch.randn(B, S, H, D, generator=g).to(dtype)
    return torch.randint(-2**30, 2**30, (B, S, H, D), generator=g, dtype=torch.int32).to(dtype)


SHAPES = [(1, 2, 8, 4, 4), (2, 2, 6, 4, 3), (3, 1, 9, 6, 5), (4, 2, 16, 28, 8), (1, 3, 7, 2, 1),
          (8, 1, 16, 8, 2)]


@pytest.mark.parametrize("P,B,S,H,D", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.int32])
def test_pack_matches_view_permute(P, B, S, H, D, dtype):
    """Brute-force index formula == an independent torch view/permute, bit for bit."""
    full = _full(B, S, H, D, dtype, seed=P * 100 + S)
    seq = seq_shards(full, P)                      # [P, B, S/P, H, D]
    head = oracle.pack(seq)                        # [P, B, S, H/P, D]
    expect = full.reshape(B, S, P, H // P, D).permute(2, 0, 1, 3, 4)
    assert torch.equal(_bits(head), _bits(expect))
    back = oracle.unpack(head)
    assert torch.equal(_bits(back), _bits(seq))


def test_pack_p1_is_identity():
    full = _full(2, 5, 3, 4, torch.bfloat16, 7)
    seq = seq_shards(full, 1)
    assert torch.equal(_bits(oracle.pack(seq)), _bits(seq))


def test_pack_rank_heads_are_contiguous_chunks():
    """Rank c receives global heads [c*H/P, (c+1)*H/P) for every gathered token."""
    P, B, S, H, D = 4, 1, 8, 8, 2
    full = torch.zeros(B, S, H, D, dtype=torch.int32)
    for t in range(S):
        for h in range(H):
            full[0, t, h, :] = 1000 * t + h
    head = oracle.pack(seq_shards(full, P))
    for c in range(P):
        for t in range(S):
            for hh in range(H // P):
                assert int(head[c, 0, t, hh, 0]) == 1000 * t + c * (H // P) + hh


# ----------------------------------------------------------------- segments

def _starts_by_nonzero(pos):
    B, S = pos.shape
    flag = pos == 0
    flag[:, 0] = True
    return torch.nonzero(flag.reshape(-1)).reshape(-1).to(torch.int32)


@pytest.mark.parametrize("B,S,P", [(1, 16, 2), (2, 12, 3), (3, 40, 4), (1, 1, 1)])
def test_segments_vs_nonzero(B, S, P):
    g = torch.Generator().manual_seed(B * 31 + S)
    pos = torch.randint(0, 4, (B, S), generator=g, dtype=torch.int64)
    gathered = oracle.gather_positions(seq_shards(pos, P))
    assert torch.equal(gathered, pos)
    cu, n, mx = oracle.segments(gathered)
    starts = _starts_by_nonzero(pos)
    assert n == starts.numel()
    assert torch.equal(cu[:-1], starts)
    assert int(cu[-1]) == B * S
    assert mx == int(torch.diff(torch.cat([starts, torch.tensor([B * S], dtype=torch.int32)])).max())


def test_segments_arange_closed_form():
    for S in (1, 7, 512, 4096):
        cu, n, mx = oracle.segments(torch.arange(S).reshape(1, S))
        assert cu.tolist() == [0, S] and n == 1 and mx == S
    cu, n, mx = oracle.segments(torch.arange(6).repeat(3, 1))
    assert cu.tolist() == [0, 6, 12, 18] and n == 3 and mx == 6


def test_segments_int32_and_int64_positions_agree():
    lens = [5, 1, 9, 3]
    pos = positions_from_doc_lengths(lens).reshape(1, -1)
    a = oracle.segments(pos)
    b = oracle.segments(pos.to(torch.int32))
    assert torch.equal(a[0], b[0]) and a[1:] == b[1:]


def test_segments_packed_config_equals_drawn_lengths():
    """The packed 32768-token workload: cu is the running sum of the drawn lengths."""
    inp = make_inputs(WORKLOADS[3], with_dout=False)
    lens = inp.doc_lengths
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, 4)))
    expect = [0] + torch.cumsum(torch.tensor(lens), 0).tolist()
    assert cu.tolist() == expect
    assert n == len(lens) and mx == max(lens)


def test_segments_golden_fixture():
    """Stored cu_seqlens of the packed workload (tests/golden/segments_packed_s32768.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "segments_packed_s32768.json")
    gold = json.load(open(path))
    inp = make_inputs(WORKLOADS[3], with_dout=False)
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, 4)))
    assert cu.tolist() == gold["cu_seqlens"] and mx == gold["max_len"] and n == gold["n_seqs"]


def test_doc_length_draw_rule():
    g = torch.Generator().manual_seed(11)
    lens = doc_lengths_uniform(g, 20000, 512, 8192)
    assert sum(lens) == 20000 and all(1 <= x <= 8192 for x in lens)
    assert all(x >= 512 for x in lens[:-1])


def test_local_shard_cu_seqlens_differ_from_gathered():
    """Negative control: cu_seqlens computed from one rank's local position shard
    do not describe the gathered sequence (the PR's 41.8% mismatch finding, in kind)."""
    inp = make_inputs(WORKLOADS[3], with_dout=False)
    shards = seq_shards(inp.positions, 4)
    good, _, _ = oracle.segments(oracle.gather_positions(shards))
    local, _, _ = oracle.segments(shards[0])
    assert local.tolist() != good.tolist()
    assert int(local[-1]) == inp.case.S // 4 != int(good[-1])


# ---------------------------------------------- KV heads fewer than ranks

@pytest.mark.parametrize("P,H,B,S,D", [(4, 2, 1, 8, 3), (8, 1, 2, 16, 4), (6, 3, 1, 12, 2), (2, 2, 1, 4, 5)])
def test_pack_replicated_matches_repeat_interleave(P, H, B, S, D):
    """Rank c receives the KV head its query heads use: with the heads of the
    full tensor repeated R = P/H times (contiguous GQA groups), rank c's share
    of the repeated tensor is one head, number c."""
    g = torch.Generator().manual_seed(1000 * P + H)
    full = torch.randn((B, S, H, D), generator=g, dtype=torch.float64).to(torch.bfloat16)
    seq = full.reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()
    rep = full.repeat_interleave(P // H, dim=2)            # [B, S, P, D]
    want = rep.permute(2, 0, 1, 3).unsqueeze(3)            # [P, B, S, 1, D]
    got = oracle.pack_replicated(seq)
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))
    if H == P:  # one head per rank: the plain pack
        assert torch.equal(got.view(torch.int16), oracle.pack(seq).view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("P,H,B,S,D", [(4, 2, 1, 8, 3), (8, 1, 2, 16, 4), (6, 3, 1, 12, 2)])
def test_reduce_replicated_is_the_rank_order_fp32_sum(P, H, B, S, D, dtype):
    g = torch.Generator().manual_seed(77 * P + H)
    head = (torch.randn((P, B, S, 1, D), generator=g, dtype=torch.float64) *
            torch.exp(2 * torch.randn((P, B, S, 1, D), generator=g, dtype=torch.float64))).to(dtype)
    got = oracle.reduce_replicated(head, H)
    R, Sl = P // H, S // P
    acc = torch.zeros((H, B, S, D), dtype=torch.float32)
    for j in range(R):                                     # rank order, fp32
        acc = acc + head[j::R, :, :, 0].float()
    want = acc.to(torch.bfloat16).permute(1, 2, 0, 3).reshape(B, P, Sl, H, D).permute(1, 0, 2, 3, 4)
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))


def test_reduce_replicated_closed_forms():
    # equal replicas sum to R times the value (exact for powers of two); R = 1 is the plain unpack
    P, H, B, S, D = 8, 2, 1, 8, 4
    base = torch.randn((H, B, S, D), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    head = base.repeat_interleave(P // H, dim=0).unsqueeze(3)   # [P, B, S, 1, D]
    got = oracle.reduce_replicated(head, H)
    want = (base.float() * 4).to(torch.bfloat16).permute(1, 2, 0, 3).reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4)
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))
    x = torch.randn((4, 1, 8, 1, 3), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    assert torch.equal(oracle.reduce_replicated(x, 4).view(torch.int16), oracle.unpack(x).view(torch.int16))
