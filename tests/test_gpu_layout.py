"""GPU parity of the layout permutation through the C ABI: single and
multi-tensor pack/unpack against the oracle's brute-force permutation,
bit-exact, for several element widths, GQA head counts and ragged shapes."""
import zlib

import pytest
import torch

import oracle
from gpu_util import bits_equal, say

pytestmark = pytest.mark.gpu

CASES = [
    # id, P, B, S, heads of each tensor, D, dtype
    ("qkv_gqa_bf16", 4, 1, 64, (8, 4, 4), 128, torch.bfloat16),
    ("qkv_b2_fp32", 2, 2, 30, (6, 2, 2), 64, torch.float32),
    ("odd_d_bf16", 2, 1, 10, (4, 2), 3, torch.bfloat16),  # runs of 6 bytes: narrow vectors
    ("one_tensor_int64", 8, 1, 16, (8,), 16, torch.int64),
]


def _rand(shape, dtype, g):
    if dtype.is_floating_point:
        return torch.randn(shape, generator=g).to(dtype)
    return torch.randint(-2 ** 62, 2 ** 62, shape, generator=g, dtype=dtype)


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_multi_pack_unpack_bit_exact(row):
    import ulysses_sequence_attention_rank_amd as uly
    name, P, B, S, heads, D, dtype = row
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    seqs = [_rand((P, B, S // P, H, D), dtype, g) for H in heads]
    dev = torch.device("cuda", 0)
    seq_d = [x.to(dev) for x in seqs]
    head_d = [torch.empty((P, B, S, H // P, D), dtype=dtype, device=dev) for H in heads]
    say(f"layout multi {name}")
    uly.a2a_pack_multi_into(seq_d, head_d, P)
    back = [torch.empty_like(x) for x in seq_d]
    uly.a2a_unpack_multi_into(head_d, back, P)
    single = [uly.a2a_pack(x) for x in seq_d]
    torch.cuda.synchronize()
    for x, h, b, s1 in zip(seqs, head_d, back, single):
        want = oracle.pack(x.view(torch.int16) if dtype == torch.bfloat16 else x)
        got = h.cpu()
        got = got.view(torch.int16) if dtype == torch.bfloat16 else got
        assert torch.equal(got, want)          # the oracle's permutation, bit for bit
        assert bits_equal(s1, h)               # one launch per tensor == one launch for all
        assert bits_equal(b, x.to(dev))        # unpack(pack(x)) == x


REP_CASES = [
    # id, P, B, S, H (KV heads, fewer than P), D, dtype
    ("rep4_bf16", 8, 1, 32, 2, 128, torch.bfloat16),
    ("rep2_b2_fp32", 4, 2, 12, 2, 64, torch.float32),
    ("rep8_one_head", 8, 1, 16, 1, 8, torch.bfloat16),
]


@pytest.mark.parametrize("row", REP_CASES, ids=[c[0] for c in REP_CASES])
def test_replicated_pack_and_gradient_sum_bit_exact(row):
    import ulysses_sequence_attention_rank_amd as uly
    name, P, B, S, H, D, dtype = row
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    seq = _rand((P, B, S // P, H, D), dtype, g)
    dev = torch.device("cuda", 0)
    head = torch.empty((P, B, S, 1, D), dtype=dtype, device=dev)
    say(f"replicated pack {name}")
    uly.a2a_pack_replicated_into(seq.to(dev), head, P)
    torch.cuda.synchronize()
    want = oracle.pack_replicated(seq)
    assert bits_equal(head, want)
    if dtype == torch.bfloat16:
        for gdt in (torch.bfloat16, torch.float32):   # replica gradients as stored
            grads = (torch.randn((P, B, S, 1, D), generator=g) *
                     torch.exp(2 * torch.randn((P, B, S, 1, D), generator=g))).to(gdt)
            out = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=dev)
            say(f"replica gradient sum {name} {gdt}")
            uly.a2a_reduce_replicated_into(grads.to(dev), out, P)
            torch.cuda.synchronize()
            assert bits_equal(out, oracle.reduce_replicated(grads, H))


# id, P, B, S, kind of positions, dtype
SEG_CASES = [
    ("every_token_starts", 2, 1, 96, "zeros", torch.int64),      # n = B*S documents of length 1
    ("one_doc", 4, 1, 4096, "arange", torch.int32),
    ("b3_ragged_chunks", 3, 3, 2997, "docs", torch.int64),      # T not a multiple of the threads
    ("long_chunks_int32", 4, 1, 262144, "docs", torch.int32),   # 256 tokens a thread: many batches
    ("dense_restarts", 2, 2, 20000, "dense", torch.int64),
    # many-work-group scan: 1024 chunks of eight 512-token rounds, documents spanning chunks
    ("multi_round_chunks", 2, 1, 4194304, "docs", torch.int64),
    # 977 chunks of twelve rounds, short documents, two batch rows, int32
    ("multi_round_dense_b2", 1, 2, 3000000, "dense", torch.int32),
]


def _positions(kind, B, S, g):
    if kind == "zeros":
        return torch.zeros(B, S, dtype=torch.int64)
    if kind == "arange":
        return torch.arange(S, dtype=torch.int64).repeat(B, 1)
    hi = 40 if kind == "dense" else 5000
    rows = []
    for _ in range(B):
        row, t = [], 0
        while t < S:
            n = min(int(torch.randint(1, hi, (1,), generator=g)), S - t)
            row.append(torch.arange(n, dtype=torch.int64))
            t += n
        rows.append(torch.cat(row))
    return torch.stack(rows)


@pytest.mark.parametrize("path", ["wide", "one_group"])
@pytest.mark.parametrize("row", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_cu_seqlens_edge_cases_bit_exact(row, path):
    """Both scans: the many-work-group one (cu_seqlens with room for its
    scratch, ulysses_cu_seqlens_capacity) and the one-work-group one (exactly
    B*S + 1 slots)."""
    import ulysses_sequence_attention_rank_amd as uly
    name, P, B, S, kind, dtype = row
    if path == "one_group" and B * S > 300000:
        pytest.skip("the one-work-group scan is exercised on the smaller cases")
    say(f"cu_seqlens {name} ({path}): P={P} B={B} S={S} {kind} {dtype}")
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    pos = _positions(kind, B, S, g)
    shards = pos.reshape(B, P, S // P).permute(1, 0, 2).contiguous().to(dtype)
    want_cu, want_n, want_mx = oracle.segments(oracle.gather_positions(shards))
    cap = uly.cu_seqlens_capacity(B, S) if path == "wide" else B * S + 1
    assert cap >= B * S + 1
    cu = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    cu, n, mx = uly.cu_seqlens_from_positions(shards.cuda(), cu=cu)
    torch.cuda.synchronize()
    assert int(n.item()) == want_n and int(mx.item()) == want_mx
    assert torch.equal(cu[: want_n + 1].cpu(), want_cu)
