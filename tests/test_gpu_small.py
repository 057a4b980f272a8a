"""GPU parity on small shapes: the whole simulated step against the fp64 oracle.

Sizes span several 128-row tiles and ragged tails; the cases cover causal,
non-causal, packed varlen (documents straddling shard and tile boundaries,
one-token documents), sliding and two-sided windows, GQA with group sizes
1, 2, 4 and 7, sinks, batch > 1 and both head dims.
"""
import zlib

import pytest
import torch

import oracle
from gpu_util import LSE_MAX, LSE_MEAN, assert_close_tol, bits_equal, say
from ulysses_inputs import seq_shards, small_case

pytestmark = pytest.mark.gpu

CASES = [
    # id, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs
    ("causal_d64_ragged", 2, 1, 200, 4, 4, 64, True, -1, -1, False, None),
    ("full_d128_gqa2", 2, 1, 256, 4, 2, 128, False, -1, -1, False, None),
    ("causal_b2_sink_swa", 4, 2, 160, 8, 4, 128, True, 37, -1, True, None),
    ("varlen_causal_d64", 2, 1, 300, 8, 2, 64, True, -1, -1, False, [[70, 1, 129, 100]]),
    ("varlen_full_sink_d128", 2, 1, 260, 4, 2, 128, False, -1, -1, True, [[130, 3, 127]]),
    ("twosided_window_d64", 2, 1, 190, 4, 2, 64, False, 20, 11, False, None),
    ("varlen_b2_causal_swa", 2, 2, 136, 4, 4, 128, True, 15, -1, True, [[60, 76], [1, 135]]),
    ("gqa7_causal_d128", 2, 1, 192, 14, 2, 128, True, -1, -1, False, None),
    ("gqa8_sink_swa_d64", 2, 1, 384, 16, 2, 64, True, 127, -1, True, None),
    ("tiny_s2", 2, 1, 2, 2, 2, 64, True, -1, -1, True, None),
    # fewer KV heads than ranks: each KV head replicated to P / Hkv ranks
    ("kvrep4_causal_sink_d128", 8, 1, 256, 16, 2, 128, True, -1, -1, True, None),
    ("kvrep2_varlen_b2_swa_d64", 4, 2, 160, 8, 2, 64, True, 33, -1, False, [[90, 70], [1, 159]]),
]


def _run(row):
    from ulysses_sequence_attention_rank_amd import sim
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp = small_case(zlib.crc32(name.encode()) % 10000, P=P, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink,
                     doc_lengths=docs)
    dev = torch.device("cuda", 0)
    bufs = sim.allocate(seq_shards(inp.q, P).to(dev), seq_shards(inp.k, P).to(dev),
                        seq_shards(inp.v, P).to(dev), seq_shards(inp.dout, P).to(dev),
                        seq_shards(inp.positions, P).to(dev),
                        None if inp.sink is None else inp.sink.to(dev))
    say(f"small step {name}")
    sim.step(bufs, causal=causal, window_left=wl, window_right=wr)
    torch.cuda.synchronize()
    return inp, bufs


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_small_step_matches_oracle(row):
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp, b = _run(row)
    # the layout steps are bit-exact against the oracle's permutation
    assert bits_equal(b.q_head, oracle.pack(seq_shards(inp.q, P)))
    kpack = oracle.pack_replicated if Hkv < P else oracle.pack
    assert bits_equal(b.k_head, kpack(seq_shards(inp.k, P)))
    assert bits_equal(b.v_head, kpack(seq_shards(inp.v, P)))
    # cu_seqlens rebuilt from the gathered positions, bit-exact
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    assert int(b.n_seqs.item()) == n and int(b.max_len.item()) == mx
    assert torch.equal(b.cu[: n + 1].cpu(), cu)
    # attention: unsharded fp64 oracle, compared in the sequence-sharded layout
    kw = dict(sink=inp.sink, cu=cu if docs is not None else None, causal=causal,
              window_left=wl, window_right=wr)
    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, **kw)
    dq, dk, dv, ds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **kw)
    shard = lambda x, H: seq_shards(x.reshape(B, S, H, D), P)
    assert_close_tol(b.o_seq, shard(o, Hq), "O")
    assert_close_tol(b.dq_seq, shard(dq, Hq), "dQ")
    assert_close_tol(b.dk_seq, shard(dk, Hkv), "dK")
    assert_close_tol(b.dv_seq, shard(dv, Hkv), "dV")
    if sink:
        assert_close_tol(b.dsink, ds, "dsink")
    # LSE per rank [P][B][hq][S] vs oracle [B*S][Hq]
    hq = Hq // P
    want = lse.reshape(B, S, P, hq).permute(2, 0, 3, 1)
    assert_close_tol(b.lse, want, "LSE", max_abs=LSE_MAX, mean_abs=LSE_MEAN)


def test_repeat_runs_are_bit_identical():
    """Every kernel is deterministic (no atomics): two runs give identical bits."""
    row = CASES[6]
    _, b1 = _run(row)
    first = [t.clone() for t in (b1.o_seq, b1.dq_seq, b1.dk_seq, b1.dv_seq, b1.dsink, b1.cu)]
    from ulysses_sequence_attention_rank_amd import sim
    say("repeat run")
    sim.step(b1, causal=True, window_left=15)
    torch.cuda.synchronize()
    for a, c in zip(first, (b1.o_seq, b1.dq_seq, b1.dk_seq, b1.dv_seq, b1.dsink, b1.cu)):
        assert bits_equal(a, c)
