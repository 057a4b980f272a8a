"""GPU parity of the fused layout: attention reading Q/K/V and writing
O/dQ/dK/dV in place in the sequence shards (and in the wrapper's
[B, H, S/P, D] form), through ulysses_attn_{fwd,bwd}_layout.

The fused step computes the same products on the same values as the
pack -> attention -> unpack step, so its outputs must be bit-identical to it;
it is also compared with the fp64 oracle directly.  Cases cover B = 1 (whose
sequence-shard rows have one stride) and B = 2 (rows that jump at every
shard and batch boundary), GQA, sinks, windows and packed documents.
"""
import zlib

import pytest
import torch

import oracle
from gpu_util import LSE_MAX, LSE_MEAN, assert_close_tol, bits_equal, say
from test_gpu_small import CASES
from ulysses_inputs import seq_shards, small_case

pytestmark = pytest.mark.gpu


def _bufs(row):
    from ulysses_sequence_attention_rank_amd import sim
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp = small_case(zlib.crc32(name.encode()) % 10000, P=P, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink,
                     doc_lengths=docs)
    dev = torch.device("cuda", 0)
    bufs = sim.allocate(seq_shards(inp.q, P).to(dev), seq_shards(inp.k, P).to(dev),
                        seq_shards(inp.v, P).to(dev), seq_shards(inp.dout, P).to(dev),
                        seq_shards(inp.positions, P).to(dev),
                        None if inp.sink is None else inp.sink.to(dev))
    return inp, bufs


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_fused_step_equals_packed_step(row):
    from ulysses_sequence_attention_rank_amd import sim
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp, b = _bufs(row)
    kw = dict(causal=causal, window_left=wl, window_right=wr)
    say(f"fused step {name}: packed")
    sim.step(b, **kw)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (b.o_seq, b.dq_seq, b.dk_seq, b.dv_seq, b.lse)]
    ref_ds = None if b.dsink is None else b.dsink.clone()
    for t in (b.o_seq, b.dq_seq, b.dk_seq, b.dv_seq, b.lse):
        t.fill_(float("nan"))
    say(f"fused step {name}: fused")
    sim.step(b, fused=True, **kw)
    torch.cuda.synchronize()
    for want, got in zip(ref, (b.o_seq, b.dq_seq, b.dk_seq, b.dv_seq, b.lse)):
        assert bits_equal(want, got)
    if ref_ds is not None:
        assert bits_equal(ref_ds, b.dsink)
    # and directly against the oracle
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    okw = dict(sink=inp.sink, cu=cu if docs is not None else None, causal=causal, window_left=wl,
               window_right=wr)
    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, **okw)
    dq, dk, dv, ds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **okw)
    shard = lambda x, H: seq_shards(x.reshape(B, S, H, D), P)
    assert_close_tol(b.o_seq, shard(o, Hq), "O")
    assert_close_tol(b.dq_seq, shard(dq, Hq), "dQ")
    assert_close_tol(b.dk_seq, shard(dk, Hkv), "dK")
    assert_close_tol(b.dv_seq, shard(dv, Hkv), "dV")
    hq = Hq // P
    assert_close_tol(b.lse, lse.reshape(B, S, P, hq).permute(2, 0, 3, 1), "LSE", max_abs=LSE_MAX,
                     mean_abs=LSE_MEAN)


@pytest.mark.parametrize("row", [CASES[2], CASES[6]], ids=[CASES[2][0], CASES[6][0]])
def test_wrapper_layout_equals_packed(row):
    """The accelerate wrapper's per-shard [B, H, S/P, D] tensors, read and
    written in place (views [P, B, S/P, h, D] of [P, B, H, S/P, D] storage)."""
    import ulysses_sequence_attention_rank_amd as uly
    from ulysses_sequence_attention_rank_amd import sim
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp, b = _bufs(row)
    kw = dict(causal=causal, window_left=wl, window_right=wr)
    sim.step(b, **kw)
    torch.cuda.synchronize()
    hq, hkv = Hq // P, Hkv // P
    # [P, B, S/P, H, D] -> storage [P, B, H, S/P, D], viewed back as [P, B, S/P, H, D]
    to_wrapper = lambda x: x.permute(0, 1, 3, 2, 4).contiguous().permute(0, 1, 3, 2, 4)
    q, k, v, do = (to_wrapper(x) for x in (b.q_seq, b.k_seq, b.v_seq, b.dout_seq))
    o, dq = to_wrapper(torch.zeros_like(b.q_seq)), to_wrapper(torch.zeros_like(b.q_seq))
    dk, dv = to_wrapper(torch.zeros_like(b.k_seq)), to_wrapper(torch.zeros_like(b.k_seq))
    lse = torch.empty_like(b.lse)
    dsink = None if b.dsink is None else torch.empty_like(b.dsink)
    say(f"wrapper layout {name}")
    for r in range(P):
        qs, ks = slice(r * hq, (r + 1) * hq), slice(r * hkv, (r + 1) * hkv)
        sk = None if b.sink is None else b.sink[qs]
        uly.attn_fwd(q[:, :, :, qs], k[:, :, :, ks], v[:, :, :, ks], sink=sk, cu_seqlens=b.cu,
                     n_seqs=b.n_seqs, out=o[:, :, :, qs], lse=lse[r], **kw)
        uly.attn_bwd(q[:, :, :, qs], k[:, :, :, ks], v[:, :, :, ks], o[:, :, :, qs],
                     do[:, :, :, qs], lse[r], sink=sk, cu_seqlens=b.cu, n_seqs=b.n_seqs,
                     dq=dq[:, :, :, qs], dk=dk[:, :, :, ks], dv=dv[:, :, :, ks],
                     dsink=None if dsink is None else dsink[qs], **kw)
    torch.cuda.synchronize()
    for want, got in ((b.o_seq, o), (b.dq_seq, dq), (b.dk_seq, dk), (b.dv_seq, dv), (b.lse, lse)):
        assert bits_equal(want, got.contiguous())
    if dsink is not None:
        assert bits_equal(b.dsink, dsink)
    # and directly against the oracle, read from the wrapper-layout storage
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    okw = dict(sink=inp.sink, cu=cu if docs is not None else None, causal=causal, window_left=wl,
               window_right=wr)
    wo, _ = oracle.attn_fwd(inp.q, inp.k, inp.v, **okw)
    wdq, wdk, wdv, wds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **okw)
    shard = lambda x, H: seq_shards(x.reshape(B, S, H, D), P)
    assert_close_tol(o, shard(wo, Hq), "wrapper O")
    assert_close_tol(dq, shard(wdq, Hq), "wrapper dQ")
    assert_close_tol(dk, shard(wdk, Hkv), "wrapper dK")
    assert_close_tol(dv, shard(wdv, Hkv), "wrapper dV")
    if dsink is not None:
        assert_close_tol(dsink, wds, "wrapper dsink")
