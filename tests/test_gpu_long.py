"""GPU parity on long single-sequence walks, element by element.

The full-size workload tests can afford the oracle only for keys near the end
of a causal sequence (few queries see them).  Here sequences of 16k-32k
tokens are compared on the keys whose dK/dV walks are the longest (key 0 of a
causal sequence is seen by every later query of every head of its group) and
on a block in the middle, against the fp64 oracle, with each of the dK/dV
kernel's schedules the launcher picks by size:

* split: 2 splits of the query walk and their fixed-order reduce (S=16384,
  GQA 7 -> 1 as a 131072-token rank has: 16384 x 7 query rows for key 0);
* unsplit with key tiles banded per XCD (S=32768, 3 KV heads);
* the balanced schedule whose long items are cut into parts (S=32768);

plus dsink on a long causal layer with sinks against the oracle over every
row, and the ring inner step at a size where its chunk forward runs unsplit.
Calls go through the plain head-layout entry points (one rank's tensors).
"""
import pytest
import torch

import oracle
from gpu_util import LSE_MAX, LSE_MEAN, assert_close_tol, say
from ulysses_inputs import small_case

pytestmark = pytest.mark.gpu

LONG = [
    # id, S, Hq, Hkv, D, sink, key blocks (start, count)
    ("split_s16384_gqa7_d128", 16384, 7, 1, 128, False, ((0, 64), (8192, 64), (16320, 64))),
    ("banded_s32768_gqa2_d64", 32768, 6, 3, 64, False, ((0, 32), (16384, 32))),
    ("balanced_s32768_gqa2_d64", 32768, 4, 2, 64, False, ((0, 32), (12800, 32), (32736, 32))),
    ("sink_split_s16384_gqa8_d64", 16384, 8, 1, 64, True, ((0, 32), (8000, 32))),
]


def _rows(S):
    rows = set(range(0, 8)) | set(range(S // 2 - 4, S // 2 + 4)) | set(range(S - 8, S))
    g = torch.Generator().manual_seed(S)
    rows |= set(torch.randint(0, S, (40,), generator=g).tolist())
    return sorted(rows)


@pytest.mark.parametrize("row", LONG, ids=[r[0] for r in LONG])
def test_long_walks_match_oracle(row):
    import ulysses_sequence_attention_rank_amd as uly
    name, S, Hq, Hkv, D, sink, blocks = row
    inp = small_case(1200 + LONG.index(row), P=1, B=1, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink)
    dev = torch.device("cuda", 0)
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.dout))
    sk = None if inp.sink is None else inp.sink.to(dev)
    say(f"long walks {name}: forward and backward")
    o, lse = uly.attn_fwd(q, k, v, sink=sk, causal=True)
    dq, dk, dv, ds = uly.attn_bwd(q, k, v, o, do, lse, sink=sk, causal=True)
    torch.cuda.synchronize()

    keys = sorted({j for s0, n in blocks for j in range(s0, min(s0 + n, S))})
    rows = _rows(S)
    say(f"long walks {name}: oracle on {len(rows)} rows and {len(keys)} keys "
        f"(key {keys[0]} sees {S - keys[0]} queries per head)")
    kw = dict(sink=inp.sink, causal=True)
    wo, wl = oracle.attn_fwd(inp.q, inp.k, inp.v, rows=rows, **kw)
    wdq, _, _, _ = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, qrows=rows, want_dkdv=False,
                                   want_dsink=False, **kw)
    _, wdk, wdv, wds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, krows=keys, want_dq=False,
                                       want_dsink=sink, **kw)
    r, kx = torch.tensor(rows), torch.tensor(keys)
    assert_close_tol(o.reshape(S, Hq, D)[r.to(dev)], wo, "O")
    assert_close_tol(lse[0].T[r.to(dev)], wl, "LSE", max_abs=LSE_MAX, mean_abs=LSE_MEAN)
    assert_close_tol(dq.reshape(S, Hq, D)[r.to(dev)], wdq, "dQ")
    assert_close_tol(dk.reshape(S, Hkv, D)[kx.to(dev)], wdk, "dK (long walks)")
    assert_close_tol(dv.reshape(S, Hkv, D)[kx.to(dev)], wdv, "dV (long walks)")
    if sink:
        assert_close_tol(ds, wds, "dsink (every row)")


def test_ring_chunks_unsplit_match_oracle():
    """The ring inner step at S=32768 (8 query heads, 1 KV head, D=128, causal):
    four KV chunks whose forward runs unsplit, merged exactly; chunk results
    and the merged output against the oracle on sampled rows."""
    import ulysses_sequence_attention_rank_amd as uly
    S, Hq, Hkv, D, C = 32768, 8, 1, 128, 4
    inp = small_case(1300, P=1, B=1, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=True)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    rows = _rows(S)
    r = torch.tensor(rows)
    Sk = S // C
    acc_o = acc_l = None
    parts = []
    for c in range(C):
        lo, hi = c * Sk, (c + 1) * Sk
        say(f"ring S={S}: chunk [{lo}, {hi})")
        o, l = uly.attn_fwd_chunk(q, k[:, lo:hi], v[:, lo:hi], lo, causal=True)
        wo, wl = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True, keys=(lo, hi), rows=rows)
        parts.append((wo, wl))
        torch.cuda.synchronize()
        go = o.reshape(S, Hq, D)[r.to(dev)]
        gl = l[0].T[r.to(dev)].double().cpu()
        assert_close_tol(go, wo, f"chunk {c} O")
        fin = torch.isfinite(wl)
        assert torch.equal(torch.isfinite(gl), fin)
        assert_close_tol(gl[fin], wl[fin], f"chunk {c} LSE", max_abs=LSE_MAX, mean_abs=LSE_MEAN)
        if acc_o is None:
            acc_o, acc_l = o.clone(), l.clone()
        else:
            uly.attn_merge(acc_o, acc_l, o, l)
    out, lse = uly.attn_merge_finish(acc_o, acc_l, sink=inp.sink.to(dev))
    torch.cuda.synchronize()
    fo, fl = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, causal=True, rows=rows)
    assert_close_tol(out.reshape(S, Hq, D)[r.to(dev)], fo, "merged O vs every key")
    assert_close_tol(lse[0].T[r.to(dev)], fl, "merged LSE vs every key", max_abs=LSE_MAX,
                     mean_abs=LSE_MEAN)
