"""GPU parity of the ring inner step: attention of the rank's queries against
one KV chunk (ulysses_attn_fwd_chunk) and the exact LSE merge of the chunks
(ulysses_attn_merge, ulysses_attn_merge_finish), against the fp64 oracle's
chunk attention and merge, and against attention over every key."""
import zlib

import pytest
import torch

import oracle
from gpu_util import LSE_MAX, LSE_MEAN, assert_close_tol, say
from ulysses_inputs import small_case

pytestmark = pytest.mark.gpu

CASES = [
    # id, B, S, Hq, Hkv, D, causal, wl, sink, docs, chunk bounds
    ("causal_docs_d128", 1, 320, 4, 2, 128, True, -1, True, [[100, 1, 219]], (0, 100, 227, 320)),
    ("full_b2_d64", 2, 200, 4, 4, 64, False, -1, False, None, (0, 64, 65, 200)),
    ("swa_b2_gqa4_d128", 2, 256, 8, 2, 128, True, 37, True, None, (0, 130, 256)),
    ("causal_many_chunks_d64", 1, 512, 2, 1, 64, True, -1, True, None, tuple(range(0, 513, 64))),
]


def _lse_close(got, want, name):
    got, want = got.double().cpu(), want.double()
    fin = torch.isfinite(want)
    assert torch.equal(torch.isfinite(got), fin), f"{name}: -inf rows differ"
    assert_close_tol(got[fin], want[fin], name, max_abs=LSE_MAX, mean_abs=LSE_MEAN)


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_chunks_and_merge_match_oracle(row):
    import ulysses_sequence_attention_rank_amd as uly
    name, B, S, Hq, Hkv, D, causal, wl, sink, docs, bounds = row
    inp = small_case(zlib.crc32(name.encode()) % 10000, P=1, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D,
                     sink=sink, doc_lengths=docs)
    dev = torch.device("cuda", 0)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    cu = n = None
    cu_cpu = None
    if docs is not None:
        cu, n, _ = uly.cu_seqlens_from_positions(inp.positions.reshape(1, B, S).to(dev))
        cu_cpu, _, _ = oracle.segments(inp.positions)
    kw = dict(causal=causal, window_left=wl)
    acc_o = acc_l = None
    parts = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        say(f"ring {name}: chunk [{lo}, {hi})")
        o, l = uly.attn_fwd_chunk(q, k[:, lo:hi], v[:, lo:hi], lo, cu_seqlens=cu, n_seqs=n, **kw)
        wo, wl_ = oracle.attn_fwd(inp.q, inp.k, inp.v, cu=cu_cpu, keys=(lo, hi), **kw)
        parts.append((wo, wl_))
        assert_close_tol(o.reshape(B * S, Hq, D), wo, f"chunk [{lo},{hi}) O")
        _lse_close(l.permute(0, 2, 1).reshape(B * S, Hq), wl_, f"chunk [{lo},{hi}) LSE")
        if acc_o is None:
            acc_o, acc_l = o.clone(), l.clone()
        else:
            uly.attn_merge(acc_o, acc_l, o, l)
    out, lse = uly.attn_merge_finish(acc_o, acc_l, sink=None if inp.sink is None else inp.sink.to(dev))
    torch.cuda.synchronize()
    mo, ml = oracle.merge_chunks([p[0] for p in parts], [p[1] for p in parts], sink=inp.sink)
    assert_close_tol(out.reshape(B * S, Hq, D), mo, "merged O")
    _lse_close(lse.permute(0, 2, 1).reshape(B * S, Hq), ml, "merged LSE")
    # and against attention over every key at once
    fo, fl = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, cu=cu_cpu, **kw)
    assert_close_tol(out.reshape(B * S, Hq, D), fo, "merged O vs full")
    _lse_close(lse.permute(0, 2, 1).reshape(B * S, Hq), fl, "merged LSE vs full")
