"""Pins of the oracle's attention forward and backward (CPU only).

Each test ties ``oracle.attn_fwd`` / ``oracle.attn_bwd`` to something other
than the oracle itself: PyTorch's own attention routines on an equivalent
problem (library special case), finite differences of the forward, closed
forms, exact identities of the method (sharded == unsharded, varlen == per
document, GQA == repeated K/V, softmax rows summing to one, zero-sum key
gradients) and a hand-worked example stored under ``tests/golden``.

Mask semantics follow the flash_attn_func argument list in the
long-context-attention issue "usage with pytorch FSDP" (causal, window_size
(left, right) with -1 unbounded); documents come from cu_seqlens rebuilt from
the gathered position_ids and the sink is one logit per head (accelerate PR
"Add an FSDP2-native Ulysses sequence parallelism backend", findings list).
"""
import json
import math
import os
import zlib

import pytest
import torch
import torch.nn.functional as F

import oracle
from ulysses_inputs import seq_shards, small_case

F64 = torch.float64


def _doc_ids(B, S, cu):
    """Document id of every flattened token, via searchsorted (independent of the oracle)."""
    t = torch.arange(B * S)
    if cu is None:
        return (t // S).reshape(B, S)
    return (torch.searchsorted(cu.to(torch.int64), t, right=True) - 1).reshape(B, S)


def _allowed(B, S, cu, causal, wl, wr):
    doc = _doc_ids(B, S, cu)
    i = torch.arange(S).reshape(S, 1)
    j = torch.arange(S).reshape(1, S)
    ok = doc[:, :, None] == doc[:, None, :]
    if causal:
        ok = ok & (j <= i)
    if wl >= 0:
        ok = ok & (i - j <= wl)
    if wr >= 0:
        ok = ok & (j - i <= wr)
    return ok  # [B, S, S]


def sdpa_reference(q, k, v, dout, sink, cu, causal, wl, wr, scale):
    """torch SDPA (fp64, CPU) on the same problem; the sink is an extra key whose
    K and V are zero and whose additive mask bias is the sink logit."""
    B, S, hq, D = q.shape
    hkv = k.shape[2]
    qt = q.to(F64).permute(0, 2, 1, 3).contiguous().requires_grad_()
    kt = k.to(F64).permute(0, 2, 1, 3).contiguous().requires_grad_()
    vt = v.to(F64).permute(0, 2, 1, 3).contiguous().requires_grad_()
    ok = _allowed(B, S, cu, causal, wl, wr)
    bias = torch.zeros(B, 1, S, S, dtype=F64).masked_fill(~ok[:, None], float("-inf"))
    bias = bias.expand(B, hq, S, S)
    kk, vv = kt, vt
    sink_col = None
    if sink is not None:
        sink_col = sink.to(F64).reshape(1, hq, 1, 1).expand(B, hq, S, 1).clone().requires_grad_()
        bias = torch.cat([bias, sink_col], dim=-1)
        kk = torch.cat([kt, torch.zeros(B, hkv, 1, D, dtype=F64)], dim=2)
        vv = torch.cat([vt, torch.zeros(B, hkv, 1, D, dtype=F64)], dim=2)
    o = F.scaled_dot_product_attention(qt, kk, vv, attn_mask=bias, scale=scale,
                                       enable_gqa=(hq != hkv))
    res = {"o": o.detach().permute(0, 2, 1, 3).reshape(B * S, hq, D)}
    if dout is not None:
        (o * dout.to(F64).permute(0, 2, 1, 3)).sum().backward()
        res["dq"] = qt.grad.permute(0, 2, 1, 3).reshape(B * S, hq, D)
        res["dk"] = kt.grad.permute(0, 2, 1, 3).reshape(B * S, hkv, D)
        res["dv"] = vt.grad.permute(0, 2, 1, 3).reshape(B * S, hkv, D)
        if sink_col is not None:
            res["dsink"] = sink_col.grad.sum(dim=(0, 2, 3))
    return res


def sdpa_lse(q, k, sink, cu, causal, wl, wr, scale):
    """Log-sum-exp from PyTorch's CPU flash-attention kernel (K/V repeated for GQA)."""
    B, S, hq, D = q.shape
    G = hq // k.shape[2]
    qt = q.to(F64).permute(0, 2, 1, 3).contiguous()
    kt = k.to(F64).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    ok = _allowed(B, S, cu, causal, wl, wr)
    bias = torch.zeros(B, 1, S, S, dtype=F64).masked_fill(~ok[:, None], float("-inf"))
    bias = bias.expand(B, hq, S, S).contiguous()
    if sink is not None:
        bias = torch.cat([bias, sink.to(F64).reshape(1, hq, 1, 1).expand(B, hq, S, 1)], -1)
        kt = torch.cat([kt, torch.zeros(B, hq, 1, D, dtype=F64)], dim=2)
    vt = torch.zeros_like(kt)
    _, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        qt, kt, vt, 0.0, False, attn_mask=bias, scale=scale)
    return lse.permute(0, 2, 1).reshape(B * S, hq)


CASES = [
    # name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, doc lengths per row
    ("mha_causal", 2, 1, 24, 4, 4, 8, True, -1, -1, False, None),
    ("mha_full", 2, 1, 20, 2, 2, 16, False, -1, -1, False, None),
    ("gqa_causal_sink", 2, 1, 32, 8, 2, 8, True, -1, -1, True, None),
    ("swa_sink", 4, 1, 40, 8, 4, 4, True, 5, -1, True, None),
    ("swa_twosided", 1, 1, 30, 2, 1, 8, False, 3, 2, False, None),
    ("varlen_causal", 4, 1, 36, 8, 2, 8, True, -1, -1, False, [[7, 12, 1, 16]]),
    ("varlen_full_sink", 2, 1, 30, 4, 2, 4, False, -1, -1, True, [[10, 3, 17]]),
    ("batch2_causal", 2, 2, 16, 4, 2, 8, True, -1, -1, True, None),
    ("batch2_varlen_swa", 2, 2, 18, 2, 2, 8, True, 4, -1, False, [[5, 13], [9, 9]]),
]


def _setup(case_row, seed):
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = case_row
    inp = small_case(seed, P=P, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink, doc_lengths=docs)
    cu = None
    if docs is not None:
        cu, _, _ = oracle.segments(inp.positions)
    return inp, cu, causal, wl, wr, D ** -0.5


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_fwd_bwd_match_torch_sdpa(row):
    inp, cu, causal, wl, wr, scale = _setup(row, seed=zlib.crc32(row[0].encode()) % 1000)
    kw = dict(sink=inp.sink, cu=cu, causal=causal, window_left=wl, window_right=wr, scale=scale)
    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, **kw)
    dq, dk, dv, ds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **kw)
    ref = sdpa_reference(inp.q, inp.k, inp.v, inp.dout, inp.sink, cu, causal, wl, wr, scale)
    torch.testing.assert_close(o, ref["o"], atol=1e-11, rtol=1e-11)
    torch.testing.assert_close(dq, ref["dq"], atol=1e-10, rtol=1e-10)
    torch.testing.assert_close(dk, ref["dk"], atol=1e-10, rtol=1e-10)
    torch.testing.assert_close(dv, ref["dv"], atol=1e-10, rtol=1e-10)
    if inp.sink is not None:
        torch.testing.assert_close(ds, ref["dsink"], atol=1e-10, rtol=1e-10)
    lse_ref = sdpa_lse(inp.q, inp.k, inp.sink, cu, causal, wl, wr, scale)
    torch.testing.assert_close(lse, lse_ref, atol=1e-10, rtol=1e-10)


def _loss(q, k, v, dout, sink, kw):
    o, _ = oracle.attn_fwd(q, k, v, sink=sink, **kw)
    B, S, hq, D = q.shape
    return float((o * dout.to(F64).reshape(B * S, hq, D)).sum())


@pytest.mark.parametrize("row", [CASES[2], CASES[3], CASES[6], CASES[8]],
                         ids=["gqa_causal_sink", "swa_sink", "varlen_full_sink", "batch2_varlen_swa"])
def test_bwd_matches_finite_differences(row):
    """Central differences of sum(O * dout) w.r.t. every input of a tiny problem."""
    name, P, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    S = min(S, 12) if docs is None else S
    row = (name, P, B, S, Hq, Hkv, min(D, 4), causal, wl, wr, sink, docs)
    inp, cu, causal, wl, wr, scale = _setup(row, seed=5)
    q, k, v, dout = (t.to(F64) for t in (inp.q, inp.k, inp.v, inp.dout))
    sk = None if inp.sink is None else inp.sink.to(F64)
    kw = dict(cu=cu, causal=causal, window_left=wl, window_right=wr, scale=scale)
    dq, dk, dv, ds = oracle.attn_bwd(q, k, v, dout, sink=sk, **kw)
    eps = 1e-6
    g = torch.Generator().manual_seed(0)
    for name_t, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = t.reshape(-1)
        idx = torch.randint(0, flat.numel(), (12,), generator=g)
        for ix in idx.tolist():
            old = float(flat[ix])
            flat[ix] = old + eps
            lp = _loss(q, k, v, dout, sk, kw)
            flat[ix] = old - eps
            lm = _loss(q, k, v, dout, sk, kw)
            flat[ix] = old
            num = (lp - lm) / (2 * eps)
            ana = float(grad.reshape(-1)[ix])
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(num)), (name_t, ix, num, ana)
    if sk is not None:
        for h in range(sk.numel()):
            old = float(sk[h])
            sk[h] = old + eps
            lp = _loss(q, k, v, dout, sk, kw)
            sk[h] = old - eps
            lm = _loss(q, k, v, dout, sk, kw)
            sk[h] = old
            assert abs((lp - lm) / (2 * eps) - float(ds[h])) <= 1e-6


# ---------------------------------------------------------------- closed forms

def test_single_token_output_is_its_value():
    inp = small_case(1, P=1, B=1, S=1, Hq=2, Hkv=1, D=8)
    for causal in (True, False):
        o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=causal)
        assert torch.equal(o[0, 0], inp.v[0, 0, 0].to(F64))
        assert torch.equal(o[0, 1], inp.v[0, 0, 0].to(F64))
        s = float((inp.q[0, 0, 0].double() * inp.k[0, 0, 0].double()).sum()) / math.sqrt(8)
        assert abs(float(lse[0, 0]) - s) < 1e-12


def test_causal_first_row_is_first_value():
    inp = small_case(2, P=2, B=1, S=16, Hq=4, Hkv=2, D=8)
    o, _ = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True)
    for h in range(4):
        assert torch.equal(o[0, h], inp.v[0, 0, h // 2].to(F64))


@pytest.mark.parametrize("with_sink", [False, True])
def test_zero_queries_average_visible_values(with_sink):
    """q = 0 makes every visible logit 0: O_i = sum_j v_j / (n_i + e^sink)."""
    S, D = 20, 4
    inp = small_case(3, P=2, B=1, S=S, Hq=2, Hkv=1, D=D, sink=with_sink)
    q = torch.zeros_like(inp.q)
    wl = 6
    o, lse = oracle.attn_fwd(q, inp.k, inp.v, sink=inp.sink, causal=True, window_left=wl)
    v = inp.v[0, :, 0].to(F64)
    for i in range(S):
        lo = max(0, i - wl)
        n = i + 1 - lo
        for h in range(2):
            extra = math.exp(float(inp.sink[h])) if with_sink else 0.0
            expect = v[lo:i + 1].sum(0) / (n + extra)
            torch.testing.assert_close(o[i, h], expect, atol=1e-14, rtol=1e-13)
            assert abs(float(lse[i, h]) - math.log(n + extra)) < 1e-13


def test_unit_values_give_one_minus_sink_probability():
    """With v = 1 every output coordinate is the total non-sink probability."""
    inp = small_case(4, P=2, B=1, S=24, Hq=4, Hkv=2, D=8, sink=True)
    v = torch.ones_like(inp.v)
    o, lse = oracle.attn_fwd(inp.q, inp.k, v, sink=inp.sink, causal=True)
    p_sink = torch.exp(inp.sink.to(F64).reshape(1, 4) - lse)
    torch.testing.assert_close(o, (1 - p_sink)[..., None].expand_as(o), atol=1e-14, rtol=1e-14)
    o2, _ = oracle.attn_fwd(inp.q, inp.k, v, causal=True)
    torch.testing.assert_close(o2, torch.ones_like(o2), atol=1e-14, rtol=0)


def test_minus_infinity_sink_is_no_sink():
    inp = small_case(5, P=2, B=1, S=20, Hq=2, Hkv=2, D=8)
    ninf = torch.full((2,), float("-inf"))
    a = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=ninf, causal=True)
    b = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_wide_window_is_full_causal():
    inp = small_case(6, P=2, B=1, S=20, Hq=2, Hkv=2, D=8)
    a = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True, window_left=20)
    b = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True)
    assert torch.equal(a[0], b[0])


def test_one_document_equals_plain():
    inp = small_case(7, P=2, B=1, S=20, Hq=2, Hkv=2, D=8)
    cu = torch.tensor([0, 20], dtype=torch.int32)
    for causal in (True, False):
        a = oracle.attn_fwd(inp.q, inp.k, inp.v, cu=cu, causal=causal)
        b = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=causal)
        assert torch.equal(a[0], b[0])


def test_varlen_equals_documents_one_by_one():
    lens = [6, 1, 11, 4]
    inp = small_case(8, P=2, B=1, S=22, Hq=4, Hkv=2, D=8, sink=True, doc_lengths=[lens])
    cu, n, mx = oracle.segments(inp.positions)
    for causal in (True, False):
        o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, cu=cu, causal=causal)
        dq, dk, dv, ds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, sink=inp.sink, cu=cu,
                                         causal=causal)
        a = 0
        ds_sum = torch.zeros(4, dtype=F64)
        for L in lens:
            sl = slice(a, a + L)
            od, ld = oracle.attn_fwd(inp.q[:, sl], inp.k[:, sl], inp.v[:, sl], sink=inp.sink,
                                     causal=causal)
            assert torch.equal(o[sl], od) and torch.equal(lse[sl], ld)
            g = oracle.attn_bwd(inp.q[:, sl], inp.k[:, sl], inp.v[:, sl], inp.dout[:, sl],
                                sink=inp.sink, causal=causal)
            assert torch.equal(dq[sl], g[0]) and torch.equal(dk[sl], g[1]) and torch.equal(dv[sl], g[2])
            ds_sum += g[3]
            a += L
        torch.testing.assert_close(ds, ds_sum, atol=1e-13, rtol=1e-13)


def test_gqa_equals_repeated_kv():
    inp = small_case(9, P=2, B=1, S=18, Hq=6, Hkv=2, D=8, sink=True)
    G = 3
    kr = inp.k.repeat_interleave(G, dim=2)
    vr = inp.v.repeat_interleave(G, dim=2)
    kw = dict(sink=inp.sink, causal=True, window_left=7)
    a = oracle.attn_fwd(inp.q, inp.k, inp.v, **kw)
    b = oracle.attn_fwd(inp.q, kr, vr, **kw)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ga = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **kw)
    gb = oracle.attn_bwd(inp.q, kr, vr, inp.dout, **kw)
    assert torch.equal(ga[0], gb[0])
    torch.testing.assert_close(ga[1], gb[1].reshape(-1, 2, G, 8).sum(2), atol=1e-13, rtol=1e-13)
    torch.testing.assert_close(ga[2], gb[2].reshape(-1, 2, G, 8).sum(2), atol=1e-13, rtol=1e-13)


def test_softmax_rows_sum_to_one():
    """sum_j P_ij + P_sink,i = 1, with P from the oracle's own LSE."""
    inp = small_case(10, P=2, B=1, S=16, Hq=2, Hkv=1, D=4, sink=True)
    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, causal=True, window_left=5)
    q, k = inp.q[0].to(F64), inp.k[0, :, 0].to(F64)
    for i in range(16):
        for h in range(2):
            tot = math.exp(float(inp.sink[h]) - float(lse[i, h]))
            for j in range(max(0, i - 5), i + 1):
                s = float((q[i, h] * k[j]).sum()) / 2.0
                tot += math.exp(s - float(lse[i, h]))
            assert abs(tot - 1.0) < 1e-12


def test_key_gradients_sum_to_zero_per_document_without_sink():
    """sum_j dS_ij = 0 for every row, hence sum_{j in doc} dK_j = 0."""
    lens = [9, 15]
    inp = small_case(11, P=2, B=1, S=24, Hq=4, Hkv=2, D=8, doc_lengths=[lens])
    cu, _, _ = oracle.segments(inp.positions)
    for causal in (True, False):
        _, dk, _, _ = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, cu=cu, causal=causal)
        assert dk[:9].sum(0).abs().max() < 1e-12
        assert dk[9:].sum(0).abs().max() < 1e-12


@pytest.mark.parametrize("P,Hq,Hkv,sink", [(2, 4, 2, False), (4, 8, 4, True), (2, 6, 2, True)])
def test_sharded_equals_unsharded(P, Hq, Hkv, sink):
    """Shard -> pack -> per-rank attention (sink sliced) -> unpack == unsharded, bit for bit."""
    S, D = 16, 8
    inp = small_case(12 + P, P=P, B=1, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink)
    kw = dict(causal=True, window_left=6)
    o_full, _ = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, **kw)
    g_full = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, sink=inp.sink, **kw)
    qh = oracle.pack(seq_shards(inp.q, P))
    kh = oracle.pack(seq_shards(inp.k, P))
    vh = oracle.pack(seq_shards(inp.v, P))
    dh = oracle.pack(seq_shards(inp.dout, P))
    hq, hkv = Hq // P, Hkv // P
    outs, dqs, dks, dvs, dss = [], [], [], [], []
    for r in range(P):
        sk = None if inp.sink is None else inp.sink[r * hq:(r + 1) * hq]
        o, _ = oracle.attn_fwd(qh[r], kh[r], vh[r], sink=sk, **kw)
        g = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], sink=sk, **kw)
        outs.append(o.reshape(1, S, hq, D))
        dqs.append(g[0].reshape(1, S, hq, D))
        dks.append(g[1].reshape(1, S, hkv, D))
        dvs.append(g[2].reshape(1, S, hkv, D))
        if sink:
            dss.append(g[3])
    o_seq = oracle.unpack(torch.stack(outs))          # [P, 1, S/P, Hq, D]
    assert torch.equal(o_seq, seq_shards(o_full.reshape(1, S, Hq, D), P))
    assert torch.equal(oracle.unpack(torch.stack(dqs)), seq_shards(g_full[0].reshape(1, S, Hq, D), P))
    assert torch.equal(oracle.unpack(torch.stack(dks)), seq_shards(g_full[1].reshape(1, S, Hkv, D), P))
    assert torch.equal(oracle.unpack(torch.stack(dvs)), seq_shards(g_full[2].reshape(1, S, Hkv, D), P))
    if sink:
        assert torch.equal(torch.cat(dss), g_full[3])


def test_local_shard_cu_seqlens_change_attention():
    """Negative control: documents taken from rank 0's local position shard (then one
    document for the rest) give a different result on the gathered sequence."""
    lens = [5, 9, 7, 11]      # boundaries at 5, 14, 21: rank 0 (tokens 0..7) sees only the first
    P, S = 4, 32
    inp = small_case(20, P=P, B=1, S=S, Hq=4, Hkv=2, D=8, doc_lengths=[lens])
    shards = seq_shards(inp.positions, P)
    good, _, _ = oracle.segments(oracle.gather_positions(shards))
    local, _, _ = oracle.segments(shards[0])
    bad = torch.cat([local[:-1], torch.tensor([S], dtype=torch.int32)])
    a, _ = oracle.attn_fwd(inp.q, inp.k, inp.v, cu=good, causal=True)
    b, _ = oracle.attn_fwd(inp.q, inp.k, inp.v, cu=bad, causal=True)
    diff = (a - b).abs()
    assert diff.max() > 0.02
    assert (diff > 0.02).float().mean() > 0.3


def test_hand_worked_golden():
    """Values worked out by hand (tests/golden/hand_attention.json)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_attention.json")
    gold = json.load(open(path))
    for ex in gold["examples"]:
        q = torch.tensor(ex["q"], dtype=F64).reshape(1, -1, 1, len(ex["q"][0]))
        k = torch.tensor(ex["k"], dtype=F64).reshape(1, -1, 1, len(ex["k"][0]))
        v = torch.tensor(ex["v"], dtype=F64).reshape(1, -1, 1, len(ex["v"][0]))
        sink = None if ex["sink"] is None else torch.tensor([ex["sink"]], dtype=F64)
        o, lse = oracle.attn_fwd(q, k, v, sink=sink, causal=ex["causal"], scale=ex["scale"])
        torch.testing.assert_close(o.reshape(-1, v.shape[-1]), torch.tensor(ex["out"], dtype=F64),
                                   atol=1e-14, rtol=1e-14)
        torch.testing.assert_close(lse.reshape(-1), torch.tensor(ex["lse"], dtype=F64),
                                   atol=1e-14, rtol=1e-14)


# ------------------------------------------- ring inner step: KV chunks + merge

CHUNK_CASES = [
    # seed, B, S, Hq, Hkv, D, causal, wl, docs, chunk bounds
    (11, 1, 48, 4, 2, 8, True, -1, None, (0, 7, 20, 33, 48)),
    (12, 2, 40, 2, 1, 4, False, -1, None, (0, 25, 40)),
    (13, 1, 64, 4, 4, 8, True, 9, [[20, 1, 43]], (0, 16, 32, 48, 64)),
]


@pytest.mark.parametrize("case", CHUNK_CASES)
def test_chunks_merged_equal_full_attention(case):
    """Attention over disjoint KV chunks, combined by the exact LSE merge (the
    sink entering once, in the merge), equals attention over every key."""
    seed, B, S, Hq, Hkv, D, causal, wl, docs, bounds = case
    inp = small_case(seed, P=1, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=True, doc_lengths=docs)
    cu = None
    if docs is not None:
        cu, _, _ = oracle.segments(inp.positions)
    kw = dict(cu=cu, causal=causal, window_left=wl)
    full_o, full_lse = oracle.attn_fwd(inp.q, inp.k, inp.v, sink=inp.sink, **kw)
    parts = [oracle.attn_fwd(inp.q, inp.k, inp.v, keys=(lo, hi), **kw)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    o, lse = oracle.merge_chunks([p[0] for p in parts], [p[1] for p in parts], sink=inp.sink)
    assert torch.allclose(o, full_o, atol=1e-12, rtol=0)
    assert torch.allclose(lse, full_lse, atol=1e-12, rtol=0)
    # without the sink: one chunk holding every key is the plain attention, exactly
    o1, l1 = oracle.attn_fwd(inp.q, inp.k, inp.v, keys=(0, S), **kw)
    o2, l2 = oracle.attn_fwd(inp.q, inp.k, inp.v, **kw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    m1, n1 = oracle.merge_chunks([o1], [l1])
    assert torch.allclose(m1, o1, atol=1e-15, rtol=0) and torch.allclose(n1, l1, atol=0, rtol=0)


def test_single_key_chunk_closed_form():
    """A chunk of one key j: rows that see j get O = v_j and LSE = scale q.k_j;
    rows that do not (causal: i < j) get O = 0 and LSE = -inf."""
    inp = small_case(21, P=1, B=1, S=16, Hq=2, Hkv=1, D=4)
    j = 5
    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, causal=True, keys=(j, j + 1))
    q, k, v = (x.double()[0] for x in (inp.q, inp.k, inp.v))
    for i in range(16):
        for h in range(2):
            if i < j:
                assert float(lse[i, h]) == float("-inf") and bool((o[i, h] == 0).all())
            else:
                assert torch.allclose(o[i, h], v[j, 0], atol=1e-14, rtol=0)
                want = 0.5 * float((q[i, h] * k[j, 0]).sum())
                assert abs(float(lse[i, h]) - want) < 1e-12
