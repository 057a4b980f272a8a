"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (the simulated step of ``ulysses_sequence_attention_rank_amd.sim``).

* pack / unpack and cu_seqlens: bit-exact against the oracle on every rank;
* attention forward (O, LSE) and dQ on sampled query rows, dK/dV on sampled
  keys, computed one by one by the fp64 oracle on the rank's head shard;
  workloads small enough (S <= 4096) are compared in full on rank 0;
* dsink against the oracle where every row's statistics are affordable
  (the sliding-window layer), else the identity dsink_h = -sum_i
  exp(sink_h - LSE_i) dO_i . O_i on the kernel's own LSE and O (a property
  that holds at any size; LSE and O themselves are checked on sampled rows);
* without sinks, sum over a document of dK is zero for every KV head.
"""
import functools

import pytest
import torch

import oracle
from gpu_util import LSE_MAX, LSE_MEAN, assert_close_tol, bits_equal, say
from ulysses_inputs import WORKLOADS, make_inputs, seq_shards

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _inputs(cfg):
    say(f"generating inputs of workload {cfg} ({WORKLOADS[cfg].name})")
    return make_inputs(WORKLOADS[cfg])


@functools.lru_cache(maxsize=1)
def _oracle_heads(cfg):
    """The oracle's own pack of the full tensors: per-rank head shards."""
    inp = _inputs(cfg)
    P = inp.case.P
    return tuple(oracle.pack(seq_shards(t, P)) for t in (inp.q, inp.k, inp.v, inp.dout))


def _device_step(cfg, variant):
    from ulysses_sequence_attention_rank_amd import sim
    inp = _inputs(cfg)
    c = inp.case
    dev = torch.device("cuda", 0)
    b = sim.allocate(seq_shards(inp.q, c.P).to(dev), seq_shards(inp.k, c.P).to(dev),
                     seq_shards(inp.v, c.P).to(dev), seq_shards(inp.dout, c.P).to(dev),
                     seq_shards(inp.positions, c.P).to(dev),
                     None if inp.sink is None else inp.sink.to(dev))
    say(f"workload {cfg} variant {variant.name}: simulated step, all {c.P} ranks")
    sim.step(b, causal=variant.causal, window_left=variant.window_left,
             window_right=variant.window_right)
    torch.cuda.synchronize()
    return b


def _sample_rows(cfg, cu, n, count=96):
    c = WORKLOADS[cfg]
    S = c.S
    rows = set(range(0, 16)) | set(range(S - 16, S))
    for r in range(1, c.P):
        rows |= {r * S // c.P - 1, r * S // c.P}
    for d in range(n):
        for x in (int(cu[d]), int(cu[d]) + 1, int(cu[d + 1]) - 1):
            if 0 <= x < S:
                rows.add(x)
    g = torch.Generator().manual_seed(1000 + cfg)
    rows |= set(torch.randint(0, S, (count,), generator=g).tolist())
    return sorted(rows)


def _sample_keys(cfg, cu, n, variant):
    """Keys whose gradients the oracle can afford: every key whose visible rows are few
    (window), the tail of the sequence, 64 keys spread over its last 2048 (the
    oracle then needs rows >= S - 2048 only), and the first keys of a document
    when the document is short enough.  (Keys with the longest walks are
    compared at 16k-32k tokens in test_gpu_long.py.)"""
    c = WORKLOADS[cfg]
    S = c.S
    keys = set(range(S - 48, S))
    if S >= 65536:
        keys |= set(range(S - 2048, S, 32))
    if variant.window_left >= 0:
        g = torch.Generator().manual_seed(2000 + cfg)
        keys |= set(range(0, 48)) | set(torch.randint(0, S, (64,), generator=g).tolist())
    for d in range(n):
        L = int(cu[d + 1]) - int(cu[d])
        if L * c.hq <= 2048 * 8:
            keys |= set(range(int(cu[d]), int(cu[d]) + 24))
    return sorted(k for k in keys if 0 <= k < S)


CASES = [(cfg, v) for cfg in (1, 2, 3, 4, 5) for v in WORKLOADS[cfg].variants]


@pytest.mark.parametrize("cfg,variant", CASES, ids=[f"w{c}-{v.name}" for c, v in CASES])
def test_workload_parity(cfg, variant):
    inp = _inputs(cfg)
    c = inp.case
    P, B, S, D = c.P, c.B, c.S, c.D
    hq, hkv = c.hq, c.hkv
    b = _device_step(cfg, variant)
    qh, kh, vh, dh = _oracle_heads(cfg)

    say("layout: pack of Q/K/V/dO and unpack of O/dQ/dK/dV, bit-exact")
    assert bits_equal(b.q_head, qh) and bits_equal(b.k_head, kh) and bits_equal(b.v_head, vh)
    assert bits_equal(b.do_head, dh)
    for name, head, seq in (("O", b.o_head, b.o_seq), ("dQ", b.dq_head, b.dq_seq),
                            ("dK", b.dk_head, b.dk_seq), ("dV", b.dv_head, b.dv_seq)):
        assert bits_equal(seq, oracle.unpack(head.cpu())), name

    say("cu_seqlens / n_seqs / max_len from the gathered positions, bit-exact")
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    assert int(b.n_seqs.item()) == n and int(b.max_len.item()) == mx
    assert torch.equal(b.cu[: n + 1].cpu(), cu)

    kw = dict(cu=cu, causal=variant.causal, window_left=variant.window_left,
              window_right=variant.window_right)
    ranks = list(range(P)) if cfg <= 3 else sorted({0, P - 1})
    for r in ranks:
        sk = None if inp.sink is None else inp.sink[r * hq:(r + 1) * hq]
        full = S <= 4096 and r == 0
        rows = None if full else _sample_rows(cfg, cu, n)
        keys = None if full else _sample_keys(cfg, cu, n, variant)
        say(f"rank {r}: oracle on {'all' if full else len(rows)} rows / "
            f"{'all' if full else len(keys)} keys")
        o, lse = oracle.attn_fwd(qh[r], kh[r], vh[r], sink=sk, rows=rows, **kw)
        dq, _, _, _ = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], sink=sk, qrows=rows,
                                      want_dkdv=False, want_dsink=False, **kw)
        _, dk, dv, _ = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], sink=sk, krows=keys,
                                       want_dq=False, want_dsink=False, **kw)
        ridx = torch.arange(B * S) if rows is None else torch.tensor(rows)
        kidx = torch.arange(B * S) if keys is None else torch.tensor(keys)
        flat = lambda t, H: t.reshape(B * S, H, D)
        assert_close_tol(flat(b.o_head[r], hq)[ridx], o, f"rank{r} O")
        assert_close_tol(b.lse[r].reshape(hq, B * S).T[ridx], lse, f"rank{r} LSE",
                         max_abs=LSE_MAX, mean_abs=LSE_MEAN)
        assert_close_tol(flat(b.dq_head[r], hq)[ridx], dq, f"rank{r} dQ")
        assert_close_tol(flat(b.dk_head[r], hkv)[kidx], dk, f"rank{r} dK")
        assert_close_tol(flat(b.dv_head[r], hkv)[kidx], dv, f"rank{r} dV")

        if inp.sink is not None:
            if variant.window_left >= 0 and variant.window_left < 1024:
                say(f"rank {r}: dsink against the oracle over every row (window layer)")
                _, _, _, ds = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], sink=sk,
                                              want_dq=False, want_dkdv=False, want_dsink=True,
                                              **kw)
                assert_close_tol(b.dsink[r * hq:(r + 1) * hq], ds, f"rank{r} dsink")
            say(f"rank {r}: dsink identity on the kernel's LSE and O")
            lse_r = b.lse[r].double().cpu()                         # [B, hq, S]
            o_r = b.o_head[r].double().cpu().permute(0, 2, 1, 3)   # [B, hq, S, D]
            do_r = dh[r].double().permute(0, 2, 1, 3)
            d_i = (o_r * do_r).sum(-1)
            p_sink = torch.exp(sk.double().reshape(1, hq, 1) - lse_r)
            want = -(p_sink * d_i).sum(dim=(0, 2))
            # the kernel's D_i uses the exact O, this one the kernel's bf16 O, off by its
            # rounding (2^-9 relative) and the kernel's own error (mean-abs scale 2e-3)
            dev_o = o_r.abs() * 2.0 ** -8 + 2e-3
            bound = (p_sink * (dev_o * do_r.abs()).sum(-1)).sum(dim=(0, 2))
            got = b.dsink[r * hq:(r + 1) * hq].double().cpu()
            print(f"  rank{r} dsink identity: |got-want|={(got - want).abs().tolist()} "
                  f"bound={bound.tolist()}", flush=True)
            assert bool(((got - want).abs() <= bound + 1e-3 * want.abs() + 1e-3).all())
        else:
            say(f"rank {r}: sum of dK over each document is zero")
            dkf = b.dk_head[r].double().cpu().reshape(B * S, hkv, D)
            for d in range(n):
                L = int(cu[d + 1]) - int(cu[d])
                sdk = dkf[int(cu[d]):int(cu[d + 1])].sum(0)
                # rounding noise of L bf16 outputs and of delta grows like sqrt(L)
                thr = 0.05 + 3e-3 * L ** 0.5
                assert float(sdk.abs().max()) < thr, (d, float(sdk.abs().max()), thr)


def test_fused_step_full_size():
    """The fused step (attention reading Q/K/V and writing O/dQ/dK/dV in the
    sequence shards in place, no pack/unpack) on the S=131072 workload, as the
    benchmark times it: bit-identical to the packed step, whose outputs the
    workload test compares with the oracle, and compared with the oracle on
    sampled rows and keys of ranks 0 and P-1 directly."""
    from ulysses_sequence_attention_rank_amd import sim
    cfg = 5
    inp = _inputs(cfg)
    c = inp.case
    P, S, D, hq, hkv = c.P, c.S, c.D, c.hq, c.hkv
    variant = c.variants[0]
    kw_step = dict(causal=variant.causal, window_left=variant.window_left,
                   window_right=variant.window_right)
    packed = _device_step(cfg, variant)
    ref = [t.clone() for t in (packed.o_seq, packed.dq_seq, packed.dk_seq, packed.dv_seq, packed.lse)]
    del packed
    torch.cuda.empty_cache()
    dev = torch.device("cuda", 0)
    b = sim.allocate(seq_shards(inp.q, P).to(dev), seq_shards(inp.k, P).to(dev),
                     seq_shards(inp.v, P).to(dev), seq_shards(inp.dout, P).to(dev),
                     seq_shards(inp.positions, P).to(dev), None)
    say(f"workload {cfg}: fused step, all {P} ranks")
    sim.step(b, fused=True, **kw_step)
    torch.cuda.synchronize()
    for name, x, y in zip(("O", "dQ", "dK", "dV", "LSE"),
                          (b.o_seq, b.dq_seq, b.dk_seq, b.dv_seq, b.lse), ref):
        assert bits_equal(x, y), f"fused {name} differs from the packed step"
    cu, n, _ = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    rows, keys = _sample_rows(cfg, cu, n, count=32), list(range(S - 48, S))
    qh, kh, vh, dh = _oracle_heads(cfg)
    kw = dict(cu=cu, **kw_step)
    ridx, kidx = torch.tensor(rows), torch.tensor(keys)
    for r in (0, P - 1):
        say(f"fused, rank {r}: oracle on {len(rows)} rows / {len(keys)} keys")
        o, _ = oracle.attn_fwd(qh[r], kh[r], vh[r], rows=rows, **kw)
        dq, dk, dv, _ = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], qrows=rows, krows=keys,
                                        want_dsink=False, **kw)
        # rank r's heads, in the sequence shards: token t of shard t // (S/P)
        seq_rows = lambda x, H, h0, idx: x.permute(1, 0, 2, 3, 4).reshape(S, -1, D)[idx, h0:h0 + H]
        assert_close_tol(seq_rows(b.o_seq, hq, r * hq, ridx), o, f"fused rank{r} O")
        assert_close_tol(seq_rows(b.dq_seq, hq, r * hq, ridx), dq, f"fused rank{r} dQ")
        assert_close_tol(seq_rows(b.dk_seq, hkv, r * hkv, kidx), dk, f"fused rank{r} dK")
        assert_close_tol(seq_rows(b.dv_seq, hkv, r * hkv, kidx), dv, f"fused rank{r} dV")


def test_workload_parity_replicated_kv():
    """The packed S=32768 workload over 16 ranks: 8 KV heads for 16 ranks, each
    replicated to 2.  Layout steps bit-exact (the replicated pack, and the
    replicas' fp32 dK/dV summed and rounded once); every rank's attention on
    sampled rows and keys; the summed dK/dV against the unsharded attention."""
    cfg = 6
    inp = _inputs(cfg)
    c = inp.case
    P, B, S, D, Hq, Hkv = c.P, c.B, c.S, c.D, c.Hq, c.Hkv
    hq, R = c.hq, c.P // c.Hkv
    variant = c.variants[0]
    b = _device_step(cfg, variant)

    say("layout: pack of Q, replicated pack of K/V, sums of the replicas' dK/dV")
    qh = oracle.pack(seq_shards(inp.q, P))
    kh = oracle.pack_replicated(seq_shards(inp.k, P))
    vh = oracle.pack_replicated(seq_shards(inp.v, P))
    dh = oracle.pack(seq_shards(inp.dout, P))
    assert bits_equal(b.q_head, qh) and bits_equal(b.k_head, kh) and bits_equal(b.v_head, vh)
    assert bits_equal(b.do_head, dh)
    assert bits_equal(b.dk_seq, oracle.reduce_replicated(b.dk_head.cpu(), Hkv))
    assert bits_equal(b.dv_seq, oracle.reduce_replicated(b.dv_head.cpu(), Hkv))

    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, P)))
    assert torch.equal(b.cu[: n + 1].cpu(), cu)
    kw = dict(cu=cu, causal=variant.causal, window_left=variant.window_left,
              window_right=variant.window_right)
    rows, keys = _sample_rows(cfg, cu, n, count=48), _sample_keys(cfg, cu, n, variant)
    ridx, kidx = torch.tensor(rows), torch.tensor(keys)
    flat = lambda t, H: t.reshape(B * S, H, D)
    for r in (0, R - 1, P - 1):   # two replicas of KV head 0, and the last rank
        say(f"rank {r}: oracle on {len(rows)} rows / {len(keys)} keys")
        o, lse = oracle.attn_fwd(qh[r], kh[r], vh[r], rows=rows, **kw)
        dq, _, _, _ = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], qrows=rows, want_dkdv=False,
                                      want_dsink=False, **kw)
        _, dk, dv, _ = oracle.attn_bwd(qh[r], kh[r], vh[r], dh[r], krows=keys, want_dq=False,
                                       want_dsink=False, **kw)
        assert_close_tol(flat(b.o_head[r], hq)[ridx], o, f"rank{r} O")
        assert_close_tol(flat(b.dq_head[r], hq)[ridx], dq, f"rank{r} dQ")
        assert_close_tol(flat(b.dk_head[r], 1)[kidx], dk, f"rank{r} dK (fp32 replica)")
        assert_close_tol(flat(b.dv_head[r], 1)[kidx], dv, f"rank{r} dV (fp32 replica)")

    say("summed dK/dV of KV head 0 against the unsharded attention of its query heads")
    G = Hq // Hkv
    _, dk0, dv0, _ = oracle.attn_bwd(inp.q[:, :, :G], inp.k[:, :, :1], inp.v[:, :, :1],
                                     inp.dout[:, :, :G], krows=keys, want_dq=False,
                                     want_dsink=False, **kw)
    dk_full = b.dk_seq.permute(1, 0, 2, 3, 4).reshape(B * S, Hkv, D)[:, :1]
    dv_full = b.dv_seq.permute(1, 0, 2, 3, 4).reshape(B * S, Hkv, D)[:, :1]
    assert_close_tol(dk_full[kidx], dk0, "summed dK")
    assert_close_tol(dv_full[kidx], dv0, "summed dV")
