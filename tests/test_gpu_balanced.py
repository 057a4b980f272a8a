"""GPU parity of the dK/dV balanced schedule, which the library uses for long
sequences on small grids (at least 256 key tiles of 128 keys, at most 512
(key tile, KV head) items, unless a sliding window narrower than 256 keys
makes every key tile's walk short).  The cases below sit in that range and add
what the five workloads do not: a ragged total length (a partial last key tile
and ragged last documents), two batch rows, non-causal packed attention, the
fp32 replica-gradient path, and the narrow-window grid at the same sizes.
dK/dV are compared with the fp64 oracle on sampled keys (every key of the
ragged tail, document starts and ends, random keys), O and dQ on sampled
rows."""
import zlib

import pytest
import torch

import oracle
from gpu_util import assert_close_tol, say

pytestmark = pytest.mark.gpu

CASES = [
    # id, B, S, hq, hkv, D, causal, window_left, packed docs, sink, fp32 dK/dV
    ("packed_ragged_causal_d128_gqa2_sink", 1, 32832, 2, 1, 128, True, -1, True, True, False),
    ("b2_window511_d64_gqa4", 2, 16448, 4, 1, 64, True, 511, False, False, False),
    # a window narrower than 256 keys takes the unsplit grid instead (same sizes)
    ("b2_window127_d64_gqa4_unsplit", 2, 16448, 4, 1, 64, True, 127, False, False, False),
    ("packed_ragged_full_d128_gqa2_f32kv", 1, 32832, 2, 1, 128, False, -1, True, False, True),
]


def _docs(T, g):
    starts, t = [], 0
    while t < T:
        starts.append(t)
        t += int(torch.randint(200, 3000, (1,), generator=g))
    return torch.tensor(starts + [T], dtype=torch.int32)


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_balanced_dkdv_parity(row):
    import ulysses_sequence_attention_rank_amd as uly
    name, B, S, hq, hkv, D, causal, wl, packed, with_sink, f32kv = row
    T = B * S
    assert (T + 127) // 128 >= 256 and (T + 127) // 128 * hkv <= 512
    g = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    rnd = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16)
    q, k, v, do = rnd(B, S, hq, D), rnd(B, S, hkv, D), rnd(B, S, hkv, D), rnd(B, S, hq, D)
    sink = torch.randn(hq, generator=g) if with_sink else None
    cu = _docs(T, g) if packed else None
    n = None if cu is None else cu.numel() - 1
    dev = torch.device("cuda", 0)
    say(f"balanced dK/dV {name}: B={B} S={S} hq={hq} hkv={hkv} D={D} causal={causal} "
        f"wl={wl} docs={n}")
    cu_d = None if cu is None else cu.to(dev)
    n_d = None if cu is None else torch.tensor([n], dtype=torch.int32, device=dev)
    sk_d = None if sink is None else sink.to(dev)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = uly.attn_fwd(qd, kd, vd, sink=sk_d, cu_seqlens=cu_d, n_seqs=n_d, causal=causal,
                          window_left=wl)
    dq, dk, dv, _ = uly.attn_bwd(qd, kd, vd, o, dod, lse, sink=sk_d, cu_seqlens=cu_d, n_seqs=n_d,
                                 causal=causal, window_left=wl, kv_grad_fp32=f32kv)
    torch.cuda.synchronize()

    keys = set(range(T - 80, T)) | set(range(0, 16))
    if cu is not None:
        for d in range(0, n, max(1, n // 6)):
            keys |= {int(cu[d]), int(cu[d]) + 1, int(cu[d + 1]) - 1}
    if B > 1:
        keys |= set(range(S - 8, S + 8))
    keys |= set(torch.randint(0, T, (24,), generator=g).tolist())
    keys = sorted(keys)
    rows = sorted(set(range(T - 8, T)) | set(torch.randint(0, T, (16,), generator=g).tolist()))
    kw = dict(sink=sink, cu=cu, causal=causal, window_left=wl)
    say(f"oracle on {len(rows)} rows / {len(keys)} keys")
    o_w, _ = oracle.attn_fwd(q, k, v, rows=rows, **kw)
    dq_w, _, _, _ = oracle.attn_bwd(q, k, v, do, qrows=rows, want_dkdv=False, want_dsink=False, **kw)
    _, dk_w, dv_w, _ = oracle.attn_bwd(q, k, v, do, krows=keys, want_dq=False, want_dsink=False,
                                       **kw)
    ridx, kidx = torch.tensor(rows), torch.tensor(keys)
    flat = lambda t, H: t.reshape(T, H, D)
    assert_close_tol(flat(o, hq)[ridx], o_w, f"{name} O")
    assert_close_tol(flat(dq, hq)[ridx], dq_w, f"{name} dQ")
    assert_close_tol(flat(dk, hkv)[kidx], dk_w, f"{name} dK")
    assert_close_tol(flat(dv, hkv)[kidx], dv_w, f"{name} dV")
