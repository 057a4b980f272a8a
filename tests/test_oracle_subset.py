"""Pins of the oracle's row and key subset mode (CPU only).

The full-size GPU parity tests ask the oracle for a sample only: the
forward of selected query rows (``attn_fwd(rows=...)``), dQ of selected rows
(``attn_bwd(qrows=..., want_dkdv=False)``) and dK/dV of selected keys
(``attn_bwd(krows=..., want_dq=False)``), for which it computes the softmax
statistics (LSE, delta) of only the rows those outputs need.  Here every such
subset result is compared, bit for bit, with the same entries of the
full-mode result, which the other oracle tests pin against PyTorch's SDPA,
finite differences and closed forms.  The oracle fills the statistics of rows
it skips with NaN, so a subset result that read one would not compare equal.

Cases cover causal, full, one- and two-sided windows, packed documents, GQA,
sinks and two batch rows; the key sets hold keys whose visible rows lie far
from them (key 0 of a causal sequence is seen by every later row).
"""
import pytest
import torch

import oracle
from ulysses_inputs import small_case

CASES = [
    # name, B, S, Hq, Hkv, D, causal, wl, wr, sink, doc lengths per row
    ("causal_gqa", 1, 96, 4, 2, 8, True, -1, -1, False, None),
    ("full_mha", 1, 80, 2, 2, 8, False, -1, -1, False, None),
    ("causal_sink_gqa7", 1, 112, 7, 1, 8, True, -1, -1, True, None),
    ("window_sink", 1, 96, 4, 1, 4, True, 9, -1, True, None),
    ("window_twosided", 1, 90, 2, 1, 8, False, 6, 4, False, None),
    ("varlen_causal", 1, 100, 4, 2, 8, True, -1, -1, False, [[31, 1, 50, 18]]),
    ("varlen_full_sink", 1, 84, 2, 1, 4, False, -1, -1, True, [[40, 3, 41]]),
    ("batch2_causal_sink", 2, 64, 4, 2, 8, True, -1, -1, True, None),
    ("batch2_varlen_window", 2, 72, 2, 2, 8, True, 11, -1, False, [[30, 42], [72]]),
]


def _setup(row):
    name, B, S, Hq, Hkv, D, causal, wl, wr, sink, docs = row
    inp = small_case(300 + CASES.index(row), P=1, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink,
                     doc_lengths=docs)
    cu = None
    if docs is not None:
        cu, _, _ = oracle.segments(inp.positions)
    kw = dict(sink=inp.sink, cu=cu, causal=causal, window_left=wl, window_right=wr)
    return inp, kw


def _subsets(B, S):
    """Query rows and keys over the flattened B*S tokens: both ends, the middle,
    document-like boundaries and a spread; deliberately unsorted, with a repeat."""
    T = B * S
    rows = [T - 1, 0, 1, T // 2, T // 3 + 1, T - 2, 5, T // 2]
    keys = [0, 1, 2, T // 2 - 1, T - 1, S - 1, 7, 0]
    if B > 1:
        rows += [S, S + 1]
        keys += [S, S + 3]
    return rows, keys


def _bits_equal(a, b):
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.int64),
                                              b.contiguous().view(torch.int64))


@pytest.mark.parametrize("row", CASES, ids=[c[0] for c in CASES])
def test_subset_mode_equals_full_mode(row):
    inp, kw = _setup(row)
    B, S = inp.q.shape[:2]
    rows, keys = _subsets(B, S)
    r, k = torch.tensor(rows), torch.tensor(keys)

    o, lse = oracle.attn_fwd(inp.q, inp.k, inp.v, **kw)
    dq, dk, dv, ds = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, **kw)
    assert torch.isfinite(o).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all()

    # forward of selected rows
    o_s, lse_s = oracle.attn_fwd(inp.q, inp.k, inp.v, rows=rows, **kw)
    assert _bits_equal(o_s, o[r]) and _bits_equal(lse_s, lse[r])

    # dQ of selected rows only (statistics of those rows only)
    dq_s, dk_n, dv_n, ds_n = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, qrows=rows,
                                             want_dkdv=False, want_dsink=False, **kw)
    assert dk_n is None and dv_n is None and ds_n is None
    assert _bits_equal(dq_s, dq[r])

    # dK/dV of selected keys only (statistics of the rows that see them)
    dq_n, dk_s, dv_s, _ = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, krows=keys,
                                          want_dq=False, want_dsink=False, **kw)
    assert dq_n is None
    assert _bits_equal(dk_s, dk[k]) and _bits_equal(dv_s, dv[k])

    # both selections in one call, and dsink alone
    dq_b, dk_b, dv_b, _ = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, qrows=rows, krows=keys,
                                          want_dsink=False, **kw)
    assert _bits_equal(dq_b, dq[r]) and _bits_equal(dk_b, dk[k]) and _bits_equal(dv_b, dv[k])
    if inp.sink is not None:
        _, _, _, ds_s = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, want_dq=False,
                                        want_dkdv=False, want_dsink=True, **kw)
        assert _bits_equal(ds_s, ds)


def test_far_key_needs_far_rows():
    """Key 0 of a causal sequence is seen by every row: its subset dK must use the
    statistics of rows far from it, and equal the full result."""
    inp = small_case(311, P=1, B=1, S=128, Hq=4, Hkv=1, D=8)
    full = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, causal=True)
    sub = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, causal=True, krows=[0], want_dq=False,
                          want_dsink=False)
    assert _bits_equal(sub[1], full[1][:1]) and _bits_equal(sub[2], full[2][:1])
    # and it is not what the rows near key 0 alone would give
    near = oracle.attn_bwd(inp.q[:, :8], inp.k[:, :8], inp.v[:, :8], inp.dout[:, :8], causal=True,
                           krows=[0], want_dq=False, want_dsink=False)
    assert not torch.allclose(near[1], sub[1], atol=1e-3)


def test_skipped_row_statistics_poison_results():
    """The statistics of rows the oracle skips are NaN (a negative control for the
    subset comparisons above): a key's dK/dV computed while only a row that
    does not see it is needed stays finite, because it reads needed rows only."""
    inp = small_case(312, P=1, B=1, S=32, Hq=2, Hkv=1, D=4)
    # key 31 is seen only by row 31 under causal masking
    _, dk, dv, _ = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, causal=True, krows=[31],
                                   want_dq=False, want_dsink=False)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
    full = oracle.attn_bwd(inp.q, inp.k, inp.v, inp.dout, causal=True)
    assert _bits_equal(dk, full[1][31:32]) and _bits_equal(dv, full[2][31:32])
