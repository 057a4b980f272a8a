"""CPU oracle (fp64, plain loops) for one Ulysses rank's hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the product package never does.
The arithmetic lives in ``orc.c`` (compiled with gcc, OpenMP over rows); this
module only marshals torch tensors in and out through ctypes.

The sequence-tiled gated MLP (fp64 torch CPU matmuls) is in ``oracle/mlp.py``.

parity unpinned: none.  Every function is pinned by the CPU tests in
``tests/test_oracle_*.py`` (library special cases, finite differences, closed
forms, brute force, a hand-worked example and invariants of the method).  The
row/key subset mode of ``attn_fwd``/``attn_bwd`` (``rows``, ``qrows``,
``krows``), which computes the softmax statistics of only the rows the
requested outputs need, is pinned bit for bit to the full mode
(``tests/test_oracle_subset.py``); statistics of skipped rows are NaN.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB = os.path.join(_HERE, "liborc.so")

__all__ = ["build", "pack", "unpack", "gather_positions", "segments", "attn_fwd", "attn_bwd",
           "num_threads"]


def build(force: bool = True) -> str:
    """Compile ``orc.c`` into ``liborc.so`` with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _Prob(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("sink", ctypes.c_void_p), ("cu", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("B", ctypes.c_int64), ("S", ctypes.c_int64), ("hq", ctypes.c_int64),
                ("hkv", ctypes.c_int64), ("D", ctypes.c_int64), ("scale", ctypes.c_double),
                ("causal", ctypes.c_int64), ("wl", ctypes.c_int64), ("wr", ctypes.c_int64),
                ("k_lo", ctypes.c_int64), ("k_hi", ctypes.c_int64)]


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.orc_pack.argtypes = [vp, vp] + [i64] * 6
        lib.orc_unpack.argtypes = [vp, vp] + [i64] * 6
        lib.orc_pack_replicated.argtypes = [vp, vp] + [i64] * 6
        lib.orc_reduce_replicated.argtypes = [vp, vp] + [i64] * 5
        lib.orc_reduce_replicated_f32.argtypes = [vp, vp] + [i64] * 5
        lib.orc_gather_positions.argtypes = [vp, vp, i64, i64, i64]
        lib.orc_segments.argtypes = [vp, i64, i64, vp, i64, vp, vp]
        lib.orc_fwd.argtypes = [ctypes.POINTER(_Prob), vp, i64, vp, vp]
        lib.orc_bwd.argtypes = [ctypes.POINTER(_Prob), vp, vp, i64, vp, vp, i64, vp, vp, vp]
        lib.orc_num_threads.argtypes = []
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_get().orc_num_threads())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def pack(seq: torch.Tensor) -> torch.Tensor:
    """``[P, B, S/P, H, D]`` sequence shards -> ``[P, B, S, H/P, D]`` head shards."""
    P, B, Sl, H, D = seq.shape
    seq = seq.contiguous()
    out = torch.empty((P, B, Sl * P, H // P, D), dtype=seq.dtype)
    rc = _get().orc_pack(_ptr(seq), _ptr(out), P, B, Sl * P, H, D, seq.element_size())
    if rc:
        raise ValueError(f"orc_pack: {rc}")
    return out


def unpack(head: torch.Tensor) -> torch.Tensor:
    """``[P, B, S, H/P, D]`` head shards -> ``[P, B, S/P, H, D]`` sequence shards."""
    P, B, S, hp, D = head.shape
    head = head.contiguous()
    out = torch.empty((P, B, S // P, hp * P, D), dtype=head.dtype)
    rc = _get().orc_unpack(_ptr(head), _ptr(out), P, B, S, hp * P, D, head.element_size())
    if rc:
        raise ValueError(f"orc_unpack: {rc}")
    return out


def pack_replicated(seq: torch.Tensor) -> torch.Tensor:
    """``[P, B, S/P, H, D]`` with H < P (P % H == 0) -> ``[P, B, S, 1, D]``: rank c
    gets KV head c // (P // H)."""
    P, B, Sl, H, D = seq.shape
    seq = seq.contiguous()
    out = torch.empty((P, B, Sl * P, 1, D), dtype=seq.dtype)
    rc = _get().orc_pack_replicated(_ptr(seq), _ptr(out), P, B, Sl * P, H, D, seq.element_size())
    if rc:
        raise ValueError(f"orc_pack_replicated: {rc}")
    return out


def reduce_replicated(head: torch.Tensor, H: int) -> torch.Tensor:
    """bf16 or fp32 ``[P, B, S, 1, D]`` replica gradients -> bf16 ``[P, B, S/P, H, D]``:
    the sum of each head's replicas in fp32, rank order, rounded once to bf16."""
    P, B, S, one, D = head.shape
    if head.dtype not in (torch.bfloat16, torch.float32) or one != 1:
        raise ValueError("reduce_replicated: bf16 or fp32 [P, B, S, 1, D]")
    head = head.contiguous()
    out = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16)
    fn = _get().orc_reduce_replicated if head.dtype == torch.bfloat16 else _get().orc_reduce_replicated_f32
    rc = fn(_ptr(head), _ptr(out), P, B, S, H, D)
    if rc:
        raise ValueError(f"orc_reduce_replicated: {rc}")
    return out


def gather_positions(shards: torch.Tensor) -> torch.Tensor:
    """``[P, B, S/P]`` position shards -> ``[B, S]`` int64 gathered positions."""
    P, B, Sl = shards.shape
    sh = shards.to(torch.int64).contiguous()
    out = torch.empty((B, P * Sl), dtype=torch.int64)
    rc = _get().orc_gather_positions(_ptr(sh), _ptr(out), P, B, P * Sl)
    if rc:
        raise ValueError(f"orc_gather_positions: {rc}")
    return out


def segments(pos: torch.Tensor) -> Tuple[torch.Tensor, int, int]:
    """Gathered ``[B, S]`` positions -> (cu_seqlens int32 [n+1], n, max_len)."""
    B, S = pos.shape
    p = pos.to(torch.int64).contiguous()
    cap = B * S + 1
    cu = torch.zeros(cap, dtype=torch.int32)
    n = ctypes.c_int32()
    mx = ctypes.c_int32()
    rc = _get().orc_segments(_ptr(p), B, S, _ptr(cu), cap, ctypes.byref(n), ctypes.byref(mx))
    if rc:
        raise ValueError(f"orc_segments: {rc}")
    return cu[: n.value + 1].clone(), n.value, mx.value


def _f64(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    return None if t is None else t.detach().to(torch.float64).contiguous()


def _prob(q, k, v, sink, cu, causal, wl, wr, scale, keys=None):
    B, S, hq, D = q.shape
    hkv = k.shape[2]
    keep = [q, k, v, sink, cu]
    k_lo, k_hi = (0, S) if keys is None else keys
    pr = _Prob(q.data_ptr(), k.data_ptr(), v.data_ptr(),
               sink.data_ptr() if sink is not None else None,
               cu.data_ptr() if cu is not None else None,
               (cu.numel() - 1) if cu is not None else 0,
               B, S, hq, hkv, D, float(scale), int(bool(causal)), int(wl), int(wr), int(k_lo),
               int(k_hi))
    return pr, keep


def _rows(rows: Optional[Sequence[int]]):
    if rows is None:
        return None
    return torch.as_tensor(list(rows) if not isinstance(rows, torch.Tensor) else rows,
                           dtype=torch.int64).contiguous()


def attn_fwd(q, k, v, *, sink=None, cu=None, causal=True, window_left=-1, window_right=-1,
             scale=None, rows=None, keys=None):
    """Exact attention of one rank's heads.

    q ``[B, S, hq, D]``, k/v ``[B, S, hkv, D]`` (any float dtype, widened to
    fp64), sink ``[hq]`` or None, cu int32 ``[n+1]`` over the flattened B*S
    tokens or None (one document per batch row).  ``rows`` selects flattened
    query rows (default: all); ``keys = (lo, hi)`` restricts the keys to those
    positions of each batch row (one KV chunk; rows that see none of them get
    O = 0, LSE = -inf).  Returns (O fp64 ``[nrows, hq, D]``, LSE fp64
    ``[nrows, hq]``).
    """
    q, k, v, sink = _f64(q), _f64(k), _f64(v), _f64(sink)
    cu = None if cu is None else cu.to(torch.int32).contiguous()
    B, S, hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    pr, keep = _prob(q, k, v, sink, cu, causal, window_left, window_right, scale, keys)
    r = _rows(rows)
    nrows = B * S if r is None else r.numel()
    out = torch.zeros((nrows, hq, D), dtype=torch.float64)
    lse = torch.zeros((nrows, hq), dtype=torch.float64)
    rc = _get().orc_fwd(ctypes.byref(pr), _ptr(r), nrows, _ptr(out), _ptr(lse))
    if rc:
        raise ValueError(f"orc_fwd: {rc}")
    return out, lse


def merge_chunks(outs, lses, sink=None):
    """Exact combination of attention over disjoint KV chunks (fp64): with
    L = log(sum_c e^{LSE_c} + e^{sink}), O = sum_c e^{LSE_c - L} O_c.
    outs ``[n, hq, D]`` and lses ``[n, hq]`` per chunk; sink ``[hq]`` or None.
    Rows with no key in any chunk and no sink get O = 0, LSE = -inf."""
    L = torch.stack([x.to(torch.float64) for x in lses])           # [C, n, hq]
    if sink is not None:
        s = sink.to(torch.float64).reshape(1, 1, -1).expand(1, L.shape[1], L.shape[2])
        L = torch.cat([L, s])
    lse = torch.logsumexp(L, dim=0)
    w = torch.exp(L[: len(outs)] - lse)                             # [C, n, hq]
    w = torch.where(torch.isfinite(lse), w, torch.zeros_like(w))
    out = sum(w[c].unsqueeze(-1) * outs[c].to(torch.float64) for c in range(len(outs)))
    return out, lse


def attn_bwd(q, k, v, dout, *, sink=None, cu=None, causal=True, window_left=-1,
             window_right=-1, scale=None, qrows=None, krows=None, want_dq=True,
             want_dkdv=True, want_dsink=None):
    """Gradients of ``sum(O * dout)`` for one rank's heads (see ``attn_fwd``).

    Returns (dQ ``[nq, hq, D]``, dK ``[nk, hkv, D]``, dV ``[nk, hkv, D]``,
    dsink ``[hq]`` or None), all fp64; ``qrows``/``krows`` select flattened
    query rows / key rows (default: all).
    """
    q, k, v, dout, sink = _f64(q), _f64(k), _f64(v), _f64(dout), _f64(sink)
    cu = None if cu is None else cu.to(torch.int32).contiguous()
    B, S, hq, D = q.shape
    hkv = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    if want_dsink is None:
        want_dsink = sink is not None
    pr, keep = _prob(q, k, v, sink, cu, causal, window_left, window_right, scale)
    qr, kr = _rows(qrows), _rows(krows)
    nq = B * S if qr is None else qr.numel()
    nk = B * S if kr is None else kr.numel()
    dq = torch.zeros((nq, hq, D), dtype=torch.float64) if want_dq else None
    dk = torch.zeros((nk, hkv, D), dtype=torch.float64) if want_dkdv else None
    dv = torch.zeros((nk, hkv, D), dtype=torch.float64) if want_dkdv else None
    ds = torch.zeros(hq, dtype=torch.float64) if want_dsink else None
    rc = _get().orc_bwd(ctypes.byref(pr), _ptr(dout), _ptr(qr), nq, _ptr(dq), _ptr(kr), nk,
                        _ptr(dk), _ptr(dv), _ptr(ds))
    if rc:
        raise ValueError(f"orc_bwd: {rc}")
    return dq, dk, dv, ds
