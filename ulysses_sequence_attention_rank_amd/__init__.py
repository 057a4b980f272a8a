"""Per-rank Ulysses sequence-parallel hot path on MI355X (gfx950).

Thin Python binding over ``libulysses.so`` (C ABI in ``include/ulysses.h``).
Every step runs in the library's HIP kernels; torch only supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing or cannot be loaded, every call raises.

Build it with ``python -m ulysses_sequence_attention_rank_amd.build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "UlyssesError", "lib_path", "load", "a2a_pack", "a2a_unpack", "a2a_pack_into",
    "a2a_unpack_into", "a2a_pack_multi_into", "a2a_unpack_multi_into", "a2a_pack_replicated_into",
    "a2a_reduce_replicated_into", "cu_seqlens_from_positions", "cu_seqlens_capacity", "attn_fwd",
    "attn_bwd",
    "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes", "Layout", "view_layout",
    "attn_fwd_chunk", "attn_merge", "attn_merge_finish", "profile_start", "profile_stop", "profile_report",
    "calibrate_mfma",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libulysses.so")
_lib = None

_STATUS = {0: "ULY_OK", -1: "ULY_ERR_NULL", -2: "ULY_ERR_SHAPE", -3: "ULY_ERR_HEADS",
           -4: "ULY_ERR_UNSUPPORTED", -5: "ULY_ERR_CAPACITY", -6: "ULY_ERR_ALIGN",
           -7: "ULY_ERR_HIP"}

EXPORTS = ("ulysses_a2a_pack", "ulysses_a2a_unpack", "ulysses_a2a_pack_multi",
           "ulysses_a2a_unpack_multi", "ulysses_a2a_pack_replicated",
           "ulysses_a2a_reduce_replicated", "ulysses_cu_seqlens_from_positions",
           "ulysses_attn_fwd", "ulysses_attn_fwd_layout", "ulysses_attn_bwd_layout",
           "ulysses_attn_bwd_layout_f32kv", "ulysses_attn_fwd_chunk", "ulysses_attn_merge",
           "ulysses_attn_merge_finish",
           "ulysses_attn_fwd_workspace_bytes", "ulysses_attn_bwd_workspace_bytes", "ulysses_attn_bwd",
           "ulysses_tiled_mlp_workspace_bytes", "ulysses_tiled_mlp_fwd", "ulysses_tiled_mlp_bwd",
           "ulysses_profile_start", "ulysses_profile_stop", "ulysses_profile_report",
           "ulysses_calibrate_mfma", "ulysses_calibrate_mfma_flops", "ulysses_last_error")


class UlyssesError(RuntimeError):
    def __init__(self, code: int, fn: str, detail: str):
        self.code = code
        super().__init__(f"{fn} failed: {_STATUS.get(code, code)}: {detail}")


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load ``libulysses.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build the HIP library first "
                           "(python -m ulysses_sequence_attention_rank_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.ulysses_a2a_pack.argtypes = [vp, vp] + [i32] * 6 + [vp]
    lib.ulysses_a2a_unpack.argtypes = [vp, vp] + [i32] * 6 + [vp]
    lib.ulysses_a2a_pack_multi.argtypes = [i32, vp, vp, vp] + [i32] * 5 + [vp]
    lib.ulysses_a2a_pack_replicated.argtypes = [vp, vp] + [i32] * 6 + [vp]
    lib.ulysses_a2a_reduce_replicated.argtypes = [vp, i32, vp] + [i32] * 5 + [vp]
    lib.ulysses_a2a_unpack_multi.argtypes = [i32, vp, vp, vp] + [i32] * 5 + [vp]
    lib.ulysses_cu_seqlens_from_positions.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.ulysses_cu_seqlens_capacity.argtypes = [i32, i32]
    lib.ulysses_attn_fwd.argtypes = [vp] * 9 + [sz] + [i32] * 5 + [f32] + [i32] * 3 + [vp]
    lib.ulysses_attn_fwd_workspace_bytes.argtypes = [i32] * 5
    lib.ulysses_attn_fwd_layout.argtypes = [vp] * 9 + [sz, vp, vp] + [i32] * 5 + [f32] + [i32] * 3 + [vp]
    lib.ulysses_attn_bwd_layout.argtypes = [vp] * 14 + [sz, vp, vp] + [i32] * 5 + [f32] + [i32] * 3 + [vp]
    lib.ulysses_attn_bwd_layout_f32kv.argtypes = lib.ulysses_attn_bwd_layout.argtypes
    lib.ulysses_attn_fwd_chunk.argtypes = [vp] * 8 + [sz, vp, vp] + [i32] * 7 + [f32] + [i32] * 3 + [vp]
    lib.ulysses_attn_merge.argtypes = [vp] * 4 + [i32] * 4 + [vp]
    lib.ulysses_attn_merge_finish.argtypes = [vp] * 5 + [i32] * 4 + [vp]
    lib.ulysses_attn_fwd_workspace_bytes.restype = sz
    lib.ulysses_attn_bwd_workspace_bytes.argtypes = [i32] * 5
    lib.ulysses_attn_bwd_workspace_bytes.restype = sz
    lib.ulysses_attn_bwd.argtypes = [vp] * 14 + [sz] + [i32] * 5 + [f32] + [i32] * 3 + [vp]
    lib.ulysses_attn_bwd_status_offset.argtypes = [i32] * 5
    lib.ulysses_attn_bwd_status_offset.restype = sz
    lib.ulysses_tiled_mlp_workspace_bytes.argtypes = [i32] * 4
    lib.ulysses_tiled_mlp_workspace_bytes.restype = sz
    lib.ulysses_tiled_mlp_fwd.argtypes = [vp] * 5 + [i32] * 4 + [vp, sz, vp]
    lib.ulysses_tiled_mlp_bwd.argtypes = [vp] * 9 + [i32] * 4 + [vp, sz, vp]
    lib.ulysses_profile_start.argtypes = [i32]
    lib.ulysses_profile_stop.argtypes = []
    lib.ulysses_profile_report.argtypes = [ctypes.c_char_p, sz]
    lib.ulysses_calibrate_mfma.argtypes = [vp, sz, i32, i32, vp]
    lib.ulysses_calibrate_mfma_flops.argtypes = [i32]
    lib.ulysses_calibrate_mfma_flops.restype = sz
    lib.ulysses_last_error.argtypes = []
    lib.ulysses_last_error.restype = ctypes.c_char_p
    for fn in EXPORTS:
        if not hasattr(lib, fn):
            raise RuntimeError(f"{_LIB_PATH} does not export {fn}")
    _lib = lib
    return lib


def _check(rc: int, fn: str):
    if rc != 0:
        raise UlyssesError(rc, fn, load().ulysses_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, strided: bool = False):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not strided and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# -------------------------------------------------------------- profiling

def profile_start(max_launches: int = 4096):
    """Record a HIP event pair around every kernel launch from now on."""
    _check(load().ulysses_profile_start(int(max_launches)), "ulysses_profile_start")


def profile_stop():
    _check(load().ulysses_profile_stop(), "ulysses_profile_stop")


def calibrate_mfma(iters: int, mode: int = 0, out: Optional[torch.Tensor] = None) -> int:
    """One launch of the matrix-core calibration (a measurement aid, on the
    current stream of ``out``'s device, default cuda:current): 512 work-groups,
    every wave ``iters`` bf16 32x32x16 products on eight accumulators; mode 0
    register operands, 1 with 8 fp32 FMAs per product, 2 one operand from LDS,
    3 both from LDS, 4 with 8 exp2 per product, 5 as 4 with multiplies in
    place of the exp2.  Returns the FLOPs it executes."""
    if out is None:
        out = torch.empty(512 * 256, dtype=torch.float32,
                          device=torch.device("cuda", torch.cuda.current_device()))
    _dev(out, "out", torch.float32)
    lib = load()
    _check(lib.ulysses_calibrate_mfma(_p(out), out.numel() * 4, int(iters), int(mode),
                                      _stream(out.device)), "ulysses_calibrate_mfma")
    return int(lib.ulysses_calibrate_mfma_flops(int(iters)))


def profile_report() -> dict:
    """{kernel: (count, total_ms, min_ms, max_ms)} of the launches recorded so far."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = load().ulysses_profile_report(buf, len(buf))
    if n < 0:
        _check(n, "ulysses_profile_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, tot, mn, mx = line.split()
        out[name] = (int(cnt), float(tot), float(mn), float(mx))
    return out


# ------------------------------------------------------------------ layout

def a2a_pack_into(seq: torch.Tensor, head: torch.Tensor, P: int):
    """``[P, B, S/P, H, D]`` sequence shards -> ``head`` ``[P, B, S, H/P, D]``."""
    _dev(seq, "seq"), _dev(head, "head")
    Pp, B, Sl, H, D = seq.shape
    if Pp != P or head.numel() != seq.numel() or head.dtype != seq.dtype:
        raise ValueError("pack: shape/dtype mismatch")
    _check(load().ulysses_a2a_pack(_p(seq), _p(head), P, B, Sl * P, H, D, seq.element_size(),
                                   _stream(seq.device)), "ulysses_a2a_pack")
    return head


def a2a_pack(seq: torch.Tensor) -> torch.Tensor:
    P, B, Sl, H, D = seq.shape
    head = torch.empty((P, B, Sl * P, H // P, D), dtype=seq.dtype, device=seq.device)
    return a2a_pack_into(seq, head, P)


def a2a_unpack_into(head: torch.Tensor, seq: torch.Tensor, P: int):
    """``[P, B, S, H/P, D]`` head shards -> ``seq`` ``[P, B, S/P, H, D]``."""
    _dev(head, "head"), _dev(seq, "seq")
    Pp, B, S, hp, D = head.shape
    if Pp != P or head.numel() != seq.numel() or head.dtype != seq.dtype:
        raise ValueError("unpack: shape/dtype mismatch")
    _check(load().ulysses_a2a_unpack(_p(head), _p(seq), P, B, S, hp * P, D, head.element_size(),
                                     _stream(head.device)), "ulysses_a2a_unpack")
    return seq


def a2a_unpack(head: torch.Tensor) -> torch.Tensor:
    P, B, S, hp, D = head.shape
    seq = torch.empty((P, B, S // P, hp * P, D), dtype=head.dtype, device=head.device)
    return a2a_unpack_into(head, seq, P)


def _multi(fn_name, srcs, dsts, P, seq_side_is_src):
    n = len(srcs)
    if n != len(dsts) or not 1 <= n <= 4:
        raise ValueError(f"{fn_name}: 1..4 source/destination pairs")
    for i, (a, b) in enumerate(zip(srcs, dsts)):
        _dev(a, f"src{i}"), _dev(b, f"dst{i}")
        if a.numel() != b.numel() or a.dtype != b.dtype or a.dtype != srcs[0].dtype:
            raise ValueError(f"{fn_name}: shape/dtype mismatch at tensor {i}")
    seqs = srcs if seq_side_is_src else dsts
    Pp, B, Sl, _, D = seqs[0].shape
    if Pp != P or any(t.shape[0] != P or t.shape[1] != B or t.shape[2] != Sl or t.shape[4] != D
                      for t in seqs):
        raise ValueError(f"{fn_name}: tensors disagree on P, B, S/P or D")
    VP = ctypes.c_void_p * n
    src_arr = VP(*[t.data_ptr() for t in srcs])
    dst_arr = VP(*[t.data_ptr() for t in dsts])
    H = (ctypes.c_int * n)(*[t.shape[3] for t in seqs])
    _check(getattr(load(), fn_name)(n, src_arr, dst_arr, H, P, B, Sl * P, D, srcs[0].element_size(),
                                    _stream(srcs[0].device)), fn_name)


def a2a_pack_multi_into(seqs, heads, P: int):
    """Pack up to four tensors of one exchange (e.g. Q, K, V) in one launch:
    ``seqs[i]`` ``[P, B, S/P, H_i, D]`` -> ``heads[i]`` ``[P, B, S, H_i/P, D]``."""
    _multi("ulysses_a2a_pack_multi", list(seqs), list(heads), P, True)
    return heads


def a2a_unpack_multi_into(heads, seqs, P: int):
    """Inverse of ``a2a_pack_multi_into`` (e.g. dQ, dK, dV in one launch)."""
    _multi("ulysses_a2a_unpack_multi", list(heads), list(seqs), P, False)
    return seqs


def a2a_pack_replicated_into(seq: torch.Tensor, head: torch.Tensor, P: int):
    """KV heads fewer than ranks: ``[P, B, S/P, H, D]`` (H < P, P % H == 0) ->
    ``head`` ``[P, B, S, 1, D]``, rank c getting head c // (P // H)."""
    _dev(seq, "seq"), _dev(head, "head")
    Pp, B, Sl, H, D = seq.shape
    if Pp != P or tuple(head.shape) != (P, B, Sl * P, 1, D) or head.dtype != seq.dtype:
        raise ValueError("pack_replicated: shape/dtype mismatch")
    _check(load().ulysses_a2a_pack_replicated(_p(seq), _p(head), P, B, Sl * P, H, D,
                                              seq.element_size(), _stream(seq.device)),
           "ulysses_a2a_pack_replicated")
    return head


def a2a_reduce_replicated_into(head: torch.Tensor, seq: torch.Tensor, P: int):
    """Gradient of ``a2a_pack_replicated_into``: each of the H heads of the bf16
    ``seq`` ``[P, B, S/P, H, D]`` gets the sum of its P // H replicas in ``head``
    (fp32 or bf16), accumulated in fp32 and rounded once."""
    _dev(head, "head"), _dev(seq, "seq", torch.bfloat16)
    if head.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("reduce_replicated: head must be fp32 or bf16")
    Pp, B, Sl, H, D = seq.shape
    if Pp != P or tuple(head.shape) != (P, B, Sl * P, 1, D):
        raise ValueError("reduce_replicated: shape mismatch")
    _check(load().ulysses_a2a_reduce_replicated(_p(head), head.element_size(), _p(seq), P, B,
                                                Sl * P, H, D, _stream(seq.device)),
           "ulysses_a2a_reduce_replicated")
    return seq


# ---------------------------------------------------------------- segments

def cu_seqlens_capacity(B: int, S: int) -> int:
    """Slots of a cu_seqlens buffer that lets the scan run on many work-groups."""
    return int(load().ulysses_cu_seqlens_capacity(B, S))


def cu_seqlens_from_positions(pos_shards: torch.Tensor, cu: Optional[torch.Tensor] = None,
                              n_seqs: Optional[torch.Tensor] = None,
                              max_len: Optional[torch.Tensor] = None):
    """``[P, B, S/P]`` int32/int64 position shards -> (cu int32 [cu_seqlens_capacity(B, S)],
    n_seqs int32 [1], max_len int32 [1]), all on the device (entries of cu past
    n_seqs are unspecified)."""
    _dev(pos_shards, "pos_shards")
    if pos_shards.dtype not in (torch.int32, torch.int64):
        raise ValueError("positions must be int32 or int64")
    P, B, Sl = pos_shards.shape
    dev = pos_shards.device
    if cu is None:
        cu = torch.empty(cu_seqlens_capacity(B, Sl * P), dtype=torch.int32, device=dev)
    if n_seqs is None:
        n_seqs = torch.empty(1, dtype=torch.int32, device=dev)
    if max_len is None:
        max_len = torch.empty(1, dtype=torch.int32, device=dev)
    _check(load().ulysses_cu_seqlens_from_positions(
        _p(pos_shards), pos_shards.element_size(), P, B, Sl * P, _p(cu), cu.numel(), _p(n_seqs),
        _p(max_len), _stream(dev)), "ulysses_cu_seqlens_from_positions")
    return cu, n_seqs, max_len


# --------------------------------------------------------------- attention

class Layout(ctypes.Structure):
    """``uly_layout``: element (b, s, h, :) at b*batch + r*shard + sl*token + h*head,
    s = r * (S / shards) + sl."""
    _fields_ = [("shards", ctypes.c_int), ("batch", ctypes.c_int64), ("shard", ctypes.c_int64),
                ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


def view_layout(t: torch.Tensor):
    """Sizes and layout of a strided view: 4-D ``[B, S, h, D]`` or 5-D
    ``[P, B, S/P, h, D]`` (P sequence shards), last dimension contiguous.
    Returns (B, S, h, D, Layout)."""
    if t.stride(-1) != 1:
        raise ValueError("the head dimension D must be contiguous")
    st = t.stride()
    if t.dim() == 4:
        B, S, h, D = t.shape
        return B, S, h, D, Layout(1, st[0], 0, st[1], st[2])
    if t.dim() == 5:
        P, B, Sl, h, D = t.shape
        return B, P * Sl, h, D, Layout(P, st[1], st[0], st[2], st[3])
    raise ValueError("expected a [B, S, h, D] or [P, B, S/P, h, D] view")


def _is_head_layout(t):
    return t.dim() == 4 and t.is_contiguous()


def _same_view(a, b, what):
    if a.shape != b.shape or a.stride() != b.stride():
        raise ValueError(f"{what} must have the same shape and strides")


def _like(t):
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)


def _shapes(q, k):
    B, S, hq, D, lq = view_layout(q)
    Bk, Sk, hkv, Dk, lk = view_layout(k)
    if (Bk, Sk, Dk) != (B, S, D):
        raise ValueError("q and k/v shapes disagree")
    return B, S, hq, hkv, D, lq, lk


def attn_fwd_workspace_bytes(B, S, hq, hkv, D) -> int:
    return int(load().ulysses_attn_fwd_workspace_bytes(B, S, hq, hkv, D))


def attn_fwd(q, k, v, *, sink=None, cu_seqlens=None, n_seqs=None, causal=True, window_left=-1,
             window_right=-1, softmax_scale=None, out=None, lse=None, workspace=None):
    """One rank's attention: q ``[B, S, hq, D]``, k/v ``[B, S, hkv, D]`` bf16, or
    strided views of the rank's heads in another layout (``view_layout``: e.g.
    ``seq[:, :, :, r*hq:(r+1)*hq]`` of the sequence shards ``[P, B, S/P, H, D]``),
    read in place; ``out`` then has q's shape and strides.
    Returns (out, lse fp32 ``[B, hq, S]``)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, torch.bfloat16, strided=True)
    B, S, hq, hkv, D, lq, lk = _shapes(q, k)
    _same_view(k, v, "k and v")
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    if out is None:
        out = _like(q)
    _same_view(q, out, "q and out")
    _dev(out, "out", torch.bfloat16, strided=True)
    if lse is None:
        lse = torch.empty((B, hq, S), dtype=torch.float32, device=q.device)
    if sink is not None:
        _dev(sink, "sink", torch.float32)
    if workspace is None:
        need = attn_fwd_workspace_bytes(B, S, hq, hkv, D)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel()
    common = (float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
              _stream(q.device))
    if all(_is_head_layout(t) for t in (q, k, v, out)):  # the plain [B, S, h, D] entry point
        _check(load().ulysses_attn_fwd(
            _p(q), _p(k), _p(v), _p(out), _p(lse), _p(sink), _p(cu_seqlens), _p(n_seqs),
            _p(workspace), ws_bytes, B, S, hq, hkv, D, *common), "ulysses_attn_fwd")
        return out, lse
    _check(load().ulysses_attn_fwd_layout(
        _p(q), _p(k), _p(v), _p(out), _p(lse), _p(sink), _p(cu_seqlens), _p(n_seqs), _p(workspace),
        ws_bytes, ctypes.byref(lq), ctypes.byref(lk), B, S, hq, hkv, D, *common),
        "ulysses_attn_fwd_layout")
    return out, lse


def attn_fwd_chunk(q, k_chunk, v_chunk, k_start: int, *, cu_seqlens=None, n_seqs=None, causal=True,
                   window_left=-1, window_right=-1, softmax_scale=None, out=None, lse=None,
                   workspace=None):
    """Attention of q (``[B, S, hq, D]`` or a strided view, as ``attn_fwd``)
    against the keys at positions ``[k_start, k_start + Sk)`` of every batch
    row, held in ``k_chunk``/``v_chunk`` ``[B, Sk, hkv, D]`` (views allowed).
    Returns (out fp32 ``[B, S, hq, D]`` normalised over the chunk, lse fp32
    ``[B, hq, S]``); rows seeing no key of the chunk get 0 and -inf."""
    for name, t in (("q", q), ("k_chunk", k_chunk), ("v_chunk", v_chunk)):
        _dev(t, name, torch.bfloat16, strided=True)
    B, S, hq, D, lq = view_layout(q)
    Bk, Sk, hkv, Dk, lk = view_layout(k_chunk)
    if (Bk, Dk) != (B, D):
        raise ValueError("q and the KV chunk disagree on B or D")
    _same_view(k_chunk, v_chunk, "k_chunk and v_chunk")
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, S, hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, hq, S), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32)
    if workspace is None:
        need = attn_fwd_workspace_bytes(B, S, hq, hkv, D)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    _check(load().ulysses_attn_fwd_chunk(
        _p(q), _p(k_chunk), _p(v_chunk), _p(out), _p(lse), _p(cu_seqlens), _p(n_seqs),
        _p(workspace), 0 if workspace is None else workspace.numel(), ctypes.byref(lq),
        ctypes.byref(lk), B, S, int(k_start), Sk, hq, hkv, D, float(softmax_scale),
        int(bool(causal)), int(window_left), int(window_right), _stream(q.device)),
        "ulysses_attn_fwd_chunk")
    return out, lse


def attn_merge(acc_out, acc_lse, out, lse):
    """acc := exact merge of acc with one more chunk's (out, lse), in place."""
    for name, t in (("acc_out", acc_out), ("acc_lse", acc_lse), ("out", out), ("lse", lse)):
        _dev(t, name, torch.float32)
    B, S, hq, D = acc_out.shape
    if out.shape != acc_out.shape or acc_lse.shape != (B, hq, S) or lse.shape != (B, hq, S):
        raise ValueError("attn_merge: shape mismatch")
    _check(load().ulysses_attn_merge(_p(acc_out), _p(acc_lse), _p(out), _p(lse), B, S, hq, D,
                                     _stream(out.device)), "ulysses_attn_merge")
    return acc_out, acc_lse


def attn_merge_finish(acc_out, acc_lse, *, sink=None, out=None, lse=None):
    """Final bf16 O and LSE from the accumulator, the sink joining once."""
    _dev(acc_out, "acc_out", torch.float32), _dev(acc_lse, "acc_lse", torch.float32)
    B, S, hq, D = acc_out.shape
    out = torch.empty((B, S, hq, D), dtype=torch.bfloat16, device=acc_out.device) if out is None else out
    lse = torch.empty_like(acc_lse) if lse is None else lse
    if sink is not None:
        _dev(sink, "sink", torch.float32)
    _check(load().ulysses_attn_merge_finish(_p(acc_out), _p(acc_lse), _p(sink), _p(out), _p(lse), B,
                                            S, hq, D, _stream(acc_out.device)),
           "ulysses_attn_merge_finish")
    return out, lse


def attn_bwd_workspace_bytes(B, S, hq, hkv, D) -> int:
    return int(load().ulysses_attn_bwd_workspace_bytes(B, S, hq, hkv, D))


def attn_bwd_status(workspace: torch.Tensor, B, S, hq, hkv, D) -> torch.Tensor:
    """The six int32 status words a backward call with these sizes left in
    ``workspace`` (a device view; read it after the call on its stream): the
    exponents of the power-of-two scales of the fp16 copies of dout, v, q and k,
    the count of copied elements that saturated, and the count of inexact ones."""
    off = int(load().ulysses_attn_bwd_status_offset(B, S, hq, hkv, D))
    return workspace[off:off + 24].view(torch.int32)


def attn_bwd(q, k, v, out, dout, lse, *, sink=None, cu_seqlens=None, n_seqs=None, causal=True,
             window_left=-1, window_right=-1, softmax_scale=None, dq=None, dk=None, dv=None,
             dsink=None, workspace=None, kv_grad_fp32=False):
    """Backward of ``attn_fwd`` for the loss ``sum(out * dout)``; views as in
    ``attn_fwd`` (out, dout, dq with q's strides, dk, dv with k's).
    ``kv_grad_fp32``: dk, dv are fp32 and unrounded (to be summed further).
    Returns (dq, dk, dv, dsink or None)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _dev(t, name, torch.bfloat16, strided=True)
    _dev(lse, "lse", torch.float32)
    B, S, hq, hkv, D, lq, lk = _shapes(q, k)
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    kv_dtype = torch.float32 if kv_grad_fp32 else torch.bfloat16
    dq = _like(q) if dq is None else dq
    if dk is None:
        dk = torch.empty_strided(k.shape, k.stride(), dtype=kv_dtype, device=k.device)
    if dv is None:
        dv = torch.empty_strided(v.shape, v.stride(), dtype=kv_dtype, device=v.device)
    for a, b, what in ((q, out, "q and out"), (q, dout, "q and dout"), (q, dq, "q and dq"),
                       (k, v, "k and v"), (k, dk, "k and dk"), (k, dv, "k and dv")):
        _same_view(a, b, what)
    _dev(dq, "dq", torch.bfloat16, strided=True)
    for name, t in (("dk", dk), ("dv", dv)):
        _dev(t, name, kv_dtype, strided=True)
    if sink is not None and dsink is None:
        dsink = torch.empty_like(sink)
    need = attn_bwd_workspace_bytes(B, S, hq, hkv, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ptrs = (_p(q), _p(k), _p(v), _p(out), _p(dout), _p(lse), _p(sink), _p(cu_seqlens), _p(n_seqs),
            _p(dq), _p(dk), _p(dv), _p(dsink), _p(workspace), workspace.numel())
    common = (float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
              _stream(q.device))
    if not kv_grad_fp32 and all(_is_head_layout(t) for t in (q, k, v, out, dout, dq, dk, dv)):
        _check(load().ulysses_attn_bwd(*ptrs, B, S, hq, hkv, D, *common), "ulysses_attn_bwd")
    else:
        fn = "ulysses_attn_bwd_layout_f32kv" if kv_grad_fp32 else "ulysses_attn_bwd_layout"
        _check(getattr(load(), fn)(*ptrs, ctypes.byref(lq), ctypes.byref(lk), B, S, hq, hkv, D,
                                   *common), fn)
    return dq, dk, dv, (dsink if sink is not None else None)


# ------------------------------------------------------------ tiled MLP

def tiled_mlp_workspace_bytes(T: int, H: int, I: int, tile: int) -> int:
    return int(load().ulysses_tiled_mlp_workspace_bytes(T, H, I, tile))


def _mlp_shapes(x, w_gate, w_up, w_down):
    for name, t in (("x", x), ("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _dev(t, name, torch.bfloat16)
    T, H = x.shape
    I = w_gate.shape[0]
    if w_gate.shape != (I, H) or w_up.shape != (I, H) or w_down.shape != (H, I):
        raise ValueError("tiled MLP: weights must be [I, H], [I, H], [H, I] for x [T, H]")
    return T, H, I


def tiled_mlp_fwd(x, w_gate, w_up, w_down, tile: int, *, y=None, workspace=None):
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T over the tokens of x ``[T, H]`` in tiles
    of ``tile`` tokens (bf16; weights ``[I, H]``, ``[I, H]``, ``[H, I]``)."""
    T, H, I = _mlp_shapes(x, w_gate, w_up, w_down)
    y = torch.empty_like(x) if y is None else y
    _dev(y, "y", torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(tiled_mlp_workspace_bytes(T, H, I, tile), dtype=torch.uint8,
                                device=x.device)
    _check(load().ulysses_tiled_mlp_fwd(_p(x), _p(w_gate), _p(w_up), _p(w_down), _p(y), T, H, I,
                                        int(tile), _p(workspace), workspace.numel(),
                                        _stream(x.device)), "ulysses_tiled_mlp_fwd")
    return y


def tiled_mlp_bwd(x, w_gate, w_up, w_down, dy, tile: int, *, dx=None, dw_gate=None, dw_up=None,
                  dw_down=None, workspace=None):
    """Backward of ``tiled_mlp_fwd`` for the loss ``sum(y * dy)``: each tile's
    activations recomputed from x, weight gradients summed in fp32 over the
    tiles.  Returns (dx bf16 ``[T, H]``, dw_gate, dw_up fp32 ``[I, H]``,
    dw_down fp32 ``[H, I]``)."""
    T, H, I = _mlp_shapes(x, w_gate, w_up, w_down)
    _dev(dy, "dy", torch.bfloat16)
    dev = x.device
    dx = torch.empty_like(x) if dx is None else dx
    dw_gate = torch.empty((I, H), dtype=torch.float32, device=dev) if dw_gate is None else dw_gate
    dw_up = torch.empty((I, H), dtype=torch.float32, device=dev) if dw_up is None else dw_up
    dw_down = torch.empty((H, I), dtype=torch.float32, device=dev) if dw_down is None else dw_down
    _dev(dx, "dx", torch.bfloat16)
    for name, t in (("dw_gate", dw_gate), ("dw_up", dw_up), ("dw_down", dw_down)):
        _dev(t, name, torch.float32)
    if workspace is None:
        workspace = torch.empty(tiled_mlp_workspace_bytes(T, H, I, tile), dtype=torch.uint8, device=dev)
    _check(load().ulysses_tiled_mlp_bwd(_p(x), _p(w_gate), _p(w_up), _p(w_down), _p(dy), _p(dx),
                                        _p(dw_gate), _p(dw_up), _p(dw_down), T, H, I, int(tile),
                                        _p(workspace), workspace.numel(), _stream(dev)),
           "ulysses_tiled_mlp_bwd")
    return dx, dw_gate, dw_up, dw_down
