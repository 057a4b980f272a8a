"""GPU: the allocation-free forward (ulysses_attn_fwd_noalloc) through the C
ABI, against ulysses_attn_fwd with a caller workspace: bit-identical outputs
on two calls in a row, the second with a smaller input (its split partials
then reuse the start of the same static array, which keeps the first call's
contents)."""
import ctypes

import pytest
import torch

from gpu_util import bits_equal, say
from ulysses_inputs import small_case

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call_pair(lib, seed, B, S, Hq, Hkv, D, causal, wl, sink):
    inp = small_case(seed, P=1, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, sink=sink)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    sk = None if inp.sink is None else inp.sink.to(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    scale = ctypes.c_float(D ** -0.5)
    need = lib.ulysses_attn_fwd_workspace_bytes(B, S, Hq, Hkv, D)
    assert 0 < need <= lib.ulysses_attn_fwd_noalloc_max_workspace(), "the case must split"
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    outs = []
    for name in ("ulysses_attn_fwd", "ulysses_attn_fwd_noalloc"):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=dev)
        say(f"{name}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} wl={wl} sink={sink}")
        if name == "ulysses_attn_fwd":
            rc = lib.ulysses_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(sk), None, None,
                                      _p(ws), ctypes.c_size_t(need), B, S, Hq, Hkv, D, scale,
                                      int(causal), wl, -1, stream)
        else:
            rc = lib.ulysses_attn_fwd_noalloc(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(sk), None,
                                              None, B, S, Hq, Hkv, D, scale, int(causal), wl, -1,
                                              stream)
        assert rc == 0, lib.ulysses_last_error()
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


def test_noalloc_forward_equals_workspace_forward():
    import ulysses_sequence_attention_rank_amd as uly
    lib = uly.load()
    lib.ulysses_attn_fwd_noalloc.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 5 + \
        [ctypes.c_float] + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    lib.ulysses_attn_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.ulysses_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ulysses_attn_fwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_size_t] + [ctypes.c_int] * 5 + \
        [ctypes.c_float] + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    lib.ulysses_last_error.restype = ctypes.c_char_p
    # the S=4096 workload's rank share (split in two over its keys), then a
    # smaller problem with a window and sinks
    for case in ((1, 4096, 6, 6, 128, True, -1, False), (1, 1000, 4, 2, 64, True, 37, True)):
        (o_ws, l_ws), (o_na, l_na) = _call_pair(lib, 77, *case)
        assert bits_equal(o_ws, o_na) and bits_equal(l_ws, l_na)
        assert torch.isfinite(o_na.float()).all()
