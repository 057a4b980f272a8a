"""The C-ABI library loads, exports every symbol ``include/ulysses.h`` declares,
and rejects bad arguments on the host before any launch (CPU only: no call
here reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import ulysses_sequence_attention_rank_amd as uly

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

OK, NULL, SHAPE, HEADS, UNSUP, CAP, ALIGN = 0, -1, -2, -3, -4, -5, -6
A = 1 << 20  # a 256-byte-aligned dummy address; never dereferenced by a rejected call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(uly.lib_path()):
        from ulysses_sequence_attention_rank_amd import build
        build.build()
    return uly.load()


def declared():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(ulysses_\w+)\s*\(", text, re.M))


def test_header_declares_the_boundary():
    assert declared() == {"ulysses_a2a_pack", "ulysses_a2a_unpack", "ulysses_a2a_pack_multi",
                          "ulysses_a2a_unpack_multi", "ulysses_a2a_pack_replicated",
                          "ulysses_a2a_reduce_replicated",
                          "ulysses_cu_seqlens_from_positions", "ulysses_cu_seqlens_capacity",
                          "ulysses_attn_fwd",
                          "ulysses_attn_fwd_layout", "ulysses_attn_bwd_layout",
                          "ulysses_attn_fwd_noalloc", "ulysses_attn_fwd_noalloc_max_workspace",
                          "ulysses_attn_bwd_layout_f32kv", "ulysses_attn_fwd_chunk",
                          "ulysses_attn_merge", "ulysses_attn_merge_finish",
                          "ulysses_attn_fwd_workspace_bytes",
                          "ulysses_attn_bwd_workspace_bytes", "ulysses_attn_bwd",
                          "ulysses_attn_bwd_status_offset",
                          "ulysses_tiled_mlp_workspace_bytes", "ulysses_tiled_mlp_fwd",
                          "ulysses_tiled_mlp_bwd",
                          "ulysses_profile_start", "ulysses_profile_stop",
                          "ulysses_profile_report", "ulysses_calibrate_mfma",
                          "ulysses_calibrate_mfma_flops", "ulysses_last_error"}


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", uly.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(ulysses_\w+)\b", out))
    assert declared() <= exported
    for name in declared():
        assert hasattr(lib, name)


def _p(x):
    return ctypes.c_void_p(x)


def test_pack_argument_errors(lib):
    f = lib.ulysses_a2a_pack
    assert f(None, _p(A), 2, 1, 8, 4, 4, 2, None) == NULL
    assert f(_p(A), _p(2 * A), 0, 1, 8, 4, 4, 2, None) == SHAPE
    assert f(_p(A), _p(2 * A), 3, 1, 8, 6, 4, 2, None) == SHAPE      # S % P
    assert f(_p(A), _p(2 * A), 2, 1, 8, 3, 4, 2, None) == HEADS      # H % P
    assert f(_p(A), _p(2 * A), 2, 1, 8, 4, 4, 3, None) == UNSUP      # elem_bytes
    assert f(_p(A + 1), _p(2 * A), 2, 1, 8, 4, 4, 2, None) == ALIGN
    assert f(_p(A), _p(A + 64), 2, 1, 8, 4, 4, 2, None) == UNSUP     # overlap
    assert b"overlap" in lib.ulysses_last_error()
    assert lib.ulysses_a2a_unpack(_p(A), _p(2 * A), 2, 1, 8, 3, 4, 2, None) == HEADS


def test_pack_multi_argument_errors(lib):
    def call(n=2, srcs=(A, 3 * A), dsts=(2 * A, 4 * A), H=(4, 2), P=2, S=8, D=2, eb=2, fn=None):
        VP = ctypes.c_void_p * max(n, 1)
        src = VP(*[ctypes.c_void_p(x) for x in srcs][:max(n, 1)])
        dst = VP(*[ctypes.c_void_p(x) for x in dsts][:max(n, 1)])
        hh = (ctypes.c_int * max(n, 1))(*H[:max(n, 1)])
        f = fn or lib.ulysses_a2a_pack_multi
        return f(n, src, dst, hh, P, 1, S, D, eb, None)
    assert call(n=0) == UNSUP
    assert call(n=5, srcs=(A,) * 5, dsts=(2 * A,) * 5, H=(2,) * 5) == UNSUP
    assert call(H=(4, 3)) == HEADS                    # 3 heads over 2 ranks
    assert call(dsts=(2 * A, 2 * A)) == UNSUP         # two destinations overlap
    assert call(dsts=(2 * A, 3 * A)) == UNSUP         # a destination overlaps a source
    assert call(S=7) == SHAPE
    assert lib.ulysses_a2a_pack_multi(1, None, None, None, 2, 1, 8, 2, 2, None) == NULL
    assert call(fn=lib.ulysses_a2a_unpack_multi, n=0) == UNSUP


def test_replicated_argument_errors(lib):
    f, g = lib.ulysses_a2a_pack_replicated, lib.ulysses_a2a_reduce_replicated
    assert f(_p(A), _p(2 * A), 4, 1, 8, 3, 8, 2, None) == HEADS     # 3 heads do not divide 4 ranks
    assert f(_p(A), _p(2 * A), 4, 1, 8, 8, 8, 2, None) == HEADS     # not fewer heads than ranks
    assert f(_p(A), _p(2 * A), 4, 1, 6, 2, 8, 2, None) == SHAPE     # S % P
    assert f(None, _p(2 * A), 4, 1, 8, 2, 8, 2, None) == NULL
    assert f(_p(A), _p(A + 64), 4, 1, 8, 2, 8, 2, None) == UNSUP    # overlap
    assert g(_p(A), 2, _p(2 * A), 4, 1, 8, 2, 12, None) == UNSUP    # D % 8
    assert g(_p(A + 2), 2, _p(2 * A), 4, 1, 8, 2, 8, None) == ALIGN
    assert g(_p(A), 3, _p(2 * A), 4, 1, 8, 2, 8, None) == UNSUP      # in_elem_bytes


def test_segments_argument_errors(lib):
    f = lib.ulysses_cu_seqlens_from_positions
    n, m, cu = _p(3 * A), _p(3 * A + 4), _p(4 * A)
    assert f(_p(A), 8, 2, 1, 8, cu, 8, n, m, None) == CAP           # needs B*S+1 = 9
    assert f(_p(A), 2, 2, 1, 8, cu, 9, n, m, None) == UNSUP         # pos_bytes
    assert f(_p(A), 8, 3, 1, 8, cu, 9, n, m, None) == SHAPE         # S % P
    assert f(None, 8, 2, 1, 8, cu, 9, n, m, None) == NULL
    assert f(_p(A + 4), 8, 2, 1, 8, cu, 9, n, m, None) == ALIGN


def _fwd(lib, q=A, k=2 * A, v=3 * A, out=4 * A, lse=5 * A, sink=None, cu=None, n=None, ws=None,
         ws_bytes=0, B=1, S=64, hq=4, hkv=2, D=128, scale=0.125, causal=1, wl=-1, wr=-1):
    return lib.ulysses_attn_fwd(_p(q), _p(k), _p(v), _p(out), _p(lse),
                                None if sink is None else _p(sink), None if cu is None else _p(cu),
                                None if n is None else _p(n), None if ws is None else _p(ws),
                                ctypes.c_size_t(ws_bytes), B, S, hq, hkv, D,
                                ctypes.c_float(scale), causal, wl, wr, None)


def test_attn_fwd_argument_errors(lib):
    assert _fwd(lib, hq=6, hkv=4) == HEADS
    assert _fwd(lib, D=96) == UNSUP
    assert _fwd(lib, wl=-2) == UNSUP
    assert _fwd(lib, scale=0.0) == UNSUP
    assert _fwd(lib, S=0) == SHAPE
    assert _fwd(lib, q=A + 8) == ALIGN
    assert _fwd(lib, cu=6 * A) == NULL       # cu_seqlens without n_seqs
    assert _fwd(lib, q=0) == NULL
    assert _fwd(lib, hq=6, hkv=4) == HEADS
    assert b"query heads" in lib.ulysses_last_error()


def test_attn_fwd_workspace(lib):
    # a small problem (few query tiles) is split over its keys and needs a workspace
    need = lib.ulysses_attn_fwd_workspace_bytes(1, 4096, 6, 6, 128)
    assert need > 4096 * 6 * 128 * 4
    assert _fwd(lib, S=4096, hq=6, hkv=6) == NULL                            # none given
    assert _fwd(lib, S=4096, hq=6, hkv=6, ws=6 * A, ws_bytes=need - 1) == CAP
    assert _fwd(lib, S=4096, hq=6, hkv=6, ws=6 * A + 16, ws_bytes=need) == ALIGN
    # a problem that fills the GPU in one pass needs none
    assert lib.ulysses_attn_fwd_workspace_bytes(1, 131072, 7, 1, 128) == 0
    assert lib.ulysses_attn_fwd_workspace_bytes(1, 4096, 6, 6, 96) == 0


def test_layout_argument_errors(lib):
    from ulysses_sequence_attention_rank_amd import Layout
    ok_q, ok_k = Layout(1, 64 * 4 * 128, 0, 4 * 128, 128), Layout(1, 64 * 2 * 128, 0, 2 * 128, 128)

    def fwd(lq=ok_q, lk=ok_k):
        return lib.ulysses_attn_fwd_layout(
            _p(A), _p(2 * A), _p(3 * A), _p(4 * A), _p(5 * A), None, None, None, None,
            ctypes.c_size_t(0), None if lq is None else ctypes.byref(lq),
            None if lk is None else ctypes.byref(lk), 1, 64, 4, 2, 128, ctypes.c_float(0.125), 1,
            -1, -1, None)
    assert fwd(lq=None) == NULL
    assert fwd(lq=Layout(3, 0, 0, 512, 128)) == SHAPE      # 3 shards do not divide S=64
    assert fwd(lk=Layout(1, 0, 0, 0, 128)) == SHAPE        # token stride 0
    assert fwd(lk=Layout(1, 0, 0, 256, -128)) == SHAPE     # negative stride
    assert fwd(lq=Layout(2, 0, 4, 512, 128)) == ALIGN      # shard stride not a multiple of 8
    rc = lib.ulysses_attn_bwd_layout(
        _p(A), _p(2 * A), _p(3 * A), _p(4 * A), _p(5 * A), _p(6 * A), None, None, None, _p(7 * A),
        _p(8 * A), _p(9 * A), None, _p(10 * A), ctypes.c_size_t(1 << 30), ctypes.byref(ok_q), None,
        1, 64, 4, 2, 128, ctypes.c_float(0.125), 1, -1, -1, None)
    assert rc == NULL


def test_chunk_and_merge_argument_errors(lib):
    from ulysses_sequence_attention_rank_amd import Layout
    lq, lk = Layout(1, 64 * 4 * 128, 0, 4 * 128, 128), Layout(1, 16 * 2 * 128, 0, 2 * 128, 128)

    def chunk(k_start=0, Sk=16):
        return lib.ulysses_attn_fwd_chunk(
            _p(A), _p(2 * A), _p(3 * A), _p(4 * A), _p(5 * A), None, None, _p(6 * A),
            ctypes.c_size_t(1 << 30), ctypes.byref(lq), ctypes.byref(lk), 1, 64, k_start, Sk, 4, 2,
            128, ctypes.c_float(0.125), 1, -1, -1, None)
    assert chunk(k_start=60, Sk=16) == SHAPE    # past the sequence end
    assert chunk(k_start=-1) == SHAPE
    assert chunk(Sk=0) == SHAPE
    m = lib.ulysses_attn_merge
    assert m(_p(A), _p(2 * A), _p(3 * A), _p(4 * A), 1, 8, 2, 12, None) == UNSUP   # D/4 = 3
    assert m(None, _p(2 * A), _p(3 * A), _p(4 * A), 1, 8, 2, 64, None) == NULL
    f = lib.ulysses_attn_merge_finish
    assert f(_p(A), _p(2 * A), None, _p(3 * A), _p(2 * A), 1, 8, 2, 64, None) == UNSUP  # lse aliases


def test_attn_bwd_argument_errors(lib):
    need = lib.ulysses_attn_bwd_workspace_bytes(1, 64, 4, 2, 128)
    assert need >= 64 * 4 * 4

    def bwd(ws_bytes=need, sink=None, dsink=None, hq=4):
        return lib.ulysses_attn_bwd(
            _p(A), _p(2 * A), _p(3 * A), _p(4 * A), _p(5 * A), _p(6 * A),
            None if sink is None else _p(sink), None, None, _p(7 * A), _p(8 * A), _p(9 * A),
            None if dsink is None else _p(dsink), _p(10 * A), ctypes.c_size_t(ws_bytes),
            1, 64, hq, 2, 128, ctypes.c_float(0.125), 1, -1, -1, None)

    assert bwd(ws_bytes=need - 1) == CAP
    assert bwd(sink=11 * A) == NULL          # sink without dsink
    assert bwd(dsink=11 * A) == NULL
    assert bwd(hq=3) == HEADS


def test_workspace_bytes_grow_with_rows(lib):
    a = lib.ulysses_attn_bwd_workspace_bytes(1, 1024, 8, 1, 64)
    b = lib.ulysses_attn_bwd_workspace_bytes(1, 2048, 8, 1, 64)
    assert b > a > 0
    assert lib.ulysses_attn_bwd_workspace_bytes(0, 1024, 8, 1, 64) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        uly.attn_fwd(q, q, q)


def test_tiled_mlp_argument_errors(lib):
    ws = lib.ulysses_tiled_mlp_workspace_bytes(200, 128, 256, 128)
    assert ws >= 128 * 256 * 2 * 5
    assert lib.ulysses_tiled_mlp_workspace_bytes(0, 128, 256, 128) == 0
    fwd = lambda T, H, I, tile, x=A, y=A, ws_ptr=A, ws_bytes=ws: lib.ulysses_tiled_mlp_fwd(
        _p(x), _p(A), _p(A), _p(A), _p(y), T, H, I, tile, _p(ws_ptr), ws_bytes, None)
    assert fwd(200, 128, 256, 128, x=0) == NULL
    assert fwd(200, 128, 256, 128, y=0) == NULL
    assert fwd(0, 128, 256, 128) == SHAPE
    assert fwd(200, 128, 256, 0) == SHAPE
    assert fwd(200, 96, 256, 128) == UNSUP
    assert fwd(200, 128, 200, 128) == UNSUP
    assert fwd(200, 128, (1 << 20) + 128, 128) == SHAPE
    assert fwd(1, (1 << 20) + 128, 128, 1) == SHAPE
    assert fwd(200, 128, 256, 128, ws_ptr=0) == NULL
    assert fwd(200, 128, 256, 128, ws_bytes=ws - 1) == CAP
    assert fwd(200, 128, 256, 128, x=A + 2) == ALIGN
    bwd = lambda dw=A: lib.ulysses_tiled_mlp_bwd(_p(A), _p(A), _p(A), _p(A), _p(A), _p(A), _p(dw),
                                                 _p(A), _p(A), 200, 128, 256, 128, _p(A), ws, None)
    assert bwd(dw=0) == NULL
    assert bwd(dw=A + 4) == ALIGN


def test_bwd_status_words_sit_inside_the_workspace(lib):
    """The status words' offset is a function of the sizes, 256-byte aligned,
    inside the workspace the same sizes ask for; 0 for rejected sizes."""
    lib.ulysses_attn_bwd_status_offset.restype = ctypes.c_size_t
    lib.ulysses_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    for B, S, hq, hkv, D in ((1, 512, 4, 4, 64), (1, 4096, 6, 6, 128), (2, 1000, 7, 1, 128),
                             (1, 131072, 7, 1, 128)):
        off = lib.ulysses_attn_bwd_status_offset(B, S, hq, hkv, D)
        need = lib.ulysses_attn_bwd_workspace_bytes(B, S, hq, hkv, D)
        assert off > 0 and off % 256 == 0 and off + 24 <= need
    assert lib.ulysses_attn_bwd_status_offset(0, 512, 4, 4, 64) == 0


def test_cu_seqlens_capacity(lib):
    """B*S + 1 plus 4 slots per chunk of at least 512 tokens, at most 1024 chunks."""
    f = lib.ulysses_cu_seqlens_capacity
    assert f(1, 512) == 512 + 1 + 4
    assert f(1, 4096) == 4096 + 1 + 4 * 8
    assert f(1, 131072) == 131072 + 1 + 4 * 256
    assert f(2, 4194304) == 8388608 + 1 + 4 * 1024
    assert f(0, 512) == 0 and f(1, 0) == 0


def test_noalloc_forward_rejects_sizes_beyond_its_scratch(lib):
    """A problem whose split partials exceed the static scratch is refused on the
    host with ULY_ERR_CAPACITY (S=8192, 12 heads, D=128 splits in two: 100 MB)."""
    lib.ulysses_attn_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.ulysses_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    cap = lib.ulysses_attn_fwd_noalloc_max_workspace()
    assert cap == 32 << 20
    assert lib.ulysses_attn_fwd_workspace_bytes(1, 8192, 12, 12, 128) > cap
    rc = lib.ulysses_attn_fwd_noalloc(_p(A), _p(A), _p(A), _p(A), _p(A), None, None, None, 1, 8192,
                                      12, 12, 128, ctypes.c_float(0.088), 1, -1, -1, None)
    assert rc == CAP and b"static scratch" in lib.ulysses_last_error()


def test_calibrate_mfma_argument_errors(lib):
    lib.ulysses_calibrate_mfma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p]
    lib.ulysses_calibrate_mfma_flops.restype = ctypes.c_size_t
    need = 512 * 256 * 4
    f = lambda out=A, nbytes=need, iters=8, mode=0: lib.ulysses_calibrate_mfma(out, nbytes, iters,
                                                                             mode, None)
    assert f(out=None) == NULL
    assert f(nbytes=need - 1) == CAP
    assert f(iters=0) == SHAPE
    assert f(iters=12) == SHAPE
    assert f(mode=6) == UNSUP
    assert f(mode=-1) == UNSUP
    assert f(out=A + 2) == ALIGN
    # 512 work-groups x 4 waves x iters x 8 accumulators x 2*32*32*16 FLOPs
    assert lib.ulysses_calibrate_mfma_flops(8) == 512 * 4 * 8 * 8 * 32768
    assert lib.ulysses_calibrate_mfma_flops(0) == 0
