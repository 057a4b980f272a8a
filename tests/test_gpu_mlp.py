"""GPU parity of the sequence-tiled gated MLP (HIP GEMM kernels) against the
fp64 oracle, through the C ABI.

Tolerance (derived from the arithmetic): x, the weights and dy are bf16 on
both sides; the GPU accumulates in fp32 and rounds at most three times on the
way to a result (the gated activation or the gated derivatives, the recomputed
projections, the output), each a relative 2^-9 (rms 1.1e-3).  Each tensor is
held to mean |err| <= 4e-3 rms(want), rms over the tensor (or, for sampled
entries, over the sample), and max |err| <= 6e-2 rms(want): the products
summed into an entry are heavy-tailed, so an entry's error follows its largest
terms, which reach several times the tensor's rms (measured up to 3.5e-2 rms
for dW_down over 64 tokens).  A wrong index or a dropped term errs by O(rms).
"""
import pytest
import torch

import oracle.mlp as om
import ulysses_sequence_attention_rank_amd as uly
from ulysses_inputs import make_mlp_inputs

from gpu_util import say

pytestmark = pytest.mark.gpu

MEAN_REL = 4e-3
MAX_REL = 6e-2


def _close(got, want, name):
    g = got.detach().to("cpu", torch.float64).reshape(-1)
    w = want.detach().to("cpu", torch.float64).reshape(-1)
    assert g.shape == w.shape, name
    assert torch.isfinite(g).all(), f"{name}: non-finite values"
    rms = float(w.pow(2).mean().sqrt())
    err = (g - w).abs()
    mx, mn = float(err.max()), float(err.mean())
    print(f"  {name}: rms={rms:.3e} max_abs={mx:.3e} ({mx / rms:.2e} rms) mean_abs={mn:.3e} "
          f"({mn / rms:.2e} rms)")
    assert mn <= MEAN_REL * rms, f"{name}: mean |err| {mn:.3e} > {MEAN_REL} rms {rms:.3e}"
    assert mx <= MAX_REL * rms, f"{name}: max |err| {mx:.3e} > {MAX_REL} rms {rms:.3e}"


CASES = [
    # (T, H, I, tile): ragged token tiles, tiles not a multiple of 64, one tile
    (200, 128, 256, 128),
    (300, 256, 384, 100),
    (64, 128, 128, 64),
    (129, 256, 128, 1000),
    (1, 128, 128, 1),
    # m tiles dealt to the XCDs in ranges (eight tiles of 256 tokens), and
    # operand widths of an odd number of 128-column halves
    (2048, 256, 1024, 2048),
    (1000, 384, 640, 512),
]


@pytest.mark.parametrize("T,H,I,tile", CASES)
def test_tiled_mlp_matches_oracle(T, H, I, tile):
    say(f"tiled_mlp T={T} H={H} I={I} tile={tile}")
    m = make_mlp_inputs(T + H + I, T, H, I, device="cuda")
    y = uly.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile)
    dx, dwg, dwu, dwd = uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile)
    torch.cuda.synchronize()
    cpu = [t.cpu() for t in (m.x, m.w_gate, m.w_up, m.w_down, m.dy)]
    want_y = om.tiled_mlp_fwd(*cpu[:4], tile=tile)
    want = om.tiled_mlp_bwd(*cpu, tile=tile)
    _close(y, want_y, "y")
    for got, w, name in zip((dx, dwg, dwu, dwd), want, ("dx", "dw_gate", "dw_up", "dw_down")):
        _close(got, w, name)


def test_tiles_do_not_change_rows():
    """A token's y and dx rows do not depend on the tiling (bitwise); the
    weight gradients, summed over tiles in another order, agree to fp32."""
    T, H, I = 300, 128, 256
    say(f"tiled_mlp tiling invariance T={T}")
    m = make_mlp_inputs(42, T, H, I, device="cuda")
    outs = []
    for tile in (300, 128, 70):
        y = uly.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile)
        outs.append((y,) + uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile))
    torch.cuda.synchronize()
    for other in outs[1:]:
        assert torch.equal(outs[0][0], other[0]) and torch.equal(outs[0][1], other[1])
        for a, b in zip(outs[0][2:], other[2:]):
            assert torch.allclose(a, b, rtol=1e-5, atol=1e-4)


def test_tiled_mlp_deterministic():
    T, H, I = 257, 128, 256
    say("tiled_mlp determinism")
    m = make_mlp_inputs(9, T, H, I, device="cuda")
    a = uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, 100)
    b = uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, 100)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_tiled_mlp_full_size_sampled():
    """The timed size (a Llama-3.2-1B-sized MLP over 32768 tokens in tiles of
    8192): sampled rows of y and dx, and sampled weight-gradient entries (each
    a sum over all tokens), against the oracle."""
    T, H, I, tile = 32768, 2048, 8192, 8192
    say(f"tiled_mlp full size T={T} H={H} I={I} tile={tile}")
    m = make_mlp_inputs(2026, T, H, I, device="cuda")
    y = uly.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile)
    dx, dwg, dwu, dwd = uly.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile)
    torch.cuda.synchronize()
    cpu = [t.cpu() for t in (m.x, m.w_gate, m.w_up, m.w_down, m.dy)]
    g = torch.Generator().manual_seed(5)
    rows = torch.cat([torch.tensor([0, tile - 1, tile, T - 1]), torch.randint(0, T, (12,), generator=g)])
    want_y = om.tiled_mlp_fwd(cpu[0][rows], *cpu[1:4], tile=len(rows))
    want_dx = om.tiled_mlp_bwd(cpu[0][rows], *cpu[1:4], cpu[4][rows], tile=len(rows))[0]
    _close(y.cpu()[rows], want_y, "y rows")
    _close(dx.cpu()[rows], want_dx, "dx rows")
    gi = torch.randint(0, I, (24,), generator=g).tolist()
    gh = torch.randint(0, H, (24,), generator=g).tolist()
    gu = list(zip(gi, gh))
    dn = list(zip(gh, gi))
    wg_e, wu_e, wd_e = om.weight_grad_entries(*cpu, gu, dn)
    dwg_c, dwu_c, dwd_c = dwg.cpu(), dwu.cpu(), dwd.cpu()
    _close(torch.tensor([float(dwg_c[i, h]) for i, h in gu]), torch.tensor(wg_e), "dw_gate entries")
    _close(torch.tensor([float(dwu_c[i, h]) for i, h in gu]), torch.tensor(wu_e), "dw_up entries")
    _close(torch.tensor([float(dwd_c[h, i]) for h, i in dn]), torch.tensor(wd_e), "dw_down entries")
