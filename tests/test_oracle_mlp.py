"""Pins of the oracle's sequence-tiled gated MLP (CPU only).

The feature is the ``TiledMLP`` / ``SequenceTiledCompute`` entry of the
DeepSpeed pull request that ports Ulysses to HF models (feature list): the
MLP of a rank's tokens computed tile by tile along the sequence, its weight
gradients added once after the tiles.  Each pin below checks the oracle
against something other than itself: the hand-worked scalar case, central
finite differences of its own forward, the untiled computation, and cases
whose result is zero by construction.
"""
import math

import pytest
import torch

from oracle import mlp as om
from ulysses_inputs import make_mlp_inputs


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_scalar_case_by_hand():
    """H = I = T = 1: y = wd * silu(wg x) * (wu x), gradients by the chain rule."""
    x, wg, wu, wd, dy = 0.75, -1.25, 0.5, 2.0, -0.375
    g, u = wg * x, wu * x
    s = _sig(g)
    silu, dsilu = g * s, s * (1.0 + g * (1.0 - s))
    y = wd * silu * u
    dh = dy * wd
    dx = dh * (dsilu * wg * u + silu * wu)
    dwg = dh * dsilu * u * x
    dwu = dh * silu * x
    dwd = dy * silu * u
    t = lambda v: torch.tensor([[v]], dtype=torch.float64)
    got_y = om.tiled_mlp_fwd(t(x), t(wg), t(wu), t(wd), tile=1)
    got = om.tiled_mlp_bwd(t(x), t(wg), t(wu), t(wd), t(dy), tile=1)
    assert got_y.item() == pytest.approx(y, rel=1e-15, abs=1e-15)
    for a, b in zip(got, (dx, dwg, dwu, dwd)):
        assert a.item() == pytest.approx(b, rel=1e-14, abs=1e-15)


def test_silu_values():
    g = torch.tensor([0.0, 1.0, -1.0, 30.0, -30.0], dtype=torch.float64)
    expect = [0.0, _sig(1.0), -_sig(-1.0), 30.0 * _sig(30.0), -30.0 * _sig(-30.0)]
    assert torch.allclose(om.silu(g), torch.tensor(expect, dtype=torch.float64), rtol=1e-14, atol=1e-300)
    # derivative by central differences
    h = 1e-6
    for v in (-3.0, -0.5, 0.0, 0.7, 4.0):
        f64 = lambda z: torch.tensor(z, dtype=torch.float64)
        num = (float(om.silu(f64(v + h))) - float(om.silu(f64(v - h)))) / (2 * h)
        assert float(om.silu_grad(torch.tensor(v, dtype=torch.float64))) == pytest.approx(num, rel=1e-8)


@pytest.mark.parametrize("T,H,I,tile", [(3, 2, 3, 2), (4, 3, 2, 1), (5, 2, 4, 3)])
def test_backward_is_the_derivative(T, H, I, tile):
    """Central finite differences of L = sum(y * dy) match every gradient."""
    m = make_mlp_inputs(T * 100 + H * 10 + I, T, H, I)
    x, wg, wu, wd, dy = (t.double() for t in (m.x, m.w_gate, m.w_up, m.w_down, m.dy))
    grads = om.tiled_mlp_bwd(x, wg, wu, wd, dy, tile)

    def loss(x_, wg_, wu_, wd_):
        return float((om.tiled_mlp_fwd(x_, wg_, wu_, wd_, tile) * dy).sum())

    eps = 1e-6
    params = [x, wg, wu, wd]
    for pi, grad in enumerate(grads):
        num = torch.zeros_like(params[pi])
        for idx in range(params[pi].numel()):
            plus = [p.clone() for p in params]
            minus = [p.clone() for p in params]
            plus[pi].view(-1)[idx] += eps
            minus[pi].view(-1)[idx] -= eps
            num.view(-1)[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert torch.allclose(grad, num, rtol=1e-6, atol=1e-8), (pi, (grad - num).abs().max())


@pytest.mark.parametrize("tile", [1, 3, 7, 10, 64])
def test_tiles_change_nothing(tile):
    """Any tile size (ragged last tile included) gives the untiled result."""
    T, H, I = 10, 6, 9
    m = make_mlp_inputs(7, T, H, I)
    ref_y = om.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile=T)
    ref = om.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile=T)
    y = om.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, m.w_down, tile=tile)
    got = om.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile=tile)
    assert torch.allclose(y, ref_y, rtol=1e-13, atol=1e-13)
    for a, b in zip(got, ref):
        assert torch.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_untiled_matches_direct_formula():
    """The one-tile oracle against the formula written out with einsum over all tokens."""
    T, H, I = 12, 5, 7
    m = make_mlp_inputs(11, T, H, I)
    x, wg, wu, wd, dy = (t.double() for t in (m.x, m.w_gate, m.w_up, m.w_down, m.dy))
    g = torch.einsum("th,ih->ti", x, wg)
    u = torch.einsum("th,ih->ti", x, wu)
    sg = 1.0 / (1.0 + torch.exp(-g))
    h = g * sg * u
    y = torch.einsum("ti,hi->th", h, wd)
    assert torch.allclose(om.tiled_mlp_fwd(x, wg, wu, wd, tile=4), y, rtol=1e-13, atol=1e-13)


def test_zero_input_and_zero_down_weight():
    T, H, I = 6, 4, 5
    m = make_mlp_inputs(3, T, H, I)
    zx = torch.zeros_like(m.x)
    y = om.tiled_mlp_fwd(zx, m.w_gate, m.w_up, m.w_down, tile=4)
    dx, dwg, dwu, dwd = om.tiled_mlp_bwd(zx, m.w_gate, m.w_up, m.w_down, m.dy, tile=4)
    assert torch.count_nonzero(y) == 0 and torch.count_nonzero(dwg) == 0
    assert torch.count_nonzero(dwu) == 0 and torch.count_nonzero(dwd) == 0 and torch.count_nonzero(dx) == 0
    zwd = torch.zeros_like(m.w_down)
    y = om.tiled_mlp_fwd(m.x, m.w_gate, m.w_up, zwd, tile=4)
    dx, dwg, dwu, dwd = om.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, zwd, m.dy, tile=4)
    assert torch.count_nonzero(y) == 0 and torch.count_nonzero(dx) == 0
    assert torch.count_nonzero(dwg) == 0 and torch.count_nonzero(dwu) == 0
    assert torch.count_nonzero(dwd) > 0   # dWd = dy^T h does not depend on Wd


def test_weight_grad_entries_match_the_full_backward():
    """The one-entry-at-a-time sums (used at full size) equal the tiled backward's entries."""
    T, H, I = 9, 5, 7
    m = make_mlp_inputs(5, T, H, I)
    _, dwg, dwu, dwd = om.tiled_mlp_bwd(m.x, m.w_gate, m.w_up, m.w_down, m.dy, tile=4)
    gu = [(0, 0), (6, 4), (3, 2)]
    dn = [(0, 0), (4, 6), (2, 3)]
    g, u, d = om.weight_grad_entries(m.x, m.w_gate, m.w_up, m.w_down, m.dy, gu, dn)
    for (i, h), a, b in zip(gu, g, u):
        assert a == pytest.approx(float(dwg[i, h]), rel=1e-12, abs=1e-13)
        assert b == pytest.approx(float(dwu[i, h]), rel=1e-12, abs=1e-13)
    for (h, i), c in zip(dn, d):
        assert c == pytest.approx(float(dwd[h, i]), rel=1e-12, abs=1e-13)
