"""CPU oracle (fp64) for the sequence-tiled MLP of one sequence-parallel rank.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the product package never does.

Reading of the pages (the DeepSpeed pull request that ports Ulysses to HF
models, feature list): ``TiledMLP`` is an autograd function that runs a
layer's MLP over the rank's tokens in tiles along the sequence, to cap the
activation memory, and the weight gradients are added once after the tiles
(the ``ds_grad_is_ready`` flag delays the per-tile addition).  The pages name
the feature only; the MLP form taken here is the gated (SwiGLU) MLP of the
Llama-family models the same pages list as verified:

    y = (silu(x Wg^T) * (x Wu^T)) Wd^T,   silu(g) = g / (1 + e^-g)

with x [T][H], Wg and Wu [I][H], Wd [H][I].  Every step is the plain
definition in fp64 (torch CPU matmuls as the library step), applied tile by
tile in the order the feature describes; the tiles change nothing but the
order in which the weight gradients are summed.

parity pins: tests/test_oracle_mlp.py (tiled equals untiled, finite
differences, a hand-worked scalar case, zero-input and zero-weight cases).
"""
from __future__ import annotations

from typing import Tuple

import torch

__all__ = ["tiled_mlp_fwd", "tiled_mlp_bwd", "weight_grad_entries", "silu", "silu_grad"]


def _f64(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to(torch.float64).cpu()


def silu(g: torch.Tensor) -> torch.Tensor:
    """silu(g) = g * sigmoid(g)."""
    return g * torch.sigmoid(g)


def silu_grad(g: torch.Tensor) -> torch.Tensor:
    """d silu / dg = sigmoid(g) * (1 + g * (1 - sigmoid(g)))."""
    s = torch.sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def _tiles(T: int, tile: int):
    if tile <= 0:
        raise ValueError("tile must be positive")
    for t0 in range(0, T, tile):
        yield t0, min(t0 + tile, T)


def tiled_mlp_fwd(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                  tile: int) -> torch.Tensor:
    """y [T][H] (fp64): each tile of tokens through the gated MLP on its own."""
    x, wg, wu, wd = _f64(x), _f64(w_gate), _f64(w_up), _f64(w_down)
    T = x.shape[0]
    y = torch.empty(T, wd.shape[0], dtype=torch.float64)
    for t0, t1 in _tiles(T, tile):
        xt = x[t0:t1]
        g = xt @ wg.T                 # gate projection
        u = xt @ wu.T                 # up projection
        h = silu(g) * u               # gated activation
        y[t0:t1] = h @ wd.T           # down projection
    return y


def tiled_mlp_bwd(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                  dy: torch.Tensor, tile: int
                  ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """(dx [T][H], dWg [I][H], dWu [I][H], dWd [H][I]), fp64.

    Per tile, the activations are recomputed from x (nothing is kept from the
    forward), dx of the tile is produced, and the tile's weight gradients are
    added to the running sums, which are returned after the last tile.
    """
    x, wg, wu, wd, dy = _f64(x), _f64(w_gate), _f64(w_up), _f64(w_down), _f64(dy)
    T = x.shape[0]
    dx = torch.empty_like(x)
    dwg = torch.zeros_like(wg)
    dwu = torch.zeros_like(wu)
    dwd = torch.zeros_like(wd)
    for t0, t1 in _tiles(T, tile):
        xt, dyt = x[t0:t1], dy[t0:t1]
        g = xt @ wg.T
        u = xt @ wu.T
        h = silu(g) * u
        dh = dyt @ wd                 # dL/dh
        dg = dh * u * silu_grad(g)    # through the gate
        du = dh * silu(g)             # through the up projection
        dx[t0:t1] = dg @ wg + du @ wu
        dwg += dg.T @ xt
        dwu += du.T @ xt
        dwd += dyt.T @ h
    return dx, dwg, dwu, dwd


def weight_grad_entries(x, w_gate, w_up, w_down, dy, gate_up_idx, down_idx):
    """Selected weight-gradient entries, each the plain sum over all tokens.

    gate_up_idx: (i, h) pairs -> (dWg[i][h], dWu[i][h]) with dWg[i][h] =
    sum_t dG[t][i] x[t][h], dG[t][i] = (dy[t] . Wd[:, i]) U[t][i] silu'(G[t][i]),
    and dWu likewise with dU = (dy[t] . Wd[:, i]) silu(G[t][i]).
    down_idx: (h, i) pairs -> dWd[h][i] = sum_t dy[t][h] silu(G[t][i]) U[t][i].
    Only the columns i involved are formed (one matvec over the tokens each).
    """
    x, wg, wu, wd, dy = _f64(x), _f64(w_gate), _f64(w_up), _f64(w_down), _f64(dy)
    cols = {}

    def col(i):
        if i not in cols:
            g = x @ wg[i]
            u = x @ wu[i]
            dh = dy @ wd[:, i]
            cols[i] = (g, u, dh)
        return cols[i]

    gate, up, down = [], [], []
    for i, h in gate_up_idx:
        g, u, dh = col(i)
        gate.append(float((dh * u * silu_grad(g)) @ x[:, h]))
        up.append(float((dh * silu(g)) @ x[:, h]))
    for h, i in down_idx:
        g, u, _ = col(i)
        down.append(float((silu(g) * u) @ dy[:, h]))
    return gate, up, down
