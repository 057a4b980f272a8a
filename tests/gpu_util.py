"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import sys

import torch

# Attention outputs and gradients vs the fp64 oracle: bf16 I/O, fp32 accumulation.
# Per element |got - want| <= MAX_ABS + |bf16(want) - want|: the stated 2e-2
# beyond the rounding of the exact value to the bf16 output format (that
# rounding alone exceeds 2e-2 for |want| >= 8).  fp32 outputs get MAX_ABS.
# Over each tensor mean |got - want| <= MEAN_ABS.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# LSE has no stated bound; it is held to fp32-accumulation accuracy because
# dsink's sink probabilities exp(sink - LSE) inherit its error.
LSE_MAX = 1e-3
LSE_MEAN = 1e-4


def say(msg: str):
    """Name the case before a GPU step (flushed, so a fault still leaves it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def assert_close_tol(got: torch.Tensor, want: torch.Tensor, name: str, max_abs=MAX_ABS,
                     mean_abs=MEAN_ABS):
    g = got.detach().to("cpu", torch.float64).reshape(-1)
    w = want.detach().to("cpu", torch.float64).reshape(-1)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    assert torch.isfinite(g).all(), f"{name}: non-finite values"
    err = (g - w).abs()
    mx = float(err.max()) if err.numel() else 0.0
    mn = float(err.mean()) if err.numel() else 0.0
    # rounding of the exact value to the output format
    wr = w.to(torch.bfloat16).double() if got.dtype == torch.bfloat16 else w
    u = (wr - w).abs()
    excess = float((err - u).max()) if err.numel() else 0.0
    msg = (f"  {name}: max_abs={mx:.3e} mean_abs={mn:.3e} beyond_rounding={excess:.3e}"
           f" (n={err.numel()})")
    if err.numel():
        i = int((err - u).argmax())
        msg += (f" worst: got={float(g[i]):.5f} want={float(w[i]):.5f};"
                f" vs bf16(oracle): max_abs={float((g - wr).abs().max()):.3e}"
                f" |oracle|max={float(w.abs().max()):.2f}")
    print(msg, flush=True)
    assert excess <= max_abs and mn <= mean_abs, \
        f"{name}: max_abs {mx:.3e} (beyond bf16 rounding {excess:.3e}), mean_abs {mn:.3e}"


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    return a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def gpu_available() -> bool:
    return torch.cuda.is_available()
