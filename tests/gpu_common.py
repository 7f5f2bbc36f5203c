"""Shared helpers for the GPU parity tests (no attention arithmetic here)."""
import sys

import numpy as np
import torch

# parity bars: float32 inputs, and bf16 inputs with float32 accumulation
F32_TOL = dict(o=1e-5, lse=1e-5)
BF16_TOL = dict(o=2e-2, lse=1e-3)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.contiguous().cuda()


def stats(got, ref):
    """max abs, max relative (to max(|ref|, 1e-3)) and RMS error over finite reference entries."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    fin = np.isfinite(r)
    # -inf entries must match exactly (empty rows)
    assert np.array_equal(g[~fin], r[~fin]), "non-finite entries differ"
    if not fin.any():
        return dict(max_abs=0.0, max_rel=0.0, rms=0.0)
    e = np.abs(g[fin] - r[fin])
    return dict(max_abs=float(e.max()), max_rel=float((e / np.maximum(np.abs(r[fin]), 1e-3)).max()),
                rms=float(np.sqrt(np.mean(e * e))))


def check(name, o, lse, o_ref, lse_ref, tol):
    so = stats(o.float().cpu().numpy() if hasattr(o, "cpu") else o, o_ref)
    sl = stats(lse.float().cpu().numpy() if hasattr(lse, "cpu") else lse, lse_ref)
    say("%s: O max_abs=%.3e max_rel=%.3e rms=%.3e | LSE max_abs=%.3e rms=%.3e"
        % (name, so["max_abs"], so["max_rel"], so["rms"], sl["max_abs"], sl["rms"]))
    assert so["max_abs"] <= tol["o"], (name, so)
    assert sl["max_abs"] <= tol["lse"], (name, sl)
    return so, sl
