"""CPU oracle of the R2LM right-to-left selective scan (fp64 numpy; test
infrastructure only, like the rest of ``oracle``).

"Bifocal Diffusion Language Models" page, sec. 2: the right-to-left stream
takes hidden states from the backbone, flips the sequence, applies a
selective scan (Mamba) and flips it back; its output is a residual
correction gated by a learnable scalar s that starts at 0, so the model at
initialisation equals the causal baseline.  During denoising the scan runs
over the generation block only.

Selective scan (the Mamba recurrence, in the order the tokens are scanned),
per batch entry, channel e and state n, from a zero state:

    h_t[e, n] = exp(delta_t[e] * A[e, n]) * h_{t-1}[e, n]
                + delta_t[e] * B_t[n] * u_t[e]
    y_t[e]    = sum_n C_t[n] * h_t[e, n] + D[e] * u_t[e]

``r2l`` flips the token axis, scans, flips back and scales by s.  Inputs are
the bf16 bit patterns (u, delta, B, C) and fp32 values (A, D) the GPU gets,
widened exactly; the arithmetic is float64.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def selective_scan(u, delta, A, Bm, Cm, Dv):
    """Forward scan.  u, delta [B, L, E]; A [E, N]; Bm, Cm [B, L, N];
    Dv [E].  Returns y [B, L, E] (float64)."""
    u, delta, A, Bm, Cm, Dv = map(_f64, (u, delta, A, Bm, Cm, Dv))
    Bsz, L, E = u.shape
    h = np.zeros((Bsz, E, A.shape[1]))
    y = np.empty((Bsz, L, E))
    for t in range(L):
        dA = np.exp(delta[:, t, :, None] * A[None])
        h = dA * h + delta[:, t, :, None] * Bm[:, t, None, :] * u[:, t, :, None]
        y[:, t] = (h * Cm[:, t, None, :]).sum(-1) + Dv[None] * u[:, t]
    return y


def r2l(u, delta, A, Bm, Cm, Dv, s):
    """The gated right-to-left correction s * flip(scan(flip(inputs)))."""
    f = lambda a: np.asarray(a)[:, ::-1]
    return float(s) * selective_scan(f(u), f(delta), A, f(Bm), f(Cm), Dv)[:, ::-1]
