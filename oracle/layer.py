"""CPU oracle of a layer's active-row projections and feed-forward (fp64
numpy; test infrastructure only, like the rest of ``oracle``).

SureLock page, sec. 2: a locked position skips its query projection and its
feed-forward sub-layer; the active rows are computed, so the dense work of a
step is O(M_t d^2).  For the rows j < m[b] of batch entry b at positions
act[b, j] of the hidden states x:

    q | k | v = x[b, act] W_qkv^T                       (heads split after)
    h         = x[b, act] + attn_out W_o^T              (attn_out head-major)
    x[b, act] = h + (silu(h W_gate^T) * (h W_up^T)) W_down^T

with silu(z) = z * sigmoid(z) and weights [out_features, in_features].  The
layer's normalisations are not part of these functions.  Inputs are the bf16
bit patterns the GPU gets, widened exactly; every product is a numpy matmul
in float64 with no intermediate rounding.  ``gated`` returns the gated
hidden rows that the down projection multiplies.
"""
from __future__ import annotations

import numpy as np


def _f64(bits):
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def rows(x_bits, act, m):
    """The active rows of batch entry b: x[b, act[b, :m[b]]] (fp64)."""
    x = _f64(x_bits)
    return [x[b, act[b, :m[b]]] for b in range(x.shape[0])]


def proj_qkv(x_bits, act, m, w_qkv_bits, Hq, Hkv, D):
    """Per batch entry: (q [Hq, m, D], k [Hkv, m, D], v [Hkv, m, D])."""
    w = _f64(w_qkv_bits)
    out = []
    for xr in rows(x_bits, act, m):
        y = xr @ w.T                                   # [m, (Hq + 2 Hkv) D]
        q = y[:, :Hq * D].reshape(-1, Hq, D).transpose(1, 0, 2)
        k = y[:, Hq * D:(Hq + Hkv) * D].reshape(-1, Hkv, D).transpose(1, 0, 2)
        v = y[:, (Hq + Hkv) * D:].reshape(-1, Hkv, D).transpose(1, 0, 2)
        out.append((q, k, v))
    return out


def proj_out(x_bits, act, m, attn_out_bits, w_o_bits):
    """Per batch entry: h [m, d] = x rows + attn_out (heads concatenated) W_o^T."""
    w = _f64(w_o_bits)
    ao = _f64(attn_out_bits)                           # [B, Hq, M, D]
    res = []
    for b, xr in enumerate(rows(x_bits, act, m)):
        a = ao[b, :, :m[b], :].transpose(1, 0, 2).reshape(m[b], ao.shape[1] * ao.shape[3])   # [m, Hq D]
        res.append(xr + a @ w.T)
    return res


def gated(h_bits, m, w_gate_bits, w_up_bits):
    """Per batch entry: silu(h W_gate^T) * (h W_up^T), [m, F]."""
    h = _f64(h_bits)
    wg, wu = _f64(w_gate_bits), _f64(w_up_bits)
    return [silu(h[b, :m[b]] @ wg.T) * (h[b, :m[b]] @ wu.T) for b in range(h.shape[0])]


def ffn(h_bits, m, w_gate_bits, w_up_bits, w_down_bits):
    """Per batch entry: h + gated(h) W_down^T, [m, d]."""
    h = _f64(h_bits)
    wd = _f64(w_down_bits)
    g = gated(h_bits, m, w_gate_bits, w_up_bits)
    return [h[b, :m[b]] + g[b] @ wd.T for b in range(h.shape[0])]
