"""GPU parity of the R2LM right-to-left selective scan against the oracle.

Bound per element: the scan runs L dependent steps in fp32, each adding a
few roundings and one exp2 ulp error to quantities no larger than the same
recurrence run on absolute values, so
    |gpu - exact| <= 16 L 2^-24 y_abs,
    y_abs = the scan of (|u|, delta, A, |B|, |C|, |D|) scaled by |s|
(the decay factors exp(delta A) are positive already).  The bf16 update of
the hidden stream adds its rounding, 2^-8 |x + y|.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import r2l as R

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd  # noqa: F401
    yield


def _bf(bits):
    from denoising_step_amd.runner import bf16_to_device
    return bf16_to_device(bits, torch.device("cuda"))


def run_and_check(c):
    import denoising_step_amd as dlm
    from denoising_step_amd.runner import bf16_to_host
    y = torch.full((c.B, c.L, c.E), float("nan"), device="cuda")
    x = _bf(c.x)
    dlm.dlm_r2l_scan(c.B, c.L, c.E, c.N, c.gate, _bf(c.u), _bf(c.delta), torch.from_numpy(c.A).cuda(),
                     _bf(c.Bm), _bf(c.Cm), torch.from_numpy(c.Dv).cuda(), y=y, x=x)
    torch.cuda.synchronize()
    yg = y.cpu().numpy().astype(np.float64)
    xg = W.bf16_bits_to_f32(bf16_to_host(x)).astype(np.float64)
    yo = R.r2l(c.u, c.delta, c.A, c.Bm, c.Cm, c.Dv, c.gate)
    absb = lambda bits: np.asarray(bits) & np.uint16(0x7fff)
    yabs = R.r2l(absb(c.u), c.delta, c.A, absb(c.Bm), absb(c.Cm), np.abs(c.Dv), abs(c.gate))
    tol = 16 * c.L * 2.0 ** -24 * yabs + 1e-30
    err = np.abs(yg - yo)
    assert np.all(np.isfinite(yg))
    ratio = (err / tol).max()
    assert ratio <= 1.0, f"y: error {err.max():.3e}, ratio to bound {ratio:.2f}"
    xs = W.bf16_bits_to_f32(c.x).astype(np.float64) + yo
    xerr = np.abs(xg - xs)
    assert np.all(xerr <= 2.0 ** -8 * np.abs(xs) + tol), f"x: error {xerr.max():.3e}"
    return ratio


@pytest.mark.parametrize("B,L,E,N", [(2, 37, 104, 16), (1, 64, 296, 8), (3, 9, 72, 8), (1, 50, 40, 32),
                                     (2, 300, 24, 32), (1, 1, 8, 16), (2, 129, 200, 16)])
def test_r2l_matches_oracle(B, L, E, N):
    _say(f"r2l B={B} L={L} E={E} N={N}")
    c = W.make_r2l("r2l_small", B=B, L=L, E=E, N=N, gate=0.8, seed=B * 100 + N)
    _say(f"  worst error / bound = {run_and_check(c):.3f}")


def test_r2l_gate_zero_leaves_stream_unchanged():
    """At initialisation (s = 0) the hidden stream is bit-identical (Bifocal
    page, sec. 2)."""
    import denoising_step_amd as dlm
    from denoising_step_amd.runner import bf16_to_host
    c = W.make_r2l("gate0", B=2, L=40, E=96, N=16, gate=0.0, seed=5)
    x = _bf(c.x)
    y = torch.full((c.B, c.L, c.E), 7.0, device="cuda")
    dlm.dlm_r2l_scan(c.B, c.L, c.E, c.N, 0.0, _bf(c.u), _bf(c.delta), torch.from_numpy(c.A).cuda(),
                     _bf(c.Bm), _bf(c.Cm), torch.from_numpy(c.Dv).cuda(), y=y, x=x)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_host(x), c.x)
    assert np.all(y.cpu().numpy() == 0.0)


def test_r2l_full_size():
    """The Bifocal page's serving shape: batch 8, a 256-token block, width
    2048, 16 states, every element against its bound."""
    c = W.r2l_bifocal()
    _say("r2l full size B=8 L=256 E=2048 N=16")
    _say(f"  worst error / bound = {run_and_check(c):.3f}")
