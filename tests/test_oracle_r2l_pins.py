"""Pins of the oracle's R2LM right-to-left selective scan.

* The gate at 0 gives exactly zero (Bifocal page, sec. 2: at initialisation
  the augmented model equals the causal baseline bit for bit).
* Closed forms: with a decay of -inf the scan has no memory; with no decay
  the state is a reverse cumulative sum (numpy cumsum).
* Brute force: the anti-causal matrix form
      y_t = sum_{s >= t} C_t . (exp(A sum_{r=t}^{s-1} delta_r) * delta_s B_s) u_s + D u_t
  computed pair by pair.
* Direction: an impulse at position p reaches only positions t <= p.
* Planted mistakes in a private copy of the oracle are caught.
"""
import importlib.util
import os

import numpy as np
import pytest

import workloads as W
from oracle import r2l as R


def _case(**kw):
    base = dict(B=2, L=12, E=5, N=4, gate=0.7, seed=3)
    base.update(kw)
    return W.make_r2l("pin", **base)


def _f(x):
    return R._f64(x)


def brute(c):
    u, dl, A, Bm, Cm, Dv = map(_f, (c.u, c.delta, c.A, c.Bm, c.Cm, c.Dv))
    y = np.zeros((c.B, c.L, c.E))
    for b in range(c.B):
        for t in range(c.L):
            for s in range(t, c.L):
                decay = np.exp(A * dl[b, t:s, :].sum(0)[:, None])             # [E, N]
                y[b, t] += (decay * (dl[b, s, :, None] * Bm[b, s][None, :]) * Cm[b, t][None, :]).sum(1) * u[b, s]
            y[b, t] += Dv * u[b, t]
    return c.gate * y


def check_gate_zero(mod):
    c = _case()
    assert np.array_equal(mod.r2l(c.u, c.delta, c.A, c.Bm, c.Cm, c.Dv, 0.0), np.zeros((c.B, c.L, c.E)))


def check_memoryless(mod):
    c = _case()
    A = np.full_like(c.A, -1e30)
    got = mod.r2l(c.u, c.delta, A, c.Bm, c.Cm, c.Dv, 1.0)
    u, dl, Bm, Cm, Dv = map(_f, (c.u, c.delta, c.Bm, c.Cm, c.Dv))
    want = dl * (Cm * Bm).sum(-1)[..., None] * u + Dv * u
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def check_no_decay(mod):
    c = _case()
    got = mod.r2l(c.u, c.delta, np.zeros_like(c.A), c.Bm, c.Cm, c.Dv, 1.0)
    u, dl, Bm, Cm, Dv = map(_f, (c.u, c.delta, c.Bm, c.Cm, c.Dv))
    term = (dl * u)[..., None] * Bm[:, :, None, :]                  # [B, L, E, N]
    h = np.cumsum(term[:, ::-1], axis=1)[:, ::-1]                     # sum over s >= t
    want = (h * Cm[:, :, None, :]).sum(-1) + Dv * u
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def check_brute(mod):
    c = _case()
    got = mod.r2l(c.u, c.delta, c.A, c.Bm, c.Cm, c.Dv, c.gate)
    assert np.allclose(got, brute(c), rtol=1e-12, atol=1e-12)


def check_direction(mod):
    c = _case(B=1, L=10)
    u = np.zeros((1, c.L, c.E), np.uint16)
    p = 6
    u[0, p] = W.to_bf16_bits(np.ones(c.E, np.float32))
    y = mod.r2l(u, c.delta, c.A, c.Bm, c.Cm, c.Dv, 1.0)
    assert np.all(y[0, p + 1:] == 0) and np.all(np.abs(y[0, :p + 1]).sum(-1) > 0)


CHECKS = (check_gate_zero, check_memoryless, check_no_decay, check_brute, check_direction)


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_r2l_pin(check):
    check(R)


SRC = os.path.join(os.path.dirname(R.__file__), "r2l.py")
MUTANTS = [
    ("output_not_flipped_back", "Cm), Dv)[:, ::-1]", "Cm), Dv)"),
    ("decay_sign", "dA = np.exp(delta[:, t, :, None] * A[None])", "dA = np.exp(-delta[:, t, :, None] * A[None])"),
    ("input_without_step", "+ delta[:, t, :, None] * Bm[:, t, None, :] * u[:, t, :, None]",
     "+ Bm[:, t, None, :] * u[:, t, :, None]"),
    ("skip_term_dropped", "(h * Cm[:, t, None, :]).sum(-1) + Dv[None] * u[:, t]", "(h * Cm[:, t, None, :]).sum(-1)"),
    ("output_reads_B", "(h * Cm[:, t, None, :])", "(h * Bm[:, t, None, :])"),
    ("gate_ignored", "return float(s) * selective_scan", "return selective_scan"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_r2l_mutant(name, old, new, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"r2l_mutant_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"r2l_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = 0
    for check in CHECKS:
        try:
            check(mod)
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
