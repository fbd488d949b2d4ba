"""Pins of the oracle's active-row projections and feed-forward.

* Closed forms: identity weights return the gathered rows themselves, zero
  weights leave only the residual, a one-unit feed-forward is worked by hand,
  and silu takes its known values.
* A second library (torch's CPU linear and silu in float64) agrees.
* The gathered computation equals the dense one over every position,
  restricted to the active rows.
* Planted mistakes in a private copy of the oracle are caught.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import layer as L


def _bits(a):
    return W.to_bf16_bits(np.asarray(a, np.float32))


def _case(**kw):
    base = dict(B=2, n_pos=40, d=128, Hq=2, Hkv=1, D=64, F=64, M=13, seed=1)
    base.update(kw)
    return W.make_layer("pin", **base)


def check_identity_qkv(mod):
    c = _case()
    n = (c.Hq + 2 * c.Hkv) * c.D
    w = np.zeros((n, c.d), np.float32)
    w[np.arange(n), np.arange(n) % c.d] = 1.0
    res = mod.proj_qkv(c.x, c.active_idx, c.m, _bits(w), c.Hq, c.Hkv, c.D)
    x = W.bf16_bits_to_f32(c.x).astype(np.float64)
    for b in range(c.B):
        xr = x[b, c.active_idx[b, :c.m[b]]]                       # [m, d]
        cols = np.arange(n) % c.d
        want = xr[:, cols]
        q, k, v = res[b]
        assert np.array_equal(q, want[:, :c.Hq * c.D].reshape(-1, c.Hq, c.D).transpose(1, 0, 2))
        assert np.array_equal(k, want[:, c.Hq * c.D:(c.Hq + c.Hkv) * c.D].reshape(-1, c.Hkv, c.D)
                              .transpose(1, 0, 2))
        assert np.array_equal(v, want[:, (c.Hq + c.Hkv) * c.D:].reshape(-1, c.Hkv, c.D).transpose(1, 0, 2))


def check_out_closed_forms(mod):
    c = _case()
    x = W.bf16_bits_to_f32(c.x).astype(np.float64)
    zero = mod.proj_out(c.x, c.active_idx, c.m, c.attn_out, _bits(np.zeros((c.d, c.Hq * c.D))))
    for b in range(c.B):
        assert np.array_equal(zero[b], x[b, c.active_idx[b, :c.m[b]]])
    # W_o picks input column (head 1, dim 3) into output column 5
    w = np.zeros((c.d, c.Hq * c.D), np.float32)
    w[5, 1 * c.D + 3] = 1.0
    one = mod.proj_out(c.x, c.active_idx, c.m, c.attn_out, _bits(w))
    ao = W.bf16_bits_to_f32(c.attn_out).astype(np.float64)
    for b in range(c.B):
        want = x[b, c.active_idx[b, :c.m[b]]].copy()
        want[:, 5] += ao[b, 1, :c.m[b], 3]
        assert np.array_equal(one[b], want)


def check_ffn_closed_forms(mod):
    # one unit: y = h + silu(h * g) * (h * u) * w, worked by hand
    h = _bits([[[2.0]]])
    got = mod.ffn(h, np.array([1]), _bits([[1.0]]), _bits([[0.25]]), _bits([[-3.0]]))[0][0, 0]
    want = 2.0 + (2.0 / (1.0 + math.exp(-2.0))) * 0.5 * -3.0
    assert abs(got - want) < 1e-15
    c = _case()
    zero = mod.ffn(c.h, c.m, c.w_gate, c.w_up, _bits(np.zeros((c.d, c.F))))
    hh = W.bf16_bits_to_f32(c.h).astype(np.float64)
    for b in range(c.B):
        assert np.array_equal(zero[b], hh[b, :c.m[b]])


def test_identity_qkv():
    check_identity_qkv(L)


def test_out_closed_forms():
    check_out_closed_forms(L)


def test_ffn_closed_forms():
    check_ffn_closed_forms(L)


def test_silu_values():
    assert L.silu(0.0) == 0.0
    assert abs(L.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(L.silu(40.0) - 40.0) < 1e-15 and abs(L.silu(-40.0)) < 1e-15


def test_against_torch_linear():
    import torch
    import torch.nn.functional as Fn
    c = _case(B=2, n_pos=50, d=192, Hq=4, Hkv=2, D=64, F=128, M=20, m=[20, 7])
    t = lambda a: torch.from_numpy(W.bf16_bits_to_f32(a).astype(np.float64))
    x, wqkv, wo, wg, wu, wd = map(t, (c.x, c.w_qkv, c.w_o, c.w_gate, c.w_up, c.w_down))
    ao, h = t(c.attn_out), t(c.h)
    qkv = L.proj_qkv(c.x, c.active_idx, c.m, c.w_qkv, c.Hq, c.Hkv, c.D)
    hout = L.proj_out(c.x, c.active_idx, c.m, c.attn_out, c.w_o)
    y = L.ffn(c.h, c.m, c.w_gate, c.w_up, c.w_down)
    for b in range(c.B):
        m = int(c.m[b])
        xr = x[b, torch.from_numpy(c.active_idx[b, :m].astype(np.int64))]
        ref = Fn.linear(xr, wqkv)
        q = ref[:, :c.Hq * c.D].reshape(m, c.Hq, c.D).permute(1, 0, 2)
        assert np.allclose(qkv[b][0], q.numpy(), rtol=1e-12, atol=1e-12)
        v = ref[:, (c.Hq + c.Hkv) * c.D:].reshape(m, c.Hkv, c.D).permute(1, 0, 2)
        assert np.allclose(qkv[b][2], v.numpy(), rtol=1e-12, atol=1e-12)
        cat = torch.cat([ao[b, hd, :m] for hd in range(c.Hq)], dim=1)
        assert np.allclose(hout[b], (xr + Fn.linear(cat, wo)).numpy(), rtol=1e-12, atol=1e-12)
        hr = h[b, :m]
        ff = hr + Fn.linear(Fn.silu(Fn.linear(hr, wg)) * Fn.linear(hr, wu), wd)
        assert np.allclose(y[b], ff.numpy(), rtol=1e-12, atol=1e-12)


def test_gathered_equals_dense_rows():
    c = _case(n_pos=30, M=11, m=[11, 4])
    allpos = np.tile(np.arange(c.n_pos, dtype=np.int32), (c.B, 1))
    full = L.proj_qkv(c.x, allpos, np.full(c.B, c.n_pos), c.w_qkv, c.Hq, c.Hkv, c.D)
    part = L.proj_qkv(c.x, c.active_idx, c.m, c.w_qkv, c.Hq, c.Hkv, c.D)
    for b in range(c.B):
        sel = c.active_idx[b, :c.m[b]]
        for i in range(3):
            assert np.array_equal(part[b][i], full[b][i][:, sel])


SRC = os.path.join(os.path.dirname(L.__file__), "layer.py")
MUTANTS = [
    ("silu_is_sigmoid", "return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    ("residual_dropped", "res.append(xr + a @ w.T)", "res.append(a @ w.T)"),
    ("gather_by_index", "return [x[b, act[b, :m[b]]] for b", "return [x[b, :m[b]] for b"),
    ("k_v_swapped", "k = y[:, Hq * D:(Hq + Hkv) * D]", "k = y[:, (Hq + Hkv) * D:]"),
    ("heads_not_concatenated", "a = ao[b, :, :m[b], :].transpose(1, 0, 2).reshape(",
     "a = ao[b, :, :m[b], :].reshape("),
    ("down_residual_dropped", "return [h[b, :m[b]] + g[b] @ wd.T", "return [g[b] @ wd.T"),
    ("up_ignored", "silu(h[b, :m[b]] @ wg.T) * (h[b, :m[b]] @ wu.T)", "silu(h[b, :m[b]] @ wg.T)"),
]


@pytest.mark.parametrize("name,old,new", [m[:3] for m in MUTANTS], ids=[m[0] for m in MUTANTS])
def test_pins_catch_layer_mutant(name, old, new, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"layer_mutant_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"layer_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = 0
    for check in (check_identity_qkv, check_out_closed_forms, check_ffn_closed_forms):
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
