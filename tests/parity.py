"""Comparison of GPU results with the oracle's, to the stated tolerances.

Floating point (fp64 oracle vs fp32/bf16 GPU):
  out     bf16, max-abs error <= 2e-2
  lse     abs <= 1e-3 (both -inf allowed)
  colsum  |g - o| <= 1e-3 |o| + 1e-6
  kl      abs <= 1e-4
  conf    abs <= 1e-5
Integer decisions must match exactly, except where the oracle's deciding
quantities tie within 1e-4 (times max(1, |value|), relative for column
sums); every excused disagreement is counted and returned.
"""
from __future__ import annotations

import numpy as np

import workloads as W

OUT_TOL = 2e-2
LSE_TOL = 1e-3
CS_REL, CS_ABS = 1e-3, 1e-6
KL_TOL = 1e-4
CONF_TOL = 1e-5
MARGIN_TOL = 1e-5       # like conf: a difference of two fp32 probabilities
ENTROPY_TOL = 1e-4      # like KL: ln sx - ex / sx from fp32 sums over the vocabulary
TIE = 1e-4


def check_attention(out_g_bits, lse_g, out_o, lse_o):
    out_g = W.bf16_bits_to_f32(out_g_bits).astype(np.float64)
    err = np.abs(out_g - out_o)
    assert np.all(np.isfinite(out_g)), "non-finite GPU output"
    assert err.max() <= OUT_TOL, f"out max-abs {err.max():.3e} > {OUT_TOL}"
    lse_g = lse_g.astype(np.float64)
    inf_o, inf_g = np.isneginf(lse_o), np.isneginf(lse_g)
    assert np.array_equal(inf_o, inf_g), "rows without visible keys differ"
    if (~inf_o).any():
        le = np.abs(lse_g[~inf_o] - lse_o[~inf_o]).max()
        assert le <= LSE_TOL, f"lse abs {le:.3e} > {LSE_TOL}"
    return float(err.max())


def check_colsum(cs_g, cs_o):
    cs_g = cs_g.astype(np.float64)
    err = np.abs(cs_g - cs_o)
    bound = CS_REL * np.abs(cs_o) + CS_ABS
    bad = err > bound
    assert not bad.any(), (f"colsum: {bad.sum()} elements out of tolerance, worst rel "
                           f"{(err / np.maximum(np.abs(cs_o), 1e-30)).max():.3e}")
    return float((err / np.maximum(np.abs(cs_o), CS_ABS)).max())


def check_posterior(kl_g, conf_g, lock_g, kl_o, conf_o, lock_o, eps, locked_in):
    """Returns the number of excused lock disagreements."""
    e = np.abs(kl_g.astype(np.float64) - kl_o).max() if kl_o.size else 0.0
    assert e <= KL_TOL, f"kl abs {e:.3e} > {KL_TOL}"
    c = np.abs(conf_g.astype(np.float64) - conf_o).max() if conf_o.size else 0.0
    assert c <= CONF_TOL, f"conf abs {c:.3e} > {CONF_TOL}"
    assert np.all(lock_g >= locked_in), "a lock was undone"
    diff = np.nonzero(lock_g != lock_o)[0]
    excused = [r for r in diff if abs(kl_o[r] - eps) <= TIE]
    assert len(excused) == len(diff), f"lock mismatch at rows {sorted(set(diff) - set(excused))[:10]}"
    return len(excused)


def _tol(v, relative):
    return TIE * abs(v) if relative else TIE * max(1.0, abs(v))


def check_scores(margin_g, entropy_g, margin_o, entropy_o, locked_in):
    """Margin and entropy per row; rows locked on entry report zeros."""
    lk = locked_in.astype(bool)
    assert np.all(margin_g[lk] == 0) and np.all(entropy_g[lk] == 0), "locked rows must report 0"
    dm = np.abs(margin_g.astype(np.float64) - margin_o)
    de = np.abs(entropy_g.astype(np.float64) - entropy_o)
    assert dm.max(initial=0) <= MARGIN_TOL, f"margin max-abs {dm.max()}"
    assert de.max(initial=0) <= ENTROPY_TOL, f"entropy max-abs {de.max()}"


def check_selection(sel_g, sel_o, mode, group_rows, tau, conf_o, score_o, locked_in, logits,
                    margin_o=None, entropy_o=None):
    """Exact match of selected rows and tokens up to oracle ties.
    Returns the number of excused disagreements."""
    if mode == W.SEL_NONE:
        assert np.all(sel_g == -1)
        return 0
    R = len(sel_o)
    by_score = mode in (W.SEL_ATTN_DYNAMIC, W.SEL_TOPK_SCORE)
    key = (score_o if by_score else margin_o if mode == W.SEL_TOPK_MARGIN else
           -entropy_o if mode == W.SEL_TOPK_LOW_ENTROPY else conf_o)
    excused = 0
    for g0 in range(0, R, group_rows):
        rows = np.arange(g0, min(R, g0 + group_rows))
        elig = rows[locked_in[rows] == 0]
        sg = set(rows[sel_g[rows] >= 0].tolist())
        so = set(rows[sel_o[rows] >= 0].tolist())
        only_g, only_o = sorted(sg - so), sorted(so - sg)
        ambiguous_group = False
        thr = -np.inf
        if mode == W.SEL_ATTN_DYNAMIC:
            ambiguous_group = any(abs(conf_o[r] - tau) <= TIE for r in elig)
            non = [r for r in elig if not conf_o[r] > tau]
            thr = max((score_o[r] for r in non), default=-np.inf)
        unmatched = []
        pool = list(only_o)
        for r in only_g:
            hit = None
            for r2 in pool:
                if abs(key[r] - key[r2]) <= _tol(key[r2], by_score):
                    hit = r2
                    break
            if hit is not None:
                pool.remove(hit)
                excused += 2
            else:
                unmatched.append(r)
        for r in unmatched + pool:
            ok = ambiguous_group
            if mode in (W.SEL_THRESH_CONF, W.SEL_ATTN_DYNAMIC) and abs(conf_o[r] - tau) <= TIE:
                ok = True
            if mode == W.SEL_ATTN_DYNAMIC and np.isfinite(thr) and abs(score_o[r] - thr) <= _tol(thr, True):
                ok = True
            assert ok, f"selection differs at row {r} (group {g0 // group_rows})"
            excused += 1
        for r in sg & so:
            if sel_g[r] != sel_o[r]:
                top2 = np.sort(logits[r].astype(np.float64))[-2:]
                assert top2[1] - top2[0] <= TIE, f"token differs at row {r}: {sel_g[r]} vs {sel_o[r]}"
                excused += 1
    return excused
