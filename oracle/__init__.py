"""CPU oracle of one masked-diffusion denoising step (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library and
its Python binding never do.  The oracle shares no code with the GPU path.

The arithmetic of one step lives in ``dlm_oracle.c`` (plain C, fp64, OpenMP
over independent rows); this module only marshals numpy arrays into it.
``block_buffer`` (the Block Buffer state machine and the compaction of the
rows to compute) and ``loop`` (the multi-step run that composes them with
the step) are plain Python.  Each function states the passage it follows.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` and ``tests/test_oracle_loop_pins.py`` against
library routines (torch SDPA, scipy, numpy), hand-worked fixtures under
``tests/golden/`` and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dlm_oracle.c")
_LIB = os.path.join(_HERE, "libdlm_oracle.so")

MASK_FULL, MASK_BLOCK_CAUSAL, MASK_GROUP = 0, 1, 2
ROW_SELECT, ROW_LOCK = 1, 2      # per-row flags of posterior() / select()


# gcc flags of the sanitizer build (host code only): address and undefined-
# behaviour checks, every finding fatal.
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math); with
    sanitize, an AddressSanitizer + UBSan build at `out` (a process that
    loads it must preload the sanitizer runtimes)."""
    lib = out or _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-Wno-unused-parameter",
                        *(SANITIZE_FLAGS if sanitize else []),
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, lib)
    return lib


_lib = None


def library_path() -> str:
    """The oracle library this process loads: DLM_ORACLE_LIB when set (a
    sanitizer build, used as it is), else the in-tree build."""
    return os.environ.get("DLM_ORACLE_LIB") or _LIB


def _load():
    global _lib
    if _lib is None:
        path = library_path()
        if path == _LIB and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I, L, Dd = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.ora_scatter.argtypes = [P, P, P, P, P, I, I, I, I, I]
        lib.ora_scatter.restype = None
        lib.ora_visible.argtypes = [I, I, I, I, I, P, P, I, I]
        lib.ora_visible.restype = I
        lib.ora_attn.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, P, P,
                                 Dd, L, P, P, P]
        lib.ora_attn.restype = None
        lib.ora_colsum.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, P, P,
                                   Dd, I, I, I, P, L, P, P]
        lib.ora_colsum.restype = None
        lib.ora_posterior.argtypes = [P, P, P, L, L, Dd, L, P, P, P, P, P, P, P, P, Dd]
        lib.ora_posterior.restype = None
        lib.ora_select.argtypes = [I, I, I, Dd, P, P, P, P, I, P, P, P, P]
        lib.ora_select.restype = None
        lib.ora_num_threads.argtypes = []
        lib.ora_num_threads.restype = I
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return _load().ora_num_threads()


def effective_kv(case):
    """The cache after the fresh K/V of the active rows are written at their
    positions (SureLock, section 2: locked rows keep cached K/V, active rows
    are recomputed).  Returns new (K, V) bf16-bit arrays; inputs untouched."""
    lib = _load()
    ck = case.cache_k.copy()
    cv = case.cache_v.copy()
    lib.ora_scatter(_p(ck), _p(cv), _p(_c(case.k, np.uint16)), _p(_c(case.v, np.uint16)),
                    _p(_c(case.active_idx, np.int32)), case.B, case.Hkv, case.n_cap,
                    case.D, case.M)
    return ck, cv


def scale_of(case) -> float:
    return case.scale if case.scale else 1.0 / np.sqrt(case.D)


def visible(case, b, i, n) -> bool:
    """Key n visible to the query at position i (MBD-LM sections 2.2/2.3,
    Bifocal dLLM section 1)."""
    lib = _load()
    st = _c(case.slot_state[b], np.uint8) if case.n_slots else None
    gr = _c(case.slot_group[b], np.int32) if case.n_slots else None
    return bool(lib.ora_visible(case.kind, case.kv_len, case.prefix_len,
                                case.block_size, case.n_slots, _p(st), _p(gr), i, n))


def attention(case, kv=None, rows=None, want_out=True):
    """Attention of active rows over visible keys of the effective cache.

    rows: flat indices ((b*Hq + h)*M + j) or None for all.  Returns
    (out [n,D] fp64 or None, lse [n] fp64).  With rows=None the arrays are
    reshaped to [B,Hq,M,D] and [B,Hq,M]."""
    lib = _load()
    K, Vv = effective_kv(case) if kv is None else kv
    n = case.B * case.Hq * case.M if rows is None else len(rows)
    rows_a = None if rows is None else _c(rows, np.int64)
    out = np.empty((n, case.D), np.float64) if want_out else None
    lse = np.empty(n, np.float64)
    st = _c(case.slot_state, np.uint8) if case.n_slots else None
    gr = _c(case.slot_group, np.int32) if case.n_slots else None
    lib.ora_attn(_p(_c(case.q, np.uint16)), _p(K), _p(Vv), _p(_c(case.active_idx, np.int32)),
                 case.B, case.Hq, case.Hkv, case.n_cap, case.D, case.M, case.kind,
                 case.kv_len, case.prefix_len, case.block_size, case.n_slots,
                 _p(st), _p(gr), scale_of(case), n, _p(rows_a), _p(out), _p(lse))
    if rows is None:
        lse = lse.reshape(case.B, case.Hq, case.M)
        if out is not None:
            out = out.reshape(case.B, case.Hq, case.M, case.D)
    return out, lse


def colsum(case, lse_all, kv=None, cols=None):
    """Attention column sums (Attn-Sampler section 2B), head-summed or per
    head, over rows whose position lies in [cs_lo, cs_hi).

    lse_all: [B,Hq,M] from ``attention`` over all rows.  cols: flat
    (b*kv_len + n) or None for all.  Returns [B,kv_len] / [B,Hq,kv_len] for
    cols=None, else [n] / [n,Hq]."""
    lib = _load()
    K, _ = effective_kv(case) if kv is None else kv
    n = case.B * case.kv_len if cols is None else len(cols)
    cols_a = None if cols is None else _c(cols, np.int64)
    res = np.empty((n, case.Hq) if case.colsum_per_head else (n,), np.float64)
    st = _c(case.slot_state, np.uint8) if case.n_slots else None
    gr = _c(case.slot_group, np.int32) if case.n_slots else None
    lib.ora_colsum(_p(_c(case.q, np.uint16)), _p(K), _p(_c(case.active_idx, np.int32)),
                   case.B, case.Hq, case.Hkv, case.n_cap, case.D, case.M, case.kind,
                   case.kv_len, case.prefix_len, case.block_size, case.n_slots,
                   _p(st), _p(gr), scale_of(case), case.cs_lo, case.cs_hi,
                   case.colsum_per_head, _p(_c(lse_all, np.float64)), n, _p(cols_a),
                   _p(res))
    if cols is None:
        if case.colsum_per_head:
            res = res.reshape(case.B, case.kv_len, case.Hq).transpose(0, 2, 1).copy()
        else:
            res = res.reshape(case.B, case.kv_len)
    return res


def posterior(logits, prev, locked, eps, rows=None, flags=None, conf_gate=0.0):
    """Per-row KL(p_t || p_{t-1}), confidence, argmax token and lock flag
    (SureLock section 2), and the margin p(top-1) - p(top-2) and entropy of
    p_t (the token-level scores named on the Attn-Sampler page, section 1).
    flags (uint8 [R] or None): only rows with bit ROW_LOCK may lock.
    conf_gate: the optional confidence gate (SureLock section 2): a row
    locks only if also conf >= conf_gate (0: no gate).
    Returns dict of kl, conf, tok, locked (new), margin, entropy."""
    lib = _load()
    logits = _c(logits, np.float32)
    prev = _c(prev, np.float32)
    locked = _c(locked, np.uint8)
    R, V = logits.shape
    n = R if rows is None else len(rows)
    rows_a = None if rows is None else _c(rows, np.int64)
    kl = np.empty(n, np.float64)
    conf = np.empty(n, np.float64)
    tok = np.empty(n, np.int32)
    lk = np.empty(n, np.uint8)
    margin = np.empty(n, np.float64)
    entropy = np.empty(n, np.float64)
    flags_a = None if flags is None else _c(flags, np.uint8)
    lib.ora_posterior(_p(logits), _p(prev), _p(locked), R, V, float(eps), n, _p(rows_a),
                      _p(kl), _p(conf), _p(tok), _p(lk), _p(margin), _p(entropy), _p(flags_a),
                      float(conf_gate))
    return {"kl": kl, "conf": conf, "tok": tok, "locked": lk, "margin": margin, "entropy": entropy}


def select(mode, k, group_rows, tau, score, conf, tok, locked_in, margin=None, entropy=None,
           flags=None):
    """Unmask selection per group of rows (confidence top-k / threshold,
    Attn-Sampler order and dynamic threshold, margin and entropy samplers).
    flags (uint8 [R] or None): only rows with bit ROW_SELECT are eligible.
    Returns sel int32 [R]."""
    lib = _load()
    conf = _c(conf, np.float64)
    R = conf.shape[0]
    zeros = np.zeros(R, np.float64)
    score_a = _c(score, np.float64) if score is not None else zeros
    margin_a = _c(margin, np.float64) if margin is not None else zeros
    entropy_a = _c(entropy, np.float64) if entropy is not None else zeros
    sel = np.empty(R, np.int32)
    lib.ora_select(int(mode), int(k), int(group_rows), float(tau), _p(score_a), _p(conf),
                   _p(_c(tok, np.int32)), _p(_c(locked_in, np.uint8)), R, _p(sel),
                   _p(margin_a), _p(entropy_a), _p(None if flags is None else _c(flags, np.uint8)))
    return sel


def step(workload, attn_rows=None):
    """The whole step on the CPU: effective K/V, attention, column sums,
    posterior, selection.  Returns a dict of fp64 results."""
    from workloads import score_for
    a, p = workload.attn, workload.post
    kv = effective_kv(a)
    out, lse = attention(a, kv=kv)
    cs = colsum(a, lse, kv=kv)
    post = posterior(p.logits, p.prev, p.locked, p.eps)
    score = score_for(p, cs if not a.colsum_per_head else cs.sum(1))
    sel = select(p.mode, p.k, p.group_rows, p.tau, score, post["conf"], post["tok"], p.locked,
                 post["margin"], post["entropy"])
    return {"cache_k": kv[0], "cache_v": kv[1], "out": out, "lse": lse, "colsum": cs,
            "score": score, "sel": sel, **post}
