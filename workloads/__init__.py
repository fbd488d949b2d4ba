"""Seeded synthetic inputs for one masked-diffusion denoising step.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds none of the method's arithmetic: only random draws,
round-to-nearest-even narrowing of the draws to bfloat16, and the index and
slot tables that describe which positions are active.

Shapes follow the pages' workloads (see ``CONFIGS``):
  * LLaDA-8B-class heads, 32 heads of width 128 (SureLock page, section 4);
  * a 512- or 1024-token generation length (SureLock page, section 4);
  * a 4096-token prompt at batch 8 (Bifocal dLLM page, section 4);
  * a 16384-token prefix (Bifocal dLLM page, section 4);
  * a running set of 2-4 consecutive blocks (MBD-LM page, section 2.1).
The pages measure on public suites with trained models; these seeded draws
stand in for them.

Every array is numpy on the host; bf16 tensors are carried as their uint16
bit patterns.  Draws are float32 standard normals scaled by the stated
standard deviation ("N(0, s)" is read as standard deviation s).
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

# Mask kinds, slot states and selection modes (same values as the C ABI).
MASK_FULL, MASK_BLOCK_CAUSAL, MASK_GROUP = 0, 1, 2
SLOT_DUMMY, SLOT_ACTIVE, SLOT_TO_CACHE, SLOT_IN_CACHE = 0, 1, 2, 3
SEL_NONE, SEL_TOPK_CONF, SEL_THRESH_CONF, SEL_ATTN_DYNAMIC, SEL_TOPK_SCORE = 0, 1, 2, 3, 4
SEL_TOPK_MARGIN, SEL_TOPK_LOW_ENTROPY = 5, 6

_STREAMS = ("q", "k", "v", "cache_k", "cache_v", "active", "logits", "noise",
            "mixture")


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  Inputs are finite by construction.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bfloat16 bit patterns exactly to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _seqs(config_id: int, seed: int):
    children = np.random.SeedSequence([config_id, seed]).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, children))


def _streams(config_id: int, seed: int):
    return {name: np.random.default_rng(s) for name, s in _seqs(config_id, seed).items()}


def _par_normal(seq, shape, std, block_rows=256) -> np.ndarray:
    """float32 N(0, std) of the given 2-D shape, filled in row blocks by
    worker threads; block i draws from the i-th child of ``seq``, so the
    result does not depend on the number of threads."""
    from concurrent.futures import ThreadPoolExecutor
    R, V = shape
    out = np.empty((R, V), np.float32)
    n_blocks = max(1, (R + block_rows - 1) // block_rows)
    kids = seq.spawn(n_blocks)

    def fill(i):
        r0, r1 = i * block_rows, min(R, (i + 1) * block_rows)
        np.random.default_rng(kids[i]).standard_normal(size=(r1 - r0, V), dtype=np.float32,
                                                       out=out[r0:r1])
        out[r0:r1] *= np.float32(std)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(n_blocks)))
    return out


def _normal_bf16(rng, shape, std) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    z *= np.float32(std)
    return to_bf16_bits(z)


@dataclasses.dataclass
class AttnCase:
    """Inputs of the attention half of one step (q, fresh k/v, cache, mask)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    n_cap: int
    kv_len: int
    prefix_len: int
    M: int
    kind: int
    block_size: int
    n_slots: int
    slot_state: np.ndarray      # uint8 [B, n_slots]
    slot_group: np.ndarray      # int32 [B, n_slots]
    cs_lo: int
    cs_hi: int
    colsum_per_head: int
    scale: float                # 0 => 1/sqrt(D)
    q: np.ndarray               # bf16 bits [B, Hq, M, D]
    k: np.ndarray               # bf16 bits [B, Hkv, M, D]
    v: np.ndarray               # bf16 bits [B, Hkv, M, D]
    cache_k: np.ndarray         # bf16 bits [B, Hkv, n_cap, D]
    cache_v: np.ndarray         # bf16 bits [B, Hkv, n_cap, D]
    active_idx: np.ndarray      # int32 [B, M], ascending, unique, >= prefix_len

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclasses.dataclass
class PostCase:
    """Inputs of the posterior half of one step (logits of two steps)."""
    name: str
    R: int
    V: int
    logits: np.ndarray          # float32 [R, V], step t
    prev: np.ndarray            # float32 [R, V], step t-1
    locked: np.ndarray          # uint8 [R], lock state before this step
    eps: float
    mode: int
    k: int
    group_rows: int
    tau: float
    # Where the selection score comes from: None, or (b, first_position):
    # score[r] = colsum[b, first_position + r] of the attention half.
    score_cols: Optional[tuple] = None
    score: Optional[np.ndarray] = None   # explicit float32 [R] score, if any


@dataclasses.dataclass
class Workload:
    attn: AttnCase
    post: PostCase
    description: str


# --------------------------------------------------------------------------
# Generic builders
# --------------------------------------------------------------------------

def make_attn(name, *, B, Hq, Hkv, D, kv_len, prefix_len, active_idx, kind,
              block_size=0, n_slots=0, slot_state=None, slot_group=None,
              cs_lo=0, cs_hi=None, colsum_per_head=0, scale=0.0, n_cap=None,
              q_std=1.0, kv_std=1.0, cache_std=1.0, garbage_rows=None,
              garbage_std=50.0, config_id=99, seed=0) -> AttnCase:
    """Draw q, fresh k/v and the cache for the given shape and active set.

    ``active_idx`` is an int array [B, M] (ascending per batch).  Cache rows
    listed in ``garbage_rows`` (a boolean [B, n_cap] mask) are drawn with
    ``garbage_std`` so that a kernel that wrongly reads them is caught.
    """
    rs = _streams(config_id, seed)
    active_idx = np.ascontiguousarray(active_idx, dtype=np.int32)
    M = active_idx.shape[1]
    n_cap = kv_len if n_cap is None else n_cap
    q = _normal_bf16(rs["q"], (B, Hq, M, D), q_std)
    k = _normal_bf16(rs["k"], (B, Hkv, M, D), kv_std)
    v = _normal_bf16(rs["v"], (B, Hkv, M, D), kv_std)
    ck = rs["cache_k"].standard_normal(size=(B, Hkv, n_cap, D), dtype=np.float32)
    cv = rs["cache_v"].standard_normal(size=(B, Hkv, n_cap, D), dtype=np.float32)
    ck *= np.float32(cache_std)
    cv *= np.float32(cache_std)
    if garbage_rows is not None:
        g = np.broadcast_to(garbage_rows[:, None, :, None], ck.shape)
        ck = np.where(g, ck * np.float32(garbage_std / cache_std), ck)
        cv = np.where(g, cv * np.float32(garbage_std / cache_std), cv)
    if slot_state is None:
        slot_state = np.zeros((B, max(n_slots, 0)), np.uint8)
    if slot_group is None:
        slot_group = np.zeros((B, max(n_slots, 0)), np.int32)
    return AttnCase(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, n_cap=n_cap, kv_len=kv_len,
        prefix_len=prefix_len, M=M, kind=kind, block_size=block_size,
        n_slots=n_slots,
        slot_state=np.ascontiguousarray(slot_state, np.uint8),
        slot_group=np.ascontiguousarray(slot_group, np.int32),
        cs_lo=cs_lo, cs_hi=kv_len if cs_hi is None else cs_hi,
        colsum_per_head=colsum_per_head, scale=scale,
        q=q, k=k, v=v, cache_k=to_bf16_bits(ck), cache_v=to_bf16_bits(cv),
        active_idx=active_idx)


def make_post(name, *, R, V, logit_std, noise_std, eps, mode, k=0,
              group_rows=None, tau=0.0, mixture=None, spike_frac=0.0,
              spike_value=30.0, locked_frac=0.0, score_cols=None,
              score_std=None, config_id=99, seed=0) -> PostCase:
    """Draw step-t logits and step-(t-1) logits = logits + noise.

    ``mixture`` = (fraction, std_a, std_b): a seeded ``fraction`` of rows
    get noise std ``std_a``, the rest ``std_b`` (``noise_std`` is then
    ignored).  ``spike_frac`` of rows get one seeded vocab entry set to
    ``spike_value`` in both arrays.  ``locked_frac`` of rows arrive locked.
    ``score_std`` draws an explicit per-row score (for posterior-only cases).
    """
    seqs = _seqs(config_id, seed)
    logits = _par_normal(seqs["logits"], (R, V), logit_std)
    noise = _par_normal(seqs["noise"], (R, V), 1.0)
    mx = np.random.default_rng(seqs["mixture"])
    if mixture is not None:
        frac, std_a, std_b = mixture
        pick = mx.random(R) < frac
        row_std = np.where(pick, np.float32(std_a), np.float32(std_b)).astype(np.float32)
        noise *= row_std[:, None]
    else:
        noise *= np.float32(noise_std)
    prev = logits + noise
    del noise
    if spike_frac > 0:
        rows = np.nonzero(mx.random(R) < spike_frac)[0]
        cols = mx.integers(0, V, size=rows.size)
        logits[rows, cols] = np.float32(spike_value)
        prev[rows, cols] = np.float32(spike_value)
    locked = (mx.random(R) < locked_frac).astype(np.uint8)
    score = None
    if score_std is not None:
        score = (mx.standard_normal(R).astype(np.float32) * np.float32(score_std)
                 + np.float32(10.0 * score_std))
    return PostCase(name=name, R=R, V=V, logits=logits, prev=prev,
                    locked=locked, eps=eps, mode=mode, k=k,
                    group_rows=R if group_rows is None else group_rows,
                    tau=tau, score_cols=score_cols, score=score)


def sorted_subset(rng, B, lo, hi, m) -> np.ndarray:
    """Per batch, a uniformly drawn ascending m-subset of [lo, hi)."""
    out = np.empty((B, m), np.int32)
    for b in range(B):
        out[b] = np.sort(rng.choice(hi - lo, size=m, replace=False)) + lo
    return out


# --------------------------------------------------------------------------
# The workloads (full sizes)
# --------------------------------------------------------------------------

def tiny(seed=0) -> Workload:
    """B=1, 2 heads of width 32, 64 positions: a 32-row clean prefix in the
    cache and a 32-token generation block, of which a seeded 16 rows are
    active (the other 16 are locked rows read from the cache).  Bidirectional.
    Posterior: 16 rows x vocab 512, logits N(0,2), prev = logits + N(0,0.05),
    eps 1e-3, unmask the top-4 by confidence."""
    cid = 1
    rs = _streams(cid, seed)
    act = sorted_subset(rs["active"], 1, 32, 64, 16)
    std = 1.0 / np.sqrt(32.0)
    a = make_attn("tiny", B=1, Hq=2, Hkv=2, D=32, kv_len=64, prefix_len=32,
                  active_idx=act, kind=MASK_FULL, cs_lo=32, cs_hi=64,
                  q_std=std, kv_std=std, cache_std=std, config_id=cid, seed=seed)
    p = make_post("tiny", R=16, V=512, logit_std=2.0, noise_std=0.05, eps=1e-3,
                  mode=SEL_TOPK_CONF, k=4, group_rows=16, config_id=cid, seed=seed)
    return Workload(a, p, "tiny: B1 H2 D32 N64, 16 active of a 32-token block")


def llada_bidirectional(seed=0, spread=False) -> Workload:
    """LLaDA-8B-like bidirectional layer: B=1, 32 heads of width 128,
    N=1024 (512 prompt + 512 generation), all 1024 queries active.  Column
    sums over the 512 masked rows.  Posterior: the first 32-row generation
    block x vocab 126464, logits N(0,3), prev + N(0,0.1), eps 1e-3, Attn-
    Sampler dynamic threshold with tau 0.9 scored by the column sums.

    ``spread=True`` draws q/k/v from N(0,1) unscaled (column sums spread out)
    and plants a 30.0 spike in 25% of posterior rows (confident rows)."""
    cid = 2 if not spread else 21
    N = 1024
    act = np.arange(N, dtype=np.int32)[None, :]
    std = 1.0 if spread else 1.0 / np.sqrt(128.0)
    a = make_attn("llada_bidirectional" + ("_spread" if spread else ""),
                  B=1, Hq=32, Hkv=32, D=128, kv_len=N, prefix_len=0,
                  active_idx=act, kind=MASK_FULL, cs_lo=512, cs_hi=1024,
                  q_std=std, kv_std=std, cache_std=std, config_id=cid, seed=seed)
    p = make_post(a.name, R=32, V=126464, logit_std=3.0, noise_std=0.1, eps=1e-3,
                  mode=SEL_ATTN_DYNAMIC, tau=0.9, group_rows=32,
                  spike_frac=0.25 if spread else 0.0,
                  score_cols=(0, 512), config_id=cid, seed=seed)
    return Workload(a, p, "LLaDA-8B-like bidirectional layer, all 1024 rows active")


def mbd_multiblock(seed=0, variant="group", B=8, Hq=32, Hkv=8, D=128, P=4096,
                   block=32, V=151936) -> Workload:
    """Multi-block diffusion running set: 4 active blocks x 32 tokens after a
    clean prefix of P rows in the cache, GQA 32 query / 8 kv heads, B=8.
    Variants: "group" (one noise group, the four blocks see each other and
    the prefix), "dummy" (six buffer slots, the last two DUMMY with garbage
    K/V), "block_causal" (each block sees the prefix and earlier blocks),
    "two_groups" (groups {0,1} and {2,3}).  Posterior: 128 rows per batch x
    vocab 151936, top-8 per 32-row block."""
    cid = {"group": 3, "dummy": 31, "block_causal": 32, "two_groups": 33}[variant]
    rs = _streams(cid, seed)
    n_active_slots = 4
    n_slots = 6 if variant == "dummy" else 4
    kv_len = P + n_slots * block
    M = n_active_slots * block
    act = np.tile(np.arange(P, P + M, dtype=np.int32), (B, 1))
    state = np.full((B, n_slots), SLOT_ACTIVE, np.uint8)
    state[:, n_active_slots:] = SLOT_DUMMY
    group = np.zeros((B, n_slots), np.int32)
    kind = MASK_GROUP
    garbage = None
    if variant == "two_groups":
        group[:] = np.array([0, 0, 1, 1], np.int32)
    elif variant == "block_causal":
        kind = MASK_BLOCK_CAUSAL
    elif variant == "dummy":
        garbage = np.zeros((B, kv_len), bool)
        garbage[:, P + M:] = True
        group[:, n_active_slots:] = 0
    a = make_attn("mbd_multiblock_" + variant, B=B, Hq=Hq, Hkv=Hkv, D=D,
                  kv_len=kv_len, prefix_len=P, active_idx=act, kind=kind,
                  block_size=block, n_slots=n_slots, slot_state=state,
                  slot_group=group, cs_lo=P, cs_hi=P + M, garbage_rows=garbage,
                  config_id=cid, seed=seed)
    del rs
    p = make_post(a.name, R=B * M, V=V, logit_std=3.0, noise_std=0.1, eps=1e-3,
                  mode=SEL_TOPK_CONF, k=8, group_rows=block, config_id=cid,
                  seed=seed)
    return Workload(a, p, f"multi-block running set ({variant}), GQA 32/8, B={B}")


def surelock_sparse(seed=0, B=4, H=32, D=128, N=8192, M=2048, V=126464) -> Workload:
    """SureLock sparse-query step: B=4, 32 heads of width 128, N=8192,
    bidirectional.  A seeded 75% of positions are locked (cache K/V); the
    2048 active rows sit at random ascending positions with fresh q/k/v
    N(0,1)/sqrt(128).  Posterior over the active rows only, vocab 126464,
    logits N(0,3); prev noise is a seeded per-row mixture (40% of rows
    N(0,0.02), 60% N(0,0.1)) so that about 40% of rows fall under eps=1e-3.
    No unmask selection (lock test only)."""
    cid = 4
    rs = _streams(cid, seed)
    act = sorted_subset(rs["active"], B, 0, N, M)
    std = 1.0 / np.sqrt(128.0)
    a = make_attn("surelock_sparse", B=B, Hq=H, Hkv=H, D=D, kv_len=N,
                  prefix_len=0, active_idx=act, kind=MASK_FULL, cs_lo=0, cs_hi=N,
                  q_std=std, kv_std=std, cache_std=std, config_id=cid, seed=seed)
    p = make_post("surelock_sparse", R=B * M, V=V, logit_std=3.0, noise_std=0.0,
                  mixture=(0.4, 0.02, 0.1), eps=1e-3, mode=SEL_NONE,
                  config_id=cid, seed=seed)
    return Workload(a, p, "SureLock sparse-query step, 2048 of 8192 rows active")


def long_prefix_sampler(seed=0, P=16384, gen=256, H=32, D=128, V=151936) -> Workload:
    """Long-context Attn-Sampler: B=1, 32 heads of width 128, a prefix of
    P=16384 rows in the cache plus a 256-token masked generation block that
    sees itself and the whole prefix.  Head-summed column sums over the 256
    generation rows rank the block; the top-16 by column sum are unmasked.
    Posterior: 256 rows x vocab 151936, logits N(0,3), prev + N(0,0.1)."""
    cid = 5
    act = np.arange(P, P + gen, dtype=np.int32)[None, :]
    a = make_attn("long_prefix_sampler", B=1, Hq=H, Hkv=H, D=D, kv_len=P + gen,
                  prefix_len=P, active_idx=act, kind=MASK_FULL, cs_lo=P,
                  cs_hi=P + gen, config_id=cid, seed=seed)
    p = make_post("long_prefix_sampler", R=gen, V=V, logit_std=3.0,
                  noise_std=0.1, eps=1e-3, mode=SEL_TOPK_SCORE, k=16,
                  group_rows=gen, score_cols=(0, P), config_id=cid, seed=seed)
    return Workload(a, p, "long-prefix Attn-Sampler, P=16384 + 256-token block")


# --------------------------------------------------------------------------
# Multi-step runs (Block Buffer loop)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LoopCase:
    """Inputs of a multi-step denoising run over a Block Buffer.  The model
    that would produce each step's queries, fresh K/V and logits is not part
    of the path: these stand in for it, for every generation position and
    step (a step reads the entries of the rows it computes)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    prefix_len: int             # clean prompt rows in the cache
    block_size: int
    n_slots: int                # generation region = n_slots * block_size positions
    max_active: int             # running-set size (most active slots at once)
    T: int                      # steps drawn
    V: int
    eps: float
    mode: int
    k: int
    tau: float
    cache_k: np.ndarray         # bf16 bits [B, Hkv, kv_len, D]
    cache_v: np.ndarray
    q: np.ndarray               # bf16 bits [T, B, Hq, n_gen, D]
    k_new: np.ndarray           # bf16 bits [T, B, Hkv, n_gen, D]
    v_new: np.ndarray
    logits: np.ndarray          # float32 [T, B, n_gen, V]
    decoded0: np.ndarray        # uint8 [B, n_gen]: positions unmasked at the start
    tokens0: np.ndarray         # int32 [B, n_gen]

    @property
    def n_gen(self) -> int:
        return self.n_slots * self.block_size

    @property
    def kv_len(self) -> int:
        return self.prefix_len + self.n_gen


def make_loop(name, *, B, Hq, Hkv, D, P, block_size, n_slots, max_active, T, V,
              eps=1e-3, mode=SEL_TOPK_CONF, k=2, tau=0.9, logit_std=3.0,
              noise_std=1.0, decay=(0.5, 0.75), qkv_std=None, n_decoded0=0,
              config_id=90, seed=0) -> LoopCase:
    """Draw a run.  Queries and fresh K/V are N(0, qkv_std) per step and
    position (default 1/sqrt(D)); the clean prompt's cache rows likewise,
    and the generation rows of the cache hold garbage N(0, 50) until a step
    writes them.  Logits of position p at step t are
        base[p] + noise_std * decay[p]**t * xi[t, p],
    base ~ N(0, logit_std), xi ~ N(0, 1) fresh each step and decay[p]
    uniform in ``decay``: each position's posterior settles geometrically at
    its own rate, so rows lock at different steps.  The first ``n_decoded0``
    positions of each sequence start unmasked (a prompt recomputed each
    step) with their base argmax as token."""
    rs = _streams(config_id, seed)
    n_gen = n_slots * block_size
    kv_len = P + n_gen
    std = (1.0 / np.sqrt(D)) if qkv_std is None else qkv_std
    q = _normal_bf16(rs["q"], (T, B, Hq, n_gen, D), std)
    kn = _normal_bf16(rs["k"], (T, B, Hkv, n_gen, D), std)
    vn = _normal_bf16(rs["v"], (T, B, Hkv, n_gen, D), std)
    ck = rs["cache_k"].standard_normal(size=(B, Hkv, kv_len, D), dtype=np.float32) * np.float32(std)
    cv = rs["cache_v"].standard_normal(size=(B, Hkv, kv_len, D), dtype=np.float32) * np.float32(std)
    ck[:, :, P:] *= np.float32(50.0 / std)
    cv[:, :, P:] *= np.float32(50.0 / std)
    lg = rs["logits"]
    base = lg.standard_normal(size=(B, n_gen, V), dtype=np.float32) * np.float32(logit_std)
    rate = rs["mixture"].uniform(decay[0], decay[1], size=(B, n_gen))
    nz = rs["noise"]
    logits = np.empty((T, B, n_gen, V), np.float32)
    for t in range(T):
        amp = (noise_std * rate ** t).astype(np.float32)
        logits[t] = base + amp[:, :, None] * nz.standard_normal(size=(B, n_gen, V), dtype=np.float32)
    dec0 = np.zeros((B, n_gen), np.uint8)
    tok0 = np.full((B, n_gen), -1, np.int32)
    dec0[:, :n_decoded0] = 1
    tok0[:, :n_decoded0] = np.argmax(base[:, :n_decoded0], axis=-1)
    return LoopCase(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, block_size=block_size,
                    n_slots=n_slots, max_active=max_active, T=T, V=V, eps=eps, mode=mode,
                    k=k, tau=tau, cache_k=to_bf16_bits(ck), cache_v=to_bf16_bits(cv),
                    q=q, k_new=kn, v_new=vn, logits=logits, decoded0=dec0, tokens0=tok0)


def loop_multiblock(seed=0) -> LoopCase:
    """Multi-block run: B=2, GQA 4/2 heads of width 64, a 48-row prompt in
    the cache, four 16-token blocks with a running set of two, vocab 1000,
    the top-2 by confidence unmasked per block and step, eps 1e-3."""
    return make_loop("loop_multiblock", B=2, Hq=4, Hkv=2, D=64, P=48, block_size=16,
                     n_slots=4, max_active=2, T=24, V=1000, mode=SEL_TOPK_CONF, k=2,
                     config_id=91, seed=seed)


def loop_surelock(seed=0) -> LoopCase:
    """SureLock-style run: B=1, 2 heads of width 128, no cached prefix, one
    80-position block of which the first 32 are an unmasked prompt that is
    recomputed until it locks; Attn-Sampler dynamic threshold (tau 0.5,
    scored by column sums), vocab 1003 (not a multiple of 4)."""
    return make_loop("loop_surelock", B=1, Hq=2, Hkv=2, D=128, P=0, block_size=80,
                     n_slots=1, max_active=1, T=64, V=1003, mode=SEL_ATTN_DYNAMIC, tau=0.5,
                     n_decoded0=32, config_id=92, seed=seed)


def loop_threshold(seed=0) -> LoopCase:
    """Six 8-token blocks, three running, GQA 8/2 heads of width 32, a
    40-row prompt, confidence threshold 0.3 (the single most confident row
    when none passes), vocab 512."""
    return make_loop("loop_threshold", B=1, Hq=8, Hkv=2, D=32, P=40, block_size=8,
                     n_slots=6, max_active=3, T=40, V=512, mode=SEL_THRESH_CONF, tau=0.3,
                     config_id=93, seed=seed)


LOOPS = {
    "loop_multiblock": loop_multiblock,
    "loop_surelock": loop_surelock,
    "loop_threshold": loop_threshold,
}


# --------------------------------------------------------------------------
# A layer's active-row projections and feed-forward
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LayerCase:
    """Inputs of one layer's active-row projections and SwiGLU feed-forward:
    hidden states, the active rows, synthetic weights [out, in] and the
    attention output / residual rows that the later calls take."""
    name: str
    B: int
    n_pos: int
    d: int
    Hq: int
    Hkv: int
    D: int
    F: int
    M: int
    x: np.ndarray               # bf16 bits [B, n_pos, d]
    active_idx: np.ndarray      # int32 [B, M], ascending
    m: np.ndarray               # int32 [B]: valid rows per batch entry
    w_qkv: np.ndarray           # bf16 bits [(Hq + 2 Hkv) D, d]
    w_o: np.ndarray             # bf16 bits [d, Hq D]
    w_gate: np.ndarray          # bf16 bits [F, d]
    w_up: np.ndarray            # bf16 bits [F, d]
    w_down: np.ndarray          # bf16 bits [d, F]
    attn_out: np.ndarray        # bf16 bits [B, Hq, M, D]
    h: np.ndarray               # bf16 bits [B, M, d]


def make_layer(name, *, B, n_pos, d, Hq, Hkv, D, F, M, m=None, config_id=95, seed=0) -> LayerCase:
    """Hidden states and residual rows N(0, 1); weights N(0, 1/sqrt(fan_in))
    (activations stay of order one); attention output N(0, 0.5).  The M
    active positions of each sequence are a seeded ascending subset."""
    rs = _streams(config_id, seed)
    act = sorted_subset(rs["active"], B, 0, n_pos, M)
    m = np.full(B, M, np.int32) if m is None else np.asarray(m, np.int32)
    wq = rs["k"]
    return LayerCase(
        name=name, B=B, n_pos=n_pos, d=d, Hq=Hq, Hkv=Hkv, D=D, F=F, M=M,
        x=_normal_bf16(rs["cache_k"], (B, n_pos, d), 1.0), active_idx=act, m=m,
        w_qkv=_normal_bf16(wq, ((Hq + 2 * Hkv) * D, d), 1.0 / np.sqrt(d)),
        w_o=_normal_bf16(wq, (d, Hq * D), 1.0 / np.sqrt(Hq * D)),
        w_gate=_normal_bf16(rs["v"], (F, d), 1.0 / np.sqrt(d)),
        w_up=_normal_bf16(rs["v"], (F, d), 1.0 / np.sqrt(d)),
        w_down=_normal_bf16(rs["v"], (d, F), 1.0 / np.sqrt(F)),
        attn_out=_normal_bf16(rs["q"], (B, Hq, M, D), 0.5),
        h=_normal_bf16(rs["cache_v"], (B, M, d), 1.0))


def layer_llada(seed=0, M=1024, n_pos=1024) -> LayerCase:
    """LLaDA-8B-shaped layer: width 4096, 32 heads of 128, feed-forward
    width 12288 (SwiGLU), B=1; M active rows of n_pos positions."""
    return make_layer("layer_llada", B=1, n_pos=n_pos, d=4096, Hq=32, Hkv=32, D=128, F=12288, M=M,
                      config_id=96, seed=seed)


# --------------------------------------------------------------------------
# R2LM right-to-left selective scan over the generation block
# --------------------------------------------------------------------------

@dataclasses.dataclass
class R2LCase:
    """Inputs of the right-to-left scan of one step: the generation block's
    hidden states and the scan's parameters (synthetic: the projections that
    produce delta, B and C are not part of the path)."""
    name: str
    B: int
    L: int
    E: int
    N: int
    u: np.ndarray               # bf16 bits [B, L, E]
    delta: np.ndarray           # bf16 bits [B, L, E], positive step sizes
    A: np.ndarray               # float32 [E, N], negative
    Bm: np.ndarray              # bf16 bits [B, L, N]
    Cm: np.ndarray              # bf16 bits [B, L, N]
    Dv: np.ndarray              # float32 [E]
    gate: float                 # the scalar s
    x: np.ndarray               # bf16 bits [B, L, E]: the hidden stream the correction joins


def make_r2l(name, *, B, L, E, N, gate=0.5, config_id=97, seed=0) -> R2LCase:
    """u, x ~ N(0, 1); delta = softplus of N(-2, 1) draws (Mamba's step-size
    parameterisation, mostly in (0.01, 1)); A[e, n] = -(n + 1) (the usual
    initialisation); B, C ~ N(0, 1); D ~ N(0, 1)."""
    rs = _streams(config_id, seed)
    d = rs["k"].standard_normal(size=(B, L, E)).astype(np.float32) - np.float32(2.0)
    delta = np.log1p(np.exp(d)).astype(np.float32)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (E, 1))
    return R2LCase(name=name, B=B, L=L, E=E, N=N,
                   u=_normal_bf16(rs["q"], (B, L, E), 1.0), delta=to_bf16_bits(delta), A=A,
                   Bm=_normal_bf16(rs["v"], (B, L, N), 1.0), Cm=_normal_bf16(rs["cache_k"], (B, L, N), 1.0),
                   Dv=rs["cache_v"].standard_normal(size=E).astype(np.float32), gate=gate,
                   x=_normal_bf16(rs["logits"], (B, L, E), 1.0))


def r2l_bifocal(seed=0) -> R2LCase:
    """The Bifocal page's serving setting: batch 8, a 256-token generation
    block, the width 2048 of its 1.7B backbone, 16 scan states."""
    return make_r2l("r2l_bifocal", B=8, L=256, E=2048, N=16, config_id=98, seed=seed)


def llada_group(seed=0) -> Workload:
    """The LLaDA-like layer's inputs under a one-block GROUP mask over the
    whole sequence (the multi-step run's mask shape at M_t = 1024): every
    key visible to every query, so it isolates what the GROUP mask itself
    costs against the FULL mask on the same shape."""
    w = llada_bidirectional(seed)
    a = w.attn
    a2 = AttnCase(**{**a.__dict__, "kind": MASK_GROUP, "prefix_len": 0, "block_size": a.kv_len,
                     "n_slots": 1, "slot_state": np.full((a.B, 1), SLOT_ACTIVE, np.uint8),
                     "slot_group": np.zeros((a.B, 1), np.int32)})
    return Workload(a2, w.post, "LLaDA-like layer under a one-block group mask")


CONFIGS = {
    "tiny": tiny,
    "llada_group": llada_group,
    "llada_bidirectional": llada_bidirectional,
    "llada_bidirectional_spread": lambda seed=0: llada_bidirectional(seed, spread=True),
    "mbd_multiblock": mbd_multiblock,
    "mbd_multiblock_dummy": lambda seed=0: mbd_multiblock(seed, "dummy"),
    "mbd_multiblock_block_causal": lambda seed=0: mbd_multiblock(seed, "block_causal"),
    "mbd_multiblock_two_groups": lambda seed=0: mbd_multiblock(seed, "two_groups"),
    "surelock_sparse": surelock_sparse,
    "long_prefix_sampler": long_prefix_sampler,
}


def get(name: str, seed: int = 0) -> Workload:
    return CONFIGS[name](seed=seed)


def score_for(post: PostCase, colsum: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """The per-row selection score: an explicit score, or a slice of the
    head-summed column sums [B, kv_len] named by ``score_cols``."""
    if post.score is not None:
        return post.score
    if post.score_cols is None:
        return None
    b, first = post.score_cols
    return np.ascontiguousarray(colsum[b, first:first + post.R])
