"""GPU parity: the HIP path through the C ABI against the oracle, element by
element on the same seeded inputs.

Reduced shapes (several tiles plus a ragged tail, every mask kind, GQA, key
splits, every selection mode, edge cases) are compared in full; the full
workloads are compared on sampled rows and columns the oracle computes one
by one, plus invariants that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (check_attention, check_colsum, check_posterior, check_scores, check_selection)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd  # noqa: F401  (raises if the library is not built)
    yield


def _device_step(w, **kw):
    from denoising_step_amd.runner import DeviceStep
    return DeviceStep(w, **kw)


# --------------------------------------------------------------------------
# reduced workloads
# --------------------------------------------------------------------------

def small_llada(spread=False, seed=0):
    N = 300
    std = 1.0 if spread else 1.0 / np.sqrt(128)
    a = W.make_attn("small_llada", B=1, Hq=4, Hkv=4, D=128, kv_len=N, prefix_len=0,
                    active_idx=np.arange(N, dtype=np.int32)[None], kind=W.MASK_FULL,
                    cs_lo=150, cs_hi=N, q_std=std, kv_std=std, cache_std=std, seed=seed)
    p = W.make_post("small_llada", R=32, V=5000, logit_std=3.0, noise_std=0.1, eps=1e-3,
                    mode=W.SEL_ATTN_DYNAMIC, tau=0.9, group_rows=32,
                    spike_frac=0.25 if spread else 0.0, score_cols=(0, 150), seed=seed)
    return W.Workload(a, p, "small llada")


def small_mbd(variant="group", D=128, per_head=0, V=8192, seed=0):
    B, Hq, Hkv, P, bs = 2, 8, 2, 333, 32
    n_slots = 6 if variant == "dummy" else 4
    kv_len = P + n_slots * bs
    M = 4 * bs
    act = np.tile(np.arange(P, P + M, dtype=np.int32), (B, 1))
    state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
    state[:, 4:] = W.SLOT_DUMMY
    state[1, 1] = W.SLOT_IN_CACHE
    group = np.zeros((B, n_slots), np.int32)
    kind = W.MASK_GROUP
    garbage = None
    if variant == "two_groups":
        group[:, :4] = [0, 0, 1, 1]
    elif variant == "block_causal":
        kind = W.MASK_BLOCK_CAUSAL
    elif variant == "dummy":
        garbage = np.zeros((B, kv_len), bool)
        garbage[:, P + M:] = True
    a = W.make_attn("small_mbd_" + variant, B=B, Hq=Hq, Hkv=Hkv, D=D, kv_len=kv_len, prefix_len=P,
                    active_idx=act, kind=kind, block_size=bs, n_slots=n_slots, slot_state=state,
                    slot_group=group, cs_lo=P, cs_hi=P + M, colsum_per_head=per_head,
                    garbage_rows=garbage, seed=seed)
    p = W.make_post(a.name, R=B * M, V=V, logit_std=3.0, noise_std=0.1, eps=1e-3,
                    mode=W.SEL_TOPK_CONF, k=8, group_rows=bs, locked_frac=0.1, seed=seed)
    return W.Workload(a, p, "small mbd " + variant)


def small_surelock(D=128, Hq=4, Hkv=4, seed=0):
    rng = np.random.default_rng(100 + seed)
    B, N, M = 2, 1000, 250
    std = 1.0 / np.sqrt(D)
    a = W.make_attn("small_surelock", B=B, Hq=Hq, Hkv=Hkv, D=D, kv_len=N, prefix_len=0,
                    active_idx=W.sorted_subset(rng, B, 0, N, M), kind=W.MASK_FULL,
                    q_std=std, kv_std=std, cache_std=std, n_cap=N + 24, seed=seed)
    p = W.make_post("small_surelock", R=B * M, V=10000, logit_std=3.0, noise_std=0.0,
                    mixture=(0.4, 0.02, 0.1), eps=1e-3, mode=W.SEL_NONE, locked_frac=0.1,
                    seed=seed)
    return W.Workload(a, p, "small surelock")


def small_long(seed=0):
    P, gen = 3000, 256
    a = W.make_attn("small_long", B=1, Hq=4, Hkv=4, D=128, kv_len=P + gen, prefix_len=P,
                    active_idx=np.arange(P, P + gen, dtype=np.int32)[None], kind=W.MASK_FULL,
                    cs_lo=P, cs_hi=P + gen, seed=seed)
    p = W.make_post("small_long", R=gen, V=20000, logit_std=3.0, noise_std=0.1, eps=1e-3,
                    mode=W.SEL_TOPK_SCORE, k=16, group_rows=gen, score_cols=(0, P), seed=seed)
    return W.Workload(a, p, "small long prefix (key splits)")


def full_check(w, check_cache=True):
    """Everything against the oracle, margin and entropy included (the
    score-tracking variant of the posterior stream)."""
    _say(f"case: {w.attn.name} / {w.post.name}")
    ora = oracle.step(w)
    ds = _device_step(w, with_scores=True)
    ds.run()
    g = ds.results()
    if check_cache:
        assert np.array_equal(g["cache_k"], ora["cache_k"]), "cache K after scatter differs"
        assert np.array_equal(g["cache_v"], ora["cache_v"]), "cache V after scatter differs"
    check_attention(g["out"], g["lse"], ora["out"], ora["lse"])
    check_colsum(g["colsum"], ora["colsum"])
    p = w.post
    lk_exc = check_posterior(g["kl"], g["conf"], g["locked"], ora["kl"], ora["conf"], ora["locked"],
                             p.eps, p.locked)
    check_scores(g["margin"], g["entropy"], ora["margin"], ora["entropy"], p.locked)
    sel_exc = check_selection(g["sel"], ora["sel"], p.mode, p.group_rows, p.tau, ora["conf"],
                              ora["score"], p.locked, p.logits, ora["margin"], ora["entropy"])
    _say(f"  excused: locks {lk_exc}, selections {sel_exc}")
    return ds, g, ora


def test_tiny():
    full_check(W.tiny())


@pytest.mark.parametrize("spread", [False, True])
def test_small_llada(spread):
    full_check(small_llada(spread))


@pytest.mark.parametrize("variant", ["group", "dummy", "block_causal", "two_groups"])
def test_small_mbd(variant):
    full_check(small_mbd(variant))


def test_small_mbd_per_head_colsum_scalar_vocab():
    full_check(small_mbd("two_groups", per_head=1, V=4099))


def test_small_surelock():
    full_check(small_surelock())


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 4, 2), (32, 6, 3), (128, 8, 1)])
def test_head_dims_and_gqa(D, Hq, Hkv):
    full_check(small_surelock(D=D, Hq=Hq, Hkv=Hkv))


def test_small_long_prefix_key_splits():
    full_check(small_long())


@pytest.mark.parametrize("kgroups", ["1", "2"])
@pytest.mark.parametrize("case", ["mbd_dummy", "surelock_d64_gqa", "surelock_d32_gqa", "long_splits",
                                  "llada_spread"])
def test_both_pass1_workgroup_shapes(kgroups, case, monkeypatch):
    """Pass 1 has two workgroup shapes (one key group of 4 waves with 64-key
    tiles, two key groups of 4 waves with 128-key tiles merged through LDS);
    the plan picks one by problem size.  Force each on the same cases."""
    monkeypatch.setenv("DLM_ATTN_KGROUPS", kgroups)
    w = {"mbd_dummy": lambda: small_mbd("dummy"),
         "surelock_d64_gqa": lambda: small_surelock(D=64, Hq=4, Hkv=2),
         "surelock_d32_gqa": lambda: small_surelock(D=32, Hq=6, Hkv=3),
         "long_splits": lambda: small_long(seed=2),
         "llada_spread": lambda: small_llada(spread=True, seed=3)}[case]()
    _say(f"DLM_ATTN_KGROUPS={kgroups}")
    full_check(w)


def mask_tiles_case(name, seed=0):
    """Shapes whose key tiles fall in each of the three mask classes:
    hidden from every row of a workgroup (skipped), visible to all of them
    (no predicate), partial.  Hidden cache rows hold large-variance garbage,
    so reading one into a sum would show."""
    B, Hq, Hkv, D = 2, 4, 2, 64
    garbage = None
    if name == "bc_early":
        # block-causal, rows in blocks 0-1 only: blocks 2-9 are hidden from every row
        P, bs, n_slots = 100, 32, 10
        act = np.tile(np.arange(P, P + 2 * bs, dtype=np.int32), (B, 1))
        state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
        group = np.zeros((B, n_slots), np.int32)
        kind = W.MASK_BLOCK_CAUSAL
        garbage = np.zeros((B, P + n_slots * bs), bool)
        garbage[:, P + 2 * bs:] = True
    elif name == "group_split":
        # groups 0,0,1,1,2,2,2,2; rows in slots 0-2, slot 3 committed: group 2 is hidden
        P, bs, n_slots = 64, 32, 8
        act = np.tile(np.arange(P, P + 3 * bs, dtype=np.int32), (B, 1))
        state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
        state[:, 3] = W.SLOT_IN_CACHE
        group = np.tile(np.array([0, 0, 1, 1, 2, 2, 2, 2], np.int32), (B, 1))
        kind = W.MASK_GROUP
        garbage = np.zeros((B, P + n_slots * bs), bool)
        garbage[:, P + 4 * bs:] = True
    elif name == "bc_odd":
        # block-causal with 37-position blocks after a 45-position prefix: block
        # boundaries fall inside key tiles at every offset
        P, bs, n_slots = 45, 37, 9
        act = np.tile(np.arange(P + 20, P + 20 + 5 * bs, dtype=np.int32), (B, 1))
        state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
        group = np.zeros((B, n_slots), np.int32)
        kind = W.MASK_BLOCK_CAUSAL
    elif name == "group_odd":
        # 23-position slots, groups 0,0,1,1,1,2,2 and a DUMMY slot: slot boundaries
        # and group changes inside tiles
        P, bs, n_slots = 70, 23, 8
        act = np.tile(np.arange(P, P + 6 * bs, dtype=np.int32), (B, 1))
        state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
        state[:, 7] = W.SLOT_DUMMY
        group = np.tile(np.array([0, 0, 1, 1, 1, 2, 2, 3], np.int32), (B, 1))
        kind = W.MASK_GROUP
        garbage = np.zeros((B, P + n_slots * bs), bool)
        garbage[:, P + 7 * bs:] = True
    elif name == "group_one_block":
        # one 256-position block, every position a row: every tile visible to all
        B, Hq, Hkv, D = 1, 4, 4, 128
        P, bs, n_slots = 0, 256, 1
        act = np.arange(bs, dtype=np.int32)[None]
        state = np.full((B, n_slots), W.SLOT_ACTIVE, np.uint8)
        group = np.zeros((B, n_slots), np.int32)
        kind = W.MASK_GROUP
    else:
        raise KeyError(name)
    kv_len = P + n_slots * bs
    M = act.shape[1]
    a = W.make_attn("mask_tiles_" + name, B=B, Hq=Hq, Hkv=Hkv, D=D, kv_len=kv_len, prefix_len=P,
                    active_idx=act, kind=kind, block_size=bs, n_slots=n_slots, slot_state=state,
                    slot_group=group, cs_lo=0, cs_hi=kv_len, garbage_rows=garbage, seed=seed)
    p = W.make_post(a.name, R=B * M, V=4096, logit_std=3.0, noise_std=0.1, eps=1e-3,
                    mode=W.SEL_TOPK_CONF, k=4, group_rows=32, seed=seed)
    return W.Workload(a, p, "mask tiles " + name)


@pytest.mark.parametrize("kgroups", ["1", "2"])
@pytest.mark.parametrize("case", ["bc_early", "group_split", "group_one_block", "bc_odd", "group_odd"])
def test_mask_tile_classes(kgroups, case, monkeypatch):
    """Tiles hidden from a whole workgroup are skipped, tiles visible to all
    its rows run without the predicate, the rest run it: all three against
    the oracle, with both pass-1 workgroup shapes.  Hidden columns get
    exactly zero column sums."""
    monkeypatch.setenv("DLM_ATTN_KGROUPS", kgroups)
    _say(f"DLM_ATTN_KGROUPS={kgroups}")
    w = mask_tiles_case(case)
    _, g, ora = full_check(w)
    if case != "group_one_block":
        a = w.attn
        first_block = {"bc_early": 2, "group_split": 4, "bc_odd": 6, "group_odd": 7}[case]
        first_hidden = a.prefix_len + first_block * a.block_size
        assert np.all(g["colsum"][:, first_hidden:] == 0)
        assert np.all(ora["colsum"][:, first_hidden:] == 0)


@pytest.mark.parametrize("mode", [True, "pass1"])
@pytest.mark.parametrize("case", ["llada_dynamic", "long_topk_score", "mbd_topk_conf"])
def test_overlapped_step_equals_serial(case, mode, monkeypatch):
    """The overlapped schedules (posterior on a second stream from the start
    of the step, or from mask_desc.pass1_done; its selection waiting for
    the column sums through select.score_ready) give the same bits as the
    serial step on the same (two-launch) posterior kernels, for both
    selection modes that read the score.  Against the serial step's
    one-launch posterior, which merges the vocabulary chunks in another
    fp32 order, the attention outputs are the same bits and the posterior
    differs by rounding only.  A selection that does not rank by the column
    sums does not wait for them and keeps the serial step's posterior
    kernels: every output is the same bits."""
    w = (small_llada(spread=True, seed=4) if case == "llada_dynamic" else
         small_long(seed=5) if case == "long_topk_score" else small_mbd(seed=6))
    by_score = w.post.mode in (W.SEL_ATTN_DYNAMIC, W.SEL_TOPK_SCORE)
    _say(f"case: overlap {case} ({mode})")
    ds = _device_step(w)
    ds.run()
    r1 = ds.results()
    monkeypatch.setenv("DLM_POST_FUSED", "0")
    ds.reset()
    ds.run()
    r0 = ds.results()
    monkeypatch.delenv("DLM_POST_FUSED")
    for rep in range(3):
        ds.reset()
        ds.colsum.fill_(float("nan"))      # a read before the sums are ready would show
        ds.run(overlap=mode)
        r2 = ds.results()
        for k in ("out", "lse", "colsum", "kl", "conf", "sel", "locked", "cache_k", "cache_v"):
            assert np.array_equal((r0 if by_score else r1)[k], r2[k], equal_nan=False), (rep, k)
        for k in ("out", "lse", "colsum", "cache_k", "cache_v"):
            assert np.array_equal(r1[k], r2[k], equal_nan=False), (rep, k)
        assert np.abs(r1["kl"].astype(np.float64) - r2["kl"]).max() <= 2e-6
        assert np.abs(r1["conf"].astype(np.float64) - r2["conf"]).max() <= 1e-6
        near = np.abs(r2["kl"].astype(np.float64) - w.post.eps) <= 1e-5   # a lock decided by rounding
        assert np.array_equal(r1["locked"][~near], r2["locked"][~near])
        # a selection decided by rounding: a confidence within 1e-6 of tau
        edge = np.abs(r2["conf"].astype(np.float64) - w.post.tau) <= 1e-6
        assert np.array_equal(r1["sel"], r2["sel"]) or edge.any()


def test_posterior_stream_variants_agree():
    """The stream kernel without margin / entropy tracking gives the same
    KL, confidence, tokens, locks and selection, bit for bit."""
    w = small_llada(spread=True, seed=8)
    _say("case: posterior variants")
    r = []
    for scores in (True, False):
        ds = _device_step(w, with_scores=scores)
        ds.run()
        r.append(ds.results())
    for k in ("kl", "conf", "sel", "locked"):
        assert np.array_equal(r[0][k], r[1][k]), k


def test_deterministic():
    w = small_long(seed=1)
    ds = _device_step(w)
    ds.run()
    r1 = ds.results()
    ds.reset()
    ds.run()
    r2 = ds.results()
    for k in ("out", "lse", "colsum", "kl", "conf", "sel", "locked"):
        assert np.array_equal(r1[k], r2[k]), k


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

def test_single_active_row_short_cache():
    a = W.make_attn("one_row", B=1, Hq=2, Hkv=1, D=128, kv_len=37, prefix_len=5,
                    active_idx=np.array([[20]], np.int32), kind=W.MASK_FULL, cs_lo=0, cs_hi=37)
    p = W.make_post("one_row", R=1, V=3, logit_std=1.0, noise_std=0.1, eps=1e-3,
                    mode=W.SEL_THRESH_CONF, tau=0.99, group_rows=1)
    full_check(W.Workload(a, p, "one row"))


def test_row_without_visible_key():
    """GROUP, no prefix: a query in a DUMMY slot of group 0 sees nothing
    (its own slot is dummy, the other slot is in a later group)."""
    bs = 16
    act = np.array([list(range(0, 8)) + list(range(bs, bs + 8))], np.int32)
    a = W.make_attn("no_key", B=1, Hq=2, Hkv=2, D=64, kv_len=2 * bs, prefix_len=0,
                    active_idx=act, kind=W.MASK_GROUP, block_size=bs, n_slots=2,
                    slot_state=np.array([[W.SLOT_DUMMY, W.SLOT_ACTIVE]], np.uint8),
                    slot_group=np.array([[0, 1]], np.int32), cs_lo=0, cs_hi=2 * bs)
    p = W.make_post("no_key", R=16, V=64, logit_std=2.0, noise_std=0.05, eps=1e-3,
                    mode=W.SEL_TOPK_CONF, k=3, group_rows=5)
    _, g, ora = full_check(W.Workload(a, p, "rows without keys"), check_cache=True)
    assert np.isneginf(ora["lse"][0, :, :8]).all()
    assert np.all(g["out"][0, :, :8] == 0)


def test_zero_active_rows():
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    B, Hkv, N, D = 2, 2, 100, 64
    ck = torch.zeros((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    cv = torch.zeros_like(ck)
    kv = dlm.KVCache(ck, cv)
    md = dlm.MaskDesc(kind=dlm.MASK_FULL, Hq=4, M=0, kv_len=N, cs_lo=0, cs_hi=N)
    md.workspace = torch.empty(max(1, dlm.dlm_step_attn_workspace_bytes(kv, md)), dtype=torch.uint8, device=dev)
    colsum = torch.full((B, N), 7.0, device=dev)
    empty_q = torch.empty((B, 4, 0, D), dtype=torch.bfloat16, device=dev)
    dlm.dlm_step_attn(empty_q, None, None, kv, torch.empty((B, 0), dtype=torch.int32, device=dev), md,
                      torch.empty((B, 4, 0, D), dtype=torch.bfloat16, device=dev),
                      torch.empty((B, 4, 0), dtype=torch.float32, device=dev), colsum)
    torch.cuda.synchronize()
    assert torch.all(colsum == 0)


def test_posterior_edge_cases():
    """Ragged last group, arrived-locked rows holding NaN (never read), argmax
    ties, every selection mode, a vocabulary that is not a multiple of 4."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(21)
    R, V = 37, 1003
    x = (rng.standard_normal((R, V)) * 2).astype(np.float32)
    x[3, [10, 500]] = 9.0          # tie for the argmax: lowest index wins
    y = (x + rng.standard_normal((R, V)) * np.where(rng.random(R) < 0.5, 0.01, 0.2)[:, None]).astype(np.float32)
    y[5] = x[5]                    # KL exactly 0
    locked = (rng.random(R) < 0.2).astype(np.uint8)
    x[locked == 1] = np.nan        # a locked row is never read
    y[locked == 1] = np.nan
    score = rng.random(R).astype(np.float32)
    ora = oracle.posterior(x, y, locked, 1e-3)
    for mode, k, tau, g in [(W.SEL_TOPK_CONF, 3, 0.0, 8), (W.SEL_THRESH_CONF, 0, 0.05, 6),
                            (W.SEL_ATTN_DYNAMIC, 0, 0.05, 10), (W.SEL_TOPK_SCORE, 4, 0.0, 37),
                            (W.SEL_NONE, 0, 0.0, 1)]:
        _say(f"case: posterior edges mode={mode}")
        s = dlm.Select(mode=mode, k=k, group_rows=g, tau=tau,
                       score=torch.from_numpy(score).to(dev))
        s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8, device=dev)
        lk = torch.from_numpy(locked.copy()).to(dev)
        sel = torch.empty(R, dtype=torch.int32, device=dev)
        kl = torch.empty(R, dtype=torch.float32, device=dev)
        conf = torch.empty(R, dtype=torch.float32, device=dev)
        dlm.dlm_posterior(torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev), lk, 1e-3, s,
                          sel, kl, conf, R, V)
        torch.cuda.synchronize()
        check_posterior(kl.cpu().numpy(), conf.cpu().numpy(), lk.cpu().numpy(), ora["kl"], ora["conf"],
                        ora["locked"], 1e-3, locked)
        sel_o = oracle.select(mode, k, g, tau, score.astype(np.float64), ora["conf"], ora["tok"], locked)
        check_selection(sel.cpu().numpy(), sel_o, mode, g, tau, ora["conf"], score.astype(np.float64),
                        locked, np.nan_to_num(x))
        assert kl.cpu().numpy()[5] == 0.0 or abs(kl.cpu().numpy()[5]) < 1e-6
        assert np.all(sel.cpu().numpy()[locked == 1] == -1)


def test_single_launch_posterior_shares_one_workspace(monkeypatch):
    """The one-launch posterior (arrival counters in the workspace, the last
    chunk of a row merges it, the last row of a group selects; taken when
    its grid is one round of workgroups) on a sequence of calls of
    different shapes and both paths sharing one workspace that was zeroed
    once: every call against the oracle, the counter block zero after every
    call, a repeated call bitwise equal, and the two-launch path (a
    score_ready event; DLM_POST_FUSED=0) on the same inputs also within the
    parity bounds of the oracle."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(77)
    cases = [
        # R, V, mode, k, tau, group, margin/entropy, flags
        (1, 151936, W.SEL_TOPK_CONF, 1, 0.0, 1, False, False),       # 38 chunks in one row
        (120, 40000, W.SEL_TOPK_MARGIN, 3, 0.0, 7, True, True),      # ragged groups, margin path
        (1600, 8192, W.SEL_TOPK_CONF, 4, 0.0, 32, False, False),     # 1600 whole rows, past one round: two launches
        (64, 1003, W.SEL_THRESH_CONF, 0, 0.05, 64, False, False),    # V not a multiple of 4
        (300, 9000, W.SEL_NONE, 0, 0.0, 1, False, True),             # no selection, 3 chunks
        (256, 70000, W.SEL_TOPK_SCORE, 16, 0.0, 256, False, False),  # one 256-row group
        (96, 20000, W.SEL_ATTN_DYNAMIC, 0, 0.3, 32, True, False),
        (8, 9001, W.SEL_TOPK_CONF, 2, 0.0, 4, True, False),          # V % 4 != 0 with 3 chunks a row
        (5, 1, W.SEL_TOPK_CONF, 2, 0.0, 5, False, False),            # V = 1
        (50, 8192, W.SEL_TOPK_LOW_ENTROPY, 2, 0.0, 10, True, False),  # every row locked below
    ]
    need = 0
    for R, V, mode, k, tau, g, sc, fl in cases:
        need = max(need, dlm.dlm_posterior_workspace_bytes(R, V, dlm.Select(mode=mode, k=k, group_rows=g)))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    ctr = 2 * 4096 * 4
    for ci, (R, V, mode, k, tau, g, sc, fl) in enumerate(cases):
        x = (rng.standard_normal((R, V)) * rng.uniform(0.5, 4.0, R)[:, None]).astype(np.float32)
        y = (x + rng.standard_normal((R, V)) * np.where(rng.random(R) < 0.4, 0.005, 0.1)[:, None]).astype(np.float32)
        locked = np.ones(R, np.uint8) if ci == len(cases) - 1 else (rng.random(R) < 0.2).astype(np.uint8)
        flags = np.where(rng.random(R) < 0.15, 2, 3).astype(np.uint8) if fl else None
        score = rng.random(R).astype(np.float32)
        ora = oracle.posterior(x, y, locked, 1e-3, flags=flags)
        sel_o = oracle.select(mode, k, g, tau, score.astype(np.float64), ora["conf"], ora["tok"], locked,
                              ora["margin"], ora["entropy"], flags=flags)
        inelig = locked if flags is None else ((locked != 0) | ((flags & 1) == 0)).astype(np.uint8)
        xd, yd, sd = (torch.from_numpy(a).to(dev) for a in (x, y, score))
        fd = torch.from_numpy(flags).to(dev) if fl else None
        runs = []
        for path in ("fused", "fused", "event", "env"):
            _say(f"case: one-launch posterior R={R} V={V} mode={mode} group={g} path={path}")
            if path == "env":
                monkeypatch.setenv("DLM_POST_FUSED", "0")
            mg = torch.empty(R, device=dev) if sc else None
            en = torch.empty(R, device=dev) if sc else None
            s = dlm.Select(mode=mode, k=k, group_rows=g, tau=tau, score=sd, margin=mg, entropy=en, row_flags=fd)
            s.workspace = ws
            if path == "event":
                ev = torch.cuda.Event()
                ev.record()
                s.score_ready = ev
            lk = torch.from_numpy(locked.copy()).to(dev)
            sel = torch.empty(R, dtype=torch.int32, device=dev)
            kl = torch.empty(R, dtype=torch.float32, device=dev)
            conf = torch.empty(R, dtype=torch.float32, device=dev)
            dlm.dlm_posterior(xd, yd, lk, 1e-3, s, sel, kl, conf, R, V)
            torch.cuda.synchronize()
            monkeypatch.delenv("DLM_POST_FUSED", raising=False)
            assert int(ws[:ctr].count_nonzero()) == 0, f"counters not left at zero after {path}"
            r = dict(kl=kl.cpu().numpy(), conf=conf.cpu().numpy(), sel=sel.cpu().numpy(), locked=lk.cpu().numpy())
            check_posterior(r["kl"], r["conf"], r["locked"], ora["kl"], ora["conf"], ora["locked"], 1e-3, locked)
            check_selection(r["sel"], sel_o, mode, g, tau, ora["conf"], score.astype(np.float64), inelig, x,
                            ora["margin"], ora["entropy"])
            if sc:
                check_scores(mg.cpu().numpy(), en.cpu().numpy(), ora["margin"], ora["entropy"], locked)
            runs.append(r)
        for key in ("kl", "conf", "sel", "locked"):
            assert np.array_equal(runs[0][key], runs[1][key]), key   # deterministic
            assert np.array_equal(runs[2][key], runs[3][key]), key   # the two-launch path, either way
        if ci == len(cases) - 1:
            assert np.all(runs[0]["sel"] == -1) and np.all(runs[0]["kl"] == 0)


def test_single_launch_posterior_graph_replays():
    """The one-launch posterior captured in a HIP graph: its arrival counters
    reset themselves (no memset node), so every replay, with eager work and
    synchronisations between replays, gives the eager call's bits."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(91)
    R, V, g = 64, 20000, 16
    x = torch.from_numpy((rng.standard_normal((R, V)) * 3).astype(np.float32)).to(dev)
    y = (x + torch.from_numpy((rng.standard_normal((R, V)) * 0.02).astype(np.float32)).to(dev)).contiguous()
    locked0 = torch.from_numpy((rng.random(R) < 0.2).astype(np.uint8)).to(dev)
    s = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=3, group_rows=g)
    s.workspace = torch.zeros(dlm.dlm_posterior_workspace_bytes(R, V, s), dtype=torch.uint8, device=dev)
    lk = locked0.clone()
    sel = torch.empty(R, dtype=torch.int32, device=dev)
    kl = torch.empty(R, dtype=torch.float32, device=dev)
    conf = torch.empty(R, dtype=torch.float32, device=dev)
    _say("case: one-launch posterior, eager")
    dlm.dlm_posterior(x, y, lk, 1e-3, s, sel, kl, conf, R, V)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (sel, kl, conf, lk)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    lk.copy_(locked0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        dlm.dlm_posterior(x, y, lk, 1e-3, s, sel, kl, conf, R, V)
    torch.cuda.synchronize()
    for rep in range(4):
        _say(f"case: one-launch posterior, graph replay {rep}")
        lk.copy_(locked0)
        sel.fill_(-7)
        kl.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((sel, kl, conf, lk), ref, ("sel", "kl", "conf", "locked")):
            assert torch.equal(got, want), (rep, name)
        assert int(s.workspace[:2 * 4096 * 4].count_nonzero()) == 0
        _ = (x[:4] * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("g,V", [(200, 600), (257, 600), (700, 600), (1024, 600), (129, 33000), (300, 40000)])
def test_large_selection_groups(g, V):
    """Groups of more than 256 rows pick by radix selection of the k-th
    largest packed key (up to 1024 rows), smaller ones by counting: every
    ranking mode on both sides of the boundary, a ragged last group, locked
    rows and rows that may not be selected.  With the larger vocabularies
    each row is also split into vocabulary chunks, so the finishing kernel
    merges several partials per row before it selects: through LDS for the
    129-row groups, straight from global memory for the 300-row ones."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(60 + g)
    R = 2 * g + 77
    x = (rng.standard_normal((R, V)) * rng.uniform(0.5, 4.0, R)[:, None]).astype(np.float32)
    y = (x + rng.standard_normal((R, V)) * 0.1).astype(np.float32)
    locked = (rng.random(R) < 0.2).astype(np.uint8)
    flags = np.where(rng.random(R) < 0.1, 2, 3).astype(np.uint8)
    score = rng.random(R).astype(np.float32)
    ora = oracle.posterior(x, y, locked, 1e-3, flags=flags)
    for mode, k, tau in [(W.SEL_TOPK_CONF, 37, 0.0), (W.SEL_TOPK_SCORE, g // 3, 0.0),
                         (W.SEL_TOPK_MARGIN, 5, 0.0), (W.SEL_TOPK_LOW_ENTROPY, 1, 0.0),
                         (W.SEL_THRESH_CONF, 0, 0.999), (W.SEL_ATTN_DYNAMIC, 0, 0.3)]:
        _say(f"case: large groups g={g} mode={mode}")
        mg = torch.empty(R, device=dev)
        en = torch.empty(R, device=dev)
        s = dlm.Select(mode=mode, k=k, group_rows=g, tau=tau, score=torch.from_numpy(score).to(dev),
                       margin=mg, entropy=en, row_flags=torch.from_numpy(flags).to(dev))
        s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8,
                                  device=dev)
        lk = torch.from_numpy(locked.copy()).to(dev)
        sel = torch.empty(R, dtype=torch.int32, device=dev)
        kl = torch.empty(R, dtype=torch.float32, device=dev)
        conf = torch.empty(R, dtype=torch.float32, device=dev)
        dlm.dlm_posterior(torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev), lk, 1e-3, s,
                          sel, kl, conf, R, V)
        torch.cuda.synchronize()
        check_posterior(kl.cpu().numpy(), conf.cpu().numpy(), lk.cpu().numpy(), ora["kl"], ora["conf"],
                        ora["locked"], 1e-3, locked)
        sel_o = oracle.select(mode, k, g, tau, score.astype(np.float64), ora["conf"], ora["tok"], locked,
                              ora["margin"], ora["entropy"], flags=flags)
        inelig = ((locked != 0) | ((flags & 1) == 0)).astype(np.uint8)
        check_selection(sel.cpu().numpy(), sel_o, mode, g, tau, ora["conf"], score.astype(np.float64),
                        inelig, x, ora["margin"], ora["entropy"])
        assert (sel_o >= 0).sum() > 0


@pytest.mark.parametrize("g,V,n_live", [(100, 40000, 30), (100, 600, 150), (700, 40000, 9), (700, 40000, 1200),
                                         (1024, 40000, 0), (1024, 126464, 16)])
def test_live_row_list(g, V, n_live):
    """A live-row list (dlm_select.live_rows / n_live / live_offset): only the
    listed rows are streamed, with the vocabulary split chosen on the device
    from the count (more chunks for fewer rows), and the finishing kernel
    merging with that same split.  Every unlisted row arrives locked; listed
    rows may arrive locked too; entries outside [0, R) (after the offset)
    and entries past the count are ignored.  Checked against the oracle on
    every row, for a staged (100-row) and a global-memory (700, 1024-row)
    merge, with no live row and with more entries than rows, under every
    selection mode (groups with at most 256 live rows rank those alone, a
    k past the live count included)."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(90 + g + n_live)
    R = 2 * g + 77 if g < 1024 else 1024
    x = (rng.standard_normal((R, V)) * rng.uniform(0.5, 4.0, R)[:, None]).astype(np.float32)
    y = (x + rng.standard_normal((R, V)) * 0.1).astype(np.float32)
    live = np.sort(rng.choice(R, size=min(n_live, R), replace=False)).astype(np.int32)
    locked = np.ones(R, np.uint8)
    locked[live] = (rng.random(len(live)) < 0.2).astype(np.uint8)    # a listed row may arrive locked
    flags = np.where(rng.random(R) < 0.1, 2, 3).astype(np.uint8)
    off = 100
    entries = list(live + off)
    if n_live >= 9:
        entries[3:3] = [-5, R + off + 7]            # outside [0, R) after the offset: ignored
    count = min(len(entries), R)
    lst = np.full(R, -1, np.int32)
    lst[:count] = np.array(entries[:count], np.int32)
    # rows that the count cuts off must arrive locked (the list's contract)
    kept = lst[:count] - off
    kept = kept[(kept >= 0) & (kept < R)]
    locked[np.setdiff1d(np.arange(R), kept)] = 1
    score = rng.random(R).astype(np.float32)
    ora = oracle.posterior(x, y, locked, 1e-3, flags=flags)
    for mode, k, tau in [(W.SEL_TOPK_CONF, 7, 0.0), (W.SEL_THRESH_CONF, 0, 0.99),
                         (W.SEL_TOPK_SCORE, 5, 0.0), (W.SEL_TOPK_MARGIN, 3, 0.0),
                         (W.SEL_TOPK_LOW_ENTROPY, 1, 0.0), (W.SEL_ATTN_DYNAMIC, 0, 0.3),
                         (W.SEL_TOPK_CONF, 300, 0.0)]:
        _say(f"case: live rows g={g} V={V} n_live={n_live} mode={mode} k={k}")
        mg = torch.empty(R, device=dev)
        en = torch.empty(R, device=dev)
        s = dlm.Select(mode=mode, k=k, group_rows=g, tau=tau, margin=mg, entropy=en,
                       score=torch.from_numpy(score).to(dev),
                       row_flags=torch.from_numpy(flags).to(dev),
                       live_rows=torch.from_numpy(lst).to(dev),
                       n_live=torch.tensor([count], dtype=torch.int32, device=dev), live_offset=off)
        s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8,
                                  device=dev)
        lk = torch.from_numpy(locked.copy()).to(dev)
        sel = torch.empty(R, dtype=torch.int32, device=dev)
        kl = torch.empty(R, dtype=torch.float32, device=dev)
        conf = torch.empty(R, dtype=torch.float32, device=dev)
        dlm.dlm_posterior(torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev), lk, 1e-3, s,
                          sel, kl, conf, R, V)
        torch.cuda.synchronize()
        check_posterior(kl.cpu().numpy(), conf.cpu().numpy(), lk.cpu().numpy(), ora["kl"], ora["conf"],
                        ora["locked"], 1e-3, locked)
        sel_o = oracle.select(mode, k, g, tau, score.astype(np.float64), ora["conf"], ora["tok"], locked,
                              ora["margin"], ora["entropy"], flags=flags)
        inelig = ((locked != 0) | ((flags & 1) == 0)).astype(np.uint8)
        check_selection(sel.cpu().numpy(), sel_o, mode, g, tau, ora["conf"], score.astype(np.float64),
                        inelig, x, ora["margin"], ora["entropy"])
        check_scores(mg.cpu().numpy(), en.cpu().numpy(), ora["margin"], ora["entropy"], locked)


@pytest.mark.parametrize("V", [1, 1003, 6000])
def test_margin_entropy_samplers(V):
    """Margin and entropy of p_t and the two token-level samplers that rank
    by them (top-k by largest margin, top-k by lowest entropy), with rows
    whose maximum repeats (margin 0), near-certain rows and locked rows."""
    import denoising_step_amd as dlm
    dev = torch.device("cuda")
    rng = np.random.default_rng(40 + V)
    R = 70
    x = (rng.standard_normal((R, V)) * np.linspace(0.2, 6.0, R)[:, None]).astype(np.float32)
    if V > 3:
        x[5, [3, V - 2]] = x[5].max() + 1.0      # repeated maximum: margin 0
        x[9, 0] = 40.0                            # near-certain row
    y = (x + rng.standard_normal((R, V)) * 0.05).astype(np.float32)
    locked = (rng.random(R) < 0.15).astype(np.uint8)
    x[locked == 1] = np.nan                       # never read
    y[locked == 1] = np.nan
    ora = oracle.posterior(x, y, locked, 1e-3)
    for mode, k, g in [(W.SEL_TOPK_MARGIN, 3, 10), (W.SEL_TOPK_LOW_ENTROPY, 2, 7),
                       (W.SEL_TOPK_MARGIN, 100, 70), (W.SEL_TOPK_LOW_ENTROPY, 1, 1)]:
        _say(f"case: samplers V={V} mode={mode} k={k} group={g}")
        mg = torch.full((R,), float("nan"), device=dev)
        en = torch.full((R,), float("nan"), device=dev)
        s = dlm.Select(mode=mode, k=k, group_rows=g, margin=mg, entropy=en)
        s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8, device=dev)
        lk = torch.from_numpy(locked.copy()).to(dev)
        sel = torch.empty(R, dtype=torch.int32, device=dev)
        kl = torch.empty(R, dtype=torch.float32, device=dev)
        conf = torch.empty(R, dtype=torch.float32, device=dev)
        dlm.dlm_posterior(torch.from_numpy(x).to(dev), torch.from_numpy(y).to(dev), lk, 1e-3, s,
                          sel, kl, conf, R, V)
        torch.cuda.synchronize()
        check_scores(mg.cpu().numpy(), en.cpu().numpy(), ora["margin"], ora["entropy"], locked)
        if V > 3:
            assert mg.cpu().numpy()[5] == 0.0 and ora["margin"][5] == 0.0
        sel_o = oracle.select(mode, k, g, 0.0, None, ora["conf"], ora["tok"], locked,
                              ora["margin"], ora["entropy"])
        exc = check_selection(sel.cpu().numpy(), sel_o, mode, g, 0.0, ora["conf"], None, locked,
                              np.nan_to_num(x), ora["margin"], ora["entropy"])
        _say(f"  excused {exc}")


def test_colsum_accumulates_over_layers():
    """colsum_accumulate = 1 adds a call's column sums to the buffer: three
    layers (different queries over the same cache) against the sum of the
    oracle's per-layer sums; a call with no active rows leaves it as is."""
    import denoising_step_amd as dlm
    base = small_mbd("two_groups", seed=7)
    a = base.attn
    rng = np.random.default_rng(77)
    layers = []
    for l in range(3):
        q = W.to_bf16_bits(rng.standard_normal(a.q.shape) * (0.5 + 0.5 * l))
        layers.append(W.AttnCase(**{**a.__dict__, "q": q}))
    want = sum(oracle.colsum(c, oracle.attention(c)[1]) for c in layers)
    ds = _device_step(W.Workload(layers[0], base.post, "layer 0"), with_posterior=False)
    for l, c in enumerate(layers):
        _say(f"case: accumulate layer {l}")
        from denoising_step_amd.runner import bf16_to_device
        ds.q = bf16_to_device(c.q, torch.device("cuda"))
        ds.md.colsum_accumulate = 0 if l == 0 else 1
        ds.run_attn()
    torch.cuda.synchronize()
    check_colsum(ds.colsum.cpu().numpy(), want)
    before = ds.colsum.clone()
    md0 = dlm.MaskDesc(kind=a.kind, Hq=a.Hq, M=0, kv_len=a.kv_len, prefix_len=a.prefix_len,
                       block_size=a.block_size, n_slots=a.n_slots, slot_state=ds.md.slot_state,
                       slot_group=ds.md.slot_group, cs_lo=a.cs_lo, cs_hi=a.cs_hi, colsum_accumulate=1)
    md0.workspace = torch.empty(max(1, dlm.dlm_step_attn_workspace_bytes(ds.kv, md0)), dtype=torch.uint8,
                                device="cuda")
    D = a.D
    dlm.dlm_step_attn(torch.empty((a.B, a.Hq, 0, D), dtype=torch.bfloat16, device="cuda"), None, None, ds.kv,
                      torch.empty((a.B, 0), dtype=torch.int32, device="cuda"), md0,
                      torch.empty((a.B, a.Hq, 0, D), dtype=torch.bfloat16, device="cuda"),
                      torch.empty((a.B, a.Hq, 0), dtype=torch.float32, device="cuda"), ds.colsum)
    torch.cuda.synchronize()
    assert torch.equal(ds.colsum, before)


# --------------------------------------------------------------------------
# full workloads: sampled outputs and invariants
# --------------------------------------------------------------------------

def _sub_batch(case, b):
    return W.AttnCase(**{**case.__dict__, "B": 1, "q": case.q[b:b + 1], "k": case.k[b:b + 1],
                         "v": case.v[b:b + 1], "cache_k": case.cache_k[b:b + 1],
                         "cache_v": case.cache_v[b:b + 1], "active_idx": case.active_idx[b:b + 1],
                         "slot_state": case.slot_state[b:b + 1], "slot_group": case.slot_group[b:b + 1]})


def _check_attn_sampled(a, g, n_rows=1024, colsum_batch=0, extra_cols=None, seed=0):
    """Sampled out/lse rows for the whole batch; every row's lse and sampled
    columns of one batch entry; the column-total invariant for every entry."""
    rng = np.random.default_rng(seed)
    kv = oracle.effective_kv(a)
    assert np.array_equal(g["cache_k"], kv[0]) and np.array_equal(g["cache_v"], kv[1])
    rows = np.sort(rng.choice(a.B * a.Hq * a.M, size=min(n_rows, a.B * a.Hq * a.M), replace=False))
    out_o, lse_o = oracle.attention(a, kv=kv, rows=rows)
    out_g = g["out"].reshape(-1, a.D)[rows]
    lse_g = g["lse"].reshape(-1)[rows]
    check_attention(out_g, lse_g, out_o, lse_o)
    # one batch entry in full for the column sums
    sb = _sub_batch(a, colsum_batch)
    kvb = (kv[0][colsum_batch:colsum_batch + 1], kv[1][colsum_batch:colsum_batch + 1])
    _, lse_b = oracle.attention(sb, kv=kvb, want_out=False)
    check_attention(np.zeros((1, 1), np.uint16), g["lse"][colsum_batch].reshape(-1),
                    np.zeros((1, 1)), lse_b.reshape(-1))
    cols = rng.choice(a.kv_len, size=min(256, a.kv_len), replace=False)
    if extra_cols is not None:
        cols = np.union1d(cols, extra_cols)
    cs_o = oracle.colsum(sb, lse_b, kv=kvb, cols=cols)
    cs_g = g["colsum"][colsum_batch][cols] if not a.colsum_per_head else g["colsum"][colsum_batch][:, cols].T
    check_colsum(cs_g, cs_o)
    # invariant: each counted row's weights sum to 1
    counted = ((a.active_idx >= a.cs_lo) & (a.active_idx < a.cs_hi)).sum(axis=1)
    tot = g["colsum"].reshape(a.B, -1).astype(np.float64).sum(axis=1)
    assert np.allclose(tot, a.Hq * counted, rtol=1e-4), (tot, a.Hq * counted)
    return cs_o, cols


def test_full_llada_bidirectional():
    full_check(W.llada_bidirectional())


def test_full_llada_bidirectional_spread():
    full_check(W.llada_bidirectional(spread=True))


def test_full_llada_group():
    """The same layer under a one-block GROUP mask: every tile classified
    visible, the results those of the FULL mask's path."""
    full_check(W.llada_group())


@pytest.mark.parametrize("variant", ["group", "dummy", "block_causal", "two_groups"])
def test_full_mbd_multiblock(variant):
    w = W.mbd_multiblock(variant=variant)
    _say(f"case: {w.attn.name} (sampled)")
    with_post = variant == "group"
    ds = _device_step(w, with_posterior=with_post)
    ds.run()
    g = ds.results()
    a = w.attn
    _check_attn_sampled(a, g, extra_cols=np.arange(a.prefix_len - 64, a.kv_len))
    if with_post:
        # every row and every selection group of the posterior
        p = w.post
        ora = oracle.posterior(p.logits, p.prev, p.locked, p.eps)
        check_posterior(g["kl"], g["conf"], g["locked"], ora["kl"], ora["conf"], ora["locked"], p.eps,
                        p.locked)
        sel_o = oracle.select(p.mode, p.k, p.group_rows, p.tau, None, ora["conf"], ora["tok"], p.locked)
        exc = check_selection(g["sel"], sel_o, p.mode, p.group_rows, p.tau, ora["conf"], None, p.locked,
                              p.logits)
        assert (g["sel"] >= 0).sum() == p.k * (p.R // p.group_rows)
        _say(f"  all {p.R // p.group_rows} groups checked; excused selections: {exc}")


def test_full_surelock_sparse():
    w = W.surelock_sparse()
    _say("case: surelock_sparse (sampled)")
    ds = _device_step(w)
    ds.run()
    g = ds.results()
    _check_attn_sampled(w.attn, g, colsum_batch=1)
    # every row of the posterior: KL, confidence and the lock decision
    p = w.post
    ora = oracle.posterior(p.logits, p.prev, p.locked, p.eps)
    check_posterior(g["kl"], g["conf"], g["locked"], ora["kl"], ora["conf"], ora["locked"], p.eps, p.locked)
    assert np.all(g["sel"] == -1)
    frac = g["locked"].mean()
    _say(f"  locked fraction after the step: {frac:.3f}")
    assert 0.3 < frac < 0.5


def test_full_long_prefix_sampler():
    w = W.long_prefix_sampler()
    _say("case: long_prefix_sampler (sampled, exact top-16)")
    ds = _device_step(w)
    ds.run()
    g = ds.results()
    a, p = w.attn, w.post
    gen_cols = np.arange(a.prefix_len, a.kv_len)
    cs_o, cols = _check_attn_sampled(a, g, extra_cols=gen_cols)
    score_o = cs_o[np.searchsorted(cols, gen_cols)]
    ora = oracle.posterior(p.logits, p.prev, p.locked, p.eps)
    check_posterior(g["kl"], g["conf"], g["locked"], ora["kl"], ora["conf"], ora["locked"], p.eps, p.locked)
    sel_o = oracle.select(p.mode, p.k, p.group_rows, p.tau, score_o, ora["conf"], ora["tok"], p.locked)
    exc = check_selection(g["sel"], sel_o, p.mode, p.group_rows, p.tau, ora["conf"], score_o, p.locked,
                          p.logits)
    assert (g["sel"] >= 0).sum() == 16
    _say(f"  excused selections: {exc}")


def test_validate_env_rejects_bad_contents(monkeypatch):
    """DLM_VALIDATE=1 checks device-array contents on a host copy and
    returns DLM_E_DESC before any launch."""
    import denoising_step_amd as dlm
    w = small_mbd("group")
    ds = _device_step(w, with_posterior=False)
    monkeypatch.setenv("DLM_VALIDATE", "1")
    ds.run_attn()                                   # valid contents pass
    torch.cuda.synchronize()
    good = ds.active_idx.clone()
    for mutate in ("duplicate", "past_kv_len", "in_prefix"):
        bad = good.clone()
        if mutate == "duplicate":
            bad[1, 7] = bad[1, 6]
        elif mutate == "past_kv_len":
            bad[0, -1] = w.attn.kv_len
        else:
            bad[0, 0] = w.attn.prefix_len - 1
        with pytest.raises(dlm.DlmError) as e:
            dlm.dlm_step_attn(ds.q, ds.k, ds.v, ds.kv, bad, ds.md, ds.out, ds.lse, ds.colsum)
        assert e.value.code == dlm.DLM_E_DESC, mutate
    bad_state = ds.md.slot_state.clone()
    bad_state[0, 0] = 7
    md = dlm.MaskDesc(**{**ds.md.__dict__, "slot_state": bad_state})
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_step_attn(ds.q, ds.k, ds.v, ds.kv, good, md, ds.out, ds.lse, ds.colsum)
    assert e.value.code == dlm.DLM_E_DESC
