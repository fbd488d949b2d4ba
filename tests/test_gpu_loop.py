"""GPU parity of the multi-step run: the Block Buffer kernel, the device row
count of dlm_step_attn, the per-row select / lock flags of dlm_posterior,
and whole runs against the oracle's loop, eagerly and replayed from one
captured HIP graph.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import block_buffer as obb
from oracle import loop as oloop
from parity import check_attention, check_colsum, check_posterior, check_selection

pytestmark = pytest.mark.gpu

BB_FIELDS = ("slot_state", "slot_group", "decoded", "tokens", "locked", "skip", "row_flags",
             "active_idx", "m_active", "n_open")


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd  # noqa: F401  (raises if the library is not built)
    yield


def _t(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _oracle_arrays(st, der):
    return {"slot_state": st.slot_state, "slot_group": st.slot_group, "decoded": st.decoded,
            "tokens": st.tokens, "locked": st.locked, "skip": der.skip, "row_flags": der.flags,
            "active_idx": der.active_idx, "m_active": der.m_active, "n_open": der.n_open}


# --------------------------------------------------------------------------
# the Block Buffer kernel
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,bs,ma,p_sel", [
    (3, 7, 3, 3, 0.3),       # several slots, small blocks
    (2, 40, 30, 4, 0.4),     # 1200 positions: two compaction rounds
    (1, 3, 700, 2, 0.5),     # 2100 positions, ragged last round
    (1, 1024, 1, 5, 0.9),    # the most slots
    (2, 1, 64, 1, 0.2),      # one block (SureLock shape)
])
def test_block_buffer_kernel_matches_oracle(B, S, bs, ma, p_sel):
    import denoising_step_amd as dlm
    _say(f"block buffer B={B} S={S} bs={bs} max_active={ma}")
    rng = np.random.default_rng(B * 1000 + S)
    n_gen, P = S * bs, 17
    dec0 = (rng.random((B, n_gen)) < 0.1).astype(np.uint8)
    tok0 = np.where(dec0 == 1, rng.integers(0, 100, (B, n_gen)), -1).astype(np.int32)
    garbage = {"slot_state": np.full((B, S), 9, np.uint8), "slot_group": np.full((B, S), -5, np.int32),
               "decoded": dec0, "tokens": tok0, "locked": np.ones((B, n_gen), np.uint8),
               "skip": np.full((B, n_gen), 7, np.uint8), "row_flags": np.full((B, n_gen), 7, np.uint8),
               "active_idx": np.full((B, n_gen), 12345, np.int32), "m_active": np.full(B, -3, np.int32),
               "n_open": np.full(B, -3, np.int32)}
    bbd = dlm.BlockBuffer(B=B, n_slots=S, block_size=bs, max_active=ma, prefix_len=P,
                          **{k: _t(v) for k, v in garbage.items()})
    sel_d = torch.empty((B, n_gen), dtype=torch.int32, device="cuda")
    dlm.dlm_block_buffer_init(bbd)
    st = obb.init(B, S, bs, ma, dec0, tok0)
    der = obb.derive(st, bs, P, None)
    for step in range(400):
        torch.cuda.synchronize()
        want = _oracle_arrays(st, der)
        for f in BB_FIELDS:
            got = getattr(bbd, f).cpu().numpy()
            assert np.array_equal(got, want[f]), (step, f)
        if int(der.n_open.sum()) == 0:
            break
        live = der.skip == 0
        sel = np.full((B, n_gen), -1, np.int32)
        pick = live & ((der.flags & obb.ROW_SELECT) != 0) & (rng.random(sel.shape) < p_sel)
        sel[pick] = rng.integers(0, 50000, int(pick.sum()))
        skip_after = der.skip.copy()
        skip_after[live & ((der.flags & obb.ROW_LOCK) != 0) & (rng.random(sel.shape) < 0.3)] = 1
        bbd.skip.copy_(_t(skip_after))
        sel_d.copy_(_t(sel))
        dlm.dlm_block_buffer_advance(bbd, sel_d)
        st, was = obb.advance(st, bs, ma, skip_after, sel)
        der = obb.derive(st, bs, P, was)
    assert int(der.n_open.sum()) == 0, "the run did not finish"


# --------------------------------------------------------------------------
# dlm_step_attn with a device row count
# --------------------------------------------------------------------------

def _truncated(a, b, m):
    """Batch entry b of an attention case, keeping its first m rows."""
    return W.AttnCase(
        name=a.name, B=1, Hq=a.Hq, Hkv=a.Hkv, D=a.D, n_cap=a.n_cap, kv_len=a.kv_len,
        prefix_len=a.prefix_len, M=m, kind=a.kind, block_size=a.block_size, n_slots=a.n_slots,
        slot_state=a.slot_state[b:b + 1], slot_group=a.slot_group[b:b + 1], cs_lo=a.cs_lo,
        cs_hi=a.cs_hi, colsum_per_head=a.colsum_per_head, scale=a.scale,
        q=np.ascontiguousarray(a.q[b:b + 1, :, :m]), k=np.ascontiguousarray(a.k[b:b + 1, :, :m]),
        v=np.ascontiguousarray(a.v[b:b + 1, :, :m]), cache_k=a.cache_k[b:b + 1],
        cache_v=a.cache_v[b:b + 1], active_idx=np.ascontiguousarray(a.active_idx[b:b + 1, :m]))


def _group_case():
    B, Hq, Hkv, P, bs, S = 2, 8, 2, 200, 32, 4
    M = S * bs
    act = np.tile(np.arange(P, P + M, dtype=np.int32), (B, 1))
    state = np.full((B, S), W.SLOT_ACTIVE, np.uint8)
    state[:, 0] = W.SLOT_IN_CACHE
    group = np.array([[0, 4, 4, 4]] * B, np.int32)
    return W.make_attn("rows_group", B=B, Hq=Hq, Hkv=Hkv, D=64, kv_len=P + M, prefix_len=P,
                       active_idx=act, kind=W.MASK_GROUP, block_size=bs, n_slots=S,
                       slot_state=state, slot_group=group, cs_lo=P, cs_hi=P + M, seed=3)


def _split_case():
    rs = np.random.default_rng(4)
    act = W.sorted_subset(rs, 1, 0, 4096, 100)
    std = 1 / np.sqrt(128)
    return W.make_attn("rows_split", B=1, Hq=2, Hkv=2, D=128, kv_len=4096, prefix_len=0,
                       active_idx=act, kind=W.MASK_FULL, cs_lo=1000, cs_hi=4096, q_std=std,
                       kv_std=std, cache_std=std, seed=4)


def _full_case():
    rs = np.random.default_rng(5)
    act = W.sorted_subset(rs, 2, 0, 700, 128)
    return W.make_attn("rows_full", B=2, Hq=4, Hkv=4, D=32, kv_len=700, prefix_len=0,
                       active_idx=act, kind=W.MASK_FULL, cs_lo=0, cs_hi=700, seed=5)


@pytest.mark.parametrize("which,counts,kgroups", [
    ("group", (77, 0), None),
    ("group", (128, 5), "1"),
    ("split", (63,), None),
    ("split", (0,), None),
    ("full", (1, 128), "2"),
    ("full", (100, 33), "1"),
])
def test_attention_device_row_count(which, counts, kgroups, monkeypatch):
    import denoising_step_amd as dlm
    from denoising_step_amd.runner import DeviceStep, bf16_to_host
    _say(f"device row count {which} {counts} kgroups={kgroups}")
    if kgroups:
        monkeypatch.setenv("DLM_ATTN_KGROUPS", kgroups)
    a = {"group": _group_case, "split": _split_case, "full": _full_case}[which]()
    w = W.Workload(a, W.make_post("none", R=1, V=8, logit_std=1, noise_std=0.1, eps=1e-3,
                                  mode=W.SEL_NONE), "row count")
    ds = DeviceStep(w, with_posterior=False)
    ds.md.m_active = torch.tensor(counts, dtype=torch.int32, device="cuda")
    # with a device row count pass 1 may split keys on the device: the
    # workspace is sized for the descriptor that carries the count
    ds.md.workspace = torch.empty(max(1, dlm.dlm_step_attn_workspace_bytes(ds.kv, ds.md)), dtype=torch.uint8,
                                  device="cuda")
    sentinel_out = torch.full_like(ds.out, 3.0)
    ds.out.copy_(sentinel_out)
    ds.lse.fill_(777.0)
    dlm.dlm_step_attn(ds.q, ds.k, ds.v, ds.kv, ds.active_idx, ds.md, ds.out, ds.lse, ds.colsum)
    torch.cuda.synchronize()
    out = bf16_to_host(ds.out)
    lse = ds.lse.cpu().numpy()
    ck = bf16_to_host(ds.cache_k)
    cs = ds.colsum.cpu().numpy()
    for b, m in enumerate(counts):
        tb = _truncated(a, b, m)
        if m > 0:
            kv = oracle.effective_kv(tb)
            o_out, o_lse = oracle.attention(tb, kv=kv)
            check_attention(out[b:b + 1, :, :m], lse[b:b + 1, :, :m], o_out, o_lse)
            check_colsum(cs[b:b + 1], oracle.colsum(tb, o_lse, kv=kv))
            assert np.array_equal(ck[b], kv[0][0])
        else:
            assert np.all(cs[b] == 0)
            assert np.array_equal(ck[b], a.cache_k[b])
        # rows past the count: not written, their cache rows untouched
        assert np.all(lse[b, :, m:] == 777.0)
        assert np.all(W.bf16_bits_to_f32(out[b, :, m:]) == 3.0)
        rest = a.active_idx[b, m:]
        assert np.array_equal(ck[b][:, rest], a.cache_k[b][:, rest])


# --------------------------------------------------------------------------
# dlm_posterior with per-row flags
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode,k,g,V", [(W.SEL_TOPK_CONF, 5, 64, 4001), (W.SEL_ATTN_DYNAMIC, 0, 100, 2048),
                                        (W.SEL_THRESH_CONF, 0, 32, 999)])
def test_posterior_row_flags(mode, k, g, V):
    import denoising_step_amd as dlm
    _say(f"row flags mode={mode} V={V}")
    R = 300
    p = W.make_post("flags", R=R, V=V, logit_std=3.0, noise_std=0.0, mixture=(0.5, 0.01, 0.2),
                    eps=1e-3, mode=mode, k=k, group_rows=g, tau=0.3, locked_frac=0.2, score_std=1.0,
                    seed=7)
    flags = np.random.default_rng(8).integers(0, 4, R).astype(np.uint8)
    o = oracle.posterior(p.logits, p.prev, p.locked, p.eps, flags=flags)
    o_sel = oracle.select(mode, k, g, p.tau, p.score, o["conf"], o["tok"], p.locked, flags=flags)
    locked = _t(p.locked)
    sel, kl, conf = (torch.empty(R, dtype=dt, device="cuda") for dt in (torch.int32, torch.float32,
                                                                       torch.float32))
    s = dlm.Select(mode=mode, k=k, group_rows=g, tau=p.tau, score=_t(p.score), row_flags=_t(flags))
    s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8,
                              device="cuda")
    dlm.dlm_posterior(_t(p.logits), _t(p.prev), locked, p.eps, s, sel, kl, conf, R, V)
    torch.cuda.synchronize()
    lk = locked.cpu().numpy()
    check_posterior(kl.cpu().numpy(), conf.cpu().numpy(), lk, o["kl"], o["conf"], o["locked"],
                    p.eps, p.locked)
    # a row without the lock flag never locks, whatever its KL
    nolock = (flags & 2) == 0
    assert np.all(lk[nolock] == p.locked[nolock])
    assert (nolock & (p.locked == 0) & (o["kl"] <= p.eps)).any()
    inelig = ((p.locked != 0) | ((flags & 1) == 0)).astype(np.uint8)
    check_selection(sel.cpu().numpy(), o_sel, mode, g, p.tau, o["conf"], p.score, inelig, p.logits)
    assert np.all(sel.cpu().numpy()[(flags & 1) == 0] == -1)


# --------------------------------------------------------------------------
# whole runs
# --------------------------------------------------------------------------

def _compare_step(dl, rec, case):
    """Compare one step's GPU results with the oracle record.  Returns False
    when an excused near-tie decision differs (later steps then diverge)."""
    from denoising_step_amd.runner import bf16_to_host
    torch.cuda.synchronize()
    out = bf16_to_host(dl.out)
    lse = dl.lse.cpu().numpy()
    for b in range(case.B):
        m = int(rec["m_active"][b])
        if m:
            check_attention(out[b, :, :m], lse[b, :, :m], rec["out"][b], rec["lse"][b])
    if dl.colsum is not None:                   # made only for a selection that ranks by them
        check_colsum(dl.colsum.cpu().numpy(), rec["colsum"])
    else:
        assert case.mode not in (W.SEL_ATTN_DYNAMIC, W.SEL_TOPK_SCORE)
    assert np.array_equal(bf16_to_host(dl.cache_k), rec["cache_k"])
    assert np.array_equal(bf16_to_host(dl.cache_v), rec["cache_v"])
    kl, conf, sel = dl.kl.cpu().numpy(), dl.conf.cpu().numpy(), dl.sel.cpu().numpy()
    st = dl.state()
    excused = 0
    for b in range(case.B):
        live = rec["skip"][b] == 0
        lock_g = np.where(live, st["locked"][b], 1).astype(np.uint8)
        lock_o = np.where(live, rec["locked"][b], 1).astype(np.uint8)
        excused += check_posterior(kl[b][live], conf[b][live], lock_g[live], rec["kl"][b][live],
                                   rec["conf"][b][live], lock_o[live], case.eps,
                                   np.zeros(int(live.sum()), np.uint8))
        inelig = ((rec["skip"][b] != 0) | ((rec["flags"][b] & 1) == 0)).astype(np.uint8)
        score = rec["colsum"][b, case.prefix_len:case.prefix_len + case.n_gen]
        excused += check_selection(sel[b], rec["sel"][b], case.mode, case.block_size, case.tau,
                                   rec["conf"][b], score, inelig, case.logits[rec["t"], b])
    if excused:
        return False
    for f in ("slot_state", "slot_group", "decoded", "tokens", "locked"):
        assert np.array_equal(st[f], rec[f]), (rec["t"], f)
    return True


def _compare_derived(dl, rec):
    st = dl.state()
    for f, g in (("active_idx", "active_idx"), ("m_active", "m_active"), ("skip", "skip"),
                 ("row_flags", "flags"), ("n_open", "n_open")):
        assert np.array_equal(st[f], rec[g]), (rec["t"], f)


@pytest.mark.parametrize("name", sorted(W.LOOPS))
def test_loop_matches_oracle(name):
    from denoising_step_amd.loop import DeviceLoop
    _say(f"loop {name}")
    case = W.LOOPS[name]()
    recs = oloop.run(case)
    dl = DeviceLoop(case)
    s = torch.cuda.Stream()
    dl.start(s)
    compared = 0
    for rec in recs:
        _compare_derived(dl, rec)
        if int(rec["n_open"].sum()) == 0:
            break
        dl.feed(rec["t"], s)
        dl.step(s)
        if not _compare_step(dl, rec, case):
            _say(f"  excused near-tie at step {rec['t']}: later steps not compared")
            break
        compared += 1
    assert compared >= (2 * (len(recs) - 1)) // 3, f"only {compared} of {len(recs) - 1} steps compared"
    _say(f"  {compared} steps compared, M_t = {[int(r['m_active'].sum()) for r in recs]}")


@pytest.mark.parametrize("name", ["loop_multiblock", "loop_surelock"])
def test_loop_graph_replay_matches_eager(name):
    """One captured step serves every step: replays (with the stand-in's
    eager work between them) reproduce the eager run bit for bit."""
    from denoising_step_amd.loop import DeviceLoop
    from denoising_step_amd.runner import bf16_to_host
    _say(f"graph replay {name}")
    case = W.LOOPS[name]()
    dl = DeviceLoop(case)
    s = torch.cuda.Stream()

    def snap():
        torch.cuda.synchronize()
        d = dl.state()
        d.update(out=bf16_to_host(dl.out), lse=dl.lse.cpu().numpy(),
                 colsum=None if dl.colsum is None else dl.colsum.cpu().numpy(),
                 kl=dl.kl.cpu().numpy(), conf=dl.conf.cpu().numpy(), sel=dl.sel.cpu().numpy(),
                 cache_k=bf16_to_host(dl.cache_k))
        return d

    eager = []
    dl.start(s)
    for t in range(case.T):
        dl.feed(t, s)
        dl.step(s)
        eager.append(snap())
        if int(eager[-1]["n_open"].sum()) == 0:
            break
    dl.start(s)
    torch.cuda.synchronize()
    g = dl.capture(s)
    for t, want in enumerate(eager):
        dl.feed(t, s)
        with torch.cuda.stream(s):
            g.replay()
        got = snap()
        for key, v in want.items():
            assert np.array_equal(got[key], v), (t, key)
    _say(f"  {len(eager)} replays equal the eager steps")
