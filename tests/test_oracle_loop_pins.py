"""Pins of the oracle's Block Buffer state machine and multi-step loop.

* The transitions are checked against traces worked by hand from the
  Multi-Block Diffusion Language Models page (sec. 2.3), stored in
  tests/golden/block_buffer.json.
* Random runs check invariants that the page's description fixes (states
  only move forward, the running set is bounded, the cached prefix stays
  contiguous, a slot leaves the running set only when fully decoded).
* Whole runs of the loop check properties fixed by the mathematics and by
  the inputs, not by the oracle: each computed row's attention sums to one
  (so the column sums add up to Hq * M_t), a lock happens exactly where
  KL (scipy) <= eps for a lockable row, a selected token is the argmax of
  that step's logits (numpy), and a cached row holds the fresh K/V of the
  last step that computed it.
* Planted mistakes in a private copy of the state machine are caught.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import block_buffer as bb
from oracle import loop as oloop

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "block_buffer.json")


def check_golden(mod):
    with open(GOLDEN) as f:
        traces = json.load(f)["traces"]
    for tr in traces:
        ns, bs, ma, P = tr["n_slots"], tr["block_size"], tr["max_active"], tr["prefix_len"]
        st = mod.init(1, ns, bs, ma)
        der = mod.derive(st, bs, P, None)
        ini = tr["init"]
        assert st.slot_state[0].tolist() == ini["slot_state"], tr["name"]
        assert st.slot_group[0].tolist() == ini["slot_group"], tr["name"]
        for key in ("skip", "flags", "active_idx"):
            assert getattr(der, key)[0].tolist() == ini[key], (tr["name"], "init", key)
        assert int(der.m_active[0]) == ini["m_active"] and int(der.n_open[0]) == ini["n_open"]
        for i, stp in enumerate(tr["steps"]):
            st, was = mod.advance(st, bs, ma, np.array([stp["skip_after"]], np.uint8),
                                  np.array([stp["sel"]], np.int32))
            der = mod.derive(st, bs, P, was)
            ex = stp["expect"]
            for key in ("slot_state", "slot_group", "decoded", "tokens", "locked"):
                assert getattr(st, key)[0].tolist() == ex[key], (tr["name"], i, key)
            for key in ("skip", "flags", "active_idx"):
                assert getattr(der, key)[0].tolist() == ex[key], (tr["name"], i, key)
            assert int(der.m_active[0]) == ex["m_active"], (tr["name"], i)
            assert int(der.n_open[0]) == ex["n_open"], (tr["name"], i)


def test_block_buffer_golden():
    check_golden(bb)


def random_run(mod, rng, B=3, n_slots=7, bs=3, max_active=3, steps=60):
    """Drive the state machine with random selections and locks that respect
    the per-row inputs it derives; yield (old state, new state, derived)."""
    st = mod.init(B, n_slots, bs, max_active)
    der = mod.derive(st, bs, 0, None)
    for _ in range(steps):
        sel = np.full(st.decoded.shape, -1, np.int32)
        skip_after = der.skip.copy()
        live = der.skip == 0
        pick = live & ((der.flags & bb.ROW_SELECT) != 0) & (rng.random(sel.shape) < 0.35)
        sel[pick] = rng.integers(0, 50, int(pick.sum()))
        lock = live & ((der.flags & bb.ROW_LOCK) != 0) & (rng.random(sel.shape) < 0.3)
        skip_after[lock] = 1
        new, was = mod.advance(st, bs, max_active, skip_after, sel)
        nder = mod.derive(new, bs, 0, was)
        yield st, new, der, nder
        st, der = new, nder


def test_block_buffer_invariants():
    rng = np.random.default_rng(21)
    order = {bb.SLOT_DUMMY: 0, bb.SLOT_ACTIVE: 1, bb.SLOT_TO_CACHE: 2, bb.SLOT_IN_CACHE: 3}
    bs = 3
    for old, new, der, nder in random_run(bb, rng, bs=bs):
        B, S = new.slot_state.shape
        for b in range(B):
            o, n = old.slot_state[b], new.slot_state[b]
            # states only move forward, one stage at most per step
            for s in range(S):
                assert 0 <= order[n[s]] - order[o[s]] <= 1
            assert np.sum(n == bb.SLOT_ACTIVE) <= 3
            # clean slots (to-cache / in-cache) form a prefix, dummy slots a suffix
            clean = [x in (bb.SLOT_TO_CACHE, bb.SLOT_IN_CACHE) for x in n]
            assert clean == sorted(clean, reverse=True)
            dummy = [x == bb.SLOT_DUMMY for x in n]
            assert dummy == sorted(dummy)
            # in-cache slots come before to-cache slots
            ic = [x == bb.SLOT_IN_CACHE for x in n]
            assert ic == sorted(ic, reverse=True)
            # a slot is clean only when every position in it is decoded
            for s in range(S):
                if clean[s]:
                    assert new.decoded[b, s * bs:(s + 1) * bs].all()
                if o[s] == bb.SLOT_TO_CACHE:
                    assert n[s] == bb.SLOT_IN_CACHE
            # locks only on decoded rows; locks and decodes are never undone
            assert np.all(new.locked[b] <= new.decoded[b])
            assert np.all(new.locked[b] >= old.locked[b]) and np.all(new.decoded[b] >= old.decoded[b])
            # the compacted rows are ascending and unique, -1 past the count
            m = int(nder.m_active[b])
            a = nder.active_idx[b]
            assert np.all(np.diff(a[:m]) > 0) and np.all(a[m:] == -1)
            # every computed row is unlocked and in an active or to-cache slot
            for p in a[:m]:
                assert not new.locked[b, p]
                assert n[p // bs] in (bb.SLOT_ACTIVE, bb.SLOT_TO_CACHE)


def test_block_buffer_terminates():
    """With at least one row selected per running block and step, every
    slot reaches in-cache; the run drains to zero rows."""
    rng = np.random.default_rng(22)
    B, S, bs, ma = 2, 5, 4, 2
    st = bb.init(B, S, bs, ma)
    der = bb.derive(st, bs, 0, None)
    for t in range(S * (bs + 2)):
        sel = np.full(st.decoded.shape, -1, np.int32)
        for b in range(B):
            for s in range(S):
                cand = [p for p in range(s * bs, (s + 1) * bs)
                        if der.skip[b, p] == 0 and der.flags[b, p] & bb.ROW_SELECT]
                if cand:
                    sel[b, cand[int(rng.integers(0, len(cand)))]] = 1
        st, was = bb.advance(st, bs, ma, der.skip, sel)
        der = bb.derive(st, bs, 0, was)
    assert np.all(st.slot_state == bb.SLOT_IN_CACHE)
    assert np.all(der.m_active == 0) and np.all(der.n_open == 0)


@pytest.mark.parametrize("name", sorted(W.LOOPS))
def test_loop_properties(name):
    from scipy.special import rel_entr, softmax
    case = W.LOOPS[name]()
    steps = oloop.run(case)
    assert int(steps[-1]["n_open"].sum()) == 0, "the run must finish within the drawn steps"
    P, bs = case.prefix_len, case.block_size
    last_k = np.full((case.B, case.Hkv, case.kv_len, case.D), -1, np.int64)
    last_v = np.full_like(last_k, -1)
    for rec in steps[:-1]:
        t = rec["t"]
        for b in range(case.B):
            m = int(rec["m_active"][b])
            # each computed row's attention sums to one over the keys it sees
            assert abs(rec["colsum"][b].sum() - case.Hq * m) < 1e-9 * max(1, m)
            rows = rec["active_idx"][b, :m]
            last_k[b][:, rows] = case.k_new[t, b][:, rows - P].astype(np.int64)
            last_v[b][:, rows] = case.v_new[t, b][:, rows - P].astype(np.int64)
            x = case.logits[t, b].astype(np.float64)
            y = case.logits[t - 1, b].astype(np.float64) if t > 0 else x
            for p in range(case.n_gen):
                if rec["skip"][b, p]:
                    assert rec["sel"][b, p] == -1
                    continue
                kl = rel_entr(softmax(x[p]), softmax(y[p])).sum()
                lockable = bool(rec["flags"][b, p] & bb.ROW_LOCK)
                assert bool(rec["skip_after"][b, p]) == (lockable and kl <= case.eps), (t, b, p)
                if rec["sel"][b, p] >= 0:
                    assert rec["flags"][b, p] & bb.ROW_SELECT
                    assert rec["sel"][b, p] == int(np.argmax(x[p]))
        # the cache: prefix rows untouched, computed rows hold their last fresh K/V
        ck = rec["cache_k"].astype(np.int64)
        assert np.array_equal(ck[:, :, :P], case.cache_k[:, :, :P].astype(np.int64))
        seen = last_k[..., 0] >= 0
        assert np.array_equal(ck[seen], last_k[seen])
        assert np.array_equal(rec["cache_v"].astype(np.int64)[seen], last_v[seen])
    # every generation position got a token
    fin = steps[-2]
    assert fin["decoded"].all() and np.all(fin["tokens"] >= 0)


def test_surelock_rows_fall():
    """In a single-block run the rows still computed never grow (SureLock
    page, sec. 3-4: M_t decreases over the steps)."""
    steps = oloop.run(W.loop_surelock())
    m = [int(r["m_active"].sum()) for r in steps]
    assert m[0] == 80 and m[-1] == 0
    assert all(a >= b for a, b in zip(m, m[1:]))


BB_SRC = os.path.join(os.path.dirname(bb.__file__), "block_buffer.py")

BB_MUTANTS = [
    ("commit_in_same_update", "        # (3) refill the running set from the lowest dummy slots\n",
     "        for s in range(n_slots):\n            if row[s] == SLOT_TO_CACHE:\n"
     "                row[s] = SLOT_IN_CACHE\n"
     "        # (3) refill the running set from the lowest dummy slots\n"),
    ("to_cache_out_of_order", "            break\n        # (3) refill",
     "            continue\n        # (3) refill"),
    ("refill_counts_to_cache", "n_act = int(np.sum(row == SLOT_ACTIVE))",
     "n_act = int(np.sum((row == SLOT_ACTIVE) | (row == SLOT_TO_CACHE)))"),
    ("active_groups_private", "g[s] = s if state_row[s] in (SLOT_TO_CACHE, SLOT_IN_CACHE) else n",
     "g[s] = s"),
    ("commit_not_computed", "if s in (SLOT_ACTIVE, SLOT_TO_CACHE) and not st.locked[b, p]:",
     "if s == SLOT_ACTIVE and not st.locked[b, p]:"),
    ("lock_without_previous_step", "elif was_active is not None and was_active[b, p]:",
     "else:"),
    ("locked_rows_computed", "if s in (SLOT_ACTIVE, SLOT_TO_CACHE) and not st.locked[b, p]:",
     "if s in (SLOT_ACTIVE, SLOT_TO_CACHE):"),
    ("select_decoded_rows", "            if not st.decoded[b, p]:\n                flags[b, p] = ROW_SELECT\n",
     "            flags[b, p] = ROW_SELECT\n            if False:\n                pass\n"),
]


@pytest.mark.parametrize("name,old,new", BB_MUTANTS, ids=[m[0] for m in BB_MUTANTS])
def test_pins_catch_block_buffer_mutant(name, old, new, tmp_path):
    with open(BB_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"bb_mutant_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"bb_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        check_golden(mod)
