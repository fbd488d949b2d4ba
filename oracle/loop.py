"""CPU oracle of the multi-step denoising loop over a Block Buffer (test
infrastructure only; small cases).

Each step, in this order (SureLock page sec. 2; "Multi-Block Diffusion
Language Models" page sec. 2.3):
  1. the rows to compute are the unlocked positions of active and to-cache
     slots, in ascending position order (the compaction of ``derive``);
  2. attention of those rows over the cache under the group mask of the slot
     table, after their fresh K/V are written into the cache (a locked row
     keeps the K/V of the last step that computed it); column sums over the
     computed rows;
  3. posterior of the positions of active slots (the others are skipped):
     KL against the previous step's logits, confidence, lock test for rows
     marked lockable, selection among rows marked selectable, one selection
     group per block, the score of a row being the column sum at its
     position;
  4. the Block Buffer advance.
The model that produces each step's queries, fresh K/V and logits is out of
scope: the case supplies them for every position and step, and a step reads
the computed rows' entries.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import block_buffer as bb


def _attn_case(case, t, b, st, rows):
    import workloads as W
    rel = rows - case.prefix_len
    return W.AttnCase(
        name=f"{case.name}_t{t}_b{b}", B=1, Hq=case.Hq, Hkv=case.Hkv, D=case.D,
        n_cap=case.kv_len, kv_len=case.kv_len, prefix_len=case.prefix_len, M=len(rows),
        kind=W.MASK_GROUP, block_size=case.block_size, n_slots=case.n_slots,
        slot_state=st.slot_state[b:b + 1].copy(), slot_group=st.slot_group[b:b + 1].copy(),
        cs_lo=case.prefix_len, cs_hi=case.kv_len, colsum_per_head=0, scale=0.0,
        q=np.ascontiguousarray(case.q[t, b:b + 1][:, :, rel]),
        k=np.ascontiguousarray(case.k_new[t, b:b + 1][:, :, rel]),
        v=np.ascontiguousarray(case.v_new[t, b:b + 1][:, :, rel]),
        cache_k=None, cache_v=None, active_idx=np.ascontiguousarray(rows[None], np.int32))


def run(case, n_steps=None):
    """Run the loop for at most n_steps (default case.T) steps or until every
    slot is in-cache.  Returns a list of per-step records (dicts of numpy
    arrays): the derived inputs the step read, its attention, posterior and
    selection results, and the buffer state after its advance."""
    T = case.T if n_steps is None else min(n_steps, case.T)
    B, P, n_gen, kv_len = case.B, case.prefix_len, case.n_gen, case.kv_len
    st = bb.init(B, case.n_slots, case.block_size, case.max_active, case.decoded0, case.tokens0)
    der = bb.derive(st, case.block_size, P, None)
    ck, cv = case.cache_k.copy(), case.cache_v.copy()
    steps = []
    for t in range(T):
        rec = {"t": t, "active_idx": der.active_idx.copy(), "m_active": der.m_active.copy(),
               "skip": der.skip.copy(), "flags": der.flags.copy(), "n_open": der.n_open.copy()}
        if int(der.n_open.sum()) == 0:
            steps.append(rec)
            break
        outs, lses = [], []
        cs = np.zeros((B, kv_len), np.float64)
        for b in range(B):
            m = int(der.m_active[b])
            if m == 0:
                outs.append(np.zeros((case.Hq, 0, case.D)))
                lses.append(np.zeros((case.Hq, 0)))
                continue
            ac = _attn_case(case, t, b, st, der.active_idx[b, :m])
            ac.cache_k, ac.cache_v = ck[b:b + 1], cv[b:b + 1]
            kv = oracle.effective_kv(ac)
            out, lse = oracle.attention(ac, kv=kv)
            cs[b] = oracle.colsum(ac, lse, kv=kv)[0]
            ck[b], cv[b] = kv[0][0], kv[1][0]
            outs.append(out[0])
            lses.append(lse[0])
        x = case.logits[t]
        y = case.logits[t - 1] if t > 0 else case.logits[0]
        kl = np.zeros((B, n_gen))
        conf = np.zeros((B, n_gen))
        skip_after = np.zeros((B, n_gen), np.uint8)
        sel = np.full((B, n_gen), -1, np.int32)
        for b in range(B):
            post = oracle.posterior(x[b], y[b], der.skip[b], case.eps, flags=der.flags[b])
            score = cs[b, P:P + n_gen]
            sel[b] = oracle.select(case.mode, case.k, case.block_size, case.tau, score,
                                   post["conf"], post["tok"], der.skip[b], post["margin"],
                                   post["entropy"], flags=der.flags[b])
            kl[b], conf[b], skip_after[b] = post["kl"], post["conf"], post["locked"]
        st, was = bb.advance(st, case.block_size, case.max_active, skip_after, sel)
        der = bb.derive(st, case.block_size, P, was)
        rec.update({"out": outs, "lse": lses, "colsum": cs, "kl": kl, "conf": conf,
                    "skip_after": skip_after, "sel": sel, "slot_state": st.slot_state.copy(),
                    "slot_group": st.slot_group.copy(), "decoded": st.decoded.copy(),
                    "tokens": st.tokens.copy(), "locked": st.locked.copy(),
                    "cache_k": ck.copy(), "cache_v": cv.copy()})
        steps.append(rec)
    return steps
