"""CPU oracle of the Block Buffer state machine, the active-set compaction and
the multi-step denoising loop (plain Python loops; small cases only).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: the GPU library and its
binding never import it, and it shares no code with them.

What it follows:
  * "Multi-Block Diffusion Language Models" page, sec. 2.3 (Block Buffer): a
    fixed number of physical slots; a slot is dummy (inactive), active (being
    decoded), to-cache (finished, not yet cached) or in-cache (committed to
    the KV cache); future blocks enter the running set by turning a dummy
    slot active, finished blocks are committed to the cache; the running set
    is bounded (sec. 2.1: a small |R_s|, e.g. 2-4 blocks); decoding and cache
    writes overlap.
  * SureLock page, sec. 2: a position whose posterior has settled (step-wise
    KL <= eps) is locked; a locked position's query and FFN are no longer
    computed and its cached K/V are reused by the others; sec. 3/4: the
    number M_t of rows still computed falls as steps go on.

Readings of points the pages leave open (each one is a plain choice):
  * The buffer covers the whole generation region: slot s holds positions
    [P + s*bs, P + (s+1)*bs).  Recycling a finished slot as a tail dummy is
    replaced by the next slot of the region, which the mask treats the same.
  * Transitions after each step, in this order: (1) to-cache -> in-cache
    (that step's forward recomputed the finished block and wrote its K/V);
    (2) the leading run of fully decoded active slots -> to-cache (a block is
    committed only after every earlier block, so the cached prefix stays
    contiguous); (3) the lowest dummy slots -> active until max_active slots
    are active.  Initially slots 0 .. max_active-1 are active.
  * Noise groups for the group mask: to-cache and in-cache slot s is group s
    (clean, block-causal), every active slot is group n_slots (one running
    noise group, mutually visible, seeing all clean blocks).
  * Rows computed by a step: every unlocked position of an active or
    to-cache slot (decode and commit share one forward).
  * The posterior covers active slots only; a position may be selected
    (unmasked) while masked, and may lock only once decoded and computed in
    the previous step (so it has a previous-step posterior).
"""
from __future__ import annotations

import dataclasses

import numpy as np

SLOT_DUMMY, SLOT_ACTIVE, SLOT_TO_CACHE, SLOT_IN_CACHE = 0, 1, 2, 3
ROW_SELECT, ROW_LOCK = 1, 2


@dataclasses.dataclass
class BufferState:
    slot_state: np.ndarray   # uint8 [B, n_slots]
    slot_group: np.ndarray   # int32 [B, n_slots]
    decoded: np.ndarray      # uint8 [B, n_gen]
    tokens: np.ndarray       # int32 [B, n_gen]
    locked: np.ndarray       # uint8 [B, n_gen]

    def copy(self):
        return BufferState(*(np.array(a) for a in dataclasses.astuple(self)))


@dataclasses.dataclass
class Derived:
    """What the next step reads: the posterior's per-row inputs and the
    compacted rows to compute."""
    skip: np.ndarray         # uint8 [B, n_gen]: posterior 'locked' input
    flags: np.ndarray        # uint8 [B, n_gen]: ROW_SELECT / ROW_LOCK
    active_idx: np.ndarray   # int32 [B, n_gen]: absolute positions, -1 past m_active
    m_active: np.ndarray     # int32 [B]
    n_open: np.ndarray       # int32 [B]: slots not yet in-cache


def slot_groups(state_row: np.ndarray) -> np.ndarray:
    n = len(state_row)
    g = np.empty(n, np.int32)
    for s in range(n):
        g[s] = s if state_row[s] in (SLOT_TO_CACHE, SLOT_IN_CACHE) else n
    return g


def init(B, n_slots, block_size, max_active, decoded0=None, tokens0=None) -> BufferState:
    n_gen = n_slots * block_size
    state = np.full((B, n_slots), SLOT_DUMMY, np.uint8)
    state[:, :min(max_active, n_slots)] = SLOT_ACTIVE
    group = np.stack([slot_groups(state[b]) for b in range(B)])
    dec = np.zeros((B, n_gen), np.uint8) if decoded0 is None else np.array(decoded0, np.uint8)
    tok = np.full((B, n_gen), -1, np.int32) if tokens0 is None else np.array(tokens0, np.int32)
    return BufferState(state, group, dec, tok, np.zeros((B, n_gen), np.uint8))


def derive(st: BufferState, block_size: int, prefix_len: int, was_active=None) -> Derived:
    """Per-row posterior inputs and the compaction of the rows to compute.
    was_active [B, n_gen] (bool): the row's slot was active during the step
    just taken (None: no step taken yet, so no row has a previous posterior)."""
    B, n_gen = st.decoded.shape
    skip = np.zeros((B, n_gen), np.uint8)
    flags = np.zeros((B, n_gen), np.uint8)
    act = np.full((B, n_gen), -1, np.int32)
    m = np.zeros(B, np.int32)
    n_open = np.zeros(B, np.int32)
    for b in range(B):
        n_open[b] = int(np.sum(st.slot_state[b] != SLOT_IN_CACHE))
        for p in range(n_gen):
            s = st.slot_state[b, p // block_size]
            skip[b, p] = 1 if (st.locked[b, p] or s != SLOT_ACTIVE) else 0
            if not st.decoded[b, p]:
                flags[b, p] = ROW_SELECT
            elif was_active is not None and was_active[b, p]:
                flags[b, p] = ROW_LOCK
            if s in (SLOT_ACTIVE, SLOT_TO_CACHE) and not st.locked[b, p]:
                act[b, m[b]] = prefix_len + p
                m[b] += 1
    return Derived(skip, flags, act, m, n_open)


def advance(st: BufferState, block_size: int, max_active: int, skip_after: np.ndarray,
            sel: np.ndarray):
    """Apply one step's posterior results and move the slots.  skip_after is
    the posterior's lock array after the step (1 for rows that arrived
    skipped or locked now); sel the selected tokens (-1: not selected).
    Returns (new state, was_active)."""
    st = st.copy()
    B, n_gen = st.decoded.shape
    n_slots = st.slot_state.shape[1]
    was_active = np.zeros((B, n_gen), bool)
    for b in range(B):
        for p in range(n_gen):
            if st.slot_state[b, p // block_size] != SLOT_ACTIVE:
                continue
            was_active[b, p] = True
            if sel[b, p] >= 0:
                st.decoded[b, p] = 1
                st.tokens[b, p] = sel[b, p]
            if skip_after[b, p]:
                st.locked[b, p] = 1
        row = st.slot_state[b]
        # (1) committed by the step just taken
        for s in range(n_slots):
            if row[s] == SLOT_TO_CACHE:
                row[s] = SLOT_IN_CACHE
        # (2) the leading run of finished active blocks
        for s in range(n_slots):
            if row[s] in (SLOT_TO_CACHE, SLOT_IN_CACHE):
                continue
            done = all(st.decoded[b, s * block_size:(s + 1) * block_size])
            if row[s] == SLOT_ACTIVE and done:
                row[s] = SLOT_TO_CACHE
                continue
            break
        # (3) refill the running set from the lowest dummy slots
        n_act = int(np.sum(row == SLOT_ACTIVE))
        for s in range(n_slots):
            if n_act >= max_active:
                break
            if row[s] == SLOT_DUMMY:
                row[s] = SLOT_ACTIVE
                n_act += 1
        st.slot_group[b] = slot_groups(row)
    return st, was_active
