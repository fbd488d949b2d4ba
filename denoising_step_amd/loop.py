"""A multi-step denoising run on the device over a Block Buffer.

``DeviceLoop`` holds a run's Block Buffer arrays, the K/V cache and the
per-step buffers, and runs one step as three C-ABI calls on one stream:

  1. ``dlm_step_attn`` over the rows the buffer chose (active_idx with its
     row count m_active on the device) under the group mask of the buffer's
     slot tables, with column sums over every computed row when the
     selection ranks by them (the Attn-Sampler modes; the other modes never
     read them, so the pass that makes them is not run);
  2. ``dlm_posterior`` per batch entry over the generation region: rows
     outside active slots and locked rows are skipped, selection groups are
     the blocks, rows carry the buffer's select / lock flags, and the score
     of a row is the column sum at its position;
  3. ``dlm_block_buffer_advance``: unmask, lock, move the slots, compact the
     next step's rows.

Nothing is read back between steps, so every step has the same launch
shapes; ``capture()`` records one step in a HIP graph that serves every
later step.

The model that would produce each step's queries, fresh K/V and logits is
not part of the path.  ``feed(t)`` stands in for it: it gathers the computed
rows' entries of the run's per-step inputs with torch and copies step t's
and step t-1's logits into the buffers the posterior reads.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MASK_GROUP, SEL_ATTN_DYNAMIC, SEL_TOPK_SCORE, BlockBuffer, KVCache, MaskDesc, Select,
               dlm_block_buffer_advance,
               dlm_block_buffer_init, dlm_posterior, dlm_posterior_workspace_bytes,
               dlm_step_attn, dlm_step_attn_workspace_bytes)
from .runner import bf16_to_device


def _on(x, dev, dtype=None, bf16=False):
    """A device tensor from a numpy array (bf16 as bit patterns) or a tensor."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.to(dev)
    if bf16:
        return bf16_to_device(x, dev)
    return torch.from_numpy(np.ascontiguousarray(x, dtype)).to(dev)


class DeviceLoop:
    def __init__(self, case, device="cuda"):
        """case: a run's inputs (``workloads.LoopCase`` fields: shapes, the
        selection rule, per-step bf16 q / k_new / v_new bit patterns and fp32
        logits for every generation position, the cache, the positions that
        start unmasked), as numpy arrays or device tensors.  The per-step
        inputs may be None when a subclass's ``feed`` makes them."""
        dev = torch.device(device)
        self.case = case
        B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
        P, S, bs = case.prefix_len, case.n_slots, case.block_size
        n_gen, kv_len, V = S * bs, P + S * bs, case.V
        self.B, self.n_gen, self.kv_len, self.V, self.P = B, n_gen, kv_len, V, P
        # stand-in inputs of every step
        self.q_all = _on(case.q, dev, bf16=True)
        self.k_all = _on(case.k_new, dev, bf16=True)
        self.v_all = _on(case.v_new, dev, bf16=True)
        self.logits_all = _on(case.logits, dev, np.float32)
        self.cache_k0 = _on(case.cache_k, dev, bf16=True)
        self.cache_v0 = _on(case.cache_v, dev, bf16=True)
        self.cache_k = self.cache_k0.clone()
        self.cache_v = self.cache_v0.clone()
        self.kv = KVCache(self.cache_k, self.cache_v)

        def z(shape, dt):
            return torch.zeros(shape, dtype=dt, device=dev)

        self.decoded0 = _on(case.decoded0, dev, np.uint8)
        self.tokens0 = _on(case.tokens0, dev, np.int32)
        self.bb = BlockBuffer(B=B, n_slots=S, block_size=bs, max_active=case.max_active, prefix_len=P,
                              slot_state=z((B, S), torch.uint8), slot_group=z((B, S), torch.int32),
                              decoded=self.decoded0.clone(), tokens=self.tokens0.clone(),
                              locked=z((B, n_gen), torch.uint8), skip=z((B, n_gen), torch.uint8),
                              row_flags=z((B, n_gen), torch.uint8),
                              active_idx=z((B, n_gen), torch.int32), m_active=z((B,), torch.int32),
                              n_open=z((B,), torch.int32))
        # per-step buffers (fixed addresses)
        self.q = z((B, Hq, n_gen, D), torch.bfloat16)
        self.k = z((B, Hkv, n_gen, D), torch.bfloat16)
        self.v = z((B, Hkv, n_gen, D), torch.bfloat16)
        self.out = z((B, Hq, n_gen, D), torch.bfloat16)
        self.lse = z((B, Hq, n_gen), torch.float32)
        # column sums only for a selection that ranks by them
        self.colsum = z((B, kv_len), torch.float32) if case.mode in (SEL_ATTN_DYNAMIC, SEL_TOPK_SCORE) else None
        self.x = z((B, n_gen, V), torch.float32)
        self.y = z((B, n_gen, V), torch.float32)
        self.sel = z((B, n_gen), torch.int32)
        self.kl = z((B, n_gen), torch.float32)
        self.conf = z((B, n_gen), torch.float32)
        self.md = MaskDesc(kind=MASK_GROUP, Hq=Hq, M=n_gen, kv_len=kv_len, prefix_len=P,
                           block_size=bs, n_slots=S, slot_state=self.bb.slot_state,
                           slot_group=self.bb.slot_group, cs_lo=P, cs_hi=kv_len,
                           m_active=self.bb.m_active)
        self.attn_ws = z((max(1, dlm_step_attn_workspace_bytes(self.kv, self.md)),), torch.uint8)
        self.md.workspace = self.attn_ws
        # The posterior streams only the step's rows: the buffer's compacted
        # active rows (every other row arrives with skip set), their count on
        # the device, so the vocabulary split follows M_t in the captured step.
        self.sels = [Select(mode=case.mode, k=case.k, group_rows=bs, tau=case.tau,
                            score=None if self.colsum is None else self.colsum[b, P:P + n_gen],
                            row_flags=self.bb.row_flags[b],
                            live_rows=self.bb.active_idx[b], n_live=self.bb.m_active[b:b + 1],
                            live_offset=P) for b in range(B)]
        self.post_ws = z((max(1, dlm_posterior_workspace_bytes(n_gen, V, self.sels[0])),), torch.uint8)
        for sl in self.sels:
            sl.workspace = self.post_ws

    def start(self, stream=None):
        """Restore the cache and the unmasked set, clear the per-step buffers
        (so two runs match bit for bit, rows past M_t included), and
        initialise the buffer."""
        with torch.cuda.stream(stream or torch.cuda.current_stream()):
            for t in (self.q, self.k, self.v, self.out, self.lse, self.colsum, self.x, self.y,
                      self.sel, self.kl, self.conf):
                if t is not None:
                    t.zero_()
            self.cache_k.copy_(self.cache_k0)
            self.cache_v.copy_(self.cache_v0)
            self.bb.decoded.copy_(self.decoded0)
            self.bb.tokens.copy_(self.tokens0)
            dlm_block_buffer_init(self.bb, stream)

    def feed(self, t, stream=None):
        """The stand-in for the model at step t (torch, on `stream`)."""
        B, n_gen = self.B, self.n_gen
        with torch.cuda.stream(stream or torch.cuda.current_stream()):
            # rows past the count gather position 0; no kernel reads them
            idx = (self.bb.active_idx - self.P).clamp_(min=0).long()
            for src, dst in ((self.q_all, self.q), (self.k_all, self.k), (self.v_all, self.v)):
                H, D = dst.shape[1], dst.shape[3]
                torch.gather(src[t], 2, idx[:, None, :, None].expand(B, H, n_gen, D), out=dst)
            self.x.copy_(self.logits_all[t])
            self.y.copy_(self.logits_all[t - 1] if t > 0 else self.logits_all[0])

    def step(self, stream=None):
        """One step of the path: attention, posterior, Block Buffer advance."""
        c = self.case
        dlm_step_attn(self.q, self.k, self.v, self.kv, self.bb.active_idx, self.md, self.out,
                      self.lse, self.colsum, stream)
        for b in range(self.B):
            dlm_posterior(self.x[b], self.y[b], self.bb.skip[b], c.eps, self.sels[b], self.sel[b],
                          self.kl[b], self.conf[b], self.n_gen, self.V, stream)
        dlm_block_buffer_advance(self.bb, self.sel, stream)

    def capture(self, stream):
        """Record one step in a HIP graph (replay it on `stream`)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            self.step(torch.cuda.current_stream())
        return g

    def state(self) -> dict:
        """Host copies of the buffer arrays (synchronises)."""
        torch.cuda.synchronize()
        names = ("slot_state", "slot_group", "decoded", "tokens", "locked", "skip", "row_flags",
                 "active_idx", "m_active", "n_open")
        return {n: getattr(self.bb, n).cpu().numpy() for n in names}
