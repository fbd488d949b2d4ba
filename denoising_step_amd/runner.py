"""Run one denoising step of a host-side workload on the GPU.

``DeviceStep`` uploads the inputs of a ``workloads.Workload`` into device
tensors, allocates outputs and workspaces once, and runs the two C-ABI calls
(``dlm_step_attn`` then ``dlm_posterior``) on a stream.  The K/V cache and
the lock flags are in/out; ``reset()`` restores their original contents so
a step can be repeated on identical inputs.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (KVCache, MaskDesc, Select, dlm_posterior, dlm_posterior_workspace_bytes,
               dlm_step_attn, dlm_step_attn_workspace_bytes)


_SIDE_STREAMS = {}


def bf16_to_device(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bf16_to_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceStep:
    def __init__(self, workload, device="cuda", with_colsum=True, with_posterior=True, with_scores=False):
        """with_scores: also compute margin and entropy of p_t (always when the
        selection mode ranks by them)."""
        a, p = workload.attn, workload.post
        self.workload = workload
        self.device = device
        dev = torch.device(device)
        self.q = bf16_to_device(a.q, dev)
        self.k = bf16_to_device(a.k, dev)
        self.v = bf16_to_device(a.v, dev)
        self.cache_k0 = bf16_to_device(a.cache_k, dev)
        self.cache_v0 = bf16_to_device(a.cache_v, dev)
        self.cache_k = self.cache_k0.clone()
        self.cache_v = self.cache_v0.clone()
        self.active_idx = torch.from_numpy(np.ascontiguousarray(a.active_idx, np.int32)).to(dev)
        slot_state = slot_group = None
        if a.kind == 2:
            slot_state = torch.from_numpy(np.ascontiguousarray(a.slot_state, np.uint8)).to(dev)
            slot_group = torch.from_numpy(np.ascontiguousarray(a.slot_group, np.int32)).to(dev)
        self.kv = KVCache(self.cache_k, self.cache_v)
        self.md = MaskDesc(kind=a.kind, Hq=a.Hq, M=a.M, kv_len=a.kv_len, prefix_len=a.prefix_len,
                           block_size=a.block_size, n_slots=a.n_slots if a.kind == 2 else 0,
                           slot_state=slot_state, slot_group=slot_group, cs_lo=a.cs_lo,
                           cs_hi=a.cs_hi, colsum_per_head=a.colsum_per_head, scale=a.scale)
        ws = dlm_step_attn_workspace_bytes(self.kv, self.md)
        self.attn_ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.md.workspace = self.attn_ws
        self.out = torch.empty((a.B, a.Hq, a.M, a.D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((a.B, a.Hq, a.M), dtype=torch.float32, device=dev)
        self.colsum = None
        if with_colsum:
            shape = (a.B, a.Hq, a.kv_len) if a.colsum_per_head else (a.B, a.kv_len)
            self.colsum = torch.empty(shape, dtype=torch.float32, device=dev)

        self.with_posterior = with_posterior
        if with_posterior:
            self.logits = torch.from_numpy(p.logits).to(dev)
            self.prev = torch.from_numpy(p.prev).to(dev)
            self.locked0 = torch.from_numpy(np.ascontiguousarray(p.locked, np.uint8)).to(dev)
            self.locked = self.locked0.clone()
            self.sel = torch.empty(p.R, dtype=torch.int32, device=dev)
            self.kl = torch.empty(p.R, dtype=torch.float32, device=dev)
            self.conf = torch.empty(p.R, dtype=torch.float32, device=dev)
            self.margin = torch.empty(p.R, dtype=torch.float32, device=dev)
            self.entropy = torch.empty(p.R, dtype=torch.float32, device=dev)
            score = None
            if p.score is not None:
                score = torch.from_numpy(p.score).to(dev)
            elif p.score_cols is not None:
                b, first = p.score_cols
                score = self.colsum[b, first:first + p.R]
            self.score = score
            scores = with_scores or p.mode in (5, 6)
            self.with_scores = scores
            self.select = Select(mode=p.mode, k=p.k, group_rows=p.group_rows, tau=p.tau, score=score,
                                 margin=self.margin if scores else None,
                                 entropy=self.entropy if scores else None)
            ws = dlm_posterior_workspace_bytes(p.R, p.V, self.select)
            self.post_ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)
            self.select.workspace = self.post_ws

    def reset(self):
        self.cache_k.copy_(self.cache_k0)
        self.cache_v.copy_(self.cache_v0)
        if self.with_posterior:
            self.locked.copy_(self.locked0)

    def run_attn(self, stream=None, fresh=True):
        dlm_step_attn(self.q, self.k if fresh else None, self.v if fresh else None, self.kv,
                      self.active_idx, self.md, self.out, self.lse, self.colsum, stream)

    def run_posterior(self, stream=None, locked=None):
        """``locked`` replaces the lock-flag buffer for this call (in/out)."""
        p = self.workload.post
        dlm_posterior(self.logits, self.prev, self.locked if locked is None else locked, p.eps,
                      self.select, self.sel, self.kl, self.conf, p.R, p.V, stream)

    def run(self, stream=None, locked=None, overlap=False):
        """One step.  With overlap, the posterior runs on a second stream and
        only its selection waits for the column sums (select.score_ready,
        for the modes that rank by them);
        the calling stream then waits for the posterior.  overlap=True
        starts its logit stream with the attention passes; overlap="pass1"
        starts it once pass 1 is done (mask_desc.pass1_done), beside the
        column-sum pass only."""
        if not (overlap and self.with_posterior):
            self.run_attn(stream)
            if self.with_posterior:
                self.run_posterior(stream, locked)
            return
        main = stream if stream is not None else torch.cuda.current_stream()
        if not hasattr(self, "_side"):
            # one side stream per device, shared by every step object: many
            # streams would spread over the few hardware queues
            if main.device not in _SIDE_STREAMS:
                _SIDE_STREAMS[main.device] = torch.cuda.Stream(device=main.device)
            self._side = _SIDE_STREAMS[main.device]
            self._ev_start, self._ev_cs, self._ev_post, self._ev_p1 = (torch.cuda.Event() for _ in range(4))
            self._ev_p1.record(main)                   # created once; the library records it
        if overlap == "pass1":
            self.md.pass1_done = self._ev_p1
            try:
                self.run_attn(main)
            finally:
                self.md.pass1_done = None
            self._side.wait_event(self._ev_p1)     # out / lse final; the column sums still running
        else:
            self._ev_start.record(main)
            self._side.wait_event(self._ev_start)  # prior work on the calling stream first
            self.run_attn(main)
        self._ev_cs.record(main)                   # column sums ready
        # only a selection that ranks by the column sums waits for them (the
        # others also keep the one-launch posterior where it applies)
        by_score = self.workload.post.mode in (3, 4)
        self.select.score_ready = self._ev_cs if by_score else None
        try:
            self.run_posterior(self._side, locked)
        finally:
            self.select.score_ready = None
        self._ev_post.record(self._side)
        main.wait_event(self._ev_post)

    def results(self) -> dict:
        torch.cuda.synchronize()
        r = {"out": bf16_to_host(self.out), "lse": self.lse.cpu().numpy(),
             "cache_k": bf16_to_host(self.cache_k), "cache_v": bf16_to_host(self.cache_v)}
        if self.colsum is not None:
            r["colsum"] = self.colsum.cpu().numpy()
        if self.with_posterior:
            r.update(sel=self.sel.cpu().numpy(), kl=self.kl.cpu().numpy(),
                     conf=self.conf.cpu().numpy(), locked=self.locked.cpu().numpy())
            if self.with_scores:
                r.update(margin=self.margin.cpu().numpy(), entropy=self.entropy.cpu().numpy())
            if self.score is not None:
                r["score"] = self.score.cpu().numpy()
        return r
