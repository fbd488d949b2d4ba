"""The allocation-free posterior (dlm_posterior_noalloc) against
dlm_posterior, through the C ABI, on the same seeded inputs.

Both run the same kernels; only where the per-(row, chunk) partials live
differs (the library's own device array against the caller's workspace),
so every output must agree bit for bit.  Two calls in a row, the second on
a smaller problem, check that the array keeps no state a later call could
read; the second workload also ranks by a score and asks for margin and
entropy (the other stream-kernel variant).  The outputs are also checked
against the oracle to the parity tolerances.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import check_posterior, check_selection

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


CASES = [
    # larger first, then a smaller one: V not a multiple of 4, selection by score
    dict(name="noalloc_topk_conf", R=768, V=50000, logit_std=3.0, noise_std=0.05, eps=1e-3,
         mode=W.SEL_TOPK_CONF, k=8, group_rows=64, locked_frac=0.2, seed=11),
    dict(name="noalloc_topk_score", R=100, V=5003, logit_std=2.0, noise_std=0.05, eps=1e-3,
         mode=W.SEL_TOPK_SCORE, k=5, group_rows=25, locked_frac=0.1, score_std=1.0, seed=12),
]


def _run(dlm, p, fn, with_scores):
    dev = torch.device("cuda")
    x = torch.from_numpy(p.logits).to(dev)
    y = torch.from_numpy(p.prev).to(dev)
    locked = torch.from_numpy(np.ascontiguousarray(p.locked, np.uint8)).to(dev)
    sel = torch.full((p.R,), -7, dtype=torch.int32, device=dev)
    kl = torch.full((p.R,), float("nan"), device=dev)
    conf = torch.full((p.R,), float("nan"), device=dev)
    margin = torch.full((p.R,), float("nan"), device=dev) if with_scores else None
    entropy = torch.full((p.R,), float("nan"), device=dev) if with_scores else None
    score = torch.from_numpy(p.score).to(dev) if p.score is not None else None
    s = dlm.Select(mode=p.mode, k=p.k, group_rows=p.group_rows, tau=p.tau, score=score,
                   margin=margin, entropy=entropy)
    if fn is dlm.dlm_posterior:
        s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(p.R, p.V, s)), dtype=torch.uint8,
                                  device=dev)
    fn(x, y, locked, p.eps, s, sel, kl, conf, p.R, p.V)
    torch.cuda.synchronize()
    out = dict(sel=sel.cpu().numpy(), kl=kl.cpu().numpy(), conf=conf.cpu().numpy(),
               locked=locked.cpu().numpy())
    if with_scores:
        out.update(margin=margin.cpu().numpy(), entropy=entropy.cpu().numpy())
    return out


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd as dlm
    for i, c in enumerate(CASES):
        c = dict(c)
        name = c.pop("name")
        p = W.make_post(name, **c)
        assert dlm.dlm_posterior_workspace_bytes(p.R, p.V, dlm.Select(mode=p.mode, k=p.k, group_rows=p.group_rows)) \
            <= dlm.NOALLOC_SCRATCH_BYTES
        with_scores = i == 1
        _say(f"case: {name} R={p.R} V={p.V} mode={p.mode} (call {i + 1} of the no-alloc entry point)")
        got = _run(dlm, p, dlm.dlm_posterior_noalloc, with_scores)
        ref = _run(dlm, p, dlm.dlm_posterior, with_scores)
        for k in ref:
            assert np.array_equal(got[k].view(np.uint32) if got[k].dtype == np.float32 else got[k],
                                  ref[k].view(np.uint32) if ref[k].dtype == np.float32 else ref[k]), k
        # and both against the oracle, to the parity tolerances
        ora = oracle.posterior(p.logits, p.prev, p.locked, p.eps)
        check_posterior(got["kl"], got["conf"], got["locked"], ora["kl"], ora["conf"], ora["locked"], p.eps,
                        p.locked)
        sel_o = oracle.select(p.mode, p.k, p.group_rows, p.tau, p.score, ora["conf"], ora["tok"], p.locked)
        check_selection(got["sel"], sel_o, p.mode, p.group_rows, p.tau, ora["conf"], p.score, p.locked,
                        p.logits)
        assert (got["sel"] >= 0).sum() > 0


def test_noalloc_rejects_a_problem_past_its_array():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd as dlm
    R, V = 200000, 4096
    dev = torch.device("cuda")
    x = torch.empty((R, V), device=dev)
    s = dlm.Select(mode=dlm.SEL_NONE)
    outs = [torch.empty(R, dtype=dt, device=dev) for dt in (torch.int32, torch.float32, torch.float32)]
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_posterior_noalloc(x, x, torch.zeros(R, dtype=torch.uint8, device=dev), 1e-3, s, *outs, R, V)
    assert e.value.code == dlm.DLM_E_WORKSPACE
