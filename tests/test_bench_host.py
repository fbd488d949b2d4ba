"""Host-side checks of bench.py (no GPU).

- The one-GPU contract: any --gpus other than 1 exits with a message and
  status 2 before anything touches a GPU.
- The algorithmic work bench.py reports (the numerator of the pass-1 and
  pass-2 rooflines) counts exactly the (query, key) pairs the mask makes
  visible: checked against the oracle's own visibility predicate pair by
  pair, for every mask kind, DUMMY slots, row subsets that feed the column
  sums and several batches with different active sets.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def _brute_pairs(a, counted_only=False):
    tot = 0
    for b in range(a.B):
        for pos in a.active_idx[b]:
            if counted_only and not (a.cs_lo <= pos < a.cs_hi):
                continue
            tot += sum(oracle.visible(a, b, int(pos), n) for n in range(a.kv_len))
    return tot * a.Hq


def _case(kind, slots, groups, act_blocks, B=2, P=40, block=8, cs=None):
    """kind with n_slots slot states ``slots`` and groups ``groups`` (per
    batch rows); active rows: the positions of the slots in act_blocks[b]."""
    n_slots = slots.shape[1]
    kv_len = P + n_slots * block
    act = [np.concatenate([np.arange(P + s * block, P + (s + 1) * block) for s in act_blocks[b]])
           for b in range(B)]
    m = max(len(x) for x in act)
    assert all(len(x) == m for x in act)
    lo, hi = cs if cs is not None else (0, kv_len)
    return W.make_attn("bench_pairs", B=B, Hq=3, Hkv=1, D=32, kv_len=kv_len, prefix_len=P,
                       active_idx=np.stack(act).astype(np.int32), kind=kind, block_size=block,
                       n_slots=n_slots, slot_state=slots, slot_group=groups, cs_lo=lo, cs_hi=hi)


CASES = {
    "full": lambda: W.tiny().attn,
    "block_causal": lambda: _case(W.MASK_BLOCK_CAUSAL,
                                  np.full((2, 4), W.SLOT_ACTIVE, np.uint8),
                                  np.zeros((2, 4), np.int32), [[0, 1, 3], [1, 2, 3]],
                                  cs=(48, 72)),
    "group_dummy": lambda: _case(W.MASK_GROUP,
                                 np.array([[1, 1, 1, 0], [1, 0, 1, 1]], np.uint8),
                                 np.array([[0, 0, 1, 0], [2, 0, 1, 2]], np.int32),
                                 [[0, 1, 2], [0, 2, 3]], cs=(40, 64)),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("counted_only", [False, True])
def test_visible_pairs_match_the_oracle_mask(name, counted_only):
    a = CASES[name]()
    assert bench.visible_pairs(a, counted_only=counted_only) == _brute_pairs(a, counted_only)


def test_stored_traffic_is_dropped_when_the_pass1_sources_change(tmp_path, monkeypatch):
    """roofline.traffic comes from a committed counter summary only while the
    digest of the pass-1 sources it records matches the sources."""
    for rel in bench.TRAFFIC_SOURCES:
        f = tmp_path / rel
        f.parent.mkdir(parents=True, exist_ok=True)
        f.write_text("source " + rel + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "attn_fwd_w_counters.md"
    summary.write_text("# counters\n\n- kernel: `k`\n"
                       f"- source_sha256: `{bench.source_digest()}`\n"
                       "- traffic_bytes_per_launch: 12345\n")
    assert bench.stored_traffic("w") == 12345
    assert bench.stored_traffic("other") is None           # no summary for it
    (tmp_path / bench.TRAFFIC_SOURCES[0]).write_text("changed\n")
    assert bench.stored_traffic("w") is None                # kernel changed since


def test_trace_and_counter_summaries(tmp_path):
    """The rocprofv3 CSV summarisers: per-kernel mean / median durations, and
    per-dispatch counter values summed over a counter's instances."""
    trace = tmp_path / "kernel_trace.csv"
    trace.write_text("Kind,Kernel_Name,Start_Timestamp,End_Timestamp\n"
                     "KERNEL_DISPATCH,kA,1000,3000\nKERNEL_DISPATCH,kA,5000,6000\n"
                     "KERNEL_DISPATCH,kA,7000,17000\nKERNEL_DISPATCH,kB,0,500\n")
    t = bench.summarize_trace(str(trace))
    assert "| `kA` | 3 | 4.33 | 2.00 | 1.00 | 10.00 | 13.0 |" in t
    assert "| `kB` | 1 | 0.50 | 0.50 |" in t
    pmc = tmp_path / "counter_collection.csv"
    pmc.write_text("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
                   "1,kA,FETCH_SIZE,10\n1,kA,FETCH_SIZE,5\n2,kA,FETCH_SIZE,20\n2,kA,FETCH_SIZE,5\n"
                   "3,kB,FETCH_SIZE,7\n")
    s = bench.summarize_pmc(str(pmc))
    assert "| `kA` | FETCH_SIZE | 2 | 20 | 20 | 15 | 25 |" in s
    assert "| `kB` | FETCH_SIZE | 1 | 7 |" in s


def test_loop_trace_summary(tmp_path):
    """The --loop trace summariser: runs split at the Block Buffer
    initialisations, per-step kernel sums of the last run (a column for each
    step kernel the trace holds), and the gaps around and inside each step
    (in microseconds)."""
    K = "void dlm::(anonymous namespace)::{}(dlm::X)"
    ev = [("block_buffer_kernel", 0, 1000),                      # run 1: initialisation
          ("feed", 2000, 3000),
          ("attn_fwd_kernel", 4000, 6000), ("posterior_stream_kernel", 6000, 9000),
          ("block_buffer_kernel", 9500, 10500),                  # step 1 of run 1 (0.5 us inside)
          ("feed", 11500, 12000),
          ("block_buffer_kernel", 13000, 14000),                 # run 2: initialisation
          ("feed", 15000, 16000),
          ("attn_fwd_kernel", 18000, 19000), ("posterior_finish_kernel", 19000, 21000),
          ("block_buffer_kernel", 21000, 22000),                 # step 1 of run 2
          ("feed", 30000, 31000)]
    trace = tmp_path / "kernel_trace.csv"
    trace.write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n" +
                     "".join(f"\"{K.format(n)}\",{a},{b}\n" for n, a, b in ev))
    t = bench.summarize_loop_trace(str(trace))
    # columns: the step kernels the trace holds (attn_fwd, posterior_stream,
    # posterior_finish, block_buffer)
    assert "| step | attn_fwd | posterior_stream | posterior_finish | block_buffer | sum |" in t
    assert "| 1 | 1.0 | 0.0 | 2.0 | 1.0 | 4.0 |" in t
    assert "| 1 | 1 | 0.006 | 0.5 | 1.00 | 1.00 |" in t
    assert "| 2 | 1 | 0.004 | 0.0 | 2.00 | 8.00 |" in t


def test_stored_counters_follow_the_kernel_sources(tmp_path, monkeypatch):
    for tag in bench.COUNTER_SOURCES:
        for rel in bench.COUNTER_SOURCES[tag]:
            f = tmp_path / rel
            f.parent.mkdir(parents=True, exist_ok=True)
            f.write_text("source " + rel + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "posterior_w_counters.md").write_text(
        "# counters\n\n- kernel: `k`\n"
        f"- source_sha256: `{bench.source_digest('posterior')}`\n"
        "- traffic_bytes_per_launch: 4096\n- fetch_scale: 1.9998\n")
    c = bench.stored_counters("posterior", "w")
    assert c["traffic_bytes_per_launch"] == 4096 and c["fetch_scale"] == 1.9998
    assert bench.stored_counters("attn_fwd", "w") is None
    (tmp_path / bench.COUNTER_SOURCES["posterior"][0]).write_text("changed\n")
    assert bench.stored_counters("posterior", "w") is None
