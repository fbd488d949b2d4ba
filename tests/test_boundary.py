"""The C-ABI library: loads, exports every declared entry point, sizes its
workspaces, and rejects bad arguments on the host before enqueuing work.

No GPU is needed: every call here fails validation (or is a workspace query)
before any HIP call, so the dummy device addresses are never dereferenced.
"""
import os
import re

import pytest

import denoising_step_amd as dlm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000          # a 16-byte aligned dummy device address, never dereferenced


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            with open(os.path.join(ROOT, "include", fn)) as f:
                text = f.read()
            names |= set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(dlm_\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert declared == set(dlm.EXPORTS), declared
    for name in declared:
        assert hasattr(dlm.lib, name), name


def _kv(B=2, Hkv=2, n_cap=128, D=64):
    return dlm.KVCache(FAKE, FAKE, B, Hkv, n_cap, D)


def _md(**kw):
    base = dict(kind=dlm.MASK_FULL, Hq=4, M=16, kv_len=100, prefix_len=10, cs_lo=0, cs_hi=100)
    base.update(kw)
    return dlm.MaskDesc(**base)


def _attn(kv=None, md=None, q=FAKE, k=FAKE, v=FAKE, active=FAKE, out=FAKE, lse=FAKE, colsum=FAKE):
    kv = kv or _kv()
    md = md or _md()
    if md.workspace is None:
        md.workspace = FAKE
        try:
            md.workspace_bytes = dlm.dlm_step_attn_workspace_bytes(kv, md)
        except dlm.DlmError:
            md.workspace_bytes = 1 << 40
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_step_attn(q, k, v, kv, active, md, out, lse, colsum, stream=0)
    return e.value.code


def test_workspace_queries():
    n = dlm.dlm_step_attn_workspace_bytes(_kv(), _md())
    assert n > 0 and n % 256 == 0
    # the long-prefix shape uses key splits: partial outputs need room
    long_kv = dlm.KVCache(FAKE, FAKE, 1, 32, 16640, 128)
    n_long = dlm.dlm_step_attn_workspace_bytes(long_kv, _md(Hq=32, M=256, kv_len=16640, prefix_len=16384))
    assert n_long >= 32 * 256 * 128 * 4 * 2
    s = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=4, group_rows=16)
    assert dlm.dlm_posterior_workspace_bytes(16, 512, s) >= 16 * 32
    assert dlm.dlm_posterior_workspace_bytes(0, 512, s) == 0
    # a live-row list sizes the partials for the largest split any count can choose
    big = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=16, group_rows=1024)
    live = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=16, group_rows=1024, live_rows=FAKE, n_live=FAKE)
    # every layout starts with the 32 KiB block of arrival counters
    ctr = 2 * 4096 * 4
    assert dlm.dlm_posterior_workspace_bytes(1024, 126464, big) == ctr + 1024 * 4 * 48
    assert dlm.dlm_posterior_workspace_bytes(1024, 126464, live) == ctr + 1024 * 31 * 48
    # groups of at most 256 rows: room for either path, here the two-launch
    # layout (4 chunks a row) is the larger (the one-launch one: per-row
    # results and 2 chunks a row)
    fz = dlm.Select(mode=dlm.SEL_TOPK_SCORE, k=16, group_rows=256, score=FAKE)
    assert dlm.dlm_posterior_workspace_bytes(256, 151936, fz) == max(ctr + 256 * 4 * 48, ctr + 256 * 16 + 256 * 2 * 48)


def test_posterior_path_per_workload_shape():
    """The posterior workspace covers both paths' layouts for the bench
    shapes: the two-launch split (about sixteen workgroups per CU, capped
    for LDS staging) and the one-launch split (about two workgroups per
    CU, whole streaming steps, 16-byte per-row results before the
    partials), both after the 32 KiB counter block."""
    ctr = 2 * 4096 * 4
    res = lambda R: (R * 16 + 255) // 256 * 256
    both = lambda R, nc2, nc1: max(ctr + R * nc2 * 48, ctr + res(R) + R * nc1 * 48)
    # LLaDA-like layer: 31 chunks a row for two launches, 16 for one
    s = dlm.Select(mode=dlm.SEL_ATTN_DYNAMIC, tau=0.9, group_rows=32, score=FAKE)
    assert dlm.dlm_posterior_workspace_bytes(32, 126464, s) == both(32, 31, 16)
    # long-prefix sampler: 4 chunks / 2 chunks
    s = dlm.Select(mode=dlm.SEL_TOPK_SCORE, k=16, group_rows=256, score=FAKE)
    assert dlm.dlm_posterior_workspace_bytes(256, 151936, s) == both(256, 4, 2)
    # multi-block: 4 chunks / whole rows
    s = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=8, group_rows=32)
    assert dlm.dlm_posterior_workspace_bytes(1024, 151936, s) == both(1024, 4, 1)
    # SureLock: whole rows on both paths
    s = dlm.Select(mode=dlm.SEL_NONE)
    assert dlm.dlm_posterior_workspace_bytes(8192, 126464, s) == both(8192, 1, 1)
    # a group of more than 256 rows: two launches only (2 chunks: V spans two steps)
    s = dlm.Select(mode=dlm.SEL_TOPK_CONF, k=8, group_rows=512)
    assert dlm.dlm_posterior_workspace_bytes(512, 8192, s) == ctr + 512 * 2 * 48


@pytest.mark.parametrize("case,code", [
    (dict(kv=_kv(D=48)), dlm.DLM_E_UNSUPPORTED),
    (dict(md=_md(Hq=3)), dlm.DLM_E_UNSUPPORTED),
    (dict(kv=_kv(B=0)), dlm.DLM_E_SHAPE),
    (dict(md=_md(kv_len=129)), dlm.DLM_E_SHAPE),
    (dict(md=_md(kv_len=0)), dlm.DLM_E_SHAPE),
    (dict(md=_md(prefix_len=101)), dlm.DLM_E_SHAPE),
    (dict(md=_md(prefix_len=-1)), dlm.DLM_E_SHAPE),
    (dict(md=_md(M=91)), dlm.DLM_E_SHAPE),
    (dict(md=_md(M=-1)), dlm.DLM_E_SHAPE),
    # 32-bit byte offsets per (batch, kv-head) slice: kv_len * D * 2 must stay below 2 GiB
    (dict(kv=_kv(B=1, Hkv=1, n_cap=1 << 24, D=128), md=_md(Hq=1, kv_len=(1 << 23) + 64, prefix_len=0)),
     dlm.DLM_E_SHAPE),
    (dict(md=_md(kind=7)), dlm.DLM_E_DESC),
    (dict(md=_md(kind=dlm.MASK_BLOCK_CAUSAL, block_size=0)), dlm.DLM_E_DESC),
    (dict(md=_md(kind=dlm.MASK_GROUP, block_size=16, n_slots=0, slot_state=FAKE, slot_group=FAKE)), dlm.DLM_E_DESC),
    (dict(md=_md(kind=dlm.MASK_GROUP, block_size=16, n_slots=2000, slot_state=FAKE, slot_group=FAKE)), dlm.DLM_E_DESC),
    (dict(md=_md(kind=dlm.MASK_GROUP, block_size=16, n_slots=6)), dlm.DLM_E_NULL),
    (dict(md=_md(kind=dlm.MASK_GROUP, block_size=16, n_slots=5, slot_state=FAKE, slot_group=FAKE)), dlm.DLM_E_DESC),
    (dict(md=_md(cs_lo=50, cs_hi=40)), dlm.DLM_E_DESC),
    (dict(md=_md(colsum_per_head=2)), dlm.DLM_E_DESC),
    (dict(md=_md(colsum_accumulate=2)), dlm.DLM_E_DESC),
    (dict(md=_md(scale=-1.0)), dlm.DLM_E_DESC),
    (dict(md=_md(scale=float("nan"))), dlm.DLM_E_DESC),
    (dict(q=None), dlm.DLM_E_NULL),
    (dict(active=None), dlm.DLM_E_NULL),
    (dict(out=None), dlm.DLM_E_NULL),
    (dict(lse=None), dlm.DLM_E_NULL),
    (dict(kv=dlm.KVCache(None, FAKE, 2, 2, 128, 64)), dlm.DLM_E_NULL),
    (dict(v=None), dlm.DLM_E_NULL),
    (dict(q=FAKE + 2), dlm.DLM_E_SHAPE),
    (dict(out=FAKE + 8), dlm.DLM_E_SHAPE),
])
def test_step_attn_rejects(case, code):
    assert _attn(**case) == code
    assert dlm.dlm_last_error() != ""


def test_step_attn_workspace_checked():
    md = _md()
    md.workspace = None
    md.workspace_bytes = 0
    md2 = _md()
    md2.workspace = FAKE
    md2.workspace_bytes = dlm.dlm_step_attn_workspace_bytes(_kv(), md2) - 1
    for m in (md, md2):
        with pytest.raises(dlm.DlmError) as e:
            dlm.dlm_step_attn(FAKE, FAKE, FAKE, _kv(), FAKE, m, FAKE, FAKE, FAKE, stream=0)
        assert e.value.code == dlm.DLM_E_WORKSPACE


def test_null_descriptors():
    import ctypes
    rc = dlm.lib.dlm_step_attn(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, None)
    assert rc == dlm.DLM_E_NULL
    n = ctypes.c_size_t(0)
    assert dlm.lib.dlm_posterior_workspace_bytes(4, 4, None, ctypes.byref(n)) == dlm.DLM_E_NULL
    assert dlm.lib.dlm_posterior(FAKE, FAKE, FAKE, 1e-3, None, FAKE, FAKE, FAKE, 4, 4, None) == dlm.DLM_E_NULL


def _post(R=16, V=512, sel=None, logits=FAKE, prev=FAKE, locked=FAKE, out=FAKE, eps=1e-3, ws=True):
    sel = sel or dlm.Select(mode=dlm.SEL_TOPK_CONF, k=4, group_rows=16)
    if ws and sel.workspace is None and R >= 0 and V >= 1:
        try:
            sel.workspace_bytes = dlm.dlm_posterior_workspace_bytes(R, V, sel)
            sel.workspace = FAKE
        except dlm.DlmError:
            pass
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_posterior(logits, prev, locked, eps, sel, out, FAKE, FAKE, R, V, stream=0)
    return e.value.code


@pytest.mark.parametrize("case,code", [
    (dict(R=-1), dlm.DLM_E_SHAPE),
    (dict(V=0), dlm.DLM_E_SHAPE),
    (dict(sel=dlm.Select(mode=9)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=7)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_MARGIN, k=-1, group_rows=16)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_LOW_ENTROPY, k=-3, group_rows=16)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_CONF, k=2, group_rows=0)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_CONF, k=2, group_rows=1025)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_CONF, k=-1, group_rows=16)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_THRESH_CONF, group_rows=16, tau=float("nan"))), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_ATTN_DYNAMIC, group_rows=16, tau=0.9)), dlm.DLM_E_NULL),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_SCORE, k=3, group_rows=16)), dlm.DLM_E_NULL),
    (dict(logits=None), dlm.DLM_E_NULL),
    (dict(prev=None), dlm.DLM_E_NULL),
    (dict(locked=None), dlm.DLM_E_NULL),
    (dict(out=None), dlm.DLM_E_NULL),
    (dict(eps=float("nan")), dlm.DLM_E_DESC),
    (dict(logits=FAKE + 4), dlm.DLM_E_SHAPE),
    (dict(ws=False), dlm.DLM_E_WORKSPACE),
])
def test_posterior_rejects(case, code):
    assert _post(**case) == code


def _post_noalloc(R=16, V=512, sel=None, logits=FAKE, prev=FAKE, locked=FAKE, out=FAKE, eps=1e-3):
    sel = sel or dlm.Select(mode=dlm.SEL_TOPK_CONF, k=4, group_rows=16)
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_posterior_noalloc(logits, prev, locked, eps, sel, out, FAKE, FAKE, R, V, stream=0)
    return e.value.code


@pytest.mark.parametrize("case,code", [
    (dict(R=-1), dlm.DLM_E_SHAPE),
    (dict(V=0), dlm.DLM_E_SHAPE),
    (dict(sel=dlm.Select(mode=9)), dlm.DLM_E_DESC),
    (dict(sel=dlm.Select(mode=dlm.SEL_TOPK_SCORE, k=3, group_rows=16)), dlm.DLM_E_NULL),
    (dict(logits=None), dlm.DLM_E_NULL),
    (dict(out=None), dlm.DLM_E_NULL),
    (dict(eps=float("nan")), dlm.DLM_E_DESC),
    (dict(logits=FAKE + 4), dlm.DLM_E_SHAPE),
    # partials past the scratch array: 200000 rows of one chunk, 48 B each
    (dict(R=200000, V=4096, sel=dlm.Select(mode=dlm.SEL_NONE)), dlm.DLM_E_WORKSPACE),
])
def test_posterior_noalloc_rejects(case, code):
    """The allocation-free posterior checks what dlm_posterior checks, and
    rejects a problem whose partials do not fit its array, before any HIP
    call (the workspace fields are ignored)."""
    assert _post_noalloc(**case) == code
    assert dlm.dlm_last_error() != ""
    big = dlm.dlm_posterior_workspace_bytes(200000, 4096, dlm.Select(mode=dlm.SEL_NONE))
    assert big > dlm.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_the_header():
    with open(os.path.join(ROOT, "include", "dlm_step.h")) as f:
        m = re.search(r"#define DLM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == dlm.NOALLOC_SCRATCH_BYTES


def test_oracle_and_library_share_no_code():
    """The GPU sources and the oracle neither include nor import each other."""
    csrc = os.path.join(ROOT, "denoising_step_amd", "csrc")
    for fn in os.listdir(csrc):
        with open(os.path.join(csrc, fn)) as f:
            assert "oracle" not in f.read().lower(), fn
    pkg = os.path.join(ROOT, "denoising_step_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            with open(os.path.join(pkg, fn)) as f:
                text = f.read()
            assert "import oracle" not in text and "from oracle" not in text, fn
    with open(os.path.join(ROOT, "oracle", "dlm_oracle.c")) as f:
        src = f.read()
    assert "dlm_step.h" not in src and "dlm_internal.h" not in src


def test_single_hip_runtime():
    """The library binds to the HIP runtime that PyTorch loaded: one runtime
    in the process, whatever was imported first."""
    import subprocess
    import sys
    code = ("import denoising_step_amd as d; print(len(d._hip_runtimes()))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip()
    assert out == "1", out


def _bb(**kw):
    base = dict(B=2, n_slots=4, block_size=16, max_active=2, prefix_len=32)
    base.update(kw)
    arrays = {f: FAKE for f in ("slot_state", "slot_group", "decoded", "tokens", "locked", "skip",
                                "row_flags", "active_idx", "m_active", "n_open")}
    for f in list(arrays):
        if f in kw:
            arrays[f] = kw.pop(f)
            base.pop(f, None)
    return dlm.BlockBuffer(**base, **arrays)


@pytest.mark.parametrize("case,code", [
    (dict(B=0), dlm.DLM_E_SHAPE),
    (dict(n_slots=0), dlm.DLM_E_SHAPE),
    (dict(n_slots=1025), dlm.DLM_E_SHAPE),
    (dict(block_size=0), dlm.DLM_E_SHAPE),
    (dict(max_active=0), dlm.DLM_E_SHAPE),
    (dict(prefix_len=-1), dlm.DLM_E_SHAPE),
    (dict(n_slots=1024, block_size=1 << 15), dlm.DLM_E_SHAPE),
    (dict(slot_state=None), dlm.DLM_E_NULL),
    (dict(active_idx=None), dlm.DLM_E_NULL),
    (dict(n_open=None), dlm.DLM_E_NULL),
])
def test_block_buffer_rejects(case, code):
    bb = _bb(**case)
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_block_buffer_init(bb, stream=0)
    assert e.value.code == code
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_block_buffer_advance(bb, FAKE, stream=0)
    assert e.value.code == code


def test_block_buffer_advance_needs_sel():
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_block_buffer_advance(_bb(), None, stream=0)
    assert e.value.code == dlm.DLM_E_NULL
    import ctypes
    assert dlm.lib.dlm_block_buffer_init(None, None) == dlm.DLM_E_NULL
    assert dlm.lib.dlm_block_buffer_advance(None, FAKE, None) == dlm.DLM_E_NULL


def _layer(**kw):
    base = dict(B=2, n_pos=100, d=256, M=40, active_idx=FAKE, Hq=4, Hkv=2, D=64, F=384)
    base.update(kw)
    return dlm.LayerDesc(**base)


@pytest.mark.parametrize("case,code", [
    (dict(B=0), dlm.DLM_E_SHAPE),
    (dict(d=0), dlm.DLM_E_SHAPE),
    (dict(M=-1), dlm.DLM_E_SHAPE),
    (dict(d=100), dlm.DLM_E_UNSUPPORTED),
    (dict(F=100), dlm.DLM_E_UNSUPPORTED),
    (dict(Hq=3), dlm.DLM_E_UNSUPPORTED),
    (dict(n_pos=1 << 20, d=4096), dlm.DLM_E_SHAPE),
    (dict(active_idx=None), dlm.DLM_E_NULL),
])
def test_layer_calls_reject(case, code):
    L = _layer(**case)
    for call in (lambda: dlm.dlm_proj_qkv(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
                 lambda: dlm.dlm_proj_out(L, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
                 lambda: dlm.dlm_ffn(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
                 lambda: dlm.dlm_layer_workspace_bytes(L)):
        with pytest.raises(dlm.DlmError) as e:
            call()
        assert e.value.code == code


def test_layer_call_specific_checks():
    with pytest.raises(dlm.DlmError) as e:          # heads of 32 do not tile the K steps of 64
        dlm.dlm_proj_out(_layer(D=32), FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == dlm.DLM_E_UNSUPPORTED
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_proj_qkv(_layer(), FAKE, None, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.code == dlm.DLM_E_NULL
    L = _layer()
    need = dlm.dlm_layer_workspace_bytes(L)
    assert need >= 2 * 40 * 384 * 2           # at least the gated hidden rows
    import ctypes
    c = dlm._c_layer(L)
    rc = dlm.lib.dlm_ffn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert rc == dlm.DLM_E_WORKSPACE
    # over 16 rows, few output tiles and a long K: K is split and the
    # projections need partial sums too (up to 16 rows one workgroup takes
    # the whole K: no partials, only the gated rows and the packed rows of h)
    assert dlm.dlm_layer_workspace_bytes(_layer(d=1024, M=8)) == 16 * 384 * 2 + 16 * 1024 * 2
    c = dlm._c_layer(_layer(d=1024, M=40))
    assert dlm.lib.dlm_proj_qkv(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == \
        dlm.DLM_E_WORKSPACE
    c = dlm._c_layer(_layer(Hq=16, Hkv=2, M=40))         # K = Hq D = 1024
    assert dlm.lib.dlm_proj_out(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == \
        dlm.DLM_E_WORKSPACE
    assert dlm.lib.dlm_proj_qkv(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == dlm.DLM_E_NULL


def test_pack_weights_rejects():
    lib = dlm.lib
    assert lib.dlm_pack_weights(FAKE, FAKE + (1 << 24), 24, 64, None) == dlm.DLM_E_UNSUPPORTED   # N % 16
    assert lib.dlm_pack_weights(FAKE, FAKE + (1 << 24), 32, 48, None) == dlm.DLM_E_UNSUPPORTED   # K % 32
    assert lib.dlm_pack_weights(FAKE, FAKE + (1 << 24), -16, 64, None) == dlm.DLM_E_SHAPE
    assert lib.dlm_pack_weights(FAKE, FAKE + (1 << 24), 1 << 16, 1 << 15, None) == dlm.DLM_E_SHAPE
    assert lib.dlm_pack_weights(None, FAKE, 32, 64, None) == dlm.DLM_E_NULL
    assert lib.dlm_pack_weights(FAKE, FAKE + 1024, 32, 64, None) == dlm.DLM_E_DESC             # overlap
    assert lib.dlm_pack_weights(None, None, 0, 64, None) == dlm.DLM_OK                           # nothing to do
    assert dlm.dlm_layer_workspace_bytes(_layer(weights_packed=True)) == dlm.dlm_layer_workspace_bytes(_layer())
    c = dlm._c_layer(_layer())
    c.weights_packed = 2
    n = __import__("ctypes").c_size_t(0)
    assert lib.dlm_layer_workspace_bytes(__import__("ctypes").byref(c), __import__("ctypes").byref(n)) == \
        dlm.DLM_E_DESC


def test_posterior_live_rows_need_a_count():
    import ctypes
    s = dlm._c_sel(dlm.Select(mode=dlm.SEL_TOPK_CONF, k=4, group_rows=16, live_rows=FAKE))
    s.workspace, s.workspace_bytes = FAKE, 1 << 20
    rc = dlm.lib.dlm_posterior(FAKE, FAKE, FAKE, 1e-3, ctypes.byref(s), FAKE, FAKE, FAKE, 16, 512, None)
    assert rc == dlm.DLM_E_NULL


def test_posterior_rejects_nan_gate():
    assert _post(sel=dlm.Select(mode=dlm.SEL_TOPK_CONF, k=2, group_rows=16, conf_gate=float("nan"))) \
        == dlm.DLM_E_DESC


@pytest.mark.parametrize("case,code", [
    (dict(B=0), dlm.DLM_E_SHAPE),
    (dict(E=0), dlm.DLM_E_SHAPE),
    (dict(L=-1), dlm.DLM_E_SHAPE),
    (dict(N=12), dlm.DLM_E_UNSUPPORTED),
    (dict(N=4), dlm.DLM_E_UNSUPPORTED),
    (dict(E=60), dlm.DLM_E_UNSUPPORTED),
    (dict(gate=float("inf")), dlm.DLM_E_DESC),
    (dict(u=None), dlm.DLM_E_NULL),
    (dict(y=None, x=None), dlm.DLM_E_NULL),
    (dict(Bm=FAKE + 8), dlm.DLM_E_SHAPE),
])
def test_r2l_scan_rejects(case, code):
    args = dict(B=2, L=16, E=64, N=16, gate=0.5, u=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, D=FAKE,
                y=FAKE, x=None)
    args.update(case)
    with pytest.raises(dlm.DlmError) as e:
        dlm.dlm_r2l_scan(stream=0, **args)
    assert e.value.code == code
