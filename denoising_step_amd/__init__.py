"""MI355X-native denoising step: Python binding of libdlm_step.so.

The binding only marshals arguments into the C ABI of include/dlm_step.h
(``dlm_step_attn``, ``dlm_posterior``, their workspace queries and the Block
Buffer calls ``dlm_block_buffer_init`` / ``dlm_block_buffer_advance``); every
step of the computation runs in the library's HIP kernels.  Tensors are
PyTorch device tensors, used for memory and streams only.  It checks tensor
shapes, dtypes and contiguity against the declared sizes so that a
mis-sized tensor can never reach a kernel.

There is no fallback: if the library is not built, importing this package
raises ImportError.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlm_step.so")

DLM_OK, DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED, DLM_E_DESC, DLM_E_WORKSPACE, DLM_E_HIP = \
    0, -1, -2, -3, -4, -5, -6
MASK_FULL, MASK_BLOCK_CAUSAL, MASK_GROUP = 0, 1, 2
SLOT_DUMMY, SLOT_ACTIVE, SLOT_TO_CACHE, SLOT_IN_CACHE = 0, 1, 2, 3
SEL_NONE, SEL_TOPK_CONF, SEL_THRESH_CONF, SEL_ATTN_DYNAMIC, SEL_TOPK_SCORE = 0, 1, 2, 3, 4
SEL_TOPK_MARGIN, SEL_TOPK_LOW_ENTROPY = 5, 6
ROW_SELECT, ROW_LOCK = 1, 2

EXPORTS = ("dlm_step_attn", "dlm_step_attn_workspace_bytes", "dlm_posterior",
           "dlm_posterior_workspace_bytes", "dlm_posterior_noalloc", "dlm_block_buffer_init", "dlm_block_buffer_advance",
           "dlm_proj_qkv", "dlm_proj_out", "dlm_ffn", "dlm_layer_workspace_bytes", "dlm_pack_weights",
           "dlm_r2l_scan",
           "dlm_last_error")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950)")

# PyTorch ships its own HIP runtime.  The library must bind to that same
# runtime (it is linked against the soname libamdhip64.so.7, which torch's
# copy carries), so torch is imported first; loading the library first would
# map a second HIP runtime into the process and torch's streams would be
# handed to the wrong one.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are mapped into this process "
                      f"({_hip_runtimes()}); import torch before loading libdlm_step")


class DlmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class _KVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("n_cap", ctypes.c_int32), ("D", ctypes.c_int32)]


class _MaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("Hq", ctypes.c_int32), ("M", ctypes.c_int32),
                ("kv_len", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("slot_state", ctypes.c_void_p), ("slot_group", ctypes.c_void_p),
                ("cs_lo", ctypes.c_int32), ("cs_hi", ctypes.c_int32),
                ("colsum_per_head", ctypes.c_int32), ("scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("colsum_accumulate", ctypes.c_int32), ("m_active", ctypes.c_void_p),
                ("pass1_done", ctypes.c_void_p)]


class _Select(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("k", ctypes.c_int32), ("group_rows", ctypes.c_int32),
                ("tau", ctypes.c_float), ("score", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("score_ready", ctypes.c_void_p), ("margin", ctypes.c_void_p),
                ("entropy", ctypes.c_void_p), ("row_flags", ctypes.c_void_p),
                ("conf_gate", ctypes.c_float), ("live_rows", ctypes.c_void_p),
                ("n_live", ctypes.c_void_p), ("live_offset", ctypes.c_int32)]


class _LayerDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_pos", ctypes.c_int32), ("d", ctypes.c_int32),
                ("M", ctypes.c_int32), ("active_idx", ctypes.c_void_p), ("m_active", ctypes.c_void_p),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("F", ctypes.c_int32), ("weights_packed", ctypes.c_int32)]


class _BlockBuffer(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_active", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
                ("slot_state", ctypes.c_void_p), ("slot_group", ctypes.c_void_p),
                ("decoded", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("locked", ctypes.c_void_p), ("skip", ctypes.c_void_p),
                ("row_flags", ctypes.c_void_p), ("active_idx", ctypes.c_void_p),
                ("m_active", ctypes.c_void_p), ("n_open", ctypes.c_void_p)]


_P = ctypes.c_void_p
lib.dlm_step_attn.argtypes = [_P, _P, _P, ctypes.POINTER(_KVCache), _P, ctypes.POINTER(_MaskDesc),
                              _P, _P, _P, _P]
lib.dlm_step_attn.restype = ctypes.c_int
lib.dlm_step_attn_workspace_bytes.argtypes = [ctypes.POINTER(_KVCache), ctypes.POINTER(_MaskDesc),
                                              ctypes.POINTER(ctypes.c_size_t)]
lib.dlm_step_attn_workspace_bytes.restype = ctypes.c_int
lib.dlm_posterior.argtypes = [_P, _P, _P, ctypes.c_float, ctypes.POINTER(_Select), _P, _P, _P,
                              ctypes.c_int32, ctypes.c_int32, _P]
lib.dlm_posterior.restype = ctypes.c_int
lib.dlm_posterior_noalloc.argtypes = lib.dlm_posterior.argtypes
lib.dlm_posterior_noalloc.restype = ctypes.c_int
lib.dlm_posterior_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Select),
                                              ctypes.POINTER(ctypes.c_size_t)]
lib.dlm_posterior_workspace_bytes.restype = ctypes.c_int
lib.dlm_block_buffer_init.argtypes = [ctypes.POINTER(_BlockBuffer), _P]
lib.dlm_block_buffer_init.restype = ctypes.c_int
lib.dlm_block_buffer_advance.argtypes = [ctypes.POINTER(_BlockBuffer), _P, _P]
lib.dlm_block_buffer_advance.restype = ctypes.c_int
class _R2LDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("gate", ctypes.c_float)]


lib.dlm_r2l_scan.argtypes = [ctypes.POINTER(_R2LDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P]
lib.dlm_r2l_scan.restype = ctypes.c_int

_LP = ctypes.POINTER(_LayerDesc)
lib.dlm_proj_qkv.argtypes = [_LP, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.dlm_proj_qkv.restype = ctypes.c_int
lib.dlm_proj_out.argtypes = [_LP, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.dlm_proj_out.restype = ctypes.c_int
lib.dlm_ffn.argtypes = [_LP, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
lib.dlm_ffn.restype = ctypes.c_int
lib.dlm_layer_workspace_bytes.argtypes = [_LP, ctypes.POINTER(ctypes.c_size_t)]
lib.dlm_layer_workspace_bytes.restype = ctypes.c_int
lib.dlm_pack_weights.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, _P]
lib.dlm_pack_weights.restype = ctypes.c_int
lib.dlm_last_error.argtypes = []
lib.dlm_last_error.restype = ctypes.c_char_p


def dlm_last_error() -> str:
    return lib.dlm_last_error().decode()


def _check(rc: int):
    if rc != DLM_OK:
        raise DlmError(rc, dlm_last_error())


# ---------------------------------------------------------------------------
# Descriptors (Python side).  Tensor fields hold torch device tensors; plain
# ints are accepted in their place by the raw entry points (tests of the
# host-side checks pass dummy addresses that are never dereferenced).
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class KVCache:
    k: object                  # bf16 [B, Hkv, n_cap, D]
    v: object
    B: int = 0
    Hkv: int = 0
    n_cap: int = 0
    D: int = 0

    def __post_init__(self):
        if hasattr(self.k, "shape") and not self.B:
            self.B, self.Hkv, self.n_cap, self.D = (int(x) for x in self.k.shape)


@dataclasses.dataclass
class MaskDesc:
    kind: int
    Hq: int
    M: int
    kv_len: int
    prefix_len: int = 0
    block_size: int = 0
    n_slots: int = 0
    slot_state: object = None  # uint8 [B, n_slots]
    slot_group: object = None  # int32 [B, n_slots]
    cs_lo: int = 0
    cs_hi: int = 0
    colsum_per_head: int = 0
    scale: float = 0.0
    workspace: object = None   # uint8 device buffer
    workspace_bytes: Optional[int] = None
    colsum_accumulate: int = 0  # 1: colsum += this call's sums (e.g. over layers)
    m_active: object = None     # optional int32 [B] device row counts
    pass1_done: object = None   # optional torch.cuda.Event (recorded once) or raw hipEvent_t


@dataclasses.dataclass
class Select:
    mode: int
    k: int = 0
    group_rows: int = 1
    tau: float = 0.0
    score: object = None       # fp32 [R]
    workspace: object = None
    workspace_bytes: Optional[int] = None
    score_ready: object = None  # torch.cuda.Event (recorded) or a raw hipEvent_t, or None
    margin: object = None       # optional fp32 [R] output
    entropy: object = None      # optional fp32 [R] output
    row_flags: object = None    # optional uint8 [R]: ROW_SELECT | ROW_LOCK per row
    conf_gate: float = 0.0      # lock only if also conf >= conf_gate (0: no gate)
    live_rows: object = None    # optional int32 [>= n]: rows that may arrive unlocked (+ live_offset)
    n_live: object = None       # int32 [1] on the device: the list's length (with live_rows)
    live_offset: int = 0        # subtracted from every live_rows entry


@dataclasses.dataclass
class LayerDesc:
    """Shapes and active rows of one layer's projections and feed-forward."""
    B: int
    n_pos: int
    d: int
    M: int
    active_idx: object = None  # int32 [B, M]
    m_active: object = None    # optional int32 [B]
    Hq: int = 1
    Hkv: int = 1
    D: int = 64
    F: int = 64
    weights_packed: bool = False   # weights in the layout of dlm_pack_weights (same shapes)


@dataclasses.dataclass
class BlockBuffer:
    """Device arrays of a multi-step run's Block Buffer (see dlm_step.h)."""
    B: int
    n_slots: int
    block_size: int
    max_active: int
    prefix_len: int
    slot_state: object = None  # uint8 [B, n_slots]
    slot_group: object = None  # int32 [B, n_slots]
    decoded: object = None     # uint8 [B, n_gen]
    tokens: object = None      # int32 [B, n_gen]
    locked: object = None      # uint8 [B, n_gen]
    skip: object = None        # uint8 [B, n_gen]
    row_flags: object = None   # uint8 [B, n_gen]
    active_idx: object = None  # int32 [B, n_gen]
    m_active: object = None    # int32 [B]
    n_open: object = None      # int32 [B]

    @property
    def n_gen(self) -> int:
        return self.n_slots * self.block_size


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return 0
    return x.numel() * x.element_size()


def _c_kv(kv: KVCache) -> _KVCache:
    return _KVCache(_ptr(kv.k), _ptr(kv.v), kv.B, kv.Hkv, kv.n_cap, kv.D)


def _event_handle(ev, what):
    if ev is None or isinstance(ev, int):
        return ev or None
    h = ev.cuda_event
    if not h:
        raise DlmError(-1, f"{what}: the event has not been created (record it once)")
    return h


def _c_mask(md: MaskDesc) -> _MaskDesc:
    wb = md.workspace_bytes if md.workspace_bytes is not None else _nbytes(md.workspace)
    return _MaskDesc(md.kind, md.Hq, md.M, md.kv_len, md.prefix_len, md.block_size, md.n_slots,
                     _ptr(md.slot_state), _ptr(md.slot_group), md.cs_lo, md.cs_hi,
                     md.colsum_per_head, md.scale, _ptr(md.workspace), wb, md.colsum_accumulate,
                     _ptr(md.m_active), _event_handle(md.pass1_done, "mask_desc.pass1_done"))


def _c_sel(s: Select) -> _Select:
    wb = s.workspace_bytes if s.workspace_bytes is not None else _nbytes(s.workspace)
    ev = s.score_ready
    if ev is not None and not isinstance(ev, int):
        ev = ev.cuda_event
        if not ev:
            raise DlmError(-1, "select.score_ready: the event has not been recorded")
    return _Select(s.mode, s.k, s.group_rows, s.tau, _ptr(s.score), _ptr(s.workspace), wb, ev or None,
                   _ptr(s.margin), _ptr(s.entropy), _ptr(s.row_flags), s.conf_gate, _ptr(s.live_rows),
                   _ptr(s.n_live), int(s.live_offset))


def _c_layer(L: LayerDesc) -> _LayerDesc:
    return _LayerDesc(L.B, L.n_pos, L.d, L.M, _ptr(L.active_idx), _ptr(L.m_active), L.Hq, L.Hkv, L.D, L.F,
                      int(bool(L.weights_packed)))


def _c_bb(bb: BlockBuffer) -> _BlockBuffer:
    return _BlockBuffer(bb.B, bb.n_slots, bb.block_size, bb.max_active, bb.prefix_len,
                        _ptr(bb.slot_state), _ptr(bb.slot_group), _ptr(bb.decoded), _ptr(bb.tokens),
                        _ptr(bb.locked), _ptr(bb.skip), _ptr(bb.row_flags), _ptr(bb.active_idx),
                        _ptr(bb.m_active), _ptr(bb.n_open))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _expect(t, name, shape, dtype):
    """Tensor argument check: device tensor, contiguous, exact shape/dtype."""
    if t is None or isinstance(t, int):
        return
    if tuple(t.shape) != tuple(shape):
        raise DlmError(DLM_E_SHAPE, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if str(t.dtype) != dtype:
        raise DlmError(DLM_E_SHAPE, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise DlmError(DLM_E_SHAPE, f"{name} must be contiguous")
    if not t.is_cuda:
        raise DlmError(DLM_E_SHAPE, f"{name} must be a device tensor")


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def dlm_step_attn_workspace_bytes(kv_cache: KVCache, mask_desc: MaskDesc) -> int:
    n = ctypes.c_size_t(0)
    kv, md = _c_kv(kv_cache), _c_mask(mask_desc)
    _check(lib.dlm_step_attn_workspace_bytes(ctypes.byref(kv), ctypes.byref(md), ctypes.byref(n)))
    return n.value


def dlm_step_attn(q, k, v, kv_cache: KVCache, active_idx, mask_desc: MaskDesc, out, lse,
                  colsum=None, stream=None) -> None:
    B, Hkv, n_cap, D = kv_cache.B, kv_cache.Hkv, kv_cache.n_cap, kv_cache.D
    Hq, M = mask_desc.Hq, mask_desc.M
    _expect(q, "q", (B, Hq, M, D), "torch.bfloat16")
    _expect(k, "k", (B, Hkv, M, D), "torch.bfloat16")
    _expect(v, "v", (B, Hkv, M, D), "torch.bfloat16")
    _expect(kv_cache.k, "kv_cache.k", (B, Hkv, n_cap, D), "torch.bfloat16")
    _expect(kv_cache.v, "kv_cache.v", (B, Hkv, n_cap, D), "torch.bfloat16")
    _expect(active_idx, "active_idx", (B, M), "torch.int32")
    _expect(out, "out", (B, Hq, M, D), "torch.bfloat16")
    _expect(lse, "lse", (B, Hq, M), "torch.float32")
    if colsum is not None:
        shape = (B, Hq, mask_desc.kv_len) if mask_desc.colsum_per_head else (B, mask_desc.kv_len)
        _expect(colsum, "colsum", shape, "torch.float32")
    if mask_desc.m_active is not None:
        _expect(mask_desc.m_active, "m_active", (B,), "torch.int32")
    if mask_desc.kind == MASK_GROUP:
        _expect(mask_desc.slot_state, "slot_state", (B, mask_desc.n_slots), "torch.uint8")
        _expect(mask_desc.slot_group, "slot_group", (B, mask_desc.n_slots), "torch.int32")
    kv, md = _c_kv(kv_cache), _c_mask(mask_desc)
    _check(lib.dlm_step_attn(_ptr(q), _ptr(k), _ptr(v), ctypes.byref(kv), _ptr(active_idx),
                             ctypes.byref(md), _ptr(out), _ptr(lse), _ptr(colsum), _stream(stream)))


def dlm_posterior_workspace_bytes(R: int, V: int, select: Select) -> int:
    n = ctypes.c_size_t(0)
    s = _c_sel(select)
    _check(lib.dlm_posterior_workspace_bytes(R, V, ctypes.byref(s), ctypes.byref(n)))
    return n.value


def _post_args(logits, prev_logits, locked, select, sel, kl, conf, R, V):
    _expect(logits, "logits", (R, V), "torch.float32")
    _expect(prev_logits, "prev_logits", (R, V), "torch.float32")
    _expect(locked, "locked", (R,), "torch.uint8")
    _expect(sel, "sel", (R,), "torch.int32")
    _expect(kl, "kl", (R,), "torch.float32")
    _expect(conf, "conf", (R,), "torch.float32")
    if select.score is not None:
        _expect(select.score, "select.score", (R,), "torch.float32")
    if select.margin is not None:
        _expect(select.margin, "select.margin", (R,), "torch.float32")
    if select.entropy is not None:
        _expect(select.entropy, "select.entropy", (R,), "torch.float32")
    if select.row_flags is not None:
        _expect(select.row_flags, "select.row_flags", (R,), "torch.uint8")
    if select.live_rows is not None:
        # R entries: the device reads at most min(n_live, R) of them
        _expect(select.live_rows, "select.live_rows", (R,), "torch.int32")
        if select.n_live is None:
            raise DlmError(DLM_E_NULL, "select.live_rows needs select.n_live")
        _expect(select.n_live, "select.n_live", (1,), "torch.int32")


def dlm_posterior(logits, prev_logits, locked, eps: float, select: Select, sel, kl, conf,
                  R: int, V: int, stream=None) -> None:
    _post_args(logits, prev_logits, locked, select, sel, kl, conf, R, V)
    s = _c_sel(select)
    _check(lib.dlm_posterior(_ptr(logits), _ptr(prev_logits), _ptr(locked), eps, ctypes.byref(s),
                             _ptr(sel), _ptr(kl), _ptr(conf), R, V, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20   # DLM_NOALLOC_SCRATCH_BYTES


def dlm_posterior_noalloc(logits, prev_logits, locked, eps: float, select: Select, sel, kl, conf,
                          R: int, V: int, stream=None) -> None:
    """dlm_posterior with its partials in the library's own device array
    (no workspace; select.workspace is ignored)."""
    _post_args(logits, prev_logits, locked, select, sel, kl, conf, R, V)
    s = _c_sel(select)
    _check(lib.dlm_posterior_noalloc(_ptr(logits), _ptr(prev_logits), _ptr(locked), eps, ctypes.byref(s),
                                     _ptr(sel), _ptr(kl), _ptr(conf), R, V, _stream(stream)))


def _expect_bb(bb: BlockBuffer):
    B, S, n = bb.B, bb.n_slots, bb.n_gen
    for name, shape, dt in (("slot_state", (B, S), "torch.uint8"), ("slot_group", (B, S), "torch.int32"),
                            ("decoded", (B, n), "torch.uint8"), ("tokens", (B, n), "torch.int32"),
                            ("locked", (B, n), "torch.uint8"), ("skip", (B, n), "torch.uint8"),
                            ("row_flags", (B, n), "torch.uint8"), ("active_idx", (B, n), "torch.int32"),
                            ("m_active", (B,), "torch.int32"), ("n_open", (B,), "torch.int32")):
        _expect(getattr(bb, name), name, shape, dt)


def dlm_block_buffer_init(bb: BlockBuffer, stream=None) -> None:
    _expect_bb(bb)
    c = _c_bb(bb)
    _check(lib.dlm_block_buffer_init(ctypes.byref(c), _stream(stream)))


def dlm_block_buffer_advance(bb: BlockBuffer, sel, stream=None) -> None:
    _expect_bb(bb)
    _expect(sel, "sel", (bb.B, bb.n_gen), "torch.int32")
    c = _c_bb(bb)
    _check(lib.dlm_block_buffer_advance(ctypes.byref(c), _ptr(sel), _stream(stream)))


def _expect_layer(L: LayerDesc):
    _expect(L.active_idx, "active_idx", (L.B, L.M), "torch.int32")
    if L.m_active is not None:
        _expect(L.m_active, "m_active", (L.B,), "torch.int32")


def dlm_proj_qkv(layer: LayerDesc, x, w_qkv, q, k, v, workspace, stream=None) -> None:
    L = layer
    _expect_layer(L)
    _expect(x, "x", (L.B, L.n_pos, L.d), "torch.bfloat16")
    _expect(w_qkv, "w_qkv", ((L.Hq + 2 * L.Hkv) * L.D, L.d), "torch.bfloat16")
    _expect(q, "q", (L.B, L.Hq, L.M, L.D), "torch.bfloat16")
    _expect(k, "k", (L.B, L.Hkv, L.M, L.D), "torch.bfloat16")
    _expect(v, "v", (L.B, L.Hkv, L.M, L.D), "torch.bfloat16")
    c = _c_layer(L)
    _check(lib.dlm_proj_qkv(ctypes.byref(c), _ptr(x), _ptr(w_qkv), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(workspace), _nbytes(workspace), _stream(stream)))


def dlm_proj_out(layer: LayerDesc, x, attn_out, w_o, h, workspace, stream=None) -> None:
    L = layer
    _expect_layer(L)
    _expect(x, "x", (L.B, L.n_pos, L.d), "torch.bfloat16")
    _expect(attn_out, "attn_out", (L.B, L.Hq, L.M, L.D), "torch.bfloat16")
    _expect(w_o, "w_o", (L.d, L.Hq * L.D), "torch.bfloat16")
    _expect(h, "h", (L.B, L.M, L.d), "torch.bfloat16")
    c = _c_layer(L)
    _check(lib.dlm_proj_out(ctypes.byref(c), _ptr(x), _ptr(attn_out), _ptr(w_o), _ptr(h),
                            _ptr(workspace), _nbytes(workspace), _stream(stream)))


def dlm_layer_workspace_bytes(layer: LayerDesc) -> int:
    n = ctypes.c_size_t(0)
    c = _c_layer(layer)
    _check(lib.dlm_layer_workspace_bytes(ctypes.byref(c), ctypes.byref(n)))
    return n.value


def dlm_pack_weights(w, packed=None, stream=None):
    """A bf16 weight [N, K] in the fragment-packed layout of the layer calls
    (see dlm_step.h), returned as a tensor of the same shape."""
    if w is None or w.dim() != 2:
        raise DlmError(DLM_E_SHAPE, "w must be a 2-d bf16 tensor")
    N, K = w.shape
    _expect(w, "w", (N, K), "torch.bfloat16")
    if packed is None:
        import torch
        packed = torch.empty_like(w)
    _expect(packed, "packed", (N, K), "torch.bfloat16")
    _check(lib.dlm_pack_weights(_ptr(w), _ptr(packed), N, K, _stream(stream)))
    return packed


def dlm_ffn(layer: LayerDesc, h, w_gate, w_up, w_down, x, workspace, stream=None) -> None:
    L = layer
    _expect_layer(L)
    _expect(h, "h", (L.B, L.M, L.d), "torch.bfloat16")
    _expect(w_gate, "w_gate", (L.F, L.d), "torch.bfloat16")
    _expect(w_up, "w_up", (L.F, L.d), "torch.bfloat16")
    _expect(w_down, "w_down", (L.d, L.F), "torch.bfloat16")
    _expect(x, "x", (L.B, L.n_pos, L.d), "torch.bfloat16")
    c = _c_layer(L)
    _check(lib.dlm_ffn(ctypes.byref(c), _ptr(h), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x),
                       _ptr(workspace), _nbytes(workspace), _stream(stream)))


def dlm_r2l_scan(B: int, L: int, E: int, N: int, gate: float, u, delta, A, Bm, Cm, D, y=None, x=None,
                 stream=None) -> None:
    """The right-to-left selective scan (see dlm_step.h)."""
    _expect(u, "u", (B, L, E), "torch.bfloat16")
    _expect(delta, "delta", (B, L, E), "torch.bfloat16")
    _expect(A, "A", (E, N), "torch.float32")
    _expect(Bm, "Bm", (B, L, N), "torch.bfloat16")
    _expect(Cm, "Cm", (B, L, N), "torch.bfloat16")
    _expect(D, "D", (E,), "torch.float32")
    if y is not None:
        _expect(y, "y", (B, L, E), "torch.float32")
    if x is not None:
        _expect(x, "x", (B, L, E), "torch.bfloat16")
    c = _R2LDesc(B, L, E, N, gate)
    _check(lib.dlm_r2l_scan(ctypes.byref(c), _ptr(u), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D),
                            _ptr(y), _ptr(x), _stream(stream)))
