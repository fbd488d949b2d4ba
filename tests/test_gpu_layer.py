"""GPU parity of the active-row projections and feed-forward (and of the
lock test's confidence gate) against the oracle, through the C ABI.

Bounds per element, from the arithmetic (fp32 accumulation of K exact bf16
products, then one round to bf16):
    |gpu - exact| <= 2^-8 |exact| + K 2^-23 sum_k |a_k w_k|
SwiGLU propagates the two products' bounds through silu (slope <= 1.1) and
the product; the down projection adds the gated rows' rounding, carried by
|W_down|.  Rows past the device row count must be left untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import layer as OL

pytestmark = pytest.mark.gpu

RND = 2.0 ** -8


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests need an MI355X")
    import denoising_step_amd  # noqa: F401
    yield


def _dev(bits):
    from denoising_step_amd.runner import bf16_to_device
    return bf16_to_device(bits, torch.device("cuda"))


def _host(t):
    from denoising_step_amd.runner import bf16_to_host
    return W.bf16_bits_to_f32(bf16_to_host(t)).astype(np.float64)


def _f(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def _check(got, want, tol, what):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    ratio = (err / tol).max() if err.size else 0.0
    assert ratio <= 1.0, f"{what}: error {err.max():.3e} over its bound (ratio {ratio:.2f})"
    return ratio


def _layer_desc(c, m_dev):
    import denoising_step_amd as dlm
    return dlm.LayerDesc(B=c.B, n_pos=c.n_pos, d=c.d, M=c.M, active_idx=torch.from_numpy(c.active_idx).cuda(),
                         m_active=m_dev, Hq=c.Hq, Hkv=c.Hkv, D=c.D, F=c.F)


CASES = {
    "d256_gqa_ragged": dict(B=2, n_pos=300, d=256, Hq=4, Hkv=2, D=64, F=384, M=150, m=[150, 77]),
    "d192_head128": dict(B=1, n_pos=200, d=192, Hq=2, Hkv=1, D=128, F=128, M=130, m=[130]),
    "all_rows": dict(B=3, n_pos=90, d=128, Hq=2, Hkv=2, D=64, F=256, M=90, m=None),
    "rows_cut": dict(B=2, n_pos=260, d=320, Hq=4, Hkv=4, D=64, F=192, M=257, m=[0, 129]),
    # few rows, long K: every product splits K (partial sums and the reduction)
    "split_k": dict(B=2, n_pos=64, d=1024, Hq=16, Hkv=4, D=64, F=1024, M=40, m=[33, 40]),
    # 17 to 64 rows in all: the 32- and 64-row tiles with their deep stage
    # rings; K splits, ragged column tiles, several batch entries sharing
    # one row tile, an entry with no rows
    "rows32_split_k": dict(B=1, n_pos=100, d=1024, Hq=16, Hkv=4, D=64, F=1024, M=24, m=[17]),
    "rows32_batches": dict(B=4, n_pos=40, d=256, Hq=4, Hkv=2, D=64, F=384, M=8, m=[8, 0, 5, 8]),
    "rows64_ragged": dict(B=2, n_pos=70, d=320, Hq=4, Hkv=4, D=64, F=192, M=30, m=[30, 11]),
    # at most 16 rows: the weight-streaming kernel (whole K per workgroup,
    # K split over its waves, the gated rows handed on packed); batch
    # entries sharing the 16 rows with one empty, five rows with waves
    # that get no K step, and 384 column tiles (eight-way K splits)
    "skinny16_batches": dict(B=4, n_pos=40, d=256, Hq=4, Hkv=2, D=64, F=384, M=4, m=[4, 0, 3, 4]),
    "skinny_rows5": dict(B=1, n_pos=70, d=320, Hq=4, Hkv=4, D=64, F=192, M=5, m=[5]),
    "skinny_kw8": dict(B=1, n_pos=64, d=512, Hq=32, Hkv=8, D=128, F=6144, M=16, m=[16]),
}


def check_layer(c, qg, kg, vg, hg, yg):
    """Compare the three calls' outputs for the valid rows of case c with
    the oracle, each element against its bound.  qg/kg/vg: [B, H, M, D];
    hg: [B, M, d]; yg: [B, M, d] (x's rows at the active positions)."""
    m = c.m
    Hq, Hkv, D = c.Hq, c.Hkv, c.D
    xa, hh, ao = _f(c.x), _f(c.h), _f(c.attn_out)
    wqkv, wo, wg, wu, wd = map(_f, (c.w_qkv, c.w_o, c.w_gate, c.w_up, c.w_down))
    ref = OL.proj_qkv(c.x, c.active_idx, m, c.w_qkv, Hq, Hkv, D)
    href = OL.proj_out(c.x, c.active_idx, m, c.attn_out, c.w_o)
    gated = OL.gated(c.h, m, c.w_gate, c.w_up)
    yref = OL.ffn(c.h, m, c.w_gate, c.w_up, c.w_down)
    worst = 0.0
    for b in range(c.B):
        mb = int(m[b])
        if mb == 0:
            continue
        s = (np.abs(xa[b, c.active_idx[b, :mb]]) @ np.abs(wqkv).T) * (c.d * 2.0 ** -23)
        split = (s[:, :Hq * D].reshape(mb, Hq, D).transpose(1, 0, 2),
                 s[:, Hq * D:(Hq + Hkv) * D].reshape(mb, Hkv, D).transpose(1, 0, 2),
                 s[:, (Hq + Hkv) * D:].reshape(mb, Hkv, D).transpose(1, 0, 2))
        for got, want, acc, nm in zip((qg[b, :, :mb], kg[b, :, :mb], vg[b, :, :mb]), ref[b], split, "qkv"):
            worst = max(worst, _check(got, want, RND * np.abs(want) + acc + 1e-30, nm))
        a = np.abs(ao[b, :, :mb].transpose(1, 0, 2).reshape(mb, -1))
        tol = RND * np.abs(href[b]) + Hq * D * 2.0 ** -23 * (a @ np.abs(wo).T) + 1e-30
        worst = max(worst, _check(hg[b, :mb], href[b], tol, "h"))
        ha = np.abs(hh[b, :mb])
        gate = hh[b, :mb] @ wg.T
        up = hh[b, :mb] @ wu.T
        eg = c.d * 2.0 ** -23 * (ha @ np.abs(wg).T)
        eu = c.d * 2.0 ** -23 * (ha @ np.abs(wu).T)
        g_tol = (RND + 2.0 ** -20) * np.abs(gated[b]) + 1.1 * np.abs(up) * eg + np.abs(OL.silu(gate)) * eu
        y_tol = (RND * np.abs(yref[b]) + g_tol @ np.abs(wd).T
                 + c.F * 2.0 ** -23 * ((np.abs(gated[b]) + g_tol) @ np.abs(wd).T) + 1e-30)
        worst = max(worst, _check(yg[b, :mb], yref[b], y_tol, "ffn"))
    return worst


def _run_layer(c, m_dev, sentinel=5.0, packed=False):
    import denoising_step_amd as dlm
    L = _layer_desc(c, m_dev)
    L.weights_packed = packed
    wt = (lambda bits: dlm.dlm_pack_weights(_dev(bits))) if packed else _dev
    x = _dev(c.x)
    q = torch.full((c.B, c.Hq, c.M, c.D), sentinel, dtype=torch.bfloat16, device="cuda")
    k = torch.full((c.B, c.Hkv, c.M, c.D), sentinel, dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, sentinel)
    h = torch.full((c.B, c.M, c.d), sentinel, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(1, dlm.dlm_layer_workspace_bytes(L)), dtype=torch.uint8, device="cuda")
    dlm.dlm_proj_qkv(L, x, wt(c.w_qkv), q, k, v, ws)
    dlm.dlm_proj_out(L, x, _dev(c.attn_out), wt(c.w_o), h, ws)
    x2 = x.clone()
    dlm.dlm_ffn(L, _dev(c.h), wt(c.w_gate), wt(c.w_up), wt(c.w_down), x2, ws)
    torch.cuda.synchronize()
    return _host(q), _host(k), _host(v), _host(h), _host(x2)


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_calls_match_oracle(name):
    kw = dict(CASES[name])
    m_list = kw.pop("m")
    c = W.make_layer(name, m=m_list, seed=7, **kw)
    _say(f"layer {name}")
    m_dev = None if m_list is None else torch.tensor(m_list, dtype=torch.int32, device="cuda")
    qg, kg, vg, hg, xg = _run_layer(c, m_dev)
    yg = np.stack([xg[b, c.active_idx[b]] for b in range(c.B)])
    worst = check_layer(c, qg, kg, vg, hg, yg)
    xa = _f(c.x)
    for b in range(c.B):
        mb = int(c.m[b])
        # rows past the count untouched; positions not computed keep their hidden state
        for t in (qg, kg, vg):
            assert np.all(t[b, :, mb:] == 5.0)
        assert np.all(hg[b, mb:] == 5.0)
        rest = np.setdiff1d(np.arange(c.n_pos), c.active_idx[b, :mb])
        assert np.array_equal(xg[b, rest], xa[b, rest]), "a row that is not active was written"
    _say(f"  worst error / bound = {worst:.3f}")


@pytest.mark.parametrize("M", [1024, 200, 100, 48, 16])
def test_layer_full_size_sampled(M):
    """The LLaDA-8B-shaped layer (width 4096, 32 heads of 128, feed-forward
    12288) with M of 2048 positions active (128-row tiles two to a CU; up
    to 256 rows, the one-per-CU deep-ring tiles with K splits; up to 16,
    the weight-streaming kernel with four- and sixteen-way K splits in the
    workgroup): sampled rows against the oracle, each element against the
    same bound."""
    c = W.layer_llada(M=M, n_pos=2048)
    _say(f"layer llada full size M={M}")
    qg, kg, vg, hg, xg = _run_layer(c, None)
    rows = np.array([0, 1, 127, 128, 511, 640, 1000, 1023]) if M == 1024 else np.array([0, 1, M // 2, M - 2, M - 1])
    sub = W.LayerCase(**{**c.__dict__, "M": len(rows), "active_idx": c.active_idx[:, rows],
                         "m": np.array([len(rows)], np.int32), "attn_out": c.attn_out[:, :, rows],
                         "h": c.h[:, rows]})
    yg = xg[:, c.active_idx[0, rows]]
    worst = check_layer(sub, qg[:, :, rows], kg[:, :, rows], vg[:, :, rows], hg[:, rows], yg)
    _say(f"  worst error / bound = {worst:.3f}")


def test_pack_weights_layout():
    """dlm_pack_weights against the layout as the header states it: element
    (n, k) at ((n / 16) (K / 32) + k / 32) 512 + ((k % 32) / 8 16 + n % 16) 8
    + k % 8, bit for bit."""
    import denoising_step_amd as dlm
    rng = np.random.default_rng(3)
    for N, K in ((16, 32), (48, 96), (4096, 4096)):
        w = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
        got = dlm.dlm_pack_weights(_dev(w))
        torch.cuda.synchronize()
        from denoising_step_amd.runner import bf16_to_host
        g = bf16_to_host(got).reshape(-1)
        n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
        pos = ((n // 16) * (K // 32) + k // 32) * 512 + ((k % 32) // 8 * 16 + n % 16) * 8 + k % 8
        want = np.empty(N * K, np.uint16)
        want[pos.reshape(-1)] = w.reshape(-1)
        assert np.array_equal(g, want), (N, K)


PACKED_CASES = ["skinny16_batches", "skinny_rows5", "skinny_kw8", "rows32_batches", "rows64_ragged",
                "rows32_split_k", "split_k", "d256_gqa_ragged", "rows_cut"]


@pytest.mark.parametrize("name", PACKED_CASES)
def test_packed_weights_bit_exact(name):
    """Weights in the packed layout give the row-major results bit for bit
    (each MFMA sees the same operands in the same order), on both product
    kernels: the weight-streaming one (up to 64 rows) and the tiled one."""
    kw = dict(CASES[name])
    m_list = kw.pop("m")
    c = W.make_layer(name, m=m_list, seed=11, **kw)
    _say(f"layer packed {name}")
    m_dev = None if m_list is None else torch.tensor(m_list, dtype=torch.int32, device="cuda")
    ref = _run_layer(c, m_dev)
    got = _run_layer(c, m_dev, packed=True)
    for r, g, nm in zip(ref, got, ("q", "k", "v", "h", "x")):
        assert np.array_equal(r, g), nm


@pytest.mark.parametrize("M", [16, 48, 200])
def test_packed_weights_full_size(M):
    """The LLaDA-8B-shaped layer with packed weights: bit for bit the
    row-major results (16 rows: the weight-streaming kernel with its four-
    and sixteen-way K splits; 48 and 200: the deep-ring tiles)."""
    c = W.layer_llada(M=M, n_pos=2048)
    _say(f"layer llada packed M={M}")
    ref = _run_layer(c, None)
    got = _run_layer(c, None, packed=True)
    for r, g, nm in zip(ref, got, ("q", "k", "v", "h", "x")):
        assert np.array_equal(r, g), nm


def test_confidence_gate():
    import denoising_step_amd as dlm
    rng = np.random.default_rng(17)
    R, V = 200, 3000
    x = (rng.standard_normal((R, V)) * np.linspace(0.5, 6.0, R)[:, None]).astype(np.float32)
    y = (x + rng.standard_normal((R, V)) * 0.005).astype(np.float32)
    locked = np.zeros(R, np.uint8)
    o0 = oracle.posterior(x, y, locked, 1e-3)
    gate = float(np.median(o0["conf"]))
    o = oracle.posterior(x, y, locked, 1e-3, conf_gate=gate)
    assert (o["locked"] != o0["locked"]).any()
    s = dlm.Select(mode=dlm.SEL_NONE, conf_gate=gate)
    s.workspace = torch.zeros(max(1, dlm.dlm_posterior_workspace_bytes(R, V, s)), dtype=torch.uint8, device="cuda")
    lk = torch.zeros(R, dtype=torch.uint8, device="cuda")
    sel = torch.empty(R, dtype=torch.int32, device="cuda")
    kl = torch.empty(R, device="cuda")
    conf = torch.empty(R, device="cuda")
    dlm.dlm_posterior(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda(), lk, 1e-3, s, sel, kl, conf, R, V)
    torch.cuda.synchronize()
    g = lk.cpu().numpy()
    assert np.abs(kl.cpu().numpy() - o["kl"]).max() <= 1e-4
    assert np.abs(conf.cpu().numpy() - o["conf"]).max() <= 1e-5
    diff = np.nonzero(g != o["locked"])[0]
    # a decision may differ only where the oracle's KL or conf sits at its threshold
    for r in diff:
        assert abs(o["kl"][r] - 1e-3) <= 1e-4 or abs(o["conf"][r] - gate) <= 1e-5, r
    _say(f"gate {gate:.4f}: {int(o['locked'].sum())} of {R} rows lock ({len(diff)} excused)")
