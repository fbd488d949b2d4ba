// dlm_api.hip -- host side of the C ABI declared in include/dlm_step.h:
// argument validation (before anything is enqueued), workspace sizing,
// launch plans, and the optional DLM_VALIDATE content check.
#include "dlm_step.h"
#include "dlm_internal.h"

#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool validate_env()
{
    const char *e = getenv("DLM_VALIDATE");
    return e && e[0] == '1';
}

// Scalar checks shared by dlm_step_attn and its workspace query.
int check_attn_scalars(const dlm_kv_cache *kc, const dlm_mask_desc *md)
{
    if (!kc) return fail(DLM_E_NULL, "kv_cache is NULL");
    if (!md) return fail(DLM_E_NULL, "mask_desc is NULL");
    if (kc->B < 1 || kc->Hkv < 1 || md->Hq < 1)
        return fail(DLM_E_SHAPE, "B=%d Hkv=%d Hq=%d must be >= 1", kc->B, kc->Hkv, md->Hq);
    if (kc->D != 32 && kc->D != 64 && kc->D != 128)
        return fail(DLM_E_UNSUPPORTED, "head dim D=%d not in {32, 64, 128}", kc->D);
    if (md->Hq % kc->Hkv != 0)
        return fail(DLM_E_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", md->Hq, kc->Hkv);
    if (md->kv_len < 1 || md->kv_len > kc->n_cap)
        return fail(DLM_E_SHAPE, "kv_len=%d must be in [1, n_cap=%d]", md->kv_len, kc->n_cap);
    if (md->prefix_len < 0 || md->prefix_len > md->kv_len)
        return fail(DLM_E_SHAPE, "prefix_len=%d must be in [0, kv_len=%d]", md->prefix_len, md->kv_len);
    if (md->M < 0 || md->M > md->kv_len - md->prefix_len)
        return fail(DLM_E_SHAPE, "M=%d must be in [0, kv_len - prefix_len = %d]", md->M,
                    md->kv_len - md->prefix_len);
    if ((long)kc->B * md->Hq * md->M > (1L << 31) - 1 ||
        (long)kc->B * kc->Hkv * kc->n_cap > (1L << 31) - 1)
        return fail(DLM_E_SHAPE, "problem too large for 32-bit row indices");
    // the kernels address one (batch, head) slice of q / K / V through
    // 32-bit byte offsets and buffer views of kv_len * D * 2 bytes
    if ((long)md->kv_len * kc->D * 2 > (long)INT_MAX - 4096)
        return fail(DLM_E_SHAPE, "kv_len=%d x D=%d bf16 is past the 2 GiB per (batch, head) slice the "
                    "kernels address with 32-bit offsets", md->kv_len, kc->D);
    if (md->kind < DLM_MASK_FULL || md->kind > DLM_MASK_GROUP)
        return fail(DLM_E_DESC, "unknown mask kind %d", md->kind);
    if (md->kind != DLM_MASK_FULL && md->block_size < 1)
        return fail(DLM_E_DESC, "block_size=%d must be >= 1 for block-causal / group masks",
                    md->block_size);
    if (md->kind == DLM_MASK_GROUP) {
        if (md->n_slots < 1 || md->n_slots > dlm::kMaxSlots)
            return fail(DLM_E_DESC, "n_slots=%d must be in [1, %d]", md->n_slots, dlm::kMaxSlots);
        if (!md->slot_state || !md->slot_group)
            return fail(DLM_E_NULL, "group mask needs slot_state and slot_group");
        if ((long)md->prefix_len + (long)md->n_slots * md->block_size < md->kv_len)
            return fail(DLM_E_DESC, "kv_len=%d exceeds prefix_len + n_slots * block_size = %ld",
                        md->kv_len, (long)md->prefix_len + (long)md->n_slots * md->block_size);
    }
    if (md->cs_lo > md->cs_hi)
        return fail(DLM_E_DESC, "cs_lo=%d > cs_hi=%d", md->cs_lo, md->cs_hi);
    if (md->colsum_per_head != 0 && md->colsum_per_head != 1)
        return fail(DLM_E_DESC, "colsum_per_head must be 0 or 1");
    if (md->colsum_accumulate != 0 && md->colsum_accumulate != 1)
        return fail(DLM_E_DESC, "colsum_accumulate must be 0 or 1");
    if (!(md->scale >= 0.f) || isinf(md->scale))
        return fail(DLM_E_DESC, "scale must be finite and >= 0 (0 selects 1/sqrt(D))");
    return DLM_OK;
}

// DLM_VALIDATE=1: check the contents of active_idx and the slot tables on a
// host copy (synchronises the stream).
int validate_contents(const dlm_kv_cache *kc, const dlm_mask_desc *md, const int32_t *active_idx,
                      hipStream_t stream)
{
    const int B = kc->B, M = md->M;
    std::vector<int32_t> act((size_t)B * M);
    std::vector<int32_t> mv((size_t)B, M);
    std::vector<uint8_t> st;
    std::vector<int32_t> gr;
    if (M > 0 && hipMemcpyAsync(act.data(), active_idx, act.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return fail(DLM_E_HIP, "DLM_VALIDATE: copy of active_idx failed");
    if (md->m_active && hipMemcpyAsync(mv.data(), md->m_active, mv.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess)
        return fail(DLM_E_HIP, "DLM_VALIDATE: copy of m_active failed");
    if (md->kind == DLM_MASK_GROUP) {
        st.resize((size_t)B * md->n_slots);
        gr.resize((size_t)B * md->n_slots);
        if (hipMemcpyAsync(st.data(), md->slot_state, st.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipMemcpyAsync(gr.data(), md->slot_group, gr.size() * 4, hipMemcpyDeviceToHost, stream) != hipSuccess)
            return fail(DLM_E_HIP, "DLM_VALIDATE: copy of slot tables failed");
    }
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(DLM_E_HIP, "DLM_VALIDATE: sync failed");
    for (int b = 0; b < B; ++b)
        if (mv[b] < 0 || mv[b] > M)
            return fail(DLM_E_DESC, "m_active[%d]=%d outside [0, M=%d]", b, mv[b], M);
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < mv[b]; ++j) {
            int p = act[(size_t)b * M + j];
            if (p < md->prefix_len || p >= md->kv_len)
                return fail(DLM_E_DESC, "active_idx[%d,%d]=%d outside [prefix_len=%d, kv_len=%d)", b, j, p,
                            md->prefix_len, md->kv_len);
            if (j > 0 && p <= act[(size_t)b * M + j - 1])
                return fail(DLM_E_DESC, "active_idx[%d] not strictly ascending at %d", b, j);
        }
    for (size_t i = 0; i < st.size(); ++i) {
        if (st[i] > DLM_SLOT_IN_CACHE) return fail(DLM_E_DESC, "slot_state[%zu]=%d unknown", i, st[i]);
        if (gr[i] < 0 || gr[i] == 0x7fffffff) return fail(DLM_E_DESC, "slot_group[%zu]=%d out of range", i, gr[i]);
    }
    return DLM_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

const char *dlm_last_error(void) { return g_err; }

int dlm_step_attn_workspace_bytes(const dlm_kv_cache *kv_cache, const dlm_mask_desc *mask_desc,
                                  size_t *bytes)
{
    g_err[0] = 0;
    if (!bytes) return fail(DLM_E_NULL, "bytes is NULL");
    int rc = check_attn_scalars(kv_cache, mask_desc);
    if (rc != DLM_OK) return rc;
    dlm::AttnPlan p = dlm::plan_attn(kv_cache->B, mask_desc->Hq, kv_cache->Hkv, kv_cache->D,
                                     mask_desc->M, mask_desc->kv_len, kv_cache->n_cap, mask_desc->m_active != nullptr);
    *bytes = p.ws_total;
    return DLM_OK;
}

int dlm_step_attn(const void *q, const void *k, const void *v, const dlm_kv_cache *kv_cache,
                  const int32_t *active_idx, const dlm_mask_desc *mask_desc, void *out, float *lse,
                  float *colsum, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_attn_scalars(kv_cache, mask_desc);
    if (rc != DLM_OK) return rc;
    const dlm_kv_cache *kc = kv_cache;
    const dlm_mask_desc *md = mask_desc;
    if (!kc->k || !kc->v) return fail(DLM_E_NULL, "the cache k/v must be non-NULL");
    if (md->M > 0 && (!q || !active_idx || !out || !lse))
        return fail(DLM_E_NULL, "q, active_idx, out and lse must be non-NULL when M > 0");
    if (md->M > 0 && (k == nullptr) != (v == nullptr))
        return fail(DLM_E_NULL, "fresh k and v must both be given or both be NULL");
    if ((md->M > 0 && (!aligned16(q) || !aligned16(out))) || !aligned16(kc->k) || !aligned16(kc->v) ||
        (k && !aligned16(k)) || (v && !aligned16(v)))
        return fail(DLM_E_SHAPE, "bf16 tensors must be 16-byte aligned");
    dlm::AttnPlan p = dlm::plan_attn(kc->B, md->Hq, kc->Hkv, kc->D, md->M, md->kv_len, kc->n_cap,
                                     md->m_active != nullptr);
    const size_t need = p.ws_total;
    if (need > 0 && (md->workspace == nullptr || md->workspace_bytes < need))
        return fail(DLM_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    md->workspace ? md->workspace_bytes : (size_t)0);
    if (validate_env()) {
        rc = validate_contents(kc, md, active_idx, stream);
        if (rc != DLM_OK) return rc;
    }

    dlm::AttnArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.ck = static_cast<uint16_t *>(kc->k);
    a.cv = static_cast<uint16_t *>(kc->v);
    a.active_idx = active_idx;
    a.slot_state = md->slot_state;
    a.slot_group = md->slot_group;
    a.out = static_cast<uint16_t *>(out);
    a.lse = lse;
    a.colsum = colsum;
    char *ws = static_cast<char *>(md->workspace);
    a.ws_o = p.ws_split_o ? reinterpret_cast<float *>(ws) : nullptr;
    a.ws_l = p.ws_split_l ? reinterpret_cast<float *>(ws + align256(p.ws_split_o)) : nullptr;
    a.ws_cs = reinterpret_cast<float *>(ws + align256(p.ws_split_o) + align256(p.ws_split_l));
    a.B = kc->B; a.Hq = md->Hq; a.Hkv = kc->Hkv; a.G = md->Hq / kc->Hkv; a.D = kc->D; a.M = md->M;
    a.n_cap = kc->n_cap; a.kv_len = md->kv_len; a.P = md->prefix_len; a.bs = md->block_size;
    a.n_slots = md->kind == DLM_MASK_GROUP ? md->n_slots : 0;
    a.kind = md->kind;
    a.m_valid = md->m_active;
    a.cs_lo = md->cs_lo; a.cs_hi = md->cs_hi; a.per_head = md->colsum_per_head;
    a.accumulate = md->colsum_accumulate;
    const float scale = md->scale > 0.f ? md->scale : 1.f / sqrtf((float)kc->D);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.n_qtiles = p.n_qtiles; a.n_kgroups = p.n_kgroups; a.n_split = p.n_split; a.split_keys = p.split_keys;
    a.n_kblocks = p.n_kblocks; a.n_rsplit = p.n_rsplit;
    a.dyn_split = p.dyn_split; a.rows_wg = p.rows_wg;

    hipError_t e = dlm::launch_step_attn(a, stream, md->pass1_done);
    if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

static int check_post_scalars(int32_t R, int32_t V, const dlm_select *s)
{
    if (!s) return fail(DLM_E_NULL, "select is NULL");
    if (R < 0) return fail(DLM_E_SHAPE, "R=%d must be >= 0", R);
    if (V < 1) return fail(DLM_E_SHAPE, "V=%d must be >= 1", V);
    if ((long)R * V > (1L << 40)) return fail(DLM_E_SHAPE, "R*V too large");
    if (s->mode < DLM_SEL_NONE || s->mode > DLM_SEL_TOPK_LOW_ENTROPY)
        return fail(DLM_E_DESC, "unknown selection mode %d", s->mode);
    if (s->mode != DLM_SEL_NONE && (s->group_rows < 1 || s->group_rows > dlm::kMaxGroupRows))
        return fail(DLM_E_DESC, "group_rows=%d must be in [1, %d]", s->group_rows, dlm::kMaxGroupRows);
    if ((s->mode == DLM_SEL_TOPK_CONF || s->mode == DLM_SEL_TOPK_SCORE || s->mode == DLM_SEL_TOPK_MARGIN ||
         s->mode == DLM_SEL_TOPK_LOW_ENTROPY) && s->k < 0)
        return fail(DLM_E_DESC, "k=%d must be >= 0", s->k);
    if ((s->mode == DLM_SEL_THRESH_CONF || s->mode == DLM_SEL_ATTN_DYNAMIC) && !isfinite(s->tau))
        return fail(DLM_E_DESC, "tau must be finite");
    if (!isfinite(s->conf_gate)) return fail(DLM_E_DESC, "conf_gate must be finite");
    return DLM_OK;
}

int dlm_posterior_workspace_bytes(int32_t R, int32_t V, const dlm_select *select, size_t *bytes)
{
    g_err[0] = 0;
    if (!bytes) return fail(DLM_E_NULL, "bytes is NULL");
    int rc = check_post_scalars(R, V, select);
    if (rc != DLM_OK) return rc;
    *bytes = dlm::post_ws_bytes(R, V, select->mode, select->group_rows, select->live_rows != nullptr);
    return DLM_OK;
}

// The posterior with its per-(row, chunk) partials at `ws` (ws_bytes of
// device memory, or NULL when none is given).
static int posterior_with(const float *logits, const float *prev_logits, uint8_t *locked, float eps,
                          const dlm_select *select, int32_t *sel, float *kl, float *conf, int32_t R,
                          int32_t V, hipStream_t stream, void *ws, size_t ws_bytes)
{
    const bool live = select->live_rows != nullptr;
    // One launch unless the selection waits for an event (the two-launch
    // path streams the logits before that wait).
    const bool fused = select->score_ready == nullptr;
    dlm::PostPlan p = dlm::plan_post(R, V, select->mode, select->group_rows, live, fused);
    const size_t need = dlm::post_ws_bytes(R, V, select->mode, select->group_rows, live);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(DLM_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    dlm::PostArgs a{};
    a.x = logits; a.y = prev_logits; a.locked = locked; a.score = select->score;
    a.sel = sel; a.kl = kl; a.conf = conf; a.margin = select->margin; a.entropy = select->entropy;
    a.flags = select->row_flags;
    a.part = reinterpret_cast<dlm::PostPartial *>(static_cast<char *>(ws) + p.off_part);
    a.R = R; a.V = V; a.mode = select->mode; a.k = select->k; a.group_rows = p.group_rows;
    a.eps = eps; a.tau = select->tau; a.conf_gate = select->conf_gate;
    a.n_chunks = p.n_chunks; a.chunk = p.chunk;
    a.live_rows = select->live_rows; a.n_live = select->n_live;
    a.live_offset = select->live_offset; a.nc_cap = p.n_chunks;
    if (p.fused) {
        char *w = static_cast<char *>(ws);
        a.rowres = reinterpret_cast<dlm::PostRowRes *>(w + p.off_rowres);
        a.row_cnt = reinterpret_cast<unsigned *>(w + p.off_row_cnt);
        a.grp_cnt = reinterpret_cast<unsigned *>(w + p.off_grp_cnt);
    }
    hipError_t e = dlm::launch_posterior(a, stream, select->score_ready);
    if (e != hipSuccess) return fail(DLM_E_HIP, "launch or event wait failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

static int check_post_call(const float *logits, const float *prev_logits, uint8_t *locked, float eps,
                           const dlm_select *select, int32_t *sel, float *kl, float *conf, int32_t R,
                           int32_t V)
{
    int rc = check_post_scalars(R, V, select);
    if (rc != DLM_OK) return rc;
    if (!logits || !prev_logits || !locked || !sel || !kl || !conf)
        return fail(DLM_E_NULL, "logits, prev_logits, locked, sel, kl and conf must be non-NULL");
    if ((select->mode == DLM_SEL_ATTN_DYNAMIC || select->mode == DLM_SEL_TOPK_SCORE) && !select->score)
        return fail(DLM_E_NULL, "selection by score needs select->score");
    if (select->live_rows && !select->n_live) return fail(DLM_E_NULL, "live_rows needs n_live");
    if (isnan(eps)) return fail(DLM_E_DESC, "eps is NaN");
    if ((V & 3) == 0 && (!aligned16(logits) || !aligned16(prev_logits)))
        return fail(DLM_E_SHAPE, "logits must be 16-byte aligned");
    return DLM_OK;
}

int dlm_posterior(const float *logits, const float *prev_logits, uint8_t *locked, float eps,
                  const dlm_select *select, int32_t *sel, float *kl, float *conf, int32_t R, int32_t V,
                  hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_post_call(logits, prev_logits, locked, eps, select, sel, kl, conf, R, V);
    if (rc != DLM_OK) return rc;
    return posterior_with(logits, prev_logits, locked, eps, select, sel, kl, conf, R, V, stream,
                          select->workspace, select->workspace_bytes);
}

// ---------------------------------------------------------------------------
// Allocation-free posterior.  The partials live in `scratch`, a file-scope
// device array: every GPU the library runs on holds its own copy from the
// first call on that device until the process ends.  In host code the
// array's name is only a host-side stand-in, so its device address is
// fetched once per device (with that device current) by
// hipGetSymbolAddress and kept; kernels get that address, never the name.
// Every call on a GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, two threads) race on it.  Nothing in it has to start
// at zero: the stream kernel writes every partial the finish kernel reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[DLM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device
}  // namespace

static int scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DLM_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DLM_E_UNSUPPORTED, "device %d is past the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(DLM_E_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return DLM_OK;
}

int dlm_posterior_noalloc(const float *logits, const float *prev_logits, uint8_t *locked, float eps,
                          const dlm_select *select, int32_t *sel, float *kl, float *conf, int32_t R,
                          int32_t V, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_post_call(logits, prev_logits, locked, eps, select, sel, kl, conf, R, V);
    if (rc != DLM_OK) return rc;
    const size_t need = dlm::post_ws_bytes(R, V, select->mode, select->group_rows, select->live_rows != nullptr);
    if (need > (size_t)DLM_NOALLOC_SCRATCH_BYTES)
        return fail(DLM_E_WORKSPACE, "R=%d V=%d needs %zu bytes of partials; the allocation-free entry "
                    "point holds %zu (use dlm_posterior with a workspace)", R, V, need,
                    (size_t)DLM_NOALLOC_SCRATCH_BYTES);
    if (R == 0) return DLM_OK;
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != DLM_OK) return rc;
    return posterior_with(logits, prev_logits, locked, eps, select, sel, kl, conf, R, V, stream, ws,
                          (size_t)DLM_NOALLOC_SCRATCH_BYTES);
}

static int check_layer(const dlm_layer_desc *L)
{
    if (!L) return fail(DLM_E_NULL, "layer descriptor is NULL");
    if (L->B < 1 || L->n_pos < 1 || L->M < 0 || L->d < 1 || L->F < 1 || L->Hq < 1 || L->Hkv < 1 || L->D < 1)
        return fail(DLM_E_SHAPE, "B=%d n_pos=%d M=%d d=%d F=%d Hq=%d Hkv=%d D=%d out of range", L->B, L->n_pos,
                    L->M, L->d, L->F, L->Hq, L->Hkv, L->D);
    if (L->d % 64 != 0 || L->F % 64 != 0)
        return fail(DLM_E_UNSUPPORTED, "d=%d and F=%d must be multiples of 64", L->d, L->F);
    if (L->Hq % L->Hkv != 0) return fail(DLM_E_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", L->Hq, L->Hkv);
    const long big = (1L << 31) - 1;
    const long rows = (long)L->B * L->M;
    const long wq = (long)(L->Hq + 2 * L->Hkv) * L->D;
    if ((long)L->B * L->n_pos * L->d * 2 > big || rows * L->F * 2 > big || rows * L->d * 2 > big ||
        rows * wq * 2 > big || wq * L->d * 2 > big || (long)L->F * L->d * 2 > big || (long)L->Hq * L->D * L->d * 2 > big)
        return fail(DLM_E_SHAPE, "a tensor of the layer exceeds 2 GiB");
    if (L->M > 0 && !L->active_idx) return fail(DLM_E_NULL, "active_idx is NULL");
    if (L->weights_packed != 0 && L->weights_packed != 1)
        return fail(DLM_E_DESC, "weights_packed=%d must be 0 or 1", L->weights_packed);
    return DLM_OK;
}

static dlm::GemmArgs gemm_base(const dlm_layer_desc *L)
{
    dlm::GemmArgs a{};
    a.act = L->active_idx; a.m_valid = L->m_active;
    a.B = L->B; a.M = L->M; a.n_pos = L->n_pos; a.Hq = L->Hq; a.Hkv = L->Hkv; a.D = L->D;
    a.w_packed = L->weights_packed;
    return a;
}

int dlm_pack_weights(const void *w, void *packed, int32_t N, int32_t K, hipStream_t stream)
{
    g_err[0] = 0;
    if (N < 0 || K < 0) return fail(DLM_E_SHAPE, "N=%d K=%d out of range", N, K);
    if (N % 16 != 0 || K % 32 != 0)
        return fail(DLM_E_UNSUPPORTED, "N=%d must be a multiple of 16 and K=%d of 32", N, K);
    if ((long)N * K * 2 > (1L << 31) - 1) return fail(DLM_E_SHAPE, "N*K=%ld exceeds 2 GiB of bf16", (long)N * K);
    if ((long)N * K == 0) return DLM_OK;
    if (!w || !packed) return fail(DLM_E_NULL, "w and packed must be non-NULL");
    const char *a = static_cast<const char *>(w), *b = static_cast<const char *>(packed);
    const long bytes = (long)N * K * 2;
    if (a < b + bytes && b < a + bytes) return fail(DLM_E_DESC, "w and packed overlap");
    hipError_t e = dlm::launch_pack_weights(static_cast<const uint16_t *>(w), static_cast<uint16_t *>(packed), N, K,
                                            stream);
    if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

static int run_gemm(const dlm::GemmArgs &a, hipStream_t stream)
{
    hipError_t e = dlm::launch_gemm(a, stream);
    if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

static int check_bb(const dlm_block_buffer *bb)
{
    if (!bb) return fail(DLM_E_NULL, "block buffer is NULL");
    if (bb->B < 1) return fail(DLM_E_SHAPE, "B=%d must be >= 1", bb->B);
    if (bb->n_slots < 1 || bb->n_slots > dlm::kMaxSlots)
        return fail(DLM_E_SHAPE, "n_slots=%d must be in [1, %d]", bb->n_slots, dlm::kMaxSlots);
    if (bb->block_size < 1) return fail(DLM_E_SHAPE, "block_size=%d must be >= 1", bb->block_size);
    if (bb->max_active < 1) return fail(DLM_E_SHAPE, "max_active=%d must be >= 1", bb->max_active);
    if (bb->prefix_len < 0) return fail(DLM_E_SHAPE, "prefix_len=%d must be >= 0", bb->prefix_len);
    const long n_gen = (long)bb->n_slots * bb->block_size;
    if (n_gen > (1L << 24) || (long)bb->prefix_len + n_gen > (1L << 31) - 1 || bb->B * n_gen > (1L << 31) - 1)
        return fail(DLM_E_SHAPE, "generation region too large (%ld positions)", n_gen);
    if (!bb->slot_state || !bb->slot_group || !bb->decoded || !bb->tokens || !bb->locked || !bb->skip ||
        !bb->row_flags || !bb->active_idx || !bb->m_active || !bb->n_open)
        return fail(DLM_E_NULL, "every array of the block buffer must be non-NULL");
    return DLM_OK;
}

static int run_bb(const dlm_block_buffer *bb, const int32_t *sel, hipStream_t stream)
{
    dlm::BBArgs a{};
    a.state = bb->slot_state; a.group = bb->slot_group; a.decoded = bb->decoded; a.tokens = bb->tokens;
    a.locked = bb->locked; a.skip = bb->skip; a.flags = bb->row_flags; a.active_idx = bb->active_idx;
    a.m_active = bb->m_active; a.n_open = bb->n_open; a.sel = sel;
    a.B = bb->B; a.n_slots = bb->n_slots; a.bs = bb->block_size; a.max_active = bb->max_active;
    a.P = bb->prefix_len; a.n_gen = bb->n_slots * bb->block_size;
    hipError_t e = dlm::launch_block_buffer(a, stream);
    if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// The products of the layer's calls and their K splits.
struct LayerPlans {
    dlm::GemmPlan qkv, out, gu, down;
    size_t g_bytes;        // gated hidden rows (bf16)
    size_t xp_bytes;       // weight-streaming products: the packed rows of x[act] and of h
    size_t total;
};
static LayerPlans plan_layer(const dlm_layer_desc *L)
{
    LayerPlans p{};
    const int rows = L->B * L->M;
    p.qkv = dlm::plan_gemm(rows, (L->Hq + 2 * L->Hkv) * L->D, L->d, false);
    p.out = dlm::plan_gemm(rows, L->d, L->Hq * L->D, false);
    p.gu = dlm::plan_gemm(rows, L->F, L->d, true);
    p.down = dlm::plan_gemm(rows, L->d, L->F, false);
    // gated hidden rows: row-major, or (weight-streaming kernel) one packed
    // 16-row operand block
    p.g_bytes = al256((size_t)(dlm::gemm_skinny(rows) ? 16 : rows) * L->F * 2);
    p.xp_bytes = dlm::gemm_skinny(rows) ? al256((size_t)16 * L->d * 2) : 0;
    size_t t = p.qkv.part_bytes > p.out.part_bytes ? p.qkv.part_bytes : p.out.part_bytes;
    if (p.xp_bytes > t) t = p.xp_bytes;
    const size_t f = p.g_bytes + p.xp_bytes +
                     (p.gu.part_bytes > p.down.part_bytes ? p.gu.part_bytes : p.down.part_bytes);
    p.total = t > f ? t : f;
    return p;
}

static int check_ws(void *ws, size_t have, size_t need)
{
    if (need > 0 && (!ws || have < need))
        return fail(DLM_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? have : (size_t)0);
    return DLM_OK;
}

static void set_plan(dlm::GemmArgs &a, const dlm::GemmPlan &p, void *part)
{
    a.splits = p.splits;
    a.kc = p.kc;
    a.part = p.splits > 1 ? static_cast<float *>(part) : nullptr;
}

int dlm_layer_workspace_bytes(const dlm_layer_desc *L, size_t *bytes)
{
    g_err[0] = 0;
    if (!bytes) return fail(DLM_E_NULL, "bytes is NULL");
    int rc = check_layer(L);
    if (rc != DLM_OK) return rc;
    *bytes = plan_layer(L).total;
    return DLM_OK;
}

int dlm_proj_qkv(const dlm_layer_desc *L, const void *x, const void *w_qkv, void *q, void *k, void *v,
                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_layer(L);
    if (rc != DLM_OK) return rc;
    if (!x || !w_qkv || (L->M > 0 && (!q || !k || !v))) return fail(DLM_E_NULL, "x, w_qkv, q, k and v must be non-NULL");
    if (L->M == 0) return DLM_OK;
    const LayerPlans P = plan_layer(L);
    rc = check_ws(workspace, workspace_bytes, P.qkv.part_bytes > P.xp_bytes ? P.qkv.part_bytes : P.xp_bytes);
    if (rc != DLM_OK) return rc;
    dlm::GemmArgs a = gemm_base(L);
    a.a = static_cast<const uint16_t *>(x);
    a.a_bytes = (long)L->B * L->n_pos * L->d * 2;
    a.a_mode = 1; a.ep_mode = 1;
    a.K = L->d; a.N = (L->Hq + 2 * L->Hkv) * L->D;
    if (P.xp_bytes) {   // gather the active rows once, as packed fragments
        hipError_t e = dlm::launch_pack_rows(a, static_cast<uint16_t *>(workspace), stream);
        if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        a.a = static_cast<const uint16_t *>(workspace);
        a.a_mode = 3;
    }
    a.w0 = static_cast<const uint16_t *>(w_qkv);
    a.out = static_cast<uint16_t *>(q); a.out_k = static_cast<uint16_t *>(k); a.out_v = static_cast<uint16_t *>(v);
    set_plan(a, P.qkv, workspace);
    return run_gemm(a, stream);
}

int dlm_proj_out(const dlm_layer_desc *L, const void *x, const void *attn_out, const void *w_o, void *h,
                 void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_layer(L);
    if (rc != DLM_OK) return rc;
    if (L->D % 64 != 0) return fail(DLM_E_UNSUPPORTED, "dlm_proj_out needs D a multiple of 64 (D=%d)", L->D);
    if (!x || !w_o || (L->M > 0 && (!attn_out || !h))) return fail(DLM_E_NULL, "x, attn_out, w_o and h must be non-NULL");
    if (L->M == 0) return DLM_OK;
    const LayerPlans P = plan_layer(L);
    rc = check_ws(workspace, workspace_bytes, P.out.part_bytes);
    if (rc != DLM_OK) return rc;
    dlm::GemmArgs a = gemm_base(L);
    a.a = static_cast<const uint16_t *>(attn_out);
    a.a_bytes = (long)L->B * L->Hq * L->M * L->D * 2;
    a.a_mode = 2; a.ep_mode = 2; a.resid_gather = 1;
    a.K = L->Hq * L->D; a.N = L->d;
    a.w0 = static_cast<const uint16_t *>(w_o);
    a.resid = static_cast<const uint16_t *>(x);
    a.out = static_cast<uint16_t *>(h);
    set_plan(a, P.out, workspace);
    return run_gemm(a, stream);
}

int dlm_ffn(const dlm_layer_desc *L, const void *h, const void *w_gate, const void *w_up, const void *w_down,
            void *x, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_layer(L);
    if (rc != DLM_OK) return rc;
    if (!w_gate || !w_up || !w_down || !x || (L->M > 0 && !h))
        return fail(DLM_E_NULL, "h, w_gate, w_up, w_down and x must be non-NULL");
    if (L->M == 0) return DLM_OK;
    const LayerPlans P = plan_layer(L);
    const size_t need = P.g_bytes + P.xp_bytes + (P.gu.part_bytes > P.down.part_bytes ? P.gu.part_bytes : P.down.part_bytes);
    rc = check_ws(workspace, workspace_bytes, need);
    if (rc != DLM_OK) return rc;
    char *ws = static_cast<char *>(workspace);
    dlm::GemmArgs g = gemm_base(L);      // gated hidden rows: silu(h Wg^T) * (h Wu^T)
    g.a = static_cast<const uint16_t *>(h);
    g.a_bytes = (long)L->B * L->M * L->d * 2;
    g.a_mode = 0; g.ep_mode = 0;
    g.K = L->d; g.N = L->F;
    g.w0 = static_cast<const uint16_t *>(w_gate); g.w1 = static_cast<const uint16_t *>(w_up);
    g.out = reinterpret_cast<uint16_t *>(ws);
    g.out_packed = dlm::gemm_skinny(L->B * L->M);   // the down projection then reads packed fragments
    set_plan(g, P.gu, ws + P.g_bytes + P.xp_bytes);
    if (P.xp_bytes) {   // h as packed fragments
        hipError_t e = dlm::launch_pack_rows(g, reinterpret_cast<uint16_t *>(ws + P.g_bytes), stream);
        if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        g.a = reinterpret_cast<const uint16_t *>(ws + P.g_bytes);
        g.a_mode = 3;
    }
    rc = run_gemm(g, stream);
    if (rc != DLM_OK) return rc;
    dlm::GemmArgs d = gemm_base(L);      // down projection + residual, back to x's active rows
    d.a = reinterpret_cast<const uint16_t *>(ws);
    d.a_bytes = (long)L->B * L->M * L->F * 2;
    d.a_mode = g.out_packed ? 3 : 0; d.ep_mode = 3; d.resid_gather = 0;
    d.K = L->F; d.N = L->d;
    d.w0 = static_cast<const uint16_t *>(w_down);
    d.resid = static_cast<const uint16_t *>(h);
    d.out = static_cast<uint16_t *>(x);
    set_plan(d, P.down, ws + P.g_bytes + P.xp_bytes);
    return run_gemm(d, stream);
}

int dlm_r2l_scan(const dlm_r2l_desc *desc, const void *u, const void *delta, const float *A, const void *Bm,
                 const void *Cm, const float *D, float *y, void *x, hipStream_t stream)
{
    g_err[0] = 0;
    if (!desc) return fail(DLM_E_NULL, "descriptor is NULL");
    const dlm_r2l_desc *d = desc;
    if (d->B < 1 || d->L < 0 || d->E < 1 || d->N < 1)
        return fail(DLM_E_SHAPE, "B=%d L=%d E=%d N=%d out of range", d->B, d->L, d->E, d->N);
    if (d->N != 8 && d->N != 16 && d->N != 32)
        return fail(DLM_E_UNSUPPORTED, "N=%d not in {8, 16, 32}", d->N);
    if (d->E % 8 != 0) return fail(DLM_E_UNSUPPORTED, "E=%d is not a multiple of 8", d->E);
    if ((long)d->B * d->L * d->E > (1L << 31) - 1) return fail(DLM_E_SHAPE, "B*L*E too large");
    if (!isfinite(d->gate)) return fail(DLM_E_DESC, "gate must be finite");
    if (!u || !delta || !A || !Bm || !Cm || !D) return fail(DLM_E_NULL, "u, delta, A, Bm, Cm and D must be non-NULL");
    if (!y && !x) return fail(DLM_E_NULL, "at least one of y and x must be given");
    if (!aligned16(u) || !aligned16(delta) || !aligned16(Bm) || !aligned16(Cm) || (x && !aligned16(x)))
        return fail(DLM_E_SHAPE, "u, delta, Bm, Cm and x must be 16-byte aligned");
    if (d->L == 0) return DLM_OK;
    dlm::R2LArgs a{};
    a.u = static_cast<const uint16_t *>(u); a.delta = static_cast<const uint16_t *>(delta);
    a.Bm = static_cast<const uint16_t *>(Bm); a.Cm = static_cast<const uint16_t *>(Cm);
    a.A = A; a.D = D; a.y = y; a.x = static_cast<uint16_t *>(x);
    a.B = d->B; a.L = d->L; a.E = d->E; a.N = d->N; a.gate = d->gate;
    hipError_t e = dlm::launch_r2l(a, stream);
    if (e != hipSuccess) return fail(DLM_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return DLM_OK;
}

int dlm_block_buffer_init(const dlm_block_buffer *bb, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_bb(bb);
    if (rc != DLM_OK) return rc;
    return run_bb(bb, nullptr, stream);
}

int dlm_block_buffer_advance(const dlm_block_buffer *bb, const int32_t *sel, hipStream_t stream)
{
    g_err[0] = 0;
    int rc = check_bb(bb);
    if (rc != DLM_OK) return rc;
    if (!sel) return fail(DLM_E_NULL, "sel is NULL");
    return run_bb(bb, sel, stream);
}

}  // extern "C"
