// attn_kernels.hip -- sparse-query attention of one denoising step on gfx950.
//
// What is computed (SureLock page, sec. 2 core mechanism; Bifocal dLLM page,
// sec. 2 inference; Attn-Sampler page, sec. 2B):
//   scatter  cache[b, g, active_idx[b, j]] <- fresh k/v of active row j
//   pass 1   per active row and q-head: s = scale * q . K over visible keys,
//            lse = logsumexp(s), out = softmax(s) V        (bf16 MFMA)
//   pass 2   colsum[b, n] = sum over heads and counted rows of
//            exp(s_n - lse)                               (bf16 MFMA recompute)
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64): operand A is 32 rows x 16
// k; lane l holds row l%32, k = 8*(l/32) .. +8.  Operand B is 16 k x 32
// columns; lane l holds column l%32, the same k.  The 32x32 fp32 result
// gives lane l column l%32 and, in element i, row 8*(i/4) + 4*(l/32) + i%4.
//
// Pass 1 computes S^T = K Q^T so each lane owns ONE query (its column): the
// online softmax is per-lane with a single exchange between the two
// half-waves, and the output O^T = V^T P^T needs P^T as operand B, which
// must hold 8 consecutive keys per lane.  The accumulator rows of S^T are
// not consecutive keys, so the LDS copy of each 32-key K sub-tile stores key
// n at row sigma(n) (bits 2 and 3 of n swapped): then accumulator element i
// of half-wave h holds key 16*(i/8) + 8*h + i%8, exactly the operand-B order.
// V is stored transposed in LDS (Vt[d][key]) so operand A of V^T P^T is one
// 16-byte read.
//
// Pass 2 computes S = Q K^T with the key as the accumulator COLUMN: each
// lane owns one key for the whole pass, so column sums accumulate in
// registers across query tiles and heads with no atomics; the two half-waves
// are added once at the end.  Partials go to a workspace and are reduced in
// a fixed order, so colsum is bitwise reproducible.
#include "dlm_internal.h"

#include <limits.h>
#include <math.h>

namespace dlm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Key code: a key is visible to a query iff key_code <= query_code.
//   FULL:          in-range keys INT_MIN; query code 0.
//   BLOCK_CAUSAL:  prefix INT_MIN; block index; query code = its block.
//   GROUP:         prefix INT_MIN; group id of the slot (INT_MAX if the slot is
//                  DUMMY); query code = group id of its slot.
// Keys at or beyond kv_len are INT_MAX.
__device__ __forceinline__ int key_code(const AttnArgs &a, const uint8_t *st, const int32_t *gr,
                                        int n)
{
    if (n >= a.kv_len) return INT_MAX;
    if (a.kind == 0 || n < a.P) return INT_MIN;
    int s = (n - a.P) / a.bs;
    if (a.kind == 1) return s;
    if (s >= a.n_slots || st[s] == 0) return INT_MAX;
    return gr[s];
}

__device__ __forceinline__ int query_code(const AttnArgs &a, const int32_t *gr, int pos)
{
    if (a.kind == 0) return 0;
    int s = (pos - a.P) / a.bs;
    if (a.kind == 1) return s;
    return (s >= 0 && s < a.n_slots) ? gr[s] : INT_MIN;
}

// ---------------------------------------------------------------------------
// Scatter: cache[b, g, active_idx[b, j], :] = fresh[b, g, j, :], 16 B/thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_scatter_kernel(AttnArgs a, long total)
{
    const int ch = a.D / 8;
    long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    int c = (int)(t % ch);
    long row = t / ch;                  // (b*Hkv + g)*M + j
    int j = (int)(row % a.M);
    long bg = row / a.M;
    int b = (int)(bg / a.Hkv);
    int pos = a.active_idx[(long)b * a.M + j];
    long dst = (bg * a.n_cap + pos) * ch + c;
    reinterpret_cast<uint4 *>(a.ck)[dst] = reinterpret_cast<const uint4 *>(a.k)[t];
    reinterpret_cast<uint4 *>(a.cv)[dst] = reinterpret_cast<const uint4 *>(a.v)[t];
}

// ---------------------------------------------------------------------------
// Pass 1.  Workgroup = 4 waves = 128 packed query rows of one (b, kv-head):
// packed row r = (q-head within the GQA group) * M + j, so the G q-heads that
// share a kv-head share every K/V tile staged in LDS.  Optional key split.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a)
{
    constexpr int KT = kKeyTile;
    constexpr int KSTR = D + 8;          // bf16 per LDS K row (16 B pad: conflict-free reads)
    constexpr int VSTR = KT + 8;         // bf16 per LDS Vt row
    constexpr int DK = D / 16;           // MFMA k-steps over the head dim
    constexpr int DT = D / 32;           // 32-row tiles of O^T
    constexpr int CH = D / 8;            // 16-byte chunks per K/V row
    constexpr int KLOADS = KT * CH / 256;        // K chunks per thread per tile
    constexpr int VGROUPS = (KT / 4) * CH;       // (4-key group, chunk) pairs per tile
    constexpr int VLOADS = (VGROUPS + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];
    __shared__ int kcode_s[KT];
    __shared__ int scode_s[kMaxSlots];

    const int tid = threadIdx.x;
    const int wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    int L = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = L % a.n_qtiles;
    L /= a.n_qtiles;
    const int split = L % a.n_split;
    const int bg = L / a.n_split;
    const int b = bg / a.Hkv, g = bg % a.Hkv;

    const uint8_t *st = a.kind == 2 ? a.slot_state + (long)b * a.n_slots : nullptr;
    const int32_t *gr = a.kind == 2 ? a.slot_group + (long)b * a.n_slots : nullptr;
    if (a.kind == 2) {
        for (int s = tid; s < a.n_slots; s += 256) scode_s[s] = st[s] == 0 ? INT_MAX : gr[s];
    }

    // This lane's query.
    const int rows_bg = a.G * a.M;
    const int r = qt * kAttnRows + wid * 32 + l32;
    const bool rv = r < rows_bg;
    const int hl = rv ? r / a.M : 0;
    const int j = rv ? r - hl * a.M : 0;
    const int h = g * a.G + hl;
    const int pos = a.active_idx[(long)b * a.M + j];
    const int qcode = rv ? query_code(a, gr, pos) : INT_MIN;

    bf16x8 qf[DK];
    {
        const uint16_t *qrow = a.q + ((long)(b * a.Hq + h) * a.M + j) * D;
        for (int kk = 0; kk < DK; ++kk) {
            if (rv) qf[kk] = *reinterpret_cast<const bf16x8 *>(qrow + kk * 16 + hh * 8);
            else qf[kk] = bf16x8{};
        }
    }

    const int k0 = split * a.split_keys;
    const int k1 = min(a.kv_len, k0 + a.split_keys);
    const uint16_t *kbase = a.ck + (long)bg * a.n_cap * D;
    const uint16_t *vbase = a.cv + (long)bg * a.n_cap * D;

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[DT];
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

    uint4 kreg[KLOADS], vreg[VLOADS][4];

    // A key row is loaded when it is below kv_len and not in a DUMMY slot
    // (DUMMY rows may hold anything; their weight is 0, their values must
    // not poison 0 * V).
    auto row_ok = [&](int n) -> bool {
        if (n >= a.kv_len) return false;
        if (a.kind != 2 || n < a.P) return true;
        int s = (n - a.P) / a.bs;
        return s < a.n_slots && scode_s[s] != INT_MAX;
    };
    auto load_tile = [&](int t0) {
        for (int u = 0; u < KLOADS; ++u) {
            int idx = tid + 256 * u;
            int n = idx / CH, c = idx % CH;
            kreg[u] = row_ok(t0 + n) ? *reinterpret_cast<const uint4 *>(kbase + (long)(t0 + n) * D + c * 8)
                                     : uint4{0, 0, 0, 0};
        }
        for (int u = 0; u < VLOADS; ++u) {
            int idx = tid + 256 * u;
            if (idx < VGROUPS) {
                int kg = idx % (KT / 4), c = idx / (KT / 4);
                for (int e = 0; e < 4; ++e) {
                    int n = t0 + kg * 4 + e;
                    vreg[u][e] = row_ok(n) ? *reinterpret_cast<const uint4 *>(vbase + (long)n * D + c * 8)
                                           : uint4{0, 0, 0, 0};
                }
            }
        }
    };
    auto store_tile = [&](int t0) {
        for (int u = 0; u < KLOADS; ++u) {
            int idx = tid + 256 * u;
            int n = idx / CH, c = idx % CH;
            int nr = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);   // sigma(n)
            *reinterpret_cast<uint4 *>(&Ks[nr * KSTR + c * 8]) = kreg[u];
        }
        for (int u = 0; u < VLOADS; ++u) {
            int idx = tid + 256 * u;
            if (idx < VGROUPS) {
                int kg = idx % (KT / 4), c = idx / (KT / 4);
                const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vreg[u][0]);
                const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vreg[u][1]);
                const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&vreg[u][2]);
                const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&vreg[u][3]);
                for (int w = 0; w < 4; ++w) {
                    // d = 8c + 2w (low halves) and 8c + 2w + 1 (high halves)
                    uint2 ev, od;
                    ev.x = (w0[w] & 0xFFFFu) | (w1[w] << 16);
                    ev.y = (w2[w] & 0xFFFFu) | (w3[w] << 16);
                    od.x = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
                    od.y = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
                    *reinterpret_cast<uint2 *>(&Vt[(c * 8 + 2 * w) * VSTR + kg * 4]) = ev;
                    *reinterpret_cast<uint2 *>(&Vt[(c * 8 + 2 * w + 1) * VSTR + kg * 4]) = od;
                }
            }
        }
        if (tid < KT) kcode_s[tid] = key_code(a, st, gr, t0 + tid);
    };

    __syncthreads();   // slot codes visible
    if (k0 < k1) load_tile(k0);
    for (int t0 = k0; t0 < k1; t0 += KT) {
        __syncthreads();
        store_tile(t0);
        __syncthreads();
        if (t0 + KT < k1) load_tile(t0 + KT);

        // S^T for two 32-key sub-tiles.
        f32x16 s[2];
        for (int sub = 0; sub < 2; ++sub) {
            s[sub] = f32x16{};
            const uint16_t *kr = &Ks[(sub * 32 + l32) * KSTR + hh * 8];
            for (int kk = 0; kk < DK; ++kk) s[sub] = mfma32(lds_frag(kr + kk * 16), qf[kk], s[sub]);
        }
        const bool all_vis = (a.kind == 0 && t0 + KT <= a.kv_len) || (t0 + KT <= a.P);
        float tmax = -INFINITY;
        for (int sub = 0; sub < 2; ++sub) {
            for (int i = 0; i < 16; ++i) {
                float v = s[sub][i] * a.scale_log2;
                if (!all_vis) {
                    int key = sub * 32 + 16 * (i >> 3) + 8 * hh + (i & 7);
                    if (kcode_s[key] > qcode) v = -INFINITY;
                }
                s[sub][i] = v;
                tmax = fmaxf(tmax, v);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        bf16x8 pf[2][2];
        for (int sub = 0; sub < 2; ++sub)
            for (int t = 0; t < 2; ++t)
                for (int e = 0; e < 8; ++e) {
                    float p = fast_exp2(s[sub][t * 8 + e] - m_use);
                    psum += p;
                    pf[sub][t][e] = (__bf16)p;
                }
        l_run = l_run * alpha + psum;
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        for (int sub = 0; sub < 2; ++sub)
            for (int t = 0; t < 2; ++t)
                for (int dt = 0; dt < DT; ++dt) {
                    bf16x8 vf = lds_frag(&Vt[(dt * 32 + l32) * VSTR + sub * 32 + t * 16 + hh * 8]);
                    o[dt] = mfma32(vf, pf[sub][t], o[dt]);
                }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!rv) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float row_lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    const long row_flat = (long)(b * a.Hq + h) * a.M + j;
    if (a.n_split == 1) {
        uint16_t *orow = a.out + row_flat * D;
        for (int dt = 0; dt < DT; ++dt)
            for (int q4 = 0; q4 < 4; ++q4) {
                __bf16 v4[4];
                for (int c = 0; c < 4; ++c) v4[c] = (__bf16)(o[dt][q4 * 4 + c] * inv);
                *reinterpret_cast<uint2 *>(orow + dt * 32 + q4 * 8 + hh * 4) =
                    *reinterpret_cast<const uint2 *>(v4);
            }
        if (hh == 0) a.lse[row_flat] = row_lse;
    } else {
        const long rows_total = (long)a.B * a.Hq * a.M;
        float *orow = a.ws_o + ((long)split * rows_total + row_flat) * D;
        for (int dt = 0; dt < DT; ++dt)
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 v;
                v.x = o[dt][q4 * 4 + 0] * inv;
                v.y = o[dt][q4 * 4 + 1] * inv;
                v.z = o[dt][q4 * 4 + 2] * inv;
                v.w = o[dt][q4 * 4 + 3] * inv;
                *reinterpret_cast<float4 *>(orow + dt * 32 + q4 * 8 + hh * 4) = v;
            }
        if (hh == 0) a.ws_l[(long)split * rows_total + row_flat] = row_lse;
    }
}

// Merge the key splits of each row in split order:
// lse = logsumexp_s lse_s, out = sum_s exp(lse_s - lse) out_s.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a)
{
    constexpr int RPB = 256 / D;        // rows per block
    const long rows_total = (long)a.B * a.Hq * a.M;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / D;
    const int d = threadIdx.x % D;
    if (row >= rows_total) return;
    float m = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, a.ws_l[s * rows_total + row]);
    float res = 0.f, L = -INFINITY;
    if (m != -INFINITY) {
        float sum = 0.f;
        for (int s = 0; s < a.n_split; ++s) sum += expf(a.ws_l[s * rows_total + row] - m);
        L = m + logf(sum);
        for (int s = 0; s < a.n_split; ++s) {
            float w = expf(a.ws_l[s * rows_total + row] - L);
            res += w * a.ws_o[(s * rows_total + row) * D + d];
        }
    }
    __bf16 bv = (__bf16)res;
    a.out[row * D + d] = *reinterpret_cast<uint16_t *>(&bv);
    if (d == 0) a.lse[row] = L;
}

// ---------------------------------------------------------------------------
// Pass 2.  Workgroup = (b, kv-head g, row split, 256-key block); wave w owns
// keys [64w, 64w+64) of the block in registers for the whole pass.  It loops
// over the G q-heads of g and over 32-row query tiles of its slice of the
// counted rows, writing one partial column sum per (q-head, row split).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void colsum_kernel(AttnArgs a)
{
    constexpr int DK = D / 16;
    constexpr int QSTR = D + 8;
    constexpr int CH = D / 8;
    constexpr int QLOADS = (kCsRows * CH + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint16_t Qs[kCsRows * QSTR];
    __shared__ float lse2_s[kCsRows];
    __shared__ int qcode_s[kCsRows];
    __shared__ int range_s[2];

    const int tid = threadIdx.x;
    const int wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;

    int L = xcd_remap(blockIdx.x, gridDim.x);
    const int kb = L % a.n_kblocks;
    L /= a.n_kblocks;
    const int rs = L % a.n_rsplit;
    L /= a.n_rsplit;
    const int g = L % a.Hkv;
    const int b = L / a.Hkv;

    const uint8_t *st = a.kind == 2 ? a.slot_state + (long)b * a.n_slots : nullptr;
    const int32_t *gr = a.kind == 2 ? a.slot_group + (long)b * a.n_slots : nullptr;
    const int32_t *act = a.active_idx + (long)b * a.M;

    // Counted rows: active rows whose position lies in [cs_lo, cs_hi);
    // active_idx is ascending, so they are the index range [j_lo, j_hi).
    if (tid < 2) {
        int target = tid == 0 ? a.cs_lo : a.cs_hi;
        int lo = 0, hi = a.M;
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (act[mid] < target) lo = mid + 1;
            else hi = mid;
        }
        range_s[tid] = lo;
    }

    // This lane's two keys and their K fragments.
    int key[2], kc[2];
    bf16x8 kf[2][DK];
    const uint16_t *kbase = a.ck + ((long)b * a.Hkv + g) * a.n_cap * D;
    for (int ct = 0; ct < 2; ++ct) {
        key[ct] = kb * kCsKeys + wid * 64 + ct * 32 + l32;
        kc[ct] = key_code(a, st, gr, key[ct]);
        const bool ok = key[ct] < a.kv_len;
        for (int kk = 0; kk < DK; ++kk) {
            if (ok) kf[ct][kk] = *reinterpret_cast<const bf16x8 *>(kbase + (long)key[ct] * D + kk * 16 + hh * 8);
            else kf[ct][kk] = bf16x8{};
        }
    }
    __syncthreads();
    const int j_lo = range_s[0], j_hi = range_s[1];
    const int cnt = max(0, j_hi - j_lo);
    const int per = ((cnt + a.n_rsplit - 1) / a.n_rsplit + kCsRows - 1) / kCsRows * kCsRows;
    const int r0 = min(j_hi, j_lo + rs * per);
    const int r1 = min(j_hi, r0 + per);

    for (int hl = 0; hl < a.G; ++hl) {
        const int h = g * a.G + hl;
        const uint16_t *qhead = a.q + ((long)b * a.Hq + h) * a.M * D;
        const float *lhead = a.lse + ((long)b * a.Hq + h) * a.M;
        float acc[2] = {0.f, 0.f};
        for (int rb = r0; rb < r1; rb += kCsRows) {
            __syncthreads();
            for (int u = 0; u < QLOADS; ++u) {
                int idx = tid + 256 * u;
                if (idx < kCsRows * CH) {
                    int rr = idx / CH, c = idx % CH;
                    uint4 v = {0, 0, 0, 0};
                    if (rb + rr < r1) v = *reinterpret_cast<const uint4 *>(qhead + (long)(rb + rr) * D + c * 8);
                    *reinterpret_cast<uint4 *>(&Qs[rr * QSTR + c * 8]) = v;
                }
            }
            if (tid < kCsRows) {
                int jr = rb + tid;
                float l2 = INFINITY;
                int qc = INT_MIN;
                if (jr < r1) {
                    float lv = lhead[jr];
                    if (lv != -INFINITY) {
                        l2 = lv * kLog2e;
                        qc = query_code(a, gr, act[jr]);
                    }
                }
                lse2_s[tid] = l2;
                qcode_s[tid] = qc;
            }
            __syncthreads();
            f32x16 s0 = f32x16{}, s1 = f32x16{};
            const uint16_t *qr = &Qs[l32 * QSTR + hh * 8];
            for (int kk = 0; kk < DK; ++kk) {
                bf16x8 qa = lds_frag(qr + kk * 16);
                s0 = mfma32(qa, kf[0][kk], s0);
                s1 = mfma32(qa, kf[1][kk], s1);
            }
            for (int i = 0; i < 16; ++i) {
                int ri = 8 * (i >> 2) + 4 * hh + (i & 3);
                float l2 = lse2_s[ri];
                int qc = qcode_s[ri];
                float p0 = fast_exp2(s0[i] * a.scale_log2 - l2);
                float p1 = fast_exp2(s1[i] * a.scale_log2 - l2);
                if (kc[0] <= qc) acc[0] += p0;
                if (kc[1] <= qc) acc[1] += p1;
            }
        }
        for (int ct = 0; ct < 2; ++ct) {
            float tot = acc[ct] + __shfl_xor(acc[ct], 32);
            if (hh == 0 && key[ct] < a.kv_len)
                a.ws_cs[(((long)b * a.Hq + h) * a.n_rsplit + rs) * a.kv_len + key[ct]] = tot;
        }
    }
}

// colsum[b, n] = sum_h sum_rs part[b, h, rs, n] (or per head: sum_rs), fixed order.
__global__ __launch_bounds__(256) void colsum_reduce_kernel(AttnArgs a)
{
    const int nh = a.per_head ? a.Hq : 1;
    const long total = (long)a.B * nh * a.kv_len;
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int n = (int)(t % a.kv_len);
    const long bh = t / a.kv_len;
    float sum = 0.f;
    if (a.per_head) {
        const float *p = a.ws_cs + bh * a.n_rsplit * a.kv_len + n;
        for (int s = 0; s < a.n_rsplit; ++s) sum += p[(long)s * a.kv_len];
    } else {
        const float *p = a.ws_cs + bh * a.Hq * a.n_rsplit * a.kv_len + n;
        for (int s = 0; s < a.Hq * a.n_rsplit; ++s) sum += p[(long)s * a.kv_len];
    }
    a.colsum[t] = sum;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, long n)
{
    long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t < n) p[t] = 0.f;
}

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t stream)
{
    if (a.M > 0 && a.k != nullptr) {
        long total = (long)a.B * a.Hkv * a.M * (D / 8);
        kv_scatter_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(a, total);
    }
    if (a.M == 0) {
        if (a.colsum) {
            long n = (long)a.B * (a.per_head ? a.Hq : 1) * a.kv_len;
            fill_zero_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a.colsum, n);
        }
        return hipGetLastError();
    }
    {
        long nwg = (long)a.B * a.Hkv * a.n_split * a.n_qtiles;
        attn_fwd_kernel<D><<<dim3((unsigned)nwg), dim3(256), 0, stream>>>(a);
    }
    if (a.n_split > 1) {
        long rows = (long)a.B * a.Hq * a.M;
        constexpr int RPB = 256 / D;
        attn_combine_kernel<D><<<dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream>>>(a);
    }
    if (a.colsum) {
        long nwg = (long)a.B * a.Hkv * a.n_rsplit * a.n_kblocks;
        colsum_kernel<D><<<dim3((unsigned)nwg), dim3(256), 0, stream>>>(a);
        long n = (long)a.B * (a.per_head ? a.Hq : 1) * a.kv_len;
        colsum_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_attn(const AttnArgs &a, hipStream_t stream)
{
    switch (a.D) {
    case 32: return launch_attn_d<32>(a, stream);
    case 64: return launch_attn_d<64>(a, stream);
    case 128: return launch_attn_d<128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

AttnPlan plan_attn(int B, int Hq, int Hkv, int D, int M, int kv_len, int n_cap)
{
    AttnPlan p{};
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.D = D; p.M = M;
    p.kv_len = kv_len; p.n_cap = n_cap;
    p.n_qtiles = (p.G * M + kAttnRows - 1) / kAttnRows;
    const long base = (long)B * Hkv * p.n_qtiles;
    const int key_tiles = (kv_len + kKeyTile - 1) / kKeyTile;
    // Split the keys until about two workgroups per CU are resident, keeping
    // at least four key tiles per split.
    int split = 1;
    if (base > 0 && base < 2L * kNumCU) {
        split = (int)((2L * kNumCU + base - 1) / base);
        split = min(split, max(1, key_tiles / 4));
    }
    int tiles_per = (key_tiles + split - 1) / split;
    p.split_keys = max(1, tiles_per) * kKeyTile;
    p.n_split = max(1, (kv_len + p.split_keys - 1) / p.split_keys);
    p.n_kblocks = (kv_len + kCsKeys - 1) / kCsKeys;
    const long cs_base = (long)B * Hkv * p.n_kblocks;
    int rsplit = 1;
    if (cs_base > 0 && cs_base < 2L * kNumCU) {
        rsplit = (int)((2L * kNumCU + cs_base - 1) / cs_base);
        rsplit = min(rsplit, max(1, M / (2 * kCsRows)));
    }
    p.n_rsplit = rsplit;
    const size_t rows_total = (size_t)B * Hq * M;
    p.ws_split_o = p.n_split > 1 ? rows_total * p.n_split * D * sizeof(float) : 0;
    p.ws_split_l = p.n_split > 1 ? rows_total * p.n_split * sizeof(float) : 0;
    p.ws_colsum = (size_t)B * Hq * p.n_rsplit * kv_len * sizeof(float);
    auto align = [](size_t x) { return (x + 255) / 256 * 256; };
    p.ws_total = align(p.ws_split_o) + align(p.ws_split_l) + align(p.ws_colsum);
    return p;
}

}  // namespace dlm
