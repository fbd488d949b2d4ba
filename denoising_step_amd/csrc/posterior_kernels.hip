// posterior_kernels.hip -- posterior, lock test and unmask selection on gfx950.
//
// What is computed, per row r not locked on entry (SureLock page, sec. 2
// core mechanism; Attn-Sampler page, sec. 1 and 2B):
//   p = softmax(x), q = softmax(y) for step-t logits x and step-(t-1) y
//   KL(p || q) = E_p[x - y] - (logsumexp x - logsumexp y)    (one pass)
//   conf = max p = 1 / sum exp(x - max x),  tok = lowest argmax x
//   lock if KL <= eps;  then a per-group selection (top-k / threshold /
//   Attn-Sampler dynamic threshold / top-k by score).
//
// The stream kernel is HBM-bound: every logit of both steps is read exactly
// once with 16-byte non-temporal loads, 4 per array in flight per thread,
// and reduced with an online (running-max) log-sum-exp.  Rows are split into
// vocabulary chunks when there are too few rows to fill the chip; each chunk
// writes one partial state, and the finishing kernel merges the partials of
// a row in chunk order (deterministic), then selects within each group.
#include "dlm_internal.h"

#include <limits.h>
#include <math.h>

namespace dlm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct RowState {
    float mx, sx, tx, my, sy, av;
    int ai;
};

__device__ __forceinline__ void rs_init(RowState &s)
{
    s.mx = -INFINITY; s.sx = 0.f; s.tx = 0.f;
    s.my = -INFINITY; s.sy = 0.f;
    s.av = -INFINITY; s.ai = INT_MAX;
}

// Merge state b into a.  Both describe disjoint element sets.
__device__ __forceinline__ void rs_merge(RowState &a, const RowState &b)
{
    float m = fmaxf(a.mx, b.mx);
    if (m != -INFINITY) {
        float ca = fast_exp2((a.mx - m) * kLog2e), cb = fast_exp2((b.mx - m) * kLog2e);
        a.sx = a.sx * ca + b.sx * cb;
        a.tx = a.tx * ca + b.tx * cb;
    }
    a.mx = m;
    float my = fmaxf(a.my, b.my);
    if (my != -INFINITY) {
        float ca = fast_exp2((a.my - my) * kLog2e), cb = fast_exp2((b.my - my) * kLog2e);
        a.sy = a.sy * ca + b.sy * cb;
    }
    a.my = my;
    if (b.av > a.av || (b.av == a.av && b.ai < a.ai)) {
        a.av = b.av;
        a.ai = b.ai;
    }
}

__device__ __forceinline__ RowState rs_shfl_xor(const RowState &s, int m)
{
    RowState o;
    o.mx = __shfl_xor(s.mx, m); o.sx = __shfl_xor(s.sx, m); o.tx = __shfl_xor(s.tx, m);
    o.my = __shfl_xor(s.my, m); o.sy = __shfl_xor(s.sy, m);
    o.av = __shfl_xor(s.av, m); o.ai = __shfl_xor(s.ai, m);
    return o;
}

// Fold a batch of n values (x[i], y[i]) at indices idx0 + stride*i into s.
template <int N>
__device__ __forceinline__ void rs_fold(RowState &s, const float (&x)[N], const float (&y)[N],
                                        const int (&idx)[N])
{
    float bx = x[0], by = y[0];
    for (int i = 1; i < N; ++i) { bx = fmaxf(bx, x[i]); by = fmaxf(by, y[i]); }
    const float mx = fmaxf(s.mx, bx), my = fmaxf(s.my, by);
    const float cx = fast_exp2((s.mx - mx) * kLog2e), cy = fast_exp2((s.my - my) * kLog2e);
    float sx = s.sx * cx, tx = s.tx * cx, sy = s.sy * cy;
    const float mxl = mx * kLog2e, myl = my * kLog2e;
    for (int i = 0; i < N; ++i) {
        float ex = fast_exp2(fmaf(x[i], kLog2e, -mxl));
        sx += ex;
        tx = fmaf(ex, x[i] - y[i], tx);
        sy += fast_exp2(fmaf(y[i], kLog2e, -myl));
        if (x[i] > s.av) { s.av = x[i]; s.ai = idx[i]; }
    }
    s.mx = mx; s.my = my; s.sx = sx; s.tx = tx; s.sy = sy;
}

template <bool VEC4>
__global__ __launch_bounds__(kPostThreads) void posterior_stream_kernel(PostArgs a)
{
    const int row = blockIdx.x / a.n_chunks;
    const int ch = blockIdx.x % a.n_chunks;
    if (a.locked[row]) return;      // a locked row is never read
    const int tid = threadIdx.x;
    const long base = (long)row * a.V;
    const float *x = a.x + base, *y = a.y + base;
    const int e0 = ch * a.chunk;
    const int e1 = min(a.V, e0 + a.chunk);

    RowState s;
    rs_init(s);
    if (VEC4) {
        // e0 and e1 are multiples of 4; 4 float4 per array per thread per step.
        constexpr int U = 4;
        const int step = kPostThreads * 4 * U;
        int e = e0;
        for (; e + step <= e1; e += step) {
            v4f xv[U], yv[U];
            for (int u = 0; u < U; ++u) {
                int off = e + (u * kPostThreads + tid) * 4;
                xv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + off));
                yv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(y + off));
            }
            float xs[4 * U], ys[4 * U];
            int is[4 * U];
            for (int u = 0; u < U; ++u) {
                int off = e + (u * kPostThreads + tid) * 4;
                xs[4 * u + 0] = xv[u].x; xs[4 * u + 1] = xv[u].y; xs[4 * u + 2] = xv[u].z; xs[4 * u + 3] = xv[u].w;
                ys[4 * u + 0] = yv[u].x; ys[4 * u + 1] = yv[u].y; ys[4 * u + 2] = yv[u].z; ys[4 * u + 3] = yv[u].w;
                is[4 * u + 0] = off; is[4 * u + 1] = off + 1; is[4 * u + 2] = off + 2; is[4 * u + 3] = off + 3;
            }
            rs_fold(s, xs, ys, is);
        }
        for (int off = e + tid * 4; off < e1; off += kPostThreads * 4) {
            v4f xv = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + off));
            v4f yv = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(y + off));
            float xs[4] = {xv.x, xv.y, xv.z, xv.w}, ys[4] = {yv.x, yv.y, yv.z, yv.w};
            int is[4] = {off, off + 1, off + 2, off + 3};
            rs_fold(s, xs, ys, is);
        }
    } else {
        for (int off = e0 + tid; off < e1; off += kPostThreads) {
            float xs[1] = {x[off]}, ys[1] = {y[off]};
            int is[1] = {off};
            rs_fold(s, xs, ys, is);
        }
    }

    // Wave, then workgroup reduction (fixed shape: deterministic).
    for (int m = 32; m >= 1; m >>= 1) rs_merge(s, rs_shfl_xor(s, m));
    __shared__ RowState red[kPostThreads / 64];
    const int wid = tid >> 6;
    if ((tid & 63) == 0) red[wid] = s;
    __syncthreads();
    if (tid == 0) {
        RowState t = red[0];
        for (int w = 1; w < kPostThreads / 64; ++w) rs_merge(t, red[w]);
        PostPartial p;
        p.mx = t.mx; p.sx = t.sx; p.tx = t.tx; p.my = t.my; p.sy = t.sy;
        p.av = t.av; p.ai = t.ai; p.pad = 0;
        a.part[(long)row * a.n_chunks + ch] = p;
    }
}

// One workgroup per selection group of rows: merge each row's chunk
// partials, finish KL / conf / tok / lock, then select within the group.
__global__ __launch_bounds__(256) void posterior_finish_kernel(PostArgs a)
{
    __shared__ float key_s[kMaxGroupRows];
    __shared__ float conf_s[kMaxGroupRows];
    __shared__ int tok_s[kMaxGroupRows];
    __shared__ uint8_t elig_s[kMaxGroupRows];
    __shared__ float thr_s;
    __shared__ int any_s;

    const int tid = threadIdx.x;
    const int g0 = blockIdx.x * a.group_rows;
    const int n = min(a.R - g0, a.group_rows);
    const bool by_score = a.mode == 3 || a.mode == 4;

    for (int t = tid; t < n; t += 256) {
        const int r = g0 + t;
        const bool was_locked = a.locked[r] != 0;
        float klv = 0.f, cf = 0.f;
        int tok = -1;
        if (!was_locked) {
            const PostPartial *pp = a.part + (long)r * a.n_chunks;
            RowState s;
            s.mx = pp[0].mx; s.sx = pp[0].sx; s.tx = pp[0].tx; s.my = pp[0].my; s.sy = pp[0].sy;
            s.av = pp[0].av; s.ai = pp[0].ai;
            for (int c = 1; c < a.n_chunks; ++c) {
                RowState o;
                o.mx = pp[c].mx; o.sx = pp[c].sx; o.tx = pp[c].tx; o.my = pp[c].my; o.sy = pp[c].sy;
                o.av = pp[c].av; o.ai = pp[c].ai;
                rs_merge(s, o);
            }
            // KL = t/sx - (mx + ln sx) + (my + ln sy)
            klv = s.tx / s.sx - (s.mx - s.my) - (logf(s.sx) - logf(s.sy));
            cf = 1.f / s.sx;
            tok = s.ai;
            a.locked[r] = klv <= a.eps ? 1 : 0;
        }
        a.kl[r] = klv;
        a.conf[r] = cf;
        conf_s[t] = cf;
        tok_s[t] = tok;
        elig_s[t] = was_locked ? 0 : 1;
        key_s[t] = by_score ? a.score[r] : cf;
    }
    if (a.mode == 0) {
        for (int t = tid; t < n; t += 256) a.sel[g0 + t] = -1;
        return;
    }
    __syncthreads();
    if (tid == 0) {
        // Dynamic threshold: the largest score of an eligible non-candidate.
        float thr = -INFINITY;
        if (a.mode == 3)
            for (int t = 0; t < n; ++t)
                if (elig_s[t] && !(conf_s[t] > a.tau)) thr = fmaxf(thr, key_s[t]);
        int any = 0;
        for (int t = 0; t < n; ++t) {
            if (!elig_s[t]) continue;
            if (a.mode == 2 && conf_s[t] > a.tau) any = 1;
            if (a.mode == 3 && conf_s[t] > a.tau && key_s[t] > thr) any = 1;
        }
        thr_s = thr;
        any_s = any;
    }
    __syncthreads();
    const float thr = thr_s;
    const int any = any_s;
    for (int t = tid; t < n; t += 256) {
        int out = -1;
        if (elig_s[t]) {
            const float kt = key_s[t];
            int rank = 0;
            for (int u = 0; u < n; ++u)
                if (elig_s[u] && (key_s[u] > kt || (key_s[u] == kt && u < t))) ++rank;
            bool pick = false;
            if (a.mode == 1 || a.mode == 4) pick = rank < a.k;
            else if (a.mode == 2) pick = any ? conf_s[t] > a.tau : rank == 0;
            else if (a.mode == 3) pick = any ? (conf_s[t] > a.tau && kt > thr) : rank == 0;
            if (pick) out = tok_s[t];
        }
        a.sel[g0 + t] = out;
    }
}

}  // namespace

hipError_t launch_posterior(const PostArgs &a, hipStream_t stream)
{
    if (a.R == 0) return hipSuccess;
    const long nwg = (long)a.R * a.n_chunks;
    if ((a.V & 3) == 0)
        posterior_stream_kernel<true><<<dim3((unsigned)nwg), dim3(kPostThreads), 0, stream>>>(a);
    else
        posterior_stream_kernel<false><<<dim3((unsigned)nwg), dim3(kPostThreads), 0, stream>>>(a);
    const int groups = (a.R + a.group_rows - 1) / a.group_rows;
    posterior_finish_kernel<<<dim3((unsigned)groups), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

PostPlan plan_post(int R, int V, int mode, int group_rows)
{
    PostPlan p{};
    // Enough workgroups for ~8 per CU, chunks of at least 16K elements.
    int chunks = 1;
    if (R > 0) {
        const long target = 8L * kNumCU;
        if (R < target) chunks = (int)((target + R - 1) / R);
        const int max_chunks = max(1, V / 16384);
        chunks = min(chunks, max_chunks);
    }
    int chunk = (V + chunks - 1) / chunks;
    chunk = (chunk + 3) / 4 * 4;
    p.chunk = max(4, chunk);
    p.n_chunks = max(1, (V + p.chunk - 1) / p.chunk);
    p.group_rows = mode == 0 ? 256 : group_rows;
    p.ws_total = (size_t)R * p.n_chunks * sizeof(PostPartial);
    return p;
}

}  // namespace dlm
