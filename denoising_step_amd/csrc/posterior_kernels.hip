// posterior_kernels.hip -- posterior, lock test and unmask selection on gfx950.
//
// What is computed, per row r not locked on entry (SureLock page, sec. 2
// core mechanism; Attn-Sampler page, sec. 1 and 2B):
//   p = softmax(x), q = softmax(y) for step-t logits x and step-(t-1) y
//   KL(p || q) = E_p[x - y] - (logsumexp x - logsumexp y)    (one pass)
//   conf = max p = 1 / sum exp(x - max x),  tok = lowest argmax x
//   lock if KL <= eps (rows the caller marks lockable: all by default);
//   then a per-group selection among rows it marks selectable (top-k /
//   threshold / Attn-Sampler dynamic threshold / top-k by score).
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
#include <stdlib.h>

namespace dlm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct RowState {
    float mx, sx, tx, my, sy, av, a2, ex;
    int ai;
};

__device__ __forceinline__ void rs_init(RowState &s)
{
    s.mx = -INFINITY; s.sx = 0.f; s.tx = 0.f;
    s.my = -INFINITY; s.sy = 0.f;
    s.av = -INFINITY; s.a2 = -INFINITY; s.ex = 0.f; s.ai = INT_MAX;
}

// Merge state b into a.  Both describe disjoint element sets.  SC: also
// the runner-up and the entropy sum (margin / entropy requested).
template <bool SC = true>
__device__ __forceinline__ void rs_merge(RowState &a, const RowState &b)
{
    float m = fmaxf(a.mx, b.mx);
    if (m != -INFINITY) {
        float ca = fast_exp2((a.mx - m) * kLog2e), cb = fast_exp2((b.mx - m) * kLog2e);
        // ex is relative to each side's own max: shift it to m (a side with
        // no element has sx = ex = 0)
        if constexpr (SC) {
            const float da = a.mx == -INFINITY ? 0.f : a.mx - m, db = b.mx == -INFINITY ? 0.f : b.mx - m;
            a.ex = (a.ex + a.sx * da) * ca + (b.ex + b.sx * db) * cb;
        }
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
    // runner-up of the union: the smaller of the two tops or either runner-up
    if constexpr (SC) a.a2 = fmaxf(fminf(a.av, b.av), fmaxf(a.a2, b.a2));
    if (b.av > a.av || (b.av == a.av && b.ai < a.ai)) {
        a.av = b.av;
        a.ai = b.ai;
    }
}

template <bool SC = true>
__device__ __forceinline__ RowState rs_shfl_xor(const RowState &s, int m)
{
    RowState o = s;
    o.mx = __shfl_xor(s.mx, m); o.sx = __shfl_xor(s.sx, m); o.tx = __shfl_xor(s.tx, m);
    o.my = __shfl_xor(s.my, m); o.sy = __shfl_xor(s.sy, m);
    o.av = __shfl_xor(s.av, m); o.ai = __shfl_xor(s.ai, m);
    if constexpr (SC) {
        o.a2 = __shfl_xor(s.a2, m);
        o.ex = __shfl_xor(s.ex, m);
    }
    return o;
}

// Fold a batch of n values (x[i], y[i]) at indices idx0 + stride*i into s.
template <bool SC, int N>
__device__ __forceinline__ void rs_fold(RowState &s, const float (&x)[N], const float (&y)[N],
                                        const int (&idx)[N])
{
    float bx = x[0], by = y[0];
    for (int i = 1; i < N; ++i) { bx = fmaxf(bx, x[i]); by = fmaxf(by, y[i]); }
    const float mx = fmaxf(s.mx, bx), my = fmaxf(s.my, by);
    const float cx = fast_exp2((s.mx - mx) * kLog2e), cy = fast_exp2((s.my - my) * kLog2e);
    const float dx = s.mx == -INFINITY ? 0.f : s.mx - mx;      // shift of ex to the new max
    float sx = s.sx * cx, tx = s.tx * cx, sy = s.sy * cy, eh = (s.ex + s.sx * dx) * cx;
    const float mxl = mx * kLog2e, myl = my * kLog2e;
    for (int i = 0; i < N; ++i) {
        float ex = fast_exp2(fmaf(x[i], kLog2e, -mxl));
        sx += ex;
        tx = fmaf(ex, x[i] - y[i], tx);
        sy += fast_exp2(fmaf(y[i], kLog2e, -myl));
        if constexpr (SC) {
            eh = fmaf(ex, x[i] - mx, eh);
            if (x[i] > s.av) { s.a2 = s.av; s.av = x[i]; s.ai = idx[i]; }
            else s.a2 = fmaxf(s.a2, x[i]);
        }
    }
    if constexpr (!SC) {
        // A new maximum can only come from a batch whose maximum beats the
        // running one; its index is the batch's lowest at that value (the
        // indices increase with i), as the element-by-element update gives.
        if (bx > s.av) {
            int ai = idx[N - 1];
            for (int i = N - 1; i >= 0; --i)
                if (x[i] == bx) ai = idx[i];
            s.av = bx;
            s.ai = ai;
        }
    }
    s.mx = mx; s.my = my; s.sx = sx; s.tx = tx; s.sy = sy;
    if constexpr (SC) s.ex = eh;
}

// As rs_fold, over the elements with ok[i] set (at least one may be unset;
// all may be).  A state that stays empty keeps mx = -inf without NaNs.
template <bool SC, int N>
__device__ __forceinline__ void rs_fold_masked(RowState &s, const float (&x)[N], const float (&y)[N],
                                               const int (&idx)[N], const bool (&ok)[N])
{
    float bx = -INFINITY, by = -INFINITY;
    for (int i = 0; i < N; ++i)
        if (ok[i]) { bx = fmaxf(bx, x[i]); by = fmaxf(by, y[i]); }
    const float mx = fmaxf(s.mx, bx), my = fmaxf(s.my, by);
    const float cx = s.mx == mx ? 1.f : fast_exp2((s.mx - mx) * kLog2e);
    const float cy = s.my == my ? 1.f : fast_exp2((s.my - my) * kLog2e);
    const float dx = (s.mx == -INFINITY || s.mx == mx) ? 0.f : s.mx - mx;
    float sx = s.sx * cx, tx = s.tx * cx, sy = s.sy * cy, eh = (s.ex + s.sx * dx) * cx;
    const float mxl = mx * kLog2e, myl = my * kLog2e;
    for (int i = 0; i < N; ++i) {
        if (!ok[i]) continue;
        float ex = fast_exp2(fmaf(x[i], kLog2e, -mxl));
        sx += ex;
        tx = fmaf(ex, x[i] - y[i], tx);
        sy += fast_exp2(fmaf(y[i], kLog2e, -myl));
        if constexpr (SC) {
            eh = fmaf(ex, x[i] - mx, eh);
            if (x[i] > s.av) { s.a2 = s.av; s.av = x[i]; s.ai = idx[i]; }
            else s.a2 = fmaxf(s.a2, x[i]);
        }
    }
    if constexpr (!SC) {
        if (bx > s.av) {           // as in rs_fold, over the valid elements
            int ai = INT_MAX;
            for (int i = N - 1; i >= 0; --i)
                if (ok[i] && x[i] == bx) ai = idx[i];
            s.av = bx;
            s.ai = ai;
        }
    }
    s.mx = mx; s.my = my; s.sx = sx; s.tx = tx; s.sy = sy;
    if constexpr (SC) s.ex = eh;
}

constexpr int kStageBytes = 48 * 1024;   // 1024 partials of 48 bytes

#ifndef DLM_POST_WGS_PER_CU
#define DLM_POST_WGS_PER_CU 16
#endif
// Least chunks per row for a selection group of more than 256 rows.
#ifndef DLM_POST_BIG_CHUNKS
#define DLM_POST_BIG_CHUNKS 4
#endif

// The split of each row's vocabulary into chunks: about sixteen streaming
// workgroups per CU over the `live` rows to stream (measured: shorter
// chunks balance the end of the stream better than four long ones per CU),
// chunks of whole streaming steps (4096 elements), capped for the
// finishing kernel by the size of the selection groups of the R rows: a
// group of up to 256 rows stages its partials in LDS in one round
// (measured best: its rows are all live); a larger group (a whole block of
// a multi-step run, most of whose rows are locked late) merges from global
// memory and keeps at least four chunks per live row.  cap > 0 bounds the
// chunk count (the partials a live-row call was sized for).  The host plan
// and, with a live-row list, both kernels evaluate this same function.
__host__ __device__ inline void post_split(long live, int R, int V, int mode, int group_rows, int cap,
                                           int &n_chunks, int &chunk)
{
    int chunks = 1;
    if (R > 0) {
        const long target = (long)DLM_POST_WGS_PER_CU * kNumCU;
        const long lv = live < 1 ? 1 : live;
        if (lv < target) chunks = (int)((target + lv - 1) / lv);
        const int max_chunks = max(1, (V + kPostThreads * kPostVec - 1) / (kPostThreads * kPostVec));
        chunks = min(chunks, max_chunks);
        const int g = min(R, mode == 0 ? 256 : group_rows);
        if (g <= 256) chunks = min(chunks, max(1, (kStageBytes / (int)sizeof(PostPartial)) / max(1, g)));
        else chunks = min(max_chunks, max(chunks, DLM_POST_BIG_CHUNKS));
        if (cap > 0) chunks = min(chunks, cap);
    }
    int ch = (V + chunks - 1) / chunks;
    // A split row gets chunks of whole streaming steps (4 float4 per array
    // per thread), so a chunk is one round of loads per step.
    constexpr int kStep = kPostThreads * kPostVec;
    ch = chunks > 1 ? (ch + kStep - 1) / kStep * kStep : (ch + 3) / 4 * 4;
    chunk = max(4, ch);
    n_chunks = max(1, (V + chunk - 1) / chunk);
}

// Workgroups per CU of the stream kernel's grid with a live-row list.
constexpr int kPostLiveGridPerCU = 16;
// Workgroups the single launch aims its vocabulary split at: two per CU.
constexpr long kPostFusedTarget = 2L * kNumCU;
// Resident workgroups per CU of the single-launch kernel: seven for the
// plain variant, five for the one that also tracks margin and entropy (its
// register use); with at most five per CU the grid is one round for both.
constexpr int kPostFusedWgsPerCU = 5;

// With a live-row list, the split this call uses (from the device count).
__device__ __forceinline__ void live_split(PostArgs &a)
{
    if (!a.live_rows) return;
    const int n = min(max(*a.n_live, 0), a.R);
    post_split(n, a.R, a.V, a.mode, a.group_rows, a.nc_cap, a.n_chunks, a.chunk);
}

// Where partial (row, chunk) lives.  The partials of selection group
// [g0, g0 + n) fill the block [g0 nc, (g0 + n) nc) of the array.  A group
// whose partials fit one LDS staging round keeps its block row-major; a
// larger one, merged straight from global memory one row per thread, keeps
// it chunk-major, so that consecutive rows of one chunk are contiguous.
// Both kernels use this one function.
__device__ __forceinline__ long part_index(const PostArgs &a, int row, int ch)
{
    const int gr = a.group_rows;        // as the finishing kernel groups rows
    const int g0 = row / gr * gr;
    const int n = min(a.R - g0, gr);
    const int nc = a.n_chunks;
    const int per_round = max(1, min(n, (kStageBytes / (int)sizeof(PostPartial)) / nc));
    return per_round < n ? (long)g0 * nc + (long)ch * n + (row - g0) : (long)row * nc + ch;
}

// Stream chunk ch of row r (elements [ch*chunk, min(V, (ch+1)*chunk))) with
// the whole workgroup and reduce it: thread 0 returns the chunk's state
// (other threads: unspecified).  Fixed reduction shape: deterministic.
template <bool VEC4, bool SC>
__device__ __forceinline__ RowState stream_chunk(const PostArgs &a, int row, int ch, RowState *red)
{
    const int tid = threadIdx.x;
    const long base = (long)row * a.V;
    const float *x = a.x + base, *y = a.y + base;
    const int e0 = ch * a.chunk;
    const int e1 = min(a.V, e0 + a.chunk);

    RowState s;
    rs_init(s);
    if (VEC4) {
        // e0 and e1 are multiples of 4; 4 float4 per array per thread per
        // step.  A partial last step issues all of its loads together too
        // (chunks are whole steps except at the end of a row).
        constexpr int U = 4;
        const int step = kPostThreads * 4 * U;
        for (int e = e0; e < e1; e += step) {
            v4f xv[U], yv[U];
            const bool full = e + step <= e1;
            for (int u = 0; u < U; ++u) {
                const int off = e + (u * kPostThreads + tid) * 4;
                if (full || off < e1) {
                    xv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + off));
                    yv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(y + off));
                } else {
                    xv[u] = v4f{0.f, 0.f, 0.f, 0.f};
                    yv[u] = v4f{0.f, 0.f, 0.f, 0.f};
                }
            }
            float xs[4 * U], ys[4 * U];
            int is[4 * U];
            for (int u = 0; u < U; ++u) {
                const int off = e + (u * kPostThreads + tid) * 4;
                xs[4 * u + 0] = xv[u].x; xs[4 * u + 1] = xv[u].y; xs[4 * u + 2] = xv[u].z; xs[4 * u + 3] = xv[u].w;
                ys[4 * u + 0] = yv[u].x; ys[4 * u + 1] = yv[u].y; ys[4 * u + 2] = yv[u].z; ys[4 * u + 3] = yv[u].w;
                is[4 * u + 0] = off; is[4 * u + 1] = off + 1; is[4 * u + 2] = off + 2; is[4 * u + 3] = off + 3;
            }
            if (full) {
                rs_fold<SC>(s, xs, ys, is);
            } else {
                bool ok[4 * U];
                for (int u = 0; u < U; ++u) {
                    const bool in = e + (u * kPostThreads + tid) * 4 < e1;   // e1 is a multiple of 4
                    ok[4 * u + 0] = in; ok[4 * u + 1] = in; ok[4 * u + 2] = in; ok[4 * u + 3] = in;
                }
                rs_fold_masked<SC>(s, xs, ys, is, ok);
            }
        }
    } else {
        for (int off = e0 + tid; off < e1; off += kPostThreads) {
            float xs[1] = {x[off]}, ys[1] = {y[off]};
            int is[1] = {off};
            rs_fold<SC>(s, xs, ys, is);
        }
    }

    // Wave, then workgroup reduction (fixed shape: deterministic).
    for (int m = 32; m >= 1; m >>= 1) rs_merge<SC>(s, rs_shfl_xor<SC>(s, m));
    const int wid = tid >> 6;
    if ((tid & 63) == 0) red[wid] = s;
    __syncthreads();
    RowState t = red[0];
    if (tid == 0)
        for (int w = 1; w < kPostThreads / 64; ++w) rs_merge<SC>(t, red[w]);
    return t;
}

__device__ __forceinline__ PostPartial to_partial(const RowState &t)
{
    PostPartial p;
    p.mx = t.mx; p.sx = t.sx; p.tx = t.tx; p.my = t.my; p.sy = t.sy;
    p.av = t.av; p.a2 = t.a2; p.ex = t.ex; p.ai = t.ai;
    p.pad[0] = p.pad[1] = p.pad[2] = 0;
    return p;
}

__device__ __forceinline__ RowState rs_load(const PostPartial &p)
{
    RowState s;
    s.mx = p.mx; s.sx = p.sx; s.tx = p.tx; s.my = p.my; s.sy = p.sy; s.av = p.av; s.ai = p.ai;
    s.a2 = p.a2; s.ex = p.ex;
    return s;
}

// One workgroup per (row, chunk); with a live-row list (LIVE), a fixed
// grid walks the (listed row, chunk) items of the device-chosen split, so
// the workgroups follow the live rows while the launch shape stays fixed.
template <bool VEC4, bool SC, bool LIVE>
__global__ __launch_bounds__(kPostThreads) void posterior_stream_kernel(PostArgs a0)
{
    __shared__ RowState red[kPostThreads / 64];
    PostArgs a = a0;
    int items = 1;
    if constexpr (LIVE) {
        live_split(a);
        items = min(max(*a.n_live, 0), a.R) * a.n_chunks;
    }
    for (int it = 0, item = blockIdx.x; LIVE ? item < items : it == 0; ++it, item += gridDim.x) {
        int row, ch;
        if constexpr (LIVE) {
            row = a.live_rows[item / a.n_chunks] - a.live_offset;
            ch = item % a.n_chunks;
            if (row < 0 || row >= a.R) continue;
        } else {
            row = blockIdx.x / a.n_chunks;
            ch = blockIdx.x % a.n_chunks;
        }
        if (a.locked[row]) continue;    // a locked row is never read
        const RowState t = stream_chunk<VEC4, SC>(a, row, ch, red);
        if (threadIdx.x == 0) a.part[part_index(a, row, ch)] = to_partial(t);
        if constexpr (LIVE) __syncthreads();   // red is rewritten by the next item
    }
}

// One workgroup per selection group of rows: merge each row's chunk
// partials, finish KL / conf / tok / lock, then select within the group.
//
// All global loads of the group (lock flags, scores, chunk partials) are
// issued before anything waits on them: the partials are staged into LDS.
// For a group of at most 128 rows, 2, 4 or 8 threads merge one row (as many
// as one pass allows): thread k takes chunks k, k+lanes, ... in order, and
// a fixed butterfly over the lanes combines them; larger groups merge one
// row per thread.
// The selection uses block-wide reductions, not a serial scan.
constexpr int kMergeLanes = 8;
#ifndef DLM_FINISH_WIDE_THREADS
#define DLM_FINISH_WIDE_THREADS 512
#endif
// Threads of the finishing workgroup of a group of more than 256 rows.
constexpr int kFinishWideThreads = DLM_FINISH_WIDE_THREADS;

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// operations are complete, then s_barrier.  Unlike __syncthreads() it does
// not wait for the wave's global stores (the kernel's outputs, which no
// other wave reads back), so those drain while the kernel goes on.  The
// "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One step of a 64-bit max across lanes: combine (hi, lo) with the lane
// the DPP control C names, in the rows of row mask RM (the other rows
// combine with themselves); all lanes active.
template <int C, int RM>
__device__ __forceinline__ void dpp_max_u64(unsigned &lo, unsigned &hi)
{
    const unsigned olo = __builtin_amdgcn_update_dpp(lo, lo, C, RM, 0xf, false);
    const unsigned ohi = __builtin_amdgcn_update_dpp(hi, hi, C, RM, 0xf, false);
    const bool gt = ohi > hi || (ohi == hi && olo > lo);
    lo = gt ? olo : lo;
    hi = gt ? ohi : hi;
}

// The maximum of a 64-bit value over the wave (every lane active), all in
// DPP: within each 16-lane row (quad swaps, half-row and row mirrors), then
// row 15 broadcast into rows 1 and 3 and lane 31 into rows 2 and 3 (GFX9
// row broadcasts), so lane 63 holds the maximum; one read out.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
    unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
    dpp_max_u64<0xB1, 0xf>(lo, hi);   // quad_perm [1,0,3,2]
    dpp_max_u64<0x4E, 0xf>(lo, hi);   // quad_perm [2,3,0,1]
    dpp_max_u64<0x141, 0xf>(lo, hi);  // row_half_mirror
    dpp_max_u64<0x140, 0xf>(lo, hi);  // row_mirror
    dpp_max_u64<0x142, 0xa>(lo, hi);  // row_bcast:15
    dpp_max_u64<0x143, 0xc>(lo, hi);  // row_bcast:31
    // readlane returns int: widen through unsigned (no sign extension)
    return ((unsigned long long)(unsigned)__builtin_amdgcn_readlane(hi, 63) << 32) |
           (unsigned long long)(unsigned)__builtin_amdgcn_readlane(lo, 63);
}

template <int NW>
__device__ __forceinline__ float block_max(float v, float *red)
{
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    const int wid = threadIdx.x >> 6;
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[wid] = v;
    lds_barrier();
    float r = red[0];
    for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
    return r;
}

// Hand-over between workgroups of one launch without cache-wide fences.
// The data are written with device-coherent stores (agent-scope atomic
// stores: write-through past this XCD's L2) and read with device-coherent
// loads; the writer waits until its stores are acknowledged before it
// counts its arrival (an agent-scope atomic add), and the reader loads only
// after it has seen the count.  This is the release / acquire sequence of
// the memory model without its L2 write-back and invalidation (buffer_wbl2
// / buffer_inv), which only plain stores and loads need and which cost
// about a microsecond per workgroup, serialised within an XCD.
__device__ __forceinline__ void st_dev(void *p, float v)
{
    __hip_atomic_store(static_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(void *p, int v)
{
    __hip_atomic_store(static_cast<unsigned *>(p), (unsigned)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f(const void *p)
{
    return __uint_as_float(__hip_atomic_load(static_cast<const unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ int ld_dev_i(const void *p)
{
    return (int)__hip_atomic_load(static_cast<const unsigned *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This wave's stores acknowledged (the "memory" clobber keeps the compiler
// from moving memory accesses across).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned arrive(unsigned *cnt)
{
    wait_stores();
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_partial(PostPartial *p, const RowState &t)
{
    st_dev(&p->mx, t.mx); st_dev(&p->sx, t.sx); st_dev(&p->tx, t.tx); st_dev(&p->my, t.my);
    st_dev(&p->sy, t.sy); st_dev(&p->av, t.av); st_dev(&p->a2, t.a2); st_dev(&p->ex, t.ex);
    st_dev(&p->ai, t.ai);
}

template <bool SC>
__device__ __forceinline__ RowState fetch_partial(const PostPartial *p)
{
    RowState s;
    s.mx = ld_dev_f(&p->mx); s.sx = ld_dev_f(&p->sx); s.tx = ld_dev_f(&p->tx); s.my = ld_dev_f(&p->my);
    s.sy = ld_dev_f(&p->sy); s.av = ld_dev_f(&p->av); s.ai = ld_dev_i(&p->ai);
    if constexpr (SC) {
        s.a2 = ld_dev_f(&p->a2);
        s.ex = ld_dev_f(&p->ex);
    } else {
        s.a2 = -INFINITY;
        s.ex = 0.f;
    }
    return s;
}

// The single launch: stream + row merge + selection.  Workgroup (row,
// chunk) streams its chunk as above and publishes the partial; the
// workgroup that arrives last at the row (an atomic count, no waiting)
// merges the row's partials in chunk order, finishes KL / conf / tok and
// the lock test, and hands the row's results on; the one that arrives last
// at the selection group (at most 256 rows) reads them back, writes the
// lock flags and runs the selection.  A row that arrives locked is handled
// by its chunk-0 workgroup alone.  Every counter is reset by its last
// arrival, so the workspace's counters are zero between calls.  Nothing
// writes a lock flag of a group before every row of the group has read its
// own: the eligibility of the selection sees the entry flags.
template <bool VEC4, bool SC>
__global__ __launch_bounds__(kPostThreads, SC ? 5 : 7) void posterior_fused_kernel(PostArgs a)
{
    __shared__ RowState red[kPostThreads / 64];
    __shared__ int row_last_s, grp_last_s, any_s;
    __shared__ float red_s[kPostThreads / 64];
    __shared__ __attribute__((aligned(16))) unsigned long long ord_s[kPostThreads];

    const int tid = threadIdx.x;
    const int nc = a.n_chunks;
    const int row = blockIdx.x / nc, ch = blockIdx.x - (blockIdx.x / nc) * nc;
    const bool was_locked = a.locked[row] != 0;
    if (was_locked && ch != 0) return;
    RowState s;
    rs_init(s);
    if (!was_locked) {
        s = stream_chunk<VEC4, SC>(a, row, ch, red);
        if (nc > 1) {
            if (tid == 0) {
                publish_partial(&a.part[(long)row * nc + ch], s);
                row_last_s = arrive(&a.row_cnt[row]) == (unsigned)(nc - 1);
            }
            __syncthreads();
            if (!row_last_s) return;
            if (tid < 64) {
                // lane l merges chunks l, l + 64, ... in order, then a fixed
                // butterfly over the wave
                RowState m;
                rs_init(m);
                for (int c = tid; c < nc; c += 64) rs_merge<SC>(m, fetch_partial<SC>(&a.part[(long)row * nc + c]));
                for (int k = 32; k >= 1; k >>= 1) rs_merge<SC>(m, rs_shfl_xor<SC>(m, k));
                s = m;
            }
            if (tid == 0) __hip_atomic_store(&a.row_cnt[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0) {
        float klv = 0.f, cf = 0.f, mg = 0.f, en = 0.f;
        int tok = -1, lock = 0;
        if (!was_locked) {
            // KL = t/sx - (mx + ln sx) + (my + ln sy)
            klv = s.tx / s.sx - (s.mx - s.my) - (logf(s.sx) - logf(s.sy));
            cf = 1.f / s.sx;
            tok = s.ai;
            const int fl = a.flags ? a.flags[row] : 3;
            lock = (klv <= a.eps && (fl & 2) && cf >= a.conf_gate) ? 1 : 0;
            // margin = conf * (1 - exp(a2 - mx)); entropy = ln sx - ex / sx
            mg = cf * (1.f - fast_exp2((s.a2 - s.mx) * kLog2e));
            en = logf(s.sx) - s.ex / s.sx;
        }
        a.kl[row] = klv;
        a.conf[row] = cf;
        if (a.margin) a.margin[row] = mg;
        if (a.entropy) a.entropy[row] = en;
        if (a.mode == 0) {
            if (!was_locked) a.locked[row] = lock;
            a.sel[row] = -1;
        } else {
            if (!was_locked) {
                PostRowRes *rr = &a.rowres[row];
                st_dev(&rr->key, a.mode == 5 ? mg : a.mode == 6 ? -en : cf);
                st_dev(&rr->conf, cf);
                st_dev(&rr->tok, tok);
                st_dev(&rr->lock, lock);
            }
            const int gi = row / a.group_rows;
            const int n = min(a.R - gi * a.group_rows, a.group_rows);
            grp_last_s = arrive(&a.grp_cnt[gi]) == (unsigned)(n - 1);
        }
    }
    if (a.mode == 0) return;
    __syncthreads();
    if (!grp_last_s) return;

    // Selection over the group's n <= 256 rows, thread t for row g0 + t.
    const int gi = row / a.group_rows;
    const int g0 = gi * a.group_rows;
    const int n = min(a.R - g0, a.group_rows);
    const bool by_score = a.mode == 3 || a.mode == 4;
    const int t = tid;
    bool elig = false;
    float key = -INFINITY, cf = 0.f;
    int tok = -1;
    if (t < n) {
        const int r = g0 + t;
        const bool lk = a.locked[r] != 0;                 // entry flag (see above)
        const int fl = a.flags ? a.flags[r] : 3;
        if (!lk) {
            const PostRowRes *rr = &a.rowres[r];
            cf = ld_dev_f(&rr->conf);
            tok = ld_dev_i(&rr->tok);
            key = by_score ? a.score[r] : ld_dev_f(&rr->key);
            a.locked[r] = (uint8_t)ld_dev_i(&rr->lock);
        }
        elig = !lk && (fl & 1);
    }
    if (tid == 0) __hip_atomic_store(&a.grp_cnt[gi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Dynamic threshold: the largest score of an eligible non-candidate.
    float thr = -INFINITY;
    if (a.mode == 3) thr = block_max<kPostThreads / 64>(elig && !(cf > a.tau) ? key : -INFINITY, red_s);
    const bool mine = elig && ((a.mode == 2 && cf > a.tau) || (a.mode == 3 && cf > a.tau && key > thr));
    if (tid == 0) any_s = 0;
    lds_barrier();
    if (mine) any_s = 1;                    // benign race: every writer stores 1
    // (key desc, row asc) as one unsigned 64-bit order, as in the
    // finishing kernel; ineligible rows take key -inf and sort last.
    const unsigned bits = __float_as_uint(elig ? key : -INFINITY);
    const unsigned ord = bits ^ ((unsigned)((int)bits >> 31) | 0x80000000u);
    const unsigned long long me = ((unsigned long long)ord << 32) | (0xffffffffu - (unsigned)t);
    ord_s[t] = t < n ? me : 0ull;
    lds_barrier();
    const int any = any_s;
    if (t >= n) return;
    int out = -1;
    if (elig) {
        typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
        int rank = 0;
#pragma unroll 16
        for (int u = 0; u < n; u += 2) {
            const u64x2 p = *reinterpret_cast<const u64x2 *>(&ord_s[u]);
            rank += (p.x > me ? 1 : 0) + (p.y > me ? 1 : 0);
        }
        const bool first = rank == 0;
        bool pick = false;
        if (a.mode == 1 || a.mode == 4 || a.mode == 5 || a.mode == 6) pick = rank < a.k;
        else if (a.mode == 2) pick = any ? cf > a.tau : first;
        else if (a.mode == 3) pick = any ? (cf > a.tau && key > thr) : first;
        if (pick) out = tok;
    }
    a.sel[g0 + t] = out;
}

template <int NT>
__global__ __launch_bounds__(NT) void posterior_finish_kernel(PostArgs a0)
{
    constexpr int NW = NT / 64;                 // waves
    constexpr int KR = kMaxGroupRows / NT;      // rows per thread of the largest group
    PostArgs a = a0;
    live_split(a);   // with a live-row list, the split the stream kernel used
    __shared__ __attribute__((aligned(16))) float key_s[kMaxGroupRows];
    __shared__ float conf_s[kMaxGroupRows];
    __shared__ int tok_s[kMaxGroupRows];
    __shared__ uint8_t elig_s[kMaxGroupRows];   // may be selected: unlocked and selectable
    __shared__ uint8_t rowf_s[kMaxGroupRows];   // bit 0 unlocked on entry, bit 2 lockable
    __shared__ __attribute__((aligned(16))) PostPartial stage_s[kStageBytes / sizeof(PostPartial)];
    __shared__ __attribute__((aligned(16))) unsigned long long ord_s[kMaxGroupRows];
    __shared__ int hist_s[256];
    __shared__ int pick_s[2];                   // radix select: digit found, count still to go
    constexpr int kSmallK = 32;                 // up to this k, a tournament instead of radix select
    __shared__ unsigned long long cand_s[NW * kSmallK + 1];
    __shared__ float red_s[NW];
    __shared__ int lrow_s[kMaxGroupRows];       // live-row list: the group's live rows, ascending
    __shared__ int lcnt_s[KR][NW];              // live-row list: live rows per (round, wave)

    const int tid = threadIdx.x;
    const int g0 = blockIdx.x * a.group_rows;
    const int n = min(a.R - g0, a.group_rows);
    const bool by_score = a.mode == 3 || a.mode == 4;
    constexpr int kStageParts = kStageBytes / (int)sizeof(PostPartial);
    const int rows_per_round = max(1, min(n, kStageParts / a.n_chunks));
    // Threads per row in the merge: the largest power of two up to
    // kMergeLanes with which one pass covers the group (1 for more than 128
    // rows, or for unsplit rows).  It depends on the shapes only, so the
    // merge order is fixed.
    int lanes = 1;
    if (a.n_chunks > 1)
        while (lanes < kMergeLanes && n * lanes * 2 <= NT) lanes *= 2;
    const bool wide = lanes > 1;

    // Issue the lock-flag and score loads together with the staging loads
    // of the partials (when they fit one round); nothing waits until the
    // barrier.
    uint8_t lk[KR], fl[KR];
    float sc[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int t = tid + NT * k;
        lk[k] = t < n ? a.locked[g0 + t] : 1;
        fl[k] = (a.flags && t < n) ? a.flags[g0 + t] : 3;
        sc[k] = (by_score && t < n) ? a.score[g0 + t] : 0.f;
    }
    // Finish row gt of the group from its merged state s.
    auto finish_row = [&](int gt, const RowState &s, bool was_locked) {
        const int r = g0 + gt;
        float klv = 0.f, cf = 0.f, mg = 0.f, en = 0.f;
        int tok = -1;
        if (!was_locked) {
            // KL = t/sx - (mx + ln sx) + (my + ln sy)
            klv = s.tx / s.sx - (s.mx - s.my) - (logf(s.sx) - logf(s.sy));
            cf = 1.f / s.sx;
            tok = s.ai;
            a.locked[r] = (klv <= a.eps && (rowf_s[gt] & 4) && cf >= a.conf_gate) ? 1 : 0;
            // margin = p(top-1) - p(top-2) = conf * (1 - exp(a2 - mx)): exactly
            // 0 on a tie, conf without a runner-up; entropy = ln sx - ex / sx
            mg = cf * (1.f - fast_exp2((s.a2 - s.mx) * kLog2e));
            en = logf(s.sx) - s.ex / s.sx;
        }
        a.kl[r] = klv;
        a.conf[r] = cf;
        if (a.margin) a.margin[r] = mg;
        if (a.entropy) a.entropy[r] = en;
        conf_s[gt] = cf;
        tok_s[gt] = tok;
        if (!by_score) key_s[gt] = a.mode == 5 ? mg : a.mode == 6 ? -en : cf;
    };
    auto set_flags = [&]() {
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            const int t = tid + NT * k;
            if (t < n) {
                elig_s[t] = (lk[k] == 0 && (fl[k] & 1)) ? 1 : 0;
                rowf_s[t] = (lk[k] == 0 ? 1 : 0) | ((fl[k] & 2) << 1);
                if (by_score) key_s[t] = sc[k];
            }
        }
    };
    int n_lrow = -1;   // the group's compacted live rows in lrow_s (live-row path only)
    if (rows_per_round < n && a.live_rows) {
        // A group of more than 256 rows under a live-row list: few rows are
        // live late in a run, each split into up to nc_cap chunks.  The live
        // rows of the group are compacted (ascending) into LDS, and `lanes`
        // threads merge each one, lane k taking chunks k, k + lanes, ... in
        // order (up to kDirect loads in flight), then a fixed butterfly over
        // the lanes; rows locked on entry get their outputs afterwards.
        constexpr int kDirect = 16;
        const int nc = a.n_chunks;
        set_flags();
        lds_barrier();
        const int lane = tid & 63, wid = tid >> 6;
        unsigned long long bal[KR];
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            const int t = tid + NT * k;
            bal[k] = __ballot(t < n && (rowf_s[t] & 1));
            if (lane == 0) lcnt_s[k][wid] = __popcll(bal[k]);
        }
        lds_barrier();
        int L = 0;
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            int before = L;
            for (int w = 0; w < NW; ++w) {
                if (w < wid) before += lcnt_s[k][w];
                L += lcnt_s[k][w];
            }
            const int t = tid + NT * k;
            if ((bal[k] >> lane) & 1ull) lrow_s[before + __popcll(bal[k] & ((1ull << lane) - 1))] = t;
        }
        n_lrow = L;
        lds_barrier();
        int lanes = 1;
        while (lanes < 32 && lanes * 2 * L <= NT && lanes * 2 <= nc) lanes *= 2;
        const int per_pass = NT / lanes;
        for (int t0 = 0; t0 < L; t0 += per_pass) {
            const int t = t0 + tid / lanes, sub = tid % lanes;
            RowState s;
            rs_init(s);
            const int gt = t < L ? lrow_s[t] : 0;
            for (int c0 = sub; t < L && c0 < nc; c0 += lanes * kDirect) {
                PostPartial q[kDirect];
#pragma unroll
                for (int u = 0; u < kDirect; ++u) {
                    const int c = c0 + u * lanes;
                    if (c < nc) q[u] = a.part[(long)g0 * nc + (long)c * n + gt];
                }
#pragma unroll
                for (int u = 0; u < kDirect; ++u)
                    if (c0 + u * lanes < nc) rs_merge(s, rs_load(q[u]));
            }
            for (int m = lanes / 2; m >= 1; m >>= 1) rs_merge(s, rs_shfl_xor(s, m));
            if (t < L && sub == 0) finish_row(gt, s, false);
        }
        for (int gt = tid; gt < n; gt += NT) {
            if (rowf_s[gt] & 1) continue;
            RowState s;
            rs_init(s);
            finish_row(gt, s, true);
        }
    } else if (rows_per_round < n) {
        // A group of more than 256 rows with split rows: its partials would
        // take several staging rounds, so each thread merges its rows
        // (gt = tid, tid + 256, ...) straight from global memory, issuing
        // the loads of up to kDirect partials (several rows when a row has
        // fewer chunks) before merging any, each row in chunk order.  The
        // first batch is issued together with the lock-flag loads (one
        // round trip); a row locked on entry is not merged.
        constexpr int kDirect = 16;
        const int nc = a.n_chunks;
        if (nc <= kDirect) {
            const int rpb = kDirect / nc;           // rows per batch
            PostPartial q[kDirect];
            auto load_batch = [&](int gt0) {
#pragma unroll
                for (int u = 0; u < kDirect; ++u) {
                    const int i = u / nc, c = u - i * nc, gt = gt0 + NT * i;
                    if (i < rpb && gt < n) q[u] = a.part[(long)g0 * nc + (long)c * n + gt];
                }
            };
            auto merge_batch = [&](int gt0) {
                RowState s;
                rs_init(s);
#pragma unroll
                for (int u = 0; u < kDirect; ++u) {
                    const int i = u / nc, c = u - i * nc, gt = gt0 + NT * i;
                    if (i < rpb && gt < n) {
                        const bool live = rowf_s[gt] & 1;   // a locked row's slots are never read
                        if (c == 0) rs_init(s);
                        if (live) rs_merge(s, rs_load(q[u]));
                        if (c == nc - 1) finish_row(gt, s, !live);
                    }
                }
            };
            // the first batch's loads go out with the lock-flag loads
            load_batch(tid);
            set_flags();
            lds_barrier();
            merge_batch(tid);
            for (int gt0 = tid + NT * rpb; gt0 < n; gt0 += NT * rpb) {
                load_batch(gt0);
                merge_batch(gt0);
            }
        } else {
            set_flags();
            lds_barrier();
            for (int gt = tid; gt < n; gt += NT) {
                const bool live = rowf_s[gt] & 1;
                RowState s;
                rs_init(s);
                for (int c0 = 0; live && c0 < nc; c0 += kDirect) {
                    PostPartial q[kDirect];
#pragma unroll
                    for (int u = 0; u < kDirect; ++u)
                        if (c0 + u < nc) q[u] = a.part[(long)g0 * nc + (long)(c0 + u) * n + gt];
#pragma unroll
                    for (int u = 0; u < kDirect; ++u)
                        if (c0 + u < nc) rs_merge(s, rs_load(q[u]));
                }
                finish_row(gt, s, !live);
            }
        }
    }
    for (int r0 = 0; rows_per_round >= n && r0 < n; r0 += rows_per_round) {
        const int nr = min(rows_per_round, n - r0);
        // Stage: the partials of rows [g0+r0, g0+r0+nr) are one contiguous
        // row-major block (part_index).
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        const v4u *src = reinterpret_cast<const v4u *>(a.part + (long)(g0 + r0) * a.n_chunks);
        v4u *dst = reinterpret_cast<v4u *>(stage_s);
        const int n16 = nr * a.n_chunks * (int)(sizeof(PostPartial) / 16);
        // up to twelve 16-byte loads in flight per thread (one round: the stage is 3072)
        for (int i0 = 0; i0 < n16; i0 += NT * 12) {
            v4u v[12];
#pragma unroll
            for (int u = 0; u < 12; ++u) {
                const int i = i0 + u * NT + tid;
                v[u] = i < n16 ? src[i] : v4u{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < 12; ++u) {
                const int i = i0 + u * NT + tid;
                if (i < n16) dst[i] = v[u];
            }
        }
        set_flags();
        lds_barrier();
        for (int t0 = 0; t0 < nr; t0 += NT / lanes) {
            const int t = t0 + tid / lanes;
            const int sub = tid % lanes;
            const bool row_ok = t < nr;
            const int gt = r0 + t;
            const bool was_locked = !row_ok || (rowf_s[gt] & 1) == 0;
            RowState s;
            rs_init(s);
            if (!was_locked) {
                const PostPartial *pp = stage_s + t * a.n_chunks;
                for (int c = sub; c < a.n_chunks; c += lanes) rs_merge(s, rs_load(pp[c]));
            }
            if (wide)
                for (int m = lanes / 2; m >= 1; m >>= 1) rs_merge(s, rs_shfl_xor(s, m));
            if (row_ok && sub == 0) finish_row(gt, s, was_locked);
        }
    }
    if (a.mode == 0) {
        for (int t = tid; t < n; t += NT) a.sel[g0 + t] = -1;
        return;
    }
    lds_barrier();   // row results (LDS) visible
    // Only rows unlocked on entry can be eligible.  When the group's live
    // rows were compacted (lrow_s) and are few, the selection runs over them
    // alone (entry i stands for row lrow_s[i]); the others are never picked
    // and order after every eligible row, so no rank changes.
    constexpr int kCountMax = 256;
    const bool lsel = n_lrow >= 0 && n_lrow <= kCountMax;
    const int ns = lsel ? n_lrow : n;
    auto row_of = [&](int i) { return lsel ? lrow_s[i] : i; };
    // Dynamic threshold: the largest score of an eligible non-candidate.
    float thr = -INFINITY;
    if (a.mode == 3) {
        float v = -INFINITY;
        for (int i = tid; i < ns; i += NT) {
            const int t = row_of(i);
            if (elig_s[t] && !(conf_s[t] > a.tau)) v = fmaxf(v, key_s[t]);
        }
        thr = block_max<NW>(v, red_s);
    }
    int mine = 0;
    for (int i = tid; i < ns; i += NT) {
        const int t = row_of(i);
        if (!elig_s[t]) continue;
        if (a.mode == 2 && conf_s[t] > a.tau) mine = 1;
        if (a.mode == 3 && conf_s[t] > a.tau && key_s[t] > thr) mine = 1;
    }
    __shared__ int any_s;
    if (tid == 0) any_s = 0;
    lds_barrier();
    if (mine) any_s = 1;                    // benign race: every writer stores 1
    lds_barrier();
    const int any = any_s;
    // rank(t) = number of eligible rows ordered before t: (key desc, row
    // asc).  Each row's (key, row) is packed into one 64-bit integer whose
    // unsigned order is exactly that order: the key's bits made
    // order-preserving (all bits flipped for a negative key, the sign bit
    // for a positive one) above the complemented row index.  Ineligible
    // rows take key -inf and sort last (eligible keys are finite: a
    // confidence or a column sum).  The packed values are distinct, so
    // rank(t) < k exactly when t's packed value is at least the k-th
    // largest.  A small group counts larger values per row (one 64-bit
    // compare and one add per pair); a larger one finds the k-th largest
    // value by radix selection over its eight bytes, most significant
    // first: a 256-bin histogram in LDS of the values that share the bytes
    // found so far, then one wave scans the bins from the top for the one
    // that holds the k-th value.  Same cost for any k.
    typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
    const bool counted = ns <= kCountMax;
    lds_barrier();
    for (int i = tid; i < ns; i += NT) {
        const int t = row_of(i);
        const unsigned bits = __float_as_uint(elig_s[t] ? key_s[t] : -INFINITY);
        const unsigned ord = bits ^ ((unsigned)((int)bits >> 31) | 0x80000000u);
        ord_s[i] = ((unsigned long long)ord << 32) | (0xffffffffu - (unsigned)t);
    }
    for (int i = ns + tid; i < ((ns + 1) & ~1); i += NT) ord_s[i] = 0;   // even count
    lds_barrier();
    // the kk-th largest packed value (kk in [1, ns]); block-uniform call
    auto kth_largest = [&](int kk) -> unsigned long long {
        unsigned long long prefix = 0;
        int krem = kk;
        for (int pass = 7; pass >= 0; --pass) {
            const int shift = pass * 8;
            if (tid < 256) hist_s[tid] = 0;
            lds_barrier();
            for (int i = tid; i < ns; i += NT) {
                const unsigned long long v = ord_s[i];
                if (pass == 7 || (v >> (shift + 8)) == prefix) atomicAdd(&hist_s[(v >> shift) & 255], 1);
            }
            lds_barrier();
            if (tid < 64) {
                // lane l holds bins 255 - 4l - j, j = 0..3 (descending)
                int c[4], sum = 0;
                for (int j = 0; j < 4; ++j) {
                    c[j] = hist_s[255 - 4 * tid - j];
                    sum += c[j];
                }
                int incl = sum;
                for (int off = 1; off < 64; off <<= 1) {
                    const int o = __shfl_up(incl, off);
                    if (tid >= off) incl += o;
                }
                int cum = incl - sum;
                if (cum < krem && krem <= incl) {
                    for (int j = 0; j < 4; ++j) {
                        if (cum + c[j] >= krem) {
                            pick_s[0] = 255 - 4 * tid - j;
                            pick_s[1] = krem - cum;
                            break;
                        }
                        cum += c[j];
                    }
                }
            }
            lds_barrier();
            prefix = (prefix << 8) | (unsigned)pick_s[0];
            krem = pick_s[1];
            lds_barrier();
        }
        return prefix;
    };
    // The kk-th largest packed value for kk <= kSmallK (block-uniform
    // call): each wave takes the kk largest of its rows (KR per lane) by
    // repeated 64-bit wave maxima (DPP steps), the one lane that holds a
    // maximum dropping it (the values are distinct; padding is 0, below any
    // packed value); the global kk largest are among these NW kk
    // candidates, and the one with exactly kk - 1 candidates above it is
    // the answer.  No atomics, three barriers.
    auto kth_small = [&](int kk) -> unsigned long long {
        const int lane = tid & 63, wid = tid >> 6;
        unsigned long long v[KR];
        for (int j = 0; j < KR; ++j) {
            const int t = wid * 64 + lane + NT * j;
            v[j] = t < ns ? ord_s[t] : 0ull;
        }
        for (int it = 0; it < kk; ++it) {
            unsigned long long mx = v[0];
            for (int j = 1; j < KR; ++j) mx = max(mx, v[j]);
            const unsigned long long m = wave_max_u64(mx);
            for (int j = 0; j < KR; ++j)
                if (v[j] == m) v[j] = 0ull;
            if (lane == 0) cand_s[wid * kk + it] = m;    // the NW kk candidates, packed
        }
        lds_barrier();
        if (tid < NW * kk) {
            const unsigned long long mine = cand_s[tid];
            int above = 0;
#pragma unroll 8
            for (int u = 0; u < NW * kk; ++u) above += cand_s[u] > mine ? 1 : 0;
            if (above == kk - 1) cand_s[NW * kSmallK] = mine;
        }
        lds_barrier();
        return cand_s[NW * kSmallK];
    };
    const bool topk = a.mode == 1 || a.mode == 4 || a.mode == 5 || a.mode == 6;
    unsigned long long kth = 0;                 // picked iff eligible and value >= kth
    if (!counted) {
        if (topk) kth = a.k <= 0 ? ~0ull : a.k >= ns ? 0ull : a.k <= kSmallK ? kth_small(a.k) : kth_largest(a.k);
        else if (!any) kth = kth_small(1);
    }
    if (lsel)
        for (int t = tid; t < n; t += NT)
            if (!(rowf_s[t] & 1)) a.sel[g0 + t] = -1;
    for (int i = tid; i < ns; i += NT) {
        const int t = row_of(i);
        int out = -1;
        if (elig_s[t]) {
            const float kt = key_s[t];
            const unsigned long long mine = ord_s[i];
            bool first = false, in_topk = false;
            if (counted) {
                int rank = 0;
                // sixteen 16-byte LDS reads in flight (one wave per SIMD:
                // nothing else hides their latency)
#pragma unroll 16
                for (int u = 0; u < ns; u += 2) {
                    const u64x2 p = *reinterpret_cast<const u64x2 *>(&ord_s[u]);
                    rank += (p.x > mine ? 1 : 0) + (p.y > mine ? 1 : 0);
                }
                first = rank == 0;
                in_topk = rank < a.k;
            } else {
                first = mine >= kth;            // kth = the largest when a fallback is needed
                in_topk = a.k > 0 && mine >= kth;
            }
            bool pick = false;
            if (topk) pick = in_topk;
            else if (a.mode == 2) pick = any ? conf_s[t] > a.tau : first;
            else if (a.mode == 3) pick = any ? (conf_s[t] > a.tau && kt > thr) : first;
            if (pick) out = tok_s[t];
        }
        a.sel[g0 + t] = out;
    }
}

}  // namespace

hipError_t launch_posterior(const PostArgs &a, hipStream_t stream, hipEvent_t finish_after)
{
    if (a.R == 0) return hipSuccess;
    long nwg = (long)a.R * a.n_chunks;
    // margin / entropy: only when an output or the selection needs them
    const bool sc = a.margin || a.entropy || a.mode == 5 || a.mode == 6;
    const bool live = a.live_rows != nullptr;
    if (live && nwg > (long)kPostLiveGridPerCU * kNumCU) nwg = (long)kPostLiveGridPerCU * kNumCU;
    const dim3 grid((unsigned)nwg), block(kPostThreads);
    if (a.rowres) {
        if ((a.V & 3) == 0) {
            if (sc) posterior_fused_kernel<true, true><<<grid, block, 0, stream>>>(a);
            else posterior_fused_kernel<true, false><<<grid, block, 0, stream>>>(a);
        } else {
            if (sc) posterior_fused_kernel<false, true><<<grid, block, 0, stream>>>(a);
            else posterior_fused_kernel<false, false><<<grid, block, 0, stream>>>(a);
        }
        return hipGetLastError();
    }
#define DLM_POST_STREAM(V4, SC_)                                                              \
    (live ? (posterior_stream_kernel<V4, SC_, true><<<grid, block, 0, stream>>>(a), 0)       \
          : (posterior_stream_kernel<V4, SC_, false><<<grid, block, 0, stream>>>(a), 0))
    if ((a.V & 3) == 0) {
        if (sc) DLM_POST_STREAM(true, true);
        else DLM_POST_STREAM(true, false);
    } else {
        if (sc) DLM_POST_STREAM(false, true);
        else DLM_POST_STREAM(false, false);
    }
#undef DLM_POST_STREAM
    if (finish_after) {
        const hipError_t e = hipStreamWaitEvent(stream, finish_after, 0);
        if (e != hipSuccess) return e;
    }
    const int groups = (a.R + a.group_rows - 1) / a.group_rows;
    // groups of more than 256 rows: a workgroup of kFinishWideThreads
    if (a.group_rows > 256)
        posterior_finish_kernel<kFinishWideThreads><<<dim3((unsigned)groups), dim3(kFinishWideThreads), 0, stream>>>(a);
    else
        posterior_finish_kernel<256><<<dim3((unsigned)groups), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

PostPlan plan_post(int R, int V, int mode, int group_rows, bool live, bool fused)
{
    PostPlan p{};
    p.group_rows = mode == 0 ? 256 : group_rows;
    const long groups = mode == 0 ? 0 : ((long)R + p.group_rows - 1) / p.group_rows;
    // The single launch: no live-row list, selection groups of at most 256
    // rows (one thread per row in its selection) and counters that fit the
    // workspace's fixed counter block; DLM_POST_FUSED=0 keeps the
    // two-launch path (measurement).
    // With a live-row list the partials are sized for the largest split a
    // call can choose (one live row), and the kernels pick the split from
    // the device count.
    post_split(live ? 1 : R, R, V, mode, group_rows, 0, p.n_chunks, p.chunk);
    // Without a selection and with whole rows per workgroup there is no
    // hand-over at all (each workgroup finishes its own row), so any grid
    // size goes (the SureLock posterior, 8192 rows: equal or 5 us faster).
    // Otherwise the single launch splits the rows into its own, fewer
    // chunks, about kPostFusedTarget workgroups in all (each hand-over, an
    // acknowledged store and an atomic round trip, costs 2-3 us, and a
    // workgroup streaming several steps keeps its loads going), and is
    // taken only when that grid is one round of resident workgroups, where
    // the hand-overs overlap other workgroups' streaming.  Measured on
    // MI355X: 32 x 126464 rows 22.1 us with the two-launch split (992
    // workgroups), 17.8-18.2 us with 8-16 chunks a row; 256 x 151936 rows
    // 61.0 us with 4 chunks, 59.8 with 2, 66.6 with 1.
    const bool base_ok = fused && !live && p.group_rows <= kPostThreads && R > 0 && groups <= kPostMaxCounters;
    bool fz = false;
    if (base_ok && mode == 0 && p.n_chunks == 1) {
        fz = true;
    } else if (base_ok) {
        constexpr int kStep = kPostThreads * kPostVec;
        const int steps = max(1, (V + kStep - 1) / kStep);
        const int c = (int)min((long)steps, max(1L, (kPostFusedTarget + R - 1) / R));
        const int ch = c > 1 ? ((V + c - 1) / c + kStep - 1) / kStep * kStep : (V + 3) / 4 * 4;
        const int nc = max(1, (V + max(4, ch) - 1) / max(4, ch));
        if ((long)R * nc <= (long)kPostFusedWgsPerCU * kNumCU && (nc == 1 || R <= kPostMaxCounters)) {
            fz = true;
            p.chunk = max(4, ch);
            p.n_chunks = nc;
        }
    }
    if (const char *e = getenv("DLM_POST_FUSED"))
        if (e[0] == '0' && e[1] == 0) fz = false;
    if (!fz) post_split(live ? 1 : R, R, V, mode, group_rows, 0, p.n_chunks, p.chunk);
    p.fused = fz ? 1 : 0;
    if (R == 0) return p;
    // Every layout starts with the counter block (row counters, then group
    // counters), so calls of any shape and either path can share a
    // workspace: only counters are ever written there, and every call
    // leaves them zero.
    size_t off = kPostCounterBytes;
    p.off_row_cnt = 0;
    p.off_grp_cnt = (size_t)kPostMaxCounters * sizeof(unsigned);
    if (fz) {
        p.off_rowres = off;
        off += ((size_t)R * sizeof(PostRowRes) + 255) / 256 * 256;
    }
    p.off_part = off;
    p.ws_total = off + (size_t)R * p.n_chunks * sizeof(PostPartial);
    return p;
}

size_t post_ws_bytes(int R, int V, int mode, int group_rows, bool live)
{
    const size_t a = plan_post(R, V, mode, group_rows, live, false).ws_total;
    const size_t b = plan_post(R, V, mode, group_rows, live, true).ws_total;
    return a > b ? a : b;
}

}  // namespace dlm
