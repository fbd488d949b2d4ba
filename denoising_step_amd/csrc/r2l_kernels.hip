// r2l_kernels.hip -- the R2LM right-to-left selective scan on gfx950.
//
// "Bifocal Diffusion Language Models" page, sec. 2: the right-to-left
// stream flips the generation block's hidden states, applies a selective
// scan (Mamba) and flips back; the result, scaled by the learnable gate s,
// is a residual correction.  Scanning the flipped sequence forward is the
// same as scanning the original from its last token down to its first, so
// the kernel walks t = L-1 .. 0 directly:
//     h[e, n] = exp(delta_t[e] A[e, n]) h[e, n] + delta_t[e] B_t[n] u_t[e]
//     y_t[e]  = s (sum_n C_t[n] h[e, n] + D[e] u_t[e])
// from a zero state at the block's right end.
//
// N is 8, 16 or 32 (a token's B row is then a whole number of 16-byte
// loads).  A thread keeps S = 4 states of one channel in registers (S = 2
// doubles the waves but measured slower: the per-token work is shared by
// fewer states); the NL = N/S threads of a channel are consecutive lanes
// and add their partial outputs with DPP (quad permutes, a row half-mirror,
// a row mirror), no LDS traffic.  A workgroup of 256 threads covers
// CW = 256/NL channels of one batch entry.
//
// The recurrence never waits on global memory: the tokens are taken in
// chunks of LC = 4096/CW (u, delta and x of a chunk are 8 KB each, B and C
// of its tokens follow), loaded straight into LDS, double-buffered so the
// next chunk is in flight while this one is scanned out of LDS.  B and C,
// shared by every channel, are widened to fp32 in LDS once per chunk.
// Each chunk's y goes to LDS and is then written out, with x += y,
// coalesced.
#include "dlm_internal.h"

namespace dlm {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kR2LThreads = 256;
constexpr int kR2LOOB = 0x7ffffff0;

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float((unsigned)v << 16); }

__device__ __forceinline__ uint16_t to_bf(float f)
{
    const __bf16 h = (__bf16)f;
    return *reinterpret_cast<const uint16_t *>(&h);
}

// lane value from the lane given by a DPP control (full rows and banks)
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the NL consecutive lanes of a channel (NL a power of two <= 16).
template <int NL>
__device__ __forceinline__ float channel_sum(float v)
{
    if (NL >= 2) v += dpp<0xB1>(v);      // quad_perm [1,0,3,2]: lane ^ 1
    if (NL >= 4) v += dpp<0x4E>(v);      // quad_perm [2,3,0,1]: lane ^ 2
    if (NL >= 8) v += dpp<0x141>(v);     // row_half_mirror: pairs the two quads of 8 lanes
    if (NL >= 16) v += dpp<0x140>(v);    // row_mirror: pairs the two halves of 16 lanes
    return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t view(const void *p, long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

#ifndef DLM_R2L_S
#define DLM_R2L_S 4
#endif
constexpr int kR2LS = DLM_R2L_S;   // states per thread (2 or 4)

// S consecutive bf16 values (4 or 8 bytes, aligned) widened to fp32
template <int S>
__device__ __forceinline__ void load_bf16s(const uint16_t *p, float (&v)[S])
{
    if constexpr (S == 2) {
        const unsigned q = *reinterpret_cast<const unsigned *>(p);
        v[0] = __uint_as_float(q << 16);
        v[1] = __uint_as_float(q & 0xffff0000u);
    } else {
        const uint2 q = *reinterpret_cast<const uint2 *>(p);
        v[0] = __uint_as_float(q.x << 16);
        v[1] = __uint_as_float(q.x & 0xffff0000u);
        v[2] = __uint_as_float(q.y << 16);
        v[3] = __uint_as_float(q.y & 0xffff0000u);
    }
}

template <int NL>
__global__ __launch_bounds__(kR2LThreads) void r2l_scan_kernel(R2LArgs a)
{
    constexpr int S = kR2LS;
    constexpr int N = S * NL;
    constexpr int CW = kR2LThreads / NL;           // channels per workgroup
    constexpr int LC = 4096 / CW;                  // tokens per chunk (8 KB per bf16 array)
    static_assert(LC % 4 == 0 && (S == 2 || S == 4), "groups of four tokens, two or four states per thread");
    constexpr int ROW = CW * 2;                    // bytes of one token's channels
    constexpr int BC = LC * N * 2;                 // bytes of a chunk's B (or C)
    constexpr int BCE = BC / 2 < 512 ? 512 : BC / 2;   // its LDS array: at least one 1-KB load
    __shared__ __attribute__((aligned(16))) uint16_t us[2][LC * CW];
    __shared__ __attribute__((aligned(16))) uint16_t ds[2][LC * CW];
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][LC * CW];
    __shared__ __attribute__((aligned(16))) uint16_t bs[2][BCE];
    __shared__ __attribute__((aligned(16))) uint16_t cs[2][BCE];
    __shared__ __attribute__((aligned(16))) float bf32[LC * N];   // the chunk's B and C widened once
    __shared__ __attribute__((aligned(16))) float cf32[LC * N];
    __shared__ float ys[LC * CW];

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int g = tid % NL, c = tid / NL;          // states S g .. S g + S-1 of local channel c
    const int cblocks = (a.E + CW - 1) / CW;
    const int b = blockIdx.x / cblocks;
    const int e0 = (blockIdx.x % cblocks) * CW;
    const int e = e0 + c;
    const int ec = e < a.E ? e : a.E - 1;

    const long tok_bytes = (long)a.B * a.L * a.E * 2;
    const __amdgpu_buffer_rsrc_t ur = view(a.u, tok_bytes), dr = view(a.delta, tok_bytes);
    const __amdgpu_buffer_rsrc_t xr = view(a.x ? (const void *)a.x : (const void *)a.u, tok_bytes);
    const __amdgpu_buffer_rsrc_t br = view(a.Bm, (long)a.B * a.L * N * 2), cr = view(a.Cm, (long)a.B * a.L * N * 2);

    // Chunk k holds tokens [hi - LC + 1, hi], hi = L - 1 - k LC; LDS row i of
    // the chunk is token lo + i.  A token before 0 reads as zeros.
    const int nch = (a.L + LC - 1) / LC;
    auto issue = [&](int k, int buf) {
        const int lo = a.L - (k + 1) * LC;
        for (int j = wid; j < 8; j += 4) {          // 8 KB per array: 8 loads of 1 KB
            const int byte = j * 1024 + lane * 16;
            const int t = lo + byte / ROW;
            const int off = t >= 0 ? (int)(((long)(b * a.L + t) * a.E + e0) * 2 + byte % ROW) : kR2LOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ur, (lds_void *)(us[buf] + j * 512), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(dr, (lds_void *)(ds[buf] + j * 512), 16, off, 0, 0, 0);
            if (a.x) __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(xs[buf] + j * 512), 16, off, 0, 0, 0);
        }
        for (int j = wid; j * 1024 < BC; j += 4) {  // B and C rows of the chunk's tokens
            const int byte = j * 1024 + lane * 16;
            const int t = lo + byte / (N * 2);
            const int off = (t >= 0 && byte < BC) ? (int)((long)(b * a.L + t) * N * 2 + byte % (N * 2)) : kR2LOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(bs[buf] + j * 512), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(cr, (lds_void *)(cs[buf] + j * 512), 16, off, 0, 0, 0);
        }
    };

    float A2[S], h[S];
    for (int i = 0; i < S; ++i) {
        A2[i] = a.A[(long)ec * N + S * g + i] * 1.4426950408889634f;
        h[i] = 0.f;
    }
    const float Dv = a.D[ec];

    // The chunk's B and C rows, shared by every channel of the batch entry,
    // are widened to fp32 once per chunk (by the whole workgroup) rather
    // than once per channel; a barrier follows.
    auto widen_bc = [&](auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        for (int i = tid; i < LC * N; i += kR2LThreads) {
            bf32[i] = bf(bs[BUF][i]);
            cf32[i] = bf(cs[BUF][i]);
        }
        __syncthreads();
    };

    // Tokens of a chunk in groups of four, last first: the group's inputs
    // are read from LDS one group ahead (their reads are in flight while the
    // previous group is scanned) and its decays exponentiated up front, so
    // only the state update is serial; the four outputs reduce as
    // independent DPP chains.  Padding rows (tokens before 0) are zeros:
    // decay 1, input 0, the state passes unchanged, and their outputs are
    // never written.
    struct Group {
        float u[4], dl[4], Bv[4][S], Cv[4][S];
    };
    auto read_group = [&](auto bufc, int i0, Group &gr) {
        constexpr int BUF = decltype(bufc)::value;
        for (int j = 0; j < 4; ++j) {
            const int i = i0 + j;
            gr.u[j] = bf(us[BUF][i * CW + c]);
            gr.dl[j] = bf(ds[BUF][i * CW + c]);
            for (int q = 0; q < S; ++q) {
                gr.Bv[j][q] = bf32[i * N + S * g + q];
                gr.Cv[j][q] = cf32[i * N + S * g + q];
            }
        }
    };
    auto scan_group = [&](const Group &gr, int i0) {
        float du[4], dA[4][S], yp[4];
        for (int j = 0; j < 4; ++j) {
            du[j] = gr.dl[j] * gr.u[j];
            for (int q = 0; q < S; ++q) dA[j][q] = __builtin_amdgcn_exp2f(gr.dl[j] * A2[q]);
        }
        for (int j = 3; j >= 0; --j) {
            yp[j] = 0.f;
            for (int q = 0; q < S; ++q) {
                h[q] = fmaf(dA[j][q], h[q], du[j] * gr.Bv[j][q]);
                yp[j] = fmaf(gr.Cv[j][q], h[q], yp[j]);
            }
        }
        for (int j = 0; j < 4; ++j) yp[j] = channel_sum<NL>(yp[j]);
        if (g == 0)
            for (int j = 0; j < 4; ++j) ys[(i0 + j) * CW + c] = a.gate * fmaf(Dv, gr.u[j], yp[j]);
    };
    // two groups' registers alternate, so no copy between them waits for
    // the reads in flight (a copy measured 12 % slower than no prefetch)
    auto scan_chunk = [&](auto bufc) {
        Group ga, gb;
        read_group(bufc, LC - 4, ga);
        for (int i0 = LC - 4; i0 >= 0; i0 -= 8) {
            if (i0 >= 4) read_group(bufc, i0 - 4, gb);
            scan_group(ga, i0);
            if (i0 < 4) break;
            if (i0 >= 8) read_group(bufc, i0 - 8, ga);
            scan_group(gb, i0 - 4);
        }
    };

    // write the chunk's y (and x + y) back, coalesced: thread = (row, channel)
    auto write_chunk = [&](auto bufc, int k) {
        constexpr int BUF = decltype(bufc)::value;
        const int lo = a.L - (k + 1) * LC;
        for (int idx = tid; idx < LC * CW; idx += kR2LThreads) {
            const int i = idx / CW, cc = idx % CW;
            const int t = lo + i, ee = e0 + cc;
            if (t < 0 || ee >= a.E) continue;
            const long o = (long)(b * a.L + t) * a.E + ee;
            const float y = ys[idx];
            if (a.y) a.y[o] = y;
            if (a.x) a.x[o] = to_bf(bf(xs[BUF][idx]) + y);
        }
    };

    issue(0, 0);
    for (int k = 0; k < nch; k += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                            // chunk k in LDS; last chunk's writes done
        if (k + 1 < nch) issue(k + 1, 1);
        widen_bc(std::integral_constant<int, 0>{});
        scan_chunk(std::integral_constant<int, 0>{});
        __syncthreads();
        write_chunk(std::integral_constant<int, 0>{}, k);
        if (k + 1 < nch) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (k + 2 < nch) issue(k + 2, 0);
            widen_bc(std::integral_constant<int, 1>{});
            scan_chunk(std::integral_constant<int, 1>{});
            __syncthreads();
            write_chunk(std::integral_constant<int, 1>{}, k + 1);
        }
    }
}

}  // namespace

hipError_t launch_r2l(const R2LArgs &a, hipStream_t stream)
{
    const int NL = a.N / kR2LS;
    const int CW = kR2LThreads / NL;
    const long grid = (long)a.B * ((a.E + CW - 1) / CW);
    if (grid == 0 || a.L == 0) return hipSuccess;
    switch (a.N) {
    case 8: r2l_scan_kernel<8 / kR2LS><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 16: r2l_scan_kernel<16 / kR2LS><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 32: r2l_scan_kernel<32 / kR2LS><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dlm
