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
// A thread keeps 4 states of one channel in registers; the N/4 threads of a
// channel are consecutive lanes and add their partial outputs with xor
// shuffles.  A workgroup of 256 threads covers 256 / (N/4) channels of one
// batch entry.  The inputs of the next U tokens are loaded before the
// current U are computed, so the loads of the dependent chain are in flight
// while it runs.  exp is the hardware exp2 of delta * A * log2(e).
#include "dlm_internal.h"

namespace dlm {

namespace {

constexpr int kR2LThreads = 256;
constexpr int kR2LU = 4;     // tokens per prefetch group

__device__ __forceinline__ float bf(uint16_t v) { return __uint_as_float((unsigned)v << 16); }

__device__ __forceinline__ uint16_t to_bf(float f)
{
    const __bf16 h = (__bf16)f;
    return *reinterpret_cast<const uint16_t *>(&h);
}

template <int NL>
__global__ __launch_bounds__(kR2LThreads) void r2l_scan_kernel(R2LArgs a)
{
    constexpr int CW = kR2LThreads / NL;           // channels per workgroup
    constexpr int U = kR2LU;
    const int tid = threadIdx.x;
    const int g = tid % NL;                        // states 4g .. 4g+3
    const int cblocks = (a.E + CW - 1) / CW;
    const int b = blockIdx.x / cblocks;
    const int e = (blockIdx.x % cblocks) * CW + tid / NL;
    const bool ok = e < a.E;
    const int ec = ok ? e : a.E - 1;               // a valid channel for the loads

    float A2[4], h[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i) A2[i] = a.A[(long)ec * a.N + 4 * g + i] * 1.4426950408889634f;
    const float Dv = a.D[ec];
    const long ue = (long)b * a.L * a.E + ec;      // u / delta / y / x at token t: ue + t * E
    const long bn = (long)b * a.L * a.N + 4 * g;   // B / C at token t: bn + t * N

    struct Tok {
        float u, dl;
        uint2 Bq, Cq;                              // 4 bf16 each
    };
    auto load = [&](int t, Tok &k) {
        k.u = bf(a.u[ue + (long)t * a.E]);
        k.dl = bf(a.delta[ue + (long)t * a.E]);
        k.Bq = *reinterpret_cast<const uint2 *>(a.Bm + bn + (long)t * a.N);
        k.Cq = *reinterpret_cast<const uint2 *>(a.Cm + bn + (long)t * a.N);
    };
    auto step = [&](int t, const Tok &k) {
        const float du = k.dl * k.u;
        const float Bv[4] = {__uint_as_float(k.Bq.x << 16), __uint_as_float(k.Bq.x & 0xffff0000u),
                             __uint_as_float(k.Bq.y << 16), __uint_as_float(k.Bq.y & 0xffff0000u)};
        const float Cv[4] = {__uint_as_float(k.Cq.x << 16), __uint_as_float(k.Cq.x & 0xffff0000u),
                             __uint_as_float(k.Cq.y << 16), __uint_as_float(k.Cq.y & 0xffff0000u)};
        float yp = 0.f;
        for (int i = 0; i < 4; ++i) {
            const float dA = __builtin_amdgcn_exp2f(k.dl * A2[i]);
            h[i] = fmaf(dA, h[i], du * Bv[i]);
            yp = fmaf(Cv[i], h[i], yp);
        }
        for (int m = 1; m < NL; m <<= 1) yp += __shfl_xor(yp, m);
        if (ok && g == 0) {
            const float y = a.gate * fmaf(Dv, k.u, yp);
            const long o = ue + (long)t * a.E;
            if (a.y) a.y[o] = y;
            if (a.x) a.x[o] = to_bf(bf(a.x[o]) + y);
        }
    };

    // tokens L-1 down to 0 in groups of U, the next group loaded first
    Tok cur[U], nxt[U];
    int t0 = a.L - 1;
    for (int u = 0; u < U; ++u)
        if (t0 - u >= 0) load(t0 - u, cur[u]);
    while (t0 >= 0) {
        const int t1 = t0 - U;
        for (int u = 0; u < U; ++u)
            if (t1 - u >= 0) load(t1 - u, nxt[u]);
        for (int u = 0; u < U; ++u)
            if (t0 - u >= 0) step(t0 - u, cur[u]);
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        t0 = t1;
    }
}

}  // namespace

hipError_t launch_r2l(const R2LArgs &a, hipStream_t stream)
{
    const int NL = a.N / 4;
    const int CW = kR2LThreads / NL;
    const long grid = (long)a.B * ((a.E + CW - 1) / CW);
    if (grid == 0 || a.L == 0) return hipSuccess;
    switch (NL) {
    case 1: r2l_scan_kernel<1><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 2: r2l_scan_kernel<2><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 4: r2l_scan_kernel<4><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 8: r2l_scan_kernel<8><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    case 16: r2l_scan_kernel<16><<<dim3((unsigned)grid), dim3(kR2LThreads), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dlm
