// gemm_kernels.hip -- the active-row projections and FFN of one layer on gfx950.
//
// SureLock page, sec. 2: a locked position skips its query projection and
// its feed-forward sub-layer, so a step's dense work is O(M_t d^2) over the
// M_t active rows only.  Every product here is
//     C[r, n] = sum_k A[r, k] * W[n, k]        (W row-major [N, K], bf16)
// with fp32 accumulation, where the rows r of A are the active rows:
//   A_GATHER  x[b, active_idx[b, j], :]                 (hidden states)
//   A_HEADS   out[b, k / D, j, k % D]                   (attention output)
//   A_PLAIN   a[r, :]                                   (compact rows)
// and the epilogue writes
//   EP_QKV      q / k / v in the attention's [B, H, M, D] layouts
//   EP_RESID    bf16(resid[r, n] + C[r, n]) to compact rows [B*M, N]
//   EP_SCATTER  bf16(resid[r, n] + C[r, n]) to x[b, active_idx[b, j], n]
//   EP_SWIGLU   bf16(silu(C_gate) * C_up), two weight matrices, one A tile.
// Row r = b * M + j is valid when j < m_active[b] (all M rows without it).
//
// Workgroup: 256 threads, a 128 x 128 output tile, K in steps of 64.  Each
// wave owns a 64 x 64 quarter as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// The A and W tiles of the next K step go straight from global memory into
// LDS (buffer loads with an LDS destination; rows past the end read as zero)
// while the current ones are multiplied.  A tile row is 128 bytes; its
// 16-byte chunks are stored at slot chunk ^ ((row >> 1) & 7), so the 16-byte
// fragment reads of 16 consecutive rows hit 16 different bank groups.
// Workgroups are ordered weight-tile major and dealt so that the row tiles
// sharing a weight tile run on one XCD (one L2).
#include "dlm_internal.h"

#include <math.h>

namespace dlm {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_view(const void *base, long bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kOOB = 0x7ffffff0;   // an offset past any view: the load returns zeros

__device__ __forceinline__ int gswz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ bool row_valid(const GemmArgs &a, int r)
{
    if (r >= a.B * a.M) return false;
    if (!a.m_valid) return true;
    const int b = r / a.M;
    return r - b * a.M < min(max(a.m_valid[b], 0), a.M);
}

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    const __bf16 h = (__bf16)f;
    return *reinterpret_cast<const uint16_t *>(&h);
}

__device__ __forceinline__ float from_bf16(uint16_t u) { return __uint_as_float((unsigned)u << 16); }

// The epilogue of element (r, n): v = C[r, n] (the gate product for
// SwiGLU), up = the up product (SwiGLU only).
__device__ __forceinline__ void store_out(const GemmArgs &a, bool swiglu, int r, int n, float v, float up)
{
    const int b = r / a.M, j = r - b * a.M;
    if (swiglu) {
        a.out[(long)r * a.N + n] = to_bf16(v / (1.f + __expf(-v)) * up);
    } else if (a.ep_mode == 1) {
        // q | k | v columns, head-major
        const int qn = a.Hq * a.D, kn = a.Hkv * a.D;
        if (n < qn)
            a.out[(((long)b * a.Hq + n / a.D) * a.M + j) * a.D + n % a.D] = to_bf16(v);
        else if (n < qn + kn)
            a.out_k[(((long)b * a.Hkv + (n - qn) / a.D) * a.M + j) * a.D + (n - qn) % a.D] = to_bf16(v);
        else
            a.out_v[(((long)b * a.Hkv + (n - qn - kn) / a.D) * a.M + j) * a.D + (n - qn - kn) % a.D] = to_bf16(v);
    } else if (a.ep_mode == 0) {
        a.out[(long)r * a.N + n] = to_bf16(v);
    } else {
        // residual: the row's own hidden state (gathered or compact)
        const long src = a.resid_gather ? ((long)b * a.n_pos + a.act[b * a.M + j]) * a.N + n : (long)r * a.N + n;
        v += from_bf16(a.resid[src]);
        const long dst = a.ep_mode == 3 ? ((long)b * a.n_pos + a.act[b * a.M + j]) * a.N + n : (long)r * a.N + n;
        a.out[dst] = to_bf16(v);
    }
}

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a)
{
    constexpr int NW = SWIGLU ? 2 : 1;     // weight matrices sharing the A tile
    __shared__ __attribute__((aligned(1024))) uint16_t As0[kBM * kBK];
    __shared__ __attribute__((aligned(1024))) uint16_t As1[kBM * kBK];
    __shared__ __attribute__((aligned(1024))) uint16_t Ws0[NW * kBN * kBK];
    __shared__ __attribute__((aligned(1024))) uint16_t Ws1[NW * kBN * kBK];

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wm = wid >> 1, wn = wid & 1;
    const int tiles_m = (a.B * a.M + kBM - 1) / kBM;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = L % tiles_m, rest = L / tiles_m;
    const int ks = rest % a.splits, nt = rest / a.splits;
    const int m0 = mt * kBM, n0 = nt * kBN;
    const int kbeg = ks * a.kc, kend = min(a.K, kbeg + a.kc);

    // A tile geometry of this thread: load u writes LDS bytes
    // (4u + wid) * 1024 + lane * 16: tile row ar[u], slot sl; the global
    // chunk it fetches is sl ^ gswz(row).
    int arow_off[4], achunk[4];
    bool any = false;
    for (int u = 0; u < 4; ++u) {
        const int byte = (4 * u + wid) * 1024 + lane * 16;
        const int row = byte >> 7, sl = (byte >> 4) & 7;
        achunk[u] = sl ^ gswz(row);
        const int r = m0 + row;
        const bool ok = row_valid(a, r);
        any |= ok;
        int off = -1;                        // -1: invalid row
        if (ok) {
            const int b = r / a.M, j = r - b * a.M;
            if (a.a_mode == 1)
                off = ((b * a.n_pos + a.act[b * a.M + j]) * a.K) * 2;
            else if (a.a_mode == 2)
                off = ((b * a.Hq * a.M + j) * a.D) * 2;
            else
                off = (r * a.K) * 2;
        }
        arow_off[u] = off;
    }
    if (!__syncthreads_or(any)) return;     // no valid row in this tile

    const __amdgpu_buffer_rsrc_t ars = gemm_view(a.a, a.a_bytes);
    const __amdgpu_buffer_rsrc_t w0 = gemm_view(a.w0, (long)a.N * a.K * 2);
    const __amdgpu_buffer_rsrc_t w1 = gemm_view(SWIGLU ? a.w1 : a.w0, (long)a.N * a.K * 2);
    int woff[4];
    for (int u = 0; u < 4; ++u) {
        const int byte = (4 * u + wid) * 1024 + lane * 16;
        const int row = byte >> 7, sl = (byte >> 4) & 7;
        const int n = n0 + row;
        woff[u] = n < a.N ? (n * a.K + (sl ^ gswz(row)) * 8) * 2 : -1;
    }

    auto issue = [&](int k0, uint16_t *as, uint16_t *ws) {
        int koff;                            // byte offset of column k0 within a row
        if (a.a_mode == 2)
            koff = ((k0 / a.D) * a.M * a.D + k0 % a.D) * 2;
        else
            koff = k0 * 2;
        for (int u = 0; u < 4; ++u) {
            const int off = arow_off[u] < 0 ? kOOB : arow_off[u] + koff + achunk[u] * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void *)(as + (4 * u + wid) * 512), 16, off, 0, 0,
                                                     0);
        }
        for (int u = 0; u < 4; ++u) {
            const int off = woff[u] < 0 ? kOOB : woff[u] + k0 * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(w0, (lds_void *)(ws + (4 * u + wid) * 512), 16, off, 0, 0,
                                                     0);
            if (SWIGLU)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(w1, (lds_void *)(ws + kBN * kBK + (4 * u + wid) * 512),
                                                         16, off, 0, 0, 0);
        }
    };

    // fragment read offsets (elements): row (wm*64 + 32i + l32), chunk 2kk + hh
    int ard[2][4], wrd[2][4];
    for (int i = 0; i < 2; ++i)
        for (int kk = 0; kk < 4; ++kk) {
            const int ra = wm * 64 + 32 * i + l32, rw = wn * 64 + 32 * i + l32;
            ard[i][kk] = ra * kBK + (((2 * kk + hh) ^ gswz(ra)) * 8);
            wrd[i][kk] = rw * kBK + (((2 * kk + hh) ^ gswz(rw)) * 8);
        }

    f32x16 acc[NW][2][2];
    for (int w = 0; w < NW; ++w)
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) acc[w][i][j] = f32x16{};

    auto compute = [&](const uint16_t *as, const uint16_t *ws) {
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(as + ard[0][kk]);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(as + ard[1][kk]);
            for (int w = 0; w < NW; ++w) {
                const uint16_t *wt = ws + w * kBN * kBK;
                const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(wt + wrd[0][kk]);
                const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(wt + wrd[1][kk]);
                acc[w][0][0] = mma(a0, b0, acc[w][0][0]);
                acc[w][0][1] = mma(a0, b1, acc[w][0][1]);
                acc[w][1][0] = mma(a1, b0, acc[w][1][0]);
                acc[w][1][1] = mma(a1, b1, acc[w][1][1]);
            }
        }
    };

    const int nk = (kend - kbeg) / kBK;
    issue(kbeg, As0, Ws0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < nk; t += 2) {
        if (t + 1 < nk) issue(kbeg + (t + 1) * kBK, As1, Ws1);
        compute(As0, Ws0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < nk) {
            if (t + 2 < nk) issue(kbeg + (t + 2) * kBK, As0, Ws0);
            compute(As1, Ws1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // Epilogue.  Accumulator element e of lane (l32, hh) in tile (i, j) is
    // row wm*64 + 32i + 8(e/4) + 4hh + e%4, column wn*64 + 32j + l32.  With
    // K splits the fp32 sums go to this split's slice of the partials.
    const long rows = (long)a.B * a.M;
    const int np = SWIGLU ? 2 * a.N : a.N;
    for (int i = 0; i < 2; ++i)
        for (int e = 0; e < 16; ++e) {
            const int r = m0 + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (!row_valid(a, r)) continue;
            for (int jj = 0; jj < 2; ++jj) {
                const int n = n0 + wn * 64 + 32 * jj + l32;
                if (n >= a.N) continue;
                const float v = acc[0][i][jj][e], up = acc[NW - 1][i][jj][e];
                if (a.splits > 1) {
                    float *p = a.part + ((long)ks * rows + r) * np + n;
                    p[0] = v;
                    if (SWIGLU) p[a.N] = up;
                } else {
                    store_out(a, SWIGLU, r, n, v, up);
                }
            }
        }
}

// Sum the K splits of each valid element in split order (deterministic)
// and apply the epilogue.  One thread per element.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a, int swiglu)
{
    const long rows = (long)a.B * a.M;
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * a.N) return;
    const int r = (int)(idx / a.N), n = (int)(idx - (long)r * a.N);
    if (!row_valid(a, r)) return;
    const int np = swiglu ? 2 * a.N : a.N;
    float v = 0.f, up = 0.f;
    for (int s = 0; s < a.splits; ++s) {
        const float *p = a.part + ((long)s * rows + r) * np + n;
        v += p[0];
        if (swiglu) up += p[a.N];
    }
    store_out(a, swiglu != 0, r, n, v, up);
}

}  // namespace

GemmPlan plan_gemm(int rows, int N, int K, bool swiglu)
{
    GemmPlan p{};
    const long tiles = (long)((rows + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    // Too few output tiles to fill the chip: split K (at least four K steps
    // per split), the partial sums then reduced by a second kernel.  From
    // 1.5 tiles per CU on, the partial-sum traffic costs more than the
    // extra parallelism gains (measured on MI355X).
    int s = 1;
    if (tiles > 0 && tiles < 3L * kNumCU / 2) {
        s = (int)((2L * kNumCU + tiles - 1) / tiles);
        s = max(1, min(s, min(16, K / (4 * kBK))));
    }
    const int steps = (K / kBK + s - 1) / s;
    p.kc = steps * kBK;
    p.splits = (K + p.kc - 1) / p.kc;
    p.part_bytes = p.splits > 1 ? (size_t)p.splits * rows * N * (swiglu ? 2 : 1) * sizeof(float) : 0;
    return p;
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    const long tiles = (long)((a.B * a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN) * a.splits;
    if (tiles == 0) return hipSuccess;
    if (a.w1)
        gemm_kernel<true><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(a);
    else
        gemm_kernel<false><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(a);
    if (a.splits > 1) {
        const long n = (long)a.B * a.M * a.N;
        gemm_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a, a.w1 ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace dlm
