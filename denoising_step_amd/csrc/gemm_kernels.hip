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
// Workgroup: 256 threads, a 128 x 128 output tile.  Each wave owns a
// 64 x 64 quarter as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.  The A and W
// tiles of the next K steps go straight from global memory into LDS (buffer
// loads with an LDS destination; rows past the end read as zero) while the
// current ones are multiplied, through a ring of LDS stages: K steps of 64
// in two stages for the plain products, of 32 in three stages for SwiGLU
// (its stage holds two weight tiles); either way 64-72 KB of LDS, so two
// workgroups share a CU (measured on MI355X against 32 x 4, 64 x 3 and
// 64 x 2 / 32 x 2 for SwiGLU).  Tile rows are stored with their 16-byte
// chunks permuted per row (gswz) so that fragment reads are free of bank
// conflicts.
// Workgroups are ordered weight-tile major and dealt so that the row tiles
// sharing a weight tile run on one XCD (one L2).
//
// Weights may also come fragment-packed (dlm_pack_weights): for each tile
// of 16 rows and each step of 32 columns, 1 KB holding the tile's 16 x 32
// block in the register order of an MFMA operand (64 lanes x 8 bf16, lane
// l: row l % 16, columns 8 (l / 16) .. + 7).  One wave load then reads 1 KB
// of contiguous memory and hands every lane its fragment; with row-major
// weights the same load touches 64 bytes in each of 16 rows, which streams
// markedly slower from HBM (measured on MI355X: about 6.3 against 5.4 TB/s
// for a bare read, 24 against 34 us for the 16-row q/k/v product).
#include "dlm_internal.h"

#include <math.h>

namespace dlm {

namespace {

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kBN = 128;
constexpr int kKQ = 64;   // split-K chunks are multiples of this many columns

// K step and LDS stages of the plain products and of the SwiGLU product
// (two weight tiles per step).  A stage holds (128 + 128 NW) x BK bf16; two
// workgroups share a CU while 2 x ST stages fit in LDS.
#ifndef DLM_GEMM_BK
#define DLM_GEMM_BK 64
#endif
#ifndef DLM_GEMM_ST
#define DLM_GEMM_ST 2
#endif
#ifndef DLM_GEMM_SW_BK
#define DLM_GEMM_SW_BK 32
#endif
#ifndef DLM_GEMM_SW_ST
#define DLM_GEMM_SW_ST 3
#endif
constexpr int kOOB = 0x7ffffff0;   // an offset past any view: the load returns zeros

// Row-tile height for a product over `rows` rows.  Up to 256 rows (two row
// tiles) the work is streaming the weights: one workgroup per CU with a
// deep ring of 64-wide K steps (as many stages as about 150 KB of LDS
// holds), so that 120-150 KB of weights are in flight per CU, and a 32-,
// 64- or 128-row tile (up to 64 rows the four waves sit side by side over
// the 128 columns).  More rows: 128-row tiles, two workgroups per CU, a
// shallower ring (measured on MI355X: the deep ring wins up to 256 rows
// and loses at 512).
__host__ __device__ constexpr int gemm_bm(int rows) { return rows <= 32 ? 32 : rows <= 64 ? 64 : 128; }
#ifndef DLM_GEMM_DEEP_MAX
#define DLM_GEMM_DEEP_MAX 256
#endif
__host__ __device__ constexpr bool gemm_deep(int rows) { return rows <= DLM_GEMM_DEEP_MAX; }
__host__ __device__ constexpr int skinny_stages(int bm, int nw)
{
    return (150 * 1024) / ((bm + nw * kBN) * 64 * 2) < 8 ? (150 * 1024) / ((bm + nw * kBN) * 64 * 2) : 8;
}

// 16-byte chunk swizzle of a tile row of BK bf16: 256 bytes hold 128 / BK
// rows, and rows that share a bank offset get distinct chunk permutations,
// so the 16-byte reads of 16 consecutive rows hit 16 different bank groups.
template <int BK>
__device__ __forceinline__ int gswz(int row)
{
    return (row / (128 / BK)) % (BK / 8);
}

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

template <bool SWIGLU, int BM, int BK, int ST>
__global__ __launch_bounds__(256, 2 * 2 * (BM + (SWIGLU ? 2 : 1) * kBN) * BK * ST <= 160 * 1024 ? 2 : 1) void
gemm_kernel(GemmArgs a)
{
    constexpr int kBM = BM;
    constexpr int NW = SWIGLU ? 2 : 1;          // weight matrices sharing the A tile
    constexpr int WM = BM == 128 ? 2 : 1;       // wave grid WM x WN over the tile
    constexpr int WN = 4 / WM;
    constexpr int TI = BM / (32 * WM);          // 32 x 32 MFMA tiles per wave: TI x TJ
    constexpr int TJ = kBN / (32 * WN);
    constexpr int CH = BK / 8;                  // 16-byte chunks per tile row
    constexpr int NA = kBM * BK / (256 * 8);    // direct 16-byte loads per thread, A tile
    constexpr int NB = kBN * BK / (256 * 8);    // the same per weight tile
    constexpr int LPS = NA + NW * NB;           // loads per thread per stage
    constexpr int KK = BK / 16;                 // MFMA K steps per stage
    static_assert(ST >= 2 && (BK == 32 || BK == 64) && NA >= 1, "tile shape");
    // stage s: the A tile, then the weight tile(s)
    constexpr int kSlot = (kBM + NW * kBN) * BK;
    __shared__ __attribute__((aligned(1024))) uint16_t Sm[ST][kSlot];

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wm = wid / WN, wn = wid % WN;
    const int tiles_m = (a.B * a.M + kBM - 1) / kBM;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = L % tiles_m, rest = L / tiles_m;
    const int ks = rest % a.splits, nt = rest / a.splits;
    const int m0 = mt * kBM, n0 = nt * kBN;
    const int kbeg = ks * a.kc, kend = min(a.K, kbeg + a.kc);

    // Tile geometry of this thread: load u writes LDS bytes
    // (4u + wid) * 1024 + lane * 16, i.e. tile row byte / (2 BK) and 16-byte
    // slot (byte / 16) % CH; the global chunk it fetches is slot ^ gswz(row).
    int arow_off[NA], achunk[NA];
    bool any = false;
    for (int u = 0; u < NA; ++u) {
        const int byte = (4 * u + wid) * 1024 + lane * 16;
        const int row = byte / (2 * BK), sl = (byte >> 4) % CH;
        achunk[u] = sl ^ gswz<BK>(row);
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

    const i32x4 ars = dma_view(a.a, a.a_bytes);
    const i32x4 w0 = dma_view(a.w0, (long)a.N * a.K * 2);
    const i32x4 w1 = dma_view(SWIGLU ? a.w1 : a.w0, (long)a.N * a.K * 2);
    int woff[NB];
    for (int u = 0; u < NB; ++u) {
        if (a.w_packed) {
            // 1 KB fragment g of the tile: 16-row group g / (BK / 32), 32-column step g % (BK / 32)
            const int g = 4 * u + wid, n16 = n0 / 16 + g / (BK / 32);
            woff[u] = 16 * n16 < a.N ? ((n16 * (a.K / 32) + g % (BK / 32)) * 512 + lane * 8) * 2 : -1;
            continue;
        }
        const int byte = (4 * u + wid) * 1024 + lane * 16;
        const int row = byte / (2 * BK), sl = (byte >> 4) % CH;
        const int n = n0 + row;
        woff[u] = n < a.N ? (n * a.K + (sl ^ gswz<BK>(row)) * 8) * 2 : -1;
    }
    const int wk = a.w_packed ? 32 : 2;      // weight bytes per column step (k0 a multiple of 32)

    // Load the K step at k0 into a slot; a step past this split's end
    // (k0 >= kend) loads zeros, so every stage issues the same loads.
    auto issue = [&](int k0, uint16_t *slot) {
        const bool live = k0 < kend;
        int koff;                            // byte offset of column k0 within a row
        if (a.a_mode == 2)
            koff = ((k0 / a.D) * a.M * a.D + k0 % a.D) * 2;
        else
            koff = k0 * 2;
        for (int u = 0; u < NA; ++u) {
            const int off = (arow_off[u] < 0 || !live) ? kOOB : arow_off[u] + koff + achunk[u] * 16;
            dma16(ars, off, slot + (4 * u + wid) * 512);
        }
        uint16_t *ws = slot + kBM * BK;
        for (int u = 0; u < NB; ++u) {
            const int off = (woff[u] < 0 || !live) ? kOOB : woff[u] + k0 * wk;
            dma16(w0, off, ws + (4 * u + wid) * 512);
            if (SWIGLU) dma16(w1, off, ws + kBN * BK + (4 * u + wid) * 512);
        }
    };

    // fragment read offsets (elements): A row wm*32TI + 32i + l32, W row
    // wn*32TJ + 32j + l32, chunk 2kk + hh
    int ard[TI][KK], wrd[TJ][KK];
    for (int kk = 0; kk < KK; ++kk) {
        for (int i = 0; i < TI; ++i) {
            const int ra = wm * 32 * TI + 32 * i + l32;
            ard[i][kk] = ra * BK + (((2 * kk + hh) ^ gswz<BK>(ra)) * 8);
        }
        for (int j = 0; j < TJ; ++j) {
            const int rw = wn * 32 * TJ + 32 * j + l32, c = 2 * kk + hh;
            wrd[j][kk] = kBM * BK + (a.w_packed ? ((rw / 16) * (BK / 32) + c / 4) * 512 + ((c % 4) * 16 + rw % 16) * 8
                                                : rw * BK + ((c ^ gswz<BK>(rw)) * 8));
        }
    }

    f32x16 acc[NW][TI][TJ];
    for (int w = 0; w < NW; ++w)
        for (int i = 0; i < TI; ++i)
            for (int j = 0; j < TJ; ++j) acc[w][i][j] = f32x16{};

    // The fragments of MFMA step kk + 1 are read before the products of
    // step kk are issued (two register buffers), so the LDS latency runs
    // under the MFMAs.
    constexpr int NRD = TI + NW * TJ;           // fragment reads per MFMA step
    auto compute = [&](const uint16_t *slot) {
        bf16x8 af[2][TI], bf[2][NW][TJ];
        auto read = [&](int kk, int p) {
            for (int i = 0; i < TI; ++i) af[p][i] = *reinterpret_cast<const bf16x8 *>(slot + ard[i][kk]);
            for (int w = 0; w < NW; ++w)
                for (int j = 0; j < TJ; ++j)
                    bf[p][w][j] = *reinterpret_cast<const bf16x8 *>(slot + w * kBN * BK + wrd[j][kk]);
        };
        read(0, 0);
        for (int kk = 0; kk < KK; ++kk) {
            const int p = kk & 1;
            if (kk + 1 < KK) read(kk + 1, p ^ 1);
            for (int w = 0; w < NW; ++w)
                for (int i = 0; i < TI; ++i)
                    for (int j = 0; j < TJ; ++j) acc[w][i][j] = mma(af[p][i], bf[p][w][j], acc[w][i][j]);
        }
        // order: the first step's reads, then per step the next step's
        // reads ahead of this step's products
        __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 1 < KK) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NW * TI * TJ, 0);
        }
    };

    // ST-stage pipeline: at step t the loads of steps t .. t+ST-2 are in
    // flight; wait for step t alone, one barrier (step t visible to every
    // wave; the slot of step t-1 free), load step t+ST-1 into that slot,
    // multiply step t.  Steps past the end load zeros and are not
    // multiplied, so the wait count is the same at every step.
    const int nk = (kend - kbeg) / BK;
    for (int q = 0; q < ST - 1; ++q) issue(kbeg + q * BK, Sm[q]);
    int rd = 0, wr = ST - 1;                 // slots of steps t and t+ST-1
    for (int t = 0; t < nk; ++t) {
        dma_wait_barrier<(ST - 2) * LPS>();
        issue(kbeg + (t + ST - 1) * BK, Sm[wr]);
        compute(Sm[rd]);
        rd = rd + 1 == ST ? 0 : rd + 1;
        wr = wr + 1 == ST ? 0 : wr + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the trailing loads of zeros

    // Epilogue.  Accumulator element e of lane (l32, hh) in tile (i, j) is
    // row wm*32TI + 32i + 8(e/4) + 4hh + e%4, column wn*32TJ + 32j + l32.
    // With K splits the fp32 sums go to this split's slice of the partials.
    const long rows = (long)a.B * a.M;
    const int np = SWIGLU ? 2 * a.N : a.N;
    for (int i = 0; i < TI; ++i)
        for (int e = 0; e < 16; ++e) {
            const int r = m0 + wm * 32 * TI + 32 * i + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (!row_valid(a, r)) continue;
            for (int jj = 0; jj < TJ; ++jj) {
                const int n = n0 + wn * 32 * TJ + 32 * jj + l32;
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

// Skinny products: at most 16 rows (late denoising steps, small M_t),
// where the work is streaming the weights once.  A workgroup owns 16 weight
// rows over the whole K (so no K-split partials and no second kernel); its
// KW waves take a KW-th of K each, and their sums are added in LDS in a
// fixed order.  KW is chosen per launch so that all waves of the grid are
// resident at once (a second, partly filled round of workgroups would
// leave the stream without enough loads in flight).  C^T = W A^T with
// v_mfma_f32_16x16x32_bf16: operand A is 16 weight rows x 32 k, lane l
// holding row l % 16, k = 8 (l / 16) .. + 7 (one packed fragment, or 64
// bytes per weight row of a row-major matrix), loaded straight into
// registers (non-temporal: each weight is read once); operand B is 32 k x
// 16 activation rows in the same lane order, read from L2 (every workgroup
// reads the same activation rows), as one 1 KB fragment per k step when
// they come packed (a_mode 3).  U k steps of loads are issued a buffer
// ahead of their MFMAs (about 12 16-byte loads per lane per buffer, two
// buffers).  With more than 16 rows the tiled kernel is faster (measured on
// MI355X with packed weights: 28 against 37 us for q/k/v at 32 rows).
constexpr int kSkinnyRows = 16;

// Packed position of element (r, n) of a 16-row activation block (the
// operand order above): k step n / 32, lane (n % 32) / 8 * 16 + r.
__device__ __forceinline__ long packed_act(int r, int n)
{
    return ((long)(n >> 5) * 64 + ((n & 31) >> 3) * 16 + r) * 8 + (n & 7);
}

template <bool SWIGLU, int KW>
__global__ __launch_bounds__(64 * KW) void skinny_kernel(GemmArgs a)
{
    constexpr int NW = SWIGLU ? 2 : 1;
    constexpr int U = SWIGLU ? 3 : 6;            // k steps (of 32) per register buffer
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    __shared__ float red_s[KW][NW][16][17];      // each wave's sums [row][n], padded

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int ksteps = a.K / 32;
    const int per = (ksteps + KW - 1) / KW;
    const int sb = min(ksteps, wid * per), se = min(ksteps, sb + per);

    // this lane's weight fragment at k step 0, and the distance of k steps
    // (in 16-byte units): packed, the tile's steps are 1 KB apart; row-major,
    // rows past N read row 0 (their sums are never stored)
    const long wbase = a.w_packed ? (long)blockIdx.x * ksteps * 512 + 8 * lane
                                  : (long)(n0 + l16 < a.N ? n0 + l16 : 0) * a.K + 8 * q4;
    const int wstep = a.w_packed ? 64 : 4;
    const v4u *wp[NW];
    wp[0] = reinterpret_cast<const v4u *>(a.w0 + wbase);
    if (SWIGLU) wp[NW - 1] = reinterpret_cast<const v4u *>(a.w1 + wbase);
    // activation row l16: element offset of this lane's first k (rows past
    // the end read row 0; their sums are never stored, and an activation row
    // only feeds its own output column)
    const int r = row_valid(a, l16) ? l16 : 0;
    const int rb = r / a.M, rj = r - rb * a.M;
    const long abase = a.a_mode == 3 ? 8L * lane
                     : (a.a_mode == 1 ? ((long)rb * a.n_pos + a.act[rb * a.M + rj]) * a.K
                      : a.a_mode == 2 ? ((long)rb * a.Hq * a.M + rj) * a.D
                                      : (long)r * a.K) + 8 * q4;
    // offset of k step st (32 columns; in mode 2 a step never straddles two
    // heads, D being a multiple of 32): the same for every lane of the wave
    auto a_step = [&](int st) -> long {
        const int kk = 32 * st;
        return a.a_mode == 3 ? 16L * kk : a.a_mode == 2 ? (long)(kk / a.D) * a.M * a.D + kk % a.D : (long)kk;
    };

    f32x4 acc[NW];
    for (int w = 0; w < NW; ++w) acc[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Two register buffers of U k steps: the loads of the next U steps are
    // issued before the MFMAs of the current ones.  Every load is
    // unconditional (a predicated load would make the compiler wait for it
    // before the zero of the other branch): steps past the wave's range
    // reload its last step and are not multiplied.
    v4u wv[2][NW][U], av[2][U];
    auto load = [&](int bi, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = min(s + u, se - 1);
            for (int w = 0; w < NW; ++w) wv[bi][w][u] = __builtin_nontemporal_load(wp[w] + wstep * st);
            av[bi][u] = *reinterpret_cast<const v4u *>(a.a + abase + a_step(st));
        }
    };
    auto mult = [&](int bi, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < se) {
                for (int w = 0; w < NW; ++w)
                    acc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        *reinterpret_cast<const bf16x8 *>(&wv[bi][w][u]),
                        *reinterpret_cast<const bf16x8 *>(&av[bi][u]), acc[w], 0, 0, 0);
            }
        }
    };
    if (sb < se) {
        load(0, sb);
        for (int s = sb; s < se; s += 2 * U) {
            if (s + U < se) load(1, s + U);
            mult(0, s);
            if (s + U >= se) break;
            if (s + 2 * U < se) load(0, s + 2 * U);
            mult(1, s + U);
        }
    }
    // lane (l16, q4) holds rows (weight) 4 q4 + i of column (activation row) l16
    for (int w = 0; w < NW; ++w)
        for (int i = 0; i < 4; ++i) red_s[wid][w][l16][4 * q4 + i] = acc[w][i];
    __syncthreads();
    for (int idx = tid; idx < 16 * 16; idx += 64 * KW) {
        const int nl = idx % 16, rr = idx / 16;
        const int nn = n0 + nl;
        if (nn >= a.N || !row_valid(a, rr)) continue;
        float v[NW];
        for (int w = 0; w < NW; ++w) {
            float t[KW];
            for (int q = 0; q < KW; ++q) t[q] = red_s[q][w][rr][nl];
            for (int h = KW / 2; h >= 1; h >>= 1)   // fixed tree order
                for (int q = 0; q < h; ++q) t[q] += t[q + h];
            v[w] = t[0];
        }
        if (SWIGLU && a.out_packed)   // gated rows straight into the down projection's operand order
            a.out[packed_act(rr, nn)] = to_bf16(v[0] / (1.f + __expf(-v[0])) * v[NW - 1]);
        else
            store_out(a, SWIGLU, rr, nn, v[0], v[NW - 1]);
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

// The activation rows of a skinny product (at most 16, a_mode 0, 1 or 2)
// as packed operand fragments: one thread per 16-byte chunk o, k step
// o / 64, lane o % 64 (row lane % 16, columns 32 step + 8 (lane / 16) ..
// + 7); rows that are not valid are written as zeros.  One read of the rows
// here saves every workgroup of the product a 16-row gather per k step.
__global__ __launch_bounds__(256) void pack_rows_kernel(GemmArgs a, uint16_t *dst)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= a.K / 32 * 64) return;
    const int lane = o % 64, r = lane % 16, k = (o / 64) * 32 + (lane / 16) * 8;
    v4u v = v4u{0u, 0u, 0u, 0u};
    if (row_valid(a, r)) {
        const int b = r / a.M, j = r - b * a.M;
        const long src = a.a_mode == 1 ? ((long)b * a.n_pos + a.act[b * a.M + j]) * a.K + k
                       : a.a_mode == 2 ? ((long)b * a.Hq * a.M + j) * a.D + (long)(k / a.D) * a.M * a.D + k % a.D
                                       : (long)r * a.K + k;
        v = *reinterpret_cast<const v4u *>(a.a + src);
    }
    reinterpret_cast<v4u *>(dst)[o] = v;
}

// One thread per 16-byte chunk of the packed layout: chunk o is lane
// o % 64 of fragment o / 64 (16-row group f / (K/32), 32-column step
// f % (K/32)); the lane holds row 16 group + lane % 16, columns
// 32 step + 8 (lane / 16) .. + 7.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t *w, uint16_t *p, int N, int K)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const long o = (long)blockIdx.x * 256 + threadIdx.x;
    if (o >= (long)N * K / 8) return;
    const long f = o / 64;
    const int lane = (int)(o % 64), ks = K / 32;
    const long row = (f / ks) * 16 + lane % 16;
    const int col = (int)(f % ks) * 32 + (lane / 16) * 8;
    reinterpret_cast<v4u *>(p)[o] = *reinterpret_cast<const v4u *>(w + row * K + col);
}

}  // namespace

hipError_t launch_pack_rows(const GemmArgs &a, uint16_t *dst, hipStream_t stream)
{
    if (!gemm_skinny(a.B * a.M) || a.a_mode == 3) return hipErrorInvalidValue;
    const int chunks = a.K / 32 * 64;
    pack_rows_kernel<<<(chunks + 255) / 256, 256, 0, stream>>>(a, dst);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const uint16_t *w, uint16_t *packed, int N, int K, hipStream_t stream)
{
    const long chunks = (long)N * K / 8;
    if (chunks == 0) return hipSuccess;
    pack_weights_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, stream>>>(w, packed, N, K);
    return hipGetLastError();
}

GemmPlan plan_gemm(int rows, int N, int K, bool swiglu)
{
    GemmPlan p{};
    if (gemm_skinny(rows)) {   // skinny_kernel: whole K per workgroup, no partials
        p.kc = K;
        p.splits = 1;
        p.part_bytes = 0;
        return p;
    }
    const int bm = gemm_bm(rows);
    const long tiles = (long)((rows + bm - 1) / bm) * ((N + kBN - 1) / kBN);
    // Too few output tiles to fill the chip: split K (at least 256 columns
    // per split), the partial sums then reduced by a second kernel.  From
    // 1.5 tiles per CU on, the partial-sum traffic costs more than the
    // extra parallelism gains (measured on MI355X).
    int s = 1;
    if (gemm_deep(rows) && tiles > 0) {
        // deep-ring tiles run one workgroup per CU: one round of
        // workgroups, each streaming as many K steps as the split allows
        // (a workgroup pays one ring fill)
        s = max(1, min((int)(kNumCU / tiles), min(16, K / 256)));
    } else if (tiles > 0 && tiles < 3L * kNumCU / 2) {
        s = (int)((2L * kNumCU + tiles - 1) / tiles);
        s = max(1, min(s, min(16, K / 256)));
    }
    const int steps = (K / kKQ + s - 1) / s;
    p.kc = steps * kKQ;
    p.splits = (K + p.kc - 1) / p.kc;
    p.part_bytes = p.splits > 1 ? (size_t)p.splits * rows * N * (swiglu ? 2 : 1) * sizeof(float) : 0;
    return p;
}

bool gemm_skinny(int rows) { return rows <= kSkinnyRows; }

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream)
{
    const int rows = a.B * a.M;
    if (rows == 0) return hipSuccess;
    if ((a.a_mode == 3 || a.out_packed) && !gemm_skinny(rows)) return hipErrorInvalidValue;
    if (gemm_skinny(rows)) {
        const int tiles = (a.N + 15) / 16;
        // four waves per SIMD fit at this kernel's register use: the widest
        // K split whose grid still fits in one round (up to 8 for the SwiGLU
        // pair, whose sums take twice the LDS)
        const long slots = 4L * kNumCU * 4;
        const int kw = !a.w1 && tiles * 16L <= slots ? 16 : tiles * 8L <= slots ? 8 : 4;
        const dim3 grid((unsigned)tiles), block(64 * kw);
        if (a.w1) {
            if (kw == 8) skinny_kernel<true, 8><<<grid, block, 0, stream>>>(a);
            else skinny_kernel<true, 4><<<grid, block, 0, stream>>>(a);
        } else {
            if (kw == 16) skinny_kernel<false, 16><<<grid, block, 0, stream>>>(a);
            else if (kw == 8) skinny_kernel<false, 8><<<grid, block, 0, stream>>>(a);
            else skinny_kernel<false, 4><<<grid, block, 0, stream>>>(a);
        }
        return hipGetLastError();
    }
    const int bm = gemm_bm(a.B * a.M);
    const long tiles = (long)((a.B * a.M + bm - 1) / bm) * ((a.N + kBN - 1) / kBN) * a.splits;
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)tiles), block(256);
    const bool deep = gemm_deep(a.B * a.M);
    if (a.w1) {
        if (bm == 32)
            gemm_kernel<true, 32, 64, skinny_stages(32, 2)><<<grid, block, 0, stream>>>(a);
        else if (bm == 64)
            gemm_kernel<true, 64, 64, skinny_stages(64, 2)><<<grid, block, 0, stream>>>(a);
        else if (deep)
            gemm_kernel<true, 128, 64, skinny_stages(128, 2)><<<grid, block, 0, stream>>>(a);
        else
            gemm_kernel<true, 128, DLM_GEMM_SW_BK, DLM_GEMM_SW_ST><<<grid, block, 0, stream>>>(a);
    } else {
        if (bm == 32)
            gemm_kernel<false, 32, 64, skinny_stages(32, 1)><<<grid, block, 0, stream>>>(a);
        else if (bm == 64)
            gemm_kernel<false, 64, 64, skinny_stages(64, 1)><<<grid, block, 0, stream>>>(a);
        else if (deep)
            gemm_kernel<false, 128, 64, skinny_stages(128, 1)><<<grid, block, 0, stream>>>(a);
        else
            gemm_kernel<false, 128, DLM_GEMM_BK, DLM_GEMM_ST><<<grid, block, 0, stream>>>(a);
    }
    if (a.splits > 1) {
        const long n = (long)a.B * a.M * a.N;
        gemm_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a, a.w1 ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace dlm
