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
#include <stdlib.h>

#include <type_traits>

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

// Raw buffer view of [base, base + bytes): 16-byte loads at or past `bytes`
// return zeros (hardware range check), so tails need no branches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return uint4{v[0], v[1], v[2], v[3]};
}

// Key code: a key is visible to a query iff key_code <= query_code.
//   FULL:          in-range keys INT_MIN; query code 0.
//   BLOCK_CAUSAL:  prefix INT_MIN; block index; query code = its block.
//   GROUP:         prefix INT_MIN; group id of the slot (INT_MAX if the slot is
//                  DUMMY); query code = group id of its slot.
// Keys at or beyond kv_len are INT_MAX.  Both passes evaluate the key code
// from a slot table staged in LDS.
__device__ __forceinline__ int query_code(const AttnArgs &a, const int32_t *gr, int pos)
{
    if (a.kind == 0) return 0;
    int s = (pos - a.P) / a.bs;
    if (a.kind == 1) return s;
    return (s >= 0 && s < a.n_slots) ? gr[s] : INT_MIN;
}

// ---------------------------------------------------------------------------
// Scatter: cache[b, g, active_idx[b, j], :] = fresh[b, g, j, :].
// The copy is cut into row blocks of 256 16-byte chunks, each inside one
// (b, kv-head): block r is (b, kv-head) r / per_bg, rows (r % per_bg) * 256 /
// (D/8) onward (wave-uniform, so scalar).  Each workgroup walks blocks
// blockIdx.x, blockIdx.x + gridDim.x, ... U at a time: a thread issues the
// loads of U chunks of K and V, then their stores, so the stores of one
// round overlap the loads of the next.  The fresh tensors are read once
// (non-temporal).
// ---------------------------------------------------------------------------
#ifndef DLM_SCATTER_UNROLL
#define DLM_SCATTER_UNROLL 2
#endif
#ifndef DLM_SCATTER_WGS
#define DLM_SCATTER_WGS 1024
#endif
constexpr int kScatterUnroll = DLM_SCATTER_UNROLL;
constexpr int kScatterWgs = DLM_SCATTER_WGS;

template <int D>
__global__ __launch_bounds__(256) void kv_scatter_kernel(AttnArgs a)
{
    constexpr int CH = D / 8;                     // chunks per row (power of 2)
    constexpr int U = kScatterUnroll;
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const int per_bg = (a.M * CH + 255) / 256;
    const int nblk = per_bg * a.B * a.Hkv;
    for (int r0 = blockIdx.x; r0 < nblk; r0 += U * gridDim.x) {
        v4u kv[U], vv[U];
        long dst[U];
        bool ok[U];
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * gridDim.x;
            const int bg = r / per_bg;
            const int t = (r - bg * per_bg) * 256 + threadIdx.x;
            const int j = t / CH, c = t % CH;
            ok[u] = r < nblk && j < a.M && j < valid_rows(a, bg / a.Hkv);
            dst[u] = 0;
            kv[u] = v4u{0u, 0u, 0u, 0u};
            vv[u] = v4u{0u, 0u, 0u, 0u};
            if (ok[u]) {
                const int b = bg / a.Hkv;
                const long src = ((long)bg * a.M + j) * CH + c;
                kv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(a.k) + src);
                vv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(a.v) + src);
                const int pos = a.active_idx[(long)b * a.M + j];
                dst[u] = ((long)bg * a.n_cap + pos) * CH + c;
            }
        }
        for (int u = 0; u < U; ++u) {
            if (ok[u]) {
                reinterpret_cast<v4u *>(a.ck)[dst[u]] = kv[u];
                reinterpret_cast<v4u *>(a.cv)[dst[u]] = vv[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 1.  A workgroup owns packed query rows of one (b, kv-head): packed
// row r = (q-head within the GQA group) * M + j, so the G q-heads that share
// a kv-head share every K/V tile staged in LDS.  Two shapes:
//   one key group (NG = 1): QW query waves of 32 rows (8 at D >= 64: 256
//     rows share each 64-key tile, halving the tile traffic per FLOP), for
//     problems with enough query tiles to fill the chip;
//   two key groups (NG = 2): 4 query waves x 2 = 8 waves on 128 rows.
//     Waves w and w + 4 own the same 32 rows; in each 128-key tile, group 0
//     takes keys 0-63 and group 1 keys 64-127.  That puts two waves on every
//     SIMD when the rows alone give one wave per SIMD.  At the end the two
//     groups exchange their (max, sum) and half of O through LDS, and each
//     merges and writes half of every row's columns.
//
// K/V tiles (64 keys per key group) go from global memory straight into
// LDS (buffer loads with the LDS destination: no registers, no LDS store
// instructions), double-buffered: the loads of tile t+1 are issued before
// tile t is
// computed, and one barrier per tile publishes them.  Rows at or past
// kv_len and rows hidden from every query of the workgroup (DUMMY slots,
// later blocks or groups) are given an out-of-range offset and read as
// zeros.
//
// Mask tiles (block-causal and group masks): the workgroup's query codes
// span [qmin, qmax] and each key tile's codes [kmin, kmax], from the slot
// table staged in LDS.  kmin > qmax: hidden from every row, skipped (no
// MFMAs; none of its rows is fetched, and leading or trailing runs of such
// tiles are not visited at all); kmax <= qmin: visible to every row, no
// predicate; otherwise partial, the per-key predicate runs.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that every lane group the
// LDS serves in one cycle hits distinct banks):
//   K: row r holds key sigma(r) (bits 2 and 3 of r swapped within each
//      32-key sub-tile), chunk c of that key at position c ^ k_swz(r).
//      The S^T accumulator then holds, in element i of half-wave h, key
//      16*(i/8) + 8*h + i%8: exactly the operand-B order of V^T P^T.
//   V: row r holds key r, chunk c at position c ^ v_swz(r).  Operand A of
//      V^T P^T (8 consecutive keys of one column per lane) is two
//      ds_read_b64_tr_b16: within each 16-lane group, source lane s points
//      at key 4e0 + s/4, column d0 + 4*(s%4), and lane j receives keys
//      4e0..4e0+3 of column d0 + j.
// The running max is only moved when it grows by more than kRescaleLog2
// (log2 units): exp2 arguments stay <= kRescaleLog2, and the O/l rescale is
// skipped on most tiles.
//
// With a key split, each workgroup writes its normalised partial (out, lse)
// to the workspace and a separate kernel merges the splits in split order.
// ---------------------------------------------------------------------------
constexpr float kRescaleLog2 = 8.f;

// Ping-pong schedule of the one-key-group pass-1 shape (see the tile loop).
#ifndef DLM_ATTN_PINGPONG
#define DLM_ATTN_PINGPONG 1
#endif
constexpr bool kPingPong = DLM_ATTN_PINGPONG != 0;

// Query waves of a one-key-group pass-1 workgroup (32 rows each).
#ifndef DLM_ATTN_QW1
#define DLM_ATTN_QW1 8
#endif
constexpr int qwaves1(int D) { return D >= 64 ? DLM_ATTN_QW1 : 4; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// XOR swizzles of the pass-1 LDS tiles (16-byte chunk index of row r).
// gfx950 serves a 16-byte LDS read 16 lanes per cycle and an 8-byte one 32
// lanes per cycle over 64 banks (8 and 16 lanes over 32 banks on older
// parts); these keep every such lane group on distinct banks under both
// models.  K: the 16 rows a lane group reads at one chunk land on 16
// distinct chunk slots.  V: the 4 rows x 4 chunks of a transposed read land
// on 16 distinct slots.  Both depend on r mod 16 only.
template <int D>
__device__ __forceinline__ int k_swz(int r)
{
    constexpr int SH = D == 128 ? 4 : D == 64 ? 3 : 2;   // log2(chunks per row)
    const int r4 = r & 15;
    return (r4 ^ (r4 >> SH)) & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int r)
{
    const int i = r & 3, par = (i ^ (i >> 1)) & 1;
    return D == 128 ? (4 * i) ^ (2 * par) : D == 64 ? 2 * i : 2 * par;
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Max over the two half-waves (lanes l and l ^ 32 hold the same query):
// v_permlane32_swap hands each half the other's values without LDS.
__device__ __forceinline__ float half_swap_max(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int NG, int QW, bool DYN>
__global__ __launch_bounds__(64 * QW * NG, 2) void attn_fwd_kernel(AttnArgs a)
{
    constexpr int KT = 64 * NG;          // keys per LDS tile; key group kg takes [64kg, 64kg + 64)
    constexpr int NT = 64 * QW * NG;     // threads: QW query waves per key group
    static_assert(NG == 1 || QW == 4, "two key groups run four query waves each");
    constexpr int ROWB = D * 2;          // bytes per K/V row
    constexpr int NLD = KT * ROWB / (NT * 16);   // 16-byte direct loads per thread per tile, per tensor
    static_assert(NLD >= 1 && NLD * NT * 16 == KT * ROWB, "tile loads must cover the tile exactly");
    constexpr int DK = D / 16;           // MFMA k-steps over the head dim
    constexpr int DT = D / 32;           // 32-row tiles of O^T
    constexpr int OOB = 0x7ffffff0;      // an offset past any buffer view

    __shared__ __attribute__((aligned(1024))) uint16_t Ks0[KT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t Ks1[KT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs0[KT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t Vs1[KT * D];
    __shared__ int kcode_s[NG == 1 && kPingPong ? 4 : 2][KT];   // key codes of partial tiles
    __shared__ int scode_s[kMaxSlots];
    __shared__ int qrange_s[2][QW];                    // each query wave's smallest / largest code
    __shared__ float ml_s[NG == 2 ? 4 * 4 * 64 : 1];   // each key group's running max and sum

    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l32 = lane & 31, hh = lane >> 5;
    const int kg = NG == 2 ? wid >> 2 : 0;   // key group
    const int wq = NG == 2 ? wid & 3 : wid;  // query wave
    const int kofs = 64 * kg;                // this group's first key in a tile

    // Work items: (query tile, key split, batch entry, kv-head).  A planned
    // launch runs one item per workgroup, ordered so that the workgroups
    // sharing K/V run on one XCD.  With a device-decided split the grid is
    // one workgroup per CU, and each walks the active items of every batch
    // entry (their query tiles and splits follow the device row counts), so
    // no workgroup is dispatched for a tile or split that is not used.
    // (DYN is a template parameter: a planned launch compiles to one pass
    // through the body.)
    for (int it = 0, item = blockIdx.x; DYN || it == 0; ++it, item += gridDim.x) {
        int qt = 0, split = 0, b = 0, g = 0;
        if constexpr (!DYN) {
            int L = xcd_remap(item, gridDim.x);
            qt = L % a.n_qtiles;
            L /= a.n_qtiles;
            split = L % a.n_split;
            L /= a.n_split;
            b = L / a.Hkv;
            g = L % a.Hkv;
        } else {
            int rem = item;
            for (; b < a.B; ++b) {
                const int qtb = (a.G * valid_rows(a, b) + 32 * QW - 1) / (32 * QW);
                const int nsb = splits_for(a, b);
                if (rem < a.Hkv * qtb * nsb) {
                    qt = rem % qtb;
                    rem /= qtb;
                    split = rem % nsb;
                    g = rem / nsb;
                    break;
                }
                rem -= a.Hkv * qtb * nsb;
            }
            if (b == a.B) break;
        }
        const int bg = b * a.Hkv + g;
        // With a device row count, a tile past the valid rows, or a split this
        // batch entry does not use, has nothing to do.
        const int Mv = valid_rows(a, b);
        const int ns = splits_for(a, b);
        if (qt * (32 * QW) >= a.G * Mv || split >= ns) continue;
        const int split_keys = ns == a.n_split ? a.split_keys : (a.kv_len + 64 * NG * ns - 1) / (64 * NG * ns) * 64 * NG;

        const uint8_t *st = a.kind == 2 ? a.slot_state + (long)b * a.n_slots : nullptr;
        const int32_t *gr = a.kind == 2 ? a.slot_group + (long)b * a.n_slots : nullptr;
        if (a.kind == 2) {
            for (int s = tid; s < a.n_slots; s += NT) scode_s[s] = st[s] == 0 ? INT_MAX : gr[s];
        }
        // The tiles need no clearing: every load of a tile writes its 16
        // bytes, and a row past kv_len or hidden from the whole workgroup is
        // given an offset past the buffer's range, for which the load writes
        // zeros (measured on MI355X), so no LDS byte read as part of a tile
        // is left over from before.

        // This lane's query: packed row r = hl * Mv + j over the Mv valid rows
        // (the row stride in memory stays M).
        const int rows_bg = a.G * Mv;
        const int r = qt * (32 * QW) + wq * 32 + l32;
        const bool rv = r < rows_bg;
        const int hl = rv ? r / Mv : 0;
        const int j = rv ? r - hl * Mv : 0;
        const int h = g * a.G + hl;
        const int pos = a.active_idx[(long)b * a.M + j];
        const int qcode = rv ? query_code(a, gr, pos) : INT_MIN;
        // The workgroup's query-code range over its valid rows: a key tile
        // whose smallest code exceeds qmax is hidden from every row and
        // skipped; one whose largest code is at most qmin is visible to every
        // row and runs without the predicate; any other tile is partial and
        // runs the per-key predicate.  Each query wave reduces its rows with
        // shuffles and leaves its range in LDS for the first barrier.
        int qmin = 0, qmax = 0;
        if (a.kind != 0) {
            int mn = rv ? qcode : INT_MAX, mx = rv ? qcode : INT_MIN;
            for (int o = 32; o >= 1; o >>= 1) {
                mn = min(mn, __shfl_xor(mn, o));
                mx = max(mx, __shfl_xor(mx, o));
            }
            if (kg == 0 && lane == 0) {
                qrange_s[0][wq] = mn;
                qrange_s[1][wq] = mx;
            }
        }

        bf16x8 qf[DK];
        {
            const uint16_t *qrow = a.q + ((long)(b * a.Hq + h) * a.M + j) * D;
            for (int kk = 0; kk < DK; ++kk) {
                if (rv) qf[kk] = *reinterpret_cast<const bf16x8 *>(qrow + kk * 16 + hh * 8);
                else qf[kk] = bf16x8{};
            }
        }

        const int k0 = split * split_keys;
        const int k1 = min(a.kv_len, k0 + split_keys);
        int kbeg = k0, kend = k1;        // the split's live tiles (set after the first barrier)
        const uint16_t *kbase = a.ck + (long)bg * a.n_cap * D;
        const uint16_t *vbase = a.cv + (long)bg * a.n_cap * D;
        const __amdgpu_buffer_rsrc_t krs = buffer_view(kbase, a.kv_len * ROWB);
        const __amdgpu_buffer_rsrc_t vrs = buffer_view(vbase, a.kv_len * ROWB);
        const float c2 = a.scale_log2;

        // Direct-load geometry of this thread: load u writes 16 bytes at LDS
        // byte (wid*NLD + u)*1024 + lane*16 of a tile, i.e. row lr, position lp.
        int ld_row[NLD], k_goff[NLD], v_goff[NLD];
        for (int u = 0; u < NLD; ++u) {
            const int byte = (wid * NLD + u) * 1024 + lane * 16;
            const int lr = byte / ROWB, lp = (byte % ROWB) / 16;
            ld_row[u] = lr;
            const int kkey = (lr & ~31) | ((lr & 19) | ((lr & 4) << 1) | ((lr & 8) >> 1));   // sigma(lr)
            k_goff[u] = (kkey * D + ((lp ^ k_swz<D>(lr)) * 8)) * 2;
            v_goff[u] = (lr * D + ((lp ^ v_swz<D>(lr)) * 8)) * 2;
        }
        // key_code from the slot codes staged in LDS: no global load, so the
        // only loads in flight in the tile loop are the tile loads themselves.
        auto key_code_lds = [&](int n) -> int {
            if (n >= a.kv_len) return INT_MAX;
            if (a.kind == 0 || n < a.P) return INT_MIN;
            const int sl = (n - a.P) / a.bs;
            if (a.kind == 1) return sl;
            return sl < a.n_slots ? scode_s[sl] : INT_MAX;
        };
        // Smallest and largest key code over keys [t0, t0 + len), keys at or
        // past kv_len counting as INT_MAX, from the staged slot codes (uniform
        // across the workgroup).  A group-mask range spanning more than eight
        // slots reports the widest range, i.e. a partial tile.
        auto key_range_lane = [&](int t0, int len, int &kmn, int &kmx) {
            const int hi = min(t0 + len, a.kv_len);
            kmn = INT_MAX;
            kmx = t0 + len > a.kv_len ? INT_MAX : INT_MIN;
            if (t0 < hi) {
                if (a.kind == 0 || t0 < a.P) kmn = INT_MIN;
                const int lo = max(t0, a.P);
                if (a.kind != 0 && lo < hi) {
                    const int s0 = (lo - a.P) / a.bs, s1 = (hi - 1 - a.P) / a.bs;
                    if (a.kind == 1) {
                        kmn = min(kmn, s0);
                        kmx = max(kmx, s1);
                    } else if (s1 - s0 >= 8) {
                        kmn = INT_MIN;
                        kmx = INT_MAX;
                    } else {
                        for (int sl = s0; sl <= s1; ++sl) {
                            const int c = sl < a.n_slots ? scode_s[sl] : INT_MAX;
                            kmn = min(kmn, c);
                            kmx = max(kmx, c);
                        }
                    }
                }
            }
        };
        auto key_range = [&](int t0, int len, int &kmn, int &kmx) {
            key_range_lane(t0, len, kmn, kmx);
            kmn = __builtin_amdgcn_readfirstlane(kmn);
            kmx = __builtin_amdgcn_readfirstlane(kmx);
        };
        // Direct loads of the K (with its key codes) or V half of the tile at t0
        // into LDS buffer buf.  In a partial block-causal or group tile, a row
        // whose key is hidden from every row of the workgroup (a DUMMY slot, a
        // later block or group) is not fetched: its out-of-range offset reads
        // zeros, and the predicate masks it anyway.  Other tiles take the plain
        // loop.
        auto issue_k = [&](int t0, int buf, bool part, int kslot) {
            uint16_t *ks = buf ? Ks1 : Ks0;
            if (part && a.kind != 0) {
                for (int u = 0; u < NLD; ++u) {
                    const int lr = ld_row[u];
                    const int kkey = (lr & ~31) | ((lr & 19) | ((lr & 4) << 1) | ((lr & 8) >> 1));
                    const int ko = key_code_lds(t0 + kkey) > qmax ? OOB : k_goff[u] + t0 * ROWB;
                    lds_void *kd = (lds_void *)(ks + (wid * NLD + u) * 512);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, ko, 0, 0, 0);
                }
            } else {
                // (the offsets are named variables: with the expression as the
                // builtin's argument, the host pass drops the kernel's stub)
                for (int u = 0; u < NLD; ++u) {
                    lds_void *kd = (lds_void *)(ks + (wid * NLD + u) * 512);
                    const int ko = k_goff[u] + t0 * ROWB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, ko, 0, 0, 0);
                }
            }
            if (part && tid < KT) kcode_s[kslot][tid] = key_code_lds(t0 + tid);
        };
        auto issue_v = [&](int t0, int buf, bool part) {
            uint16_t *vs = buf ? Vs1 : Vs0;
            if (part && a.kind != 0) {
                for (int u = 0; u < NLD; ++u) {
                    const int vo = key_code_lds(t0 + ld_row[u]) > qmax ? OOB : v_goff[u] + t0 * ROWB;
                    lds_void *vd = (lds_void *)(vs + (wid * NLD + u) * 512);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, 0, 0, 0);
                }
            } else {
                for (int u = 0; u < NLD; ++u) {
                    lds_void *vd = (lds_void *)(vs + (wid * NLD + u) * 512);
                    const int vo = v_goff[u] + t0 * ROWB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, 0, 0, 0);
                }
            }
        };

        // Loop-invariant LDS read offsets (elements) of this lane.
        int k_rd[DK];                                          // K chunk 2kk+hh of row l32
        for (int kk = 0; kk < DK; ++kk) k_rd[kk] = l32 * D + (((2 * kk + hh) ^ k_swz<D>(l32)) * 8);
        const int s16 = lane & 15, g16 = lane >> 4;
        int v_rd[DT];                                          // column tile dt, first row of the group
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (g16 & 1) + ((s16 & 3) >> 1);
            const int row = 8 * (g16 >> 1) + (s16 >> 2);      // row mod 4 = s16 / 4
            v_rd[dt] = row * D + ((chunk ^ v_swz<D>(row)) * 8) + (s16 & 1) * 4;
        }

        // Running max and sum; m_use is the exponent offset (the running max,
        // 0 before the lane's first visible key) and g_thr how far a tile's
        // max may pass it before O and l are rescaled (any finite max at the
        // first visible key, kRescaleLog2 afterwards).
        float m_run = -INFINITY, l_run = 0.f, m_use = 0.f, g_thr = -INFINITY;
        f32x16 o[DT];
        for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

        // O^T += V^T P^T over one 32-key sub-tile at vt: two transposed reads
        // give keys 16t + 8hh + (0..7) of column 32dt + l32 (operand A).
        auto pv_mfma = [&](const uint16_t *vt, int t, int dt, const bf16x8 &p) {
            const uint16_t *vp = vt + 16 * t * D + v_rd[dt];
            const s16x4 lo = lds_read_tr(vp);
            const s16x4 hi = lds_read_tr(vp + 4 * D);
            const s16x4 v8[2] = {lo, hi};
            o[dt] = mfma32(*reinterpret_cast<const bf16x8 *>(v8), p, o[dt]);
        };

        // S^T of this group's two 32-key sub-tiles of a tile (K at ks), the two
        // MFMA chains interleaved and the K fragments read two k-steps ahead.
        auto qk = [&](const uint16_t *ks, f32x16 &s0, f32x16 &s1) {
            s0 = f32x16{};
            s1 = f32x16{};
            bf16x8 r0[2], r1[2];
            for (int kk = 0; kk < 2 && kk < DK; ++kk) {
                r0[kk] = lds_frag(ks + k_rd[kk]);
                r1[kk] = lds_frag(ks + 32 * D + k_rd[kk]);
            }
            for (int kk = 0; kk < DK; ++kk) {
                const bf16x8 a0 = r0[kk & 1], a1 = r1[kk & 1];
                if (kk + 2 < DK) {
                    r0[kk & 1] = lds_frag(ks + k_rd[kk + 2]);
                    r1[kk & 1] = lds_frag(ks + 32 * D + k_rd[kk + 2]);
                }
                s0 = mfma32(a0, qf[kk], s0);
                s1 = mfma32(a1, qf[kk], s1);
            }
            // keep that order: 4 reads, then (2 MFMAs, 2 reads) ..., 4 MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, DK >= 2 ? 4 : 2, 0);
            for (int kk = 0; kk + 2 < DK; ++kk) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, DK >= 2 ? 4 : 2, 0);
        };

        // Mask, then the exponent arguments u = s * scale * log2(e) - m_use
        // (written over the scores) and their max: taking the max of FMA results rather than raw MFMA outputs
        // spares the NaN canonicalisation of every input.  The running max
        // moves only when the tile's max exceeds g_thr (more than kRescaleLog2
        // above it, or any visible key at the lane's first); then O and l are
        // rescaled and u shifted.
        auto prep = [&](f32x16 &s0, f32x16 &s1, const int *kc, bool all_vis) {
            if (!all_vis) {
                for (int i = 0; i < 16; ++i) {
                    const int key = 16 * (i >> 3) + 8 * hh + (i & 7);
                    if (kc[key] > qcode) s0[i] = -INFINITY;
                    if (kc[32 + key] > qcode) s1[i] = -INFINITY;
                }
            }
            f32x16 &u0 = s0, &u1 = s1;       // the arguments replace the scores in place
            for (int i = 0; i < 16; ++i) {
                u0[i] = fmaf(s0[i], c2, -m_use);
                u1[i] = fmaf(s1[i], c2, -m_use);
            }
            // the max of the 32 arguments as a tree of 3-input maxima (16 ops)
            float t1[12];
            for (int k = 0; k < 5; ++k) {
                t1[k] = max3f(u0[3 * k], u0[3 * k + 1], u0[3 * k + 2]);
                t1[5 + k] = max3f(u1[3 * k], u1[3 * k + 1], u1[3 * k + 2]);
            }
            t1[10] = u0[15];
            t1[11] = u1[15];
            const float t2[4] = {max3f(t1[0], t1[1], t1[2]), max3f(t1[3], t1[4], t1[5]), max3f(t1[6], t1[7], t1[8]),
                                 max3f(t1[9], t1[10], t1[11])};
            const float tmax = half_swap_max(fmaxf(max3f(t2[0], t2[1], t2[2]), t2[3]));
            const bool grow = tmax > g_thr;
            if (__any(grow)) {
                const float d = grow ? tmax : 0.f;                 // new max - m_use
                const float alpha = grow ? fast_exp2(m_run - (m_use + d)) : 1.f;   // 0 when m_run = -inf
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
                l_run *= alpha;
                if (grow) {
                    m_run = m_use + d;
                    m_use = m_run;
                    g_thr = kRescaleLog2;
                }
                for (int i = 0; i < 16; ++i) {
                    u0[i] -= d;
                    u1[i] -= d;
                }
            }
        };

        // The classes of the split's tiles (read once kbeg and kend are final),
        // 64 tiles at a time with one tile per lane: the slot-code reads run in
        // parallel and outside the tile pipeline, where a uniform LDS read would
        // wait for every LDS read in flight.  Bit i of window w, tile
        // kbeg + (64 w + i) KT: cls_part, partial for the workgroup (its loads
        // check rows); cls_vis / cls_live, this wave's keys of the tile are
        // visible to every row / to some row.  A tile is partial when it is not
        // visible to every row of the workgroup (a ragged tail, or block-causal
        // / group keys some row does not see): only partial tiles stage key
        // codes for the predicate and check their rows.
        unsigned long long cls_part = 0, cls_vis = 0, cls_live = 0;
        int cls_win = -1;
        auto tile_class = [&](int j, bool &part, bool &vis, bool &live) {
            const int w = j >> 6;
            if (w != cls_win) {
                const int t0 = kbeg + (64 * w + lane) * KT;
                bool pt = false, vs = true, lv = true;
                if (t0 < kend) {
                    int kmn, kmx;
                    key_range_lane(t0, KT, kmn, kmx);
                    pt = t0 + KT > a.P && kmx > qmin;
                    if (NG == 2) key_range_lane(t0 + kofs, 64, kmn, kmx);
                    const bool v0 = (a.kind == 0 && t0 + KT <= a.kv_len) || t0 + KT <= a.P;
                    vs = v0 || kmx <= qmin;
                    lv = v0 || kmn <= qmax;
                }
                cls_part = __ballot(pt);
                cls_vis = __ballot(vs);
                cls_live = __ballot(lv);
                cls_win = w;
            }
            part = (cls_part >> (j & 63)) & 1;
            vis = (cls_vis >> (j & 63)) & 1;
            live = (cls_live >> (j & 63)) & 1;
        };
        auto tile_part = [&](int j) -> bool {
            bool p, v, l;
            tile_class(j, p, v, l);
            return p;
        };
        // One tile: compute on LDS buffer BUF while tile t0 + KT streams into
        // the other one.  BUF is a compile-time constant, so the compiler sees
        // that the reads and the in-flight LDS loads touch different arrays and
        // does not wait for the loads before reading.  The PV products of
        // sub-tile 0 are interleaved with the exponentials of sub-tile 1.
        // Prefix tiles and whole in-range tiles of a full mask are visible to
        // every row; any other tile is classified by this key group's 64 keys:
        // skipped when hidden from every row, no predicate when visible to all.
        auto tile_step = [&](auto bufc, int t0) {
            constexpr int BUF = decltype(bufc)::value;
            const int j = (t0 - kbeg) / KT;
            if (t0 + KT < kend) {
                const bool part = tile_part(j + 1);
                issue_k(t0 + KT, BUF ^ 1, part, BUF ^ 1);
                issue_v(t0 + KT, BUF ^ 1, part);
            }
            bool part_, vis, live;
            tile_class(j, part_, vis, live);
            if (live) {
                const uint16_t *ks = (BUF ? Ks1 : Ks0) + kofs * D;
                const uint16_t *vs = (BUF ? Vs1 : Vs0) + kofs * D;
                f32x16 s0, s1;
                qk(ks, s0, s1);
                prep(s0, s1, kcode_s[BUF] + kofs, vis);
                const f32x16 &u0 = s0, &u1 = s1;
                float psum = 0.f;
                bf16x8 p0[2], p1[2];
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(u0[i]);
                    psum += p;
                    p0[i >> 3][i & 7] = (__bf16)p;
                }
                constexpr int PER = 16 / (2 * DT);   // exps of sub-tile 1 per PV product
                for (int q = 0; q < 2 * DT; ++q) {
                    pv_mfma(vs, q / DT, q % DT, p0[q / DT]);
                    for (int e = 0; e < PER; ++e) {
                        const int i = q * PER + e;
                        const float p = fast_exp2(u1[i]);
                        psum += p;
                        p1[i >> 3][i & 7] = (__bf16)p;
                    }
                }
                l_run += psum;
                for (int q = 0; q < 2 * DT; ++q) pv_mfma(vs + 32 * D, q / DT, q % DT, p1[q / DT]);
            }
            __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next tile landed
            __syncthreads();
        };

        __syncthreads();   // slot codes and the query waves' code ranges visible
        if (a.kind != 0) {
            qmin = INT_MAX;
            qmax = INT_MIN;
            for (int w = 0; w < QW; ++w) {
                qmin = min(qmin, qrange_s[0][w]);
                qmax = max(qmax, qrange_s[1][w]);
            }
            qmin = __builtin_amdgcn_readfirstlane(qmin);
            qmax = __builtin_amdgcn_readfirstlane(qmax);
        }
        // Leading and trailing tiles of the split that are hidden from every
        // row (later blocks or groups, DUMMY slots past the last live one) are
        // never visited: no loads, no MFMAs.  A hidden tile between live ones
        // is visited, but its rows are not fetched and its MFMAs are skipped.
        if (a.kind != 0) {
            int kmn, kmx;
            for (; kbeg < kend; kbeg += KT) {
                key_range(kbeg, KT, kmn, kmx);
                if (kmn <= qmax) break;
            }
            while (kend > kbeg) {
                const int tl = kbeg + (kend - 1 - kbeg) / KT * KT;   // start of the last tile
                key_range(tl, KT, kmn, kmx);
                if (kmn <= qmax) break;
                kend = tl;
            }
            kbeg = __builtin_amdgcn_readfirstlane(kbeg);
            kend = __builtin_amdgcn_readfirstlane(kend);
        }
        if constexpr (NG == 1 && kPingPong) {
            // Ping-pong.  Waves [0, QW/2) (group A) and [QW/2, QW) (group B) run
            // the same sequence of tiles one phase apart.  A phase is either all
            // MFMA (PV of tile j - 1 and QK of tile j) or all VALU (the softmax of
            // tile j), so on every SIMD one wave's matrix work overlaps the other
            // wave's vector work.  LDS slot j (buffer j % 2) holds K(j) and
            // V(j - 1): group A uses it in phase 2j, group B in phase 2j + 1;
            // slot j + 2 is loaded from the start of phase 2j + 2 and waited for
            // at the end of phase 2j + 3.  Key codes of partial tiles go to a
            // ring of four (tile j's are read up to phase 2j + 2).
            const int grp = wid >= QW / 2 ? 1 : 0;
            const int T = (kend - kbeg + KT - 1) / KT;
            f32x16 s0 = f32x16{}, s1 = f32x16{};   // S^T of the tile between its QK and softmax phases
            bf16x8 p0[2], p1[2];                   // P of the tile between its softmax and PV phases
            auto load_slot = [&](auto bufc, int js) __attribute__((always_inline)) {
                constexpr int SB = decltype(bufc)::value;
                if (js < T) {
                    const int t0 = kbeg + js * KT;
                    issue_k(t0, SB, tile_part(js), js & 3);
                }
                if (js >= 1 && js <= T) {
                    const int t0 = kbeg + (js - 1) * KT;
                    issue_v(t0, SB, tile_part(js - 1));
                }
            };
            auto mfma_phase = [&](auto bufc, int jq) __attribute__((always_inline)) {   // PV of tile jq - 1, QK of tile jq (slot jq)
                constexpr int SB = decltype(bufc)::value;
                const uint16_t *ks = SB ? Ks1 : Ks0;
                const uint16_t *vs = SB ? Vs1 : Vs0;
                if (jq >= 1 && jq <= T) {
                    for (int q = 0; q < 2 * DT; ++q) pv_mfma(vs, q / DT, q % DT, p0[q / DT]);
                    for (int q = 0; q < 2 * DT; ++q) pv_mfma(vs + 32 * D, q / DT, q % DT, p1[q / DT]);
                }
                if (jq < T) qk(ks, s0, s1);
            };
            auto softmax_phase = [&](int jq) __attribute__((always_inline)) {           // tile jq: P and the running max and sum
                if (jq >= T) return;
                bool part, vis, live;
                tile_class(jq, part, vis, live);
                prep(s0, s1, kcode_s[jq & 3], vis);
                float psum = 0.f;
                for (int i = 0; i < 16; ++i) {
                    const float e = fast_exp2(s0[i]);
                    psum += e;
                    p0[i >> 3][i & 7] = (__bf16)e;
                }
                for (int i = 0; i < 16; ++i) {
                    const float e = fast_exp2(s1[i]);
                    psum += e;
                    p1[i >> 3][i & 7] = (__bf16)e;
                }
                l_run += psum;
            };
            // Barriers ending a phase: after an even (global) phase the slot loads
            // issued at its start stay in flight; after an odd one they have
            // landed.
            auto bar_nowait = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0) only
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            };
            auto bar_wait = [&]() __attribute__((always_inline)) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            };
            load_slot(std::integral_constant<int, 0>{}, 0);
            load_slot(std::integral_constant<int, 1>{}, 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // Each group runs its own loop over local phases 2jq (MFMA, slot jq)
            // and 2jq + 1 (softmax of tile jq); group B is one phase behind, so
            // global phase p is A's phase p and B's phase p - 1.  Global phase
            // 2s - 2 (s >= 2) issues slot s: A at the start of its MFMA phase
            // s - 1, B at the start of its softmax phase s - 2.  Both groups end
            // after 2T + 2 barriers.  Unrolled by two tiles so every LDS buffer
            // index is a constant.
            if (grp == 0) {
                for (int jq = 0; jq <= T; jq += 2) {
                    if (jq >= 1) load_slot(std::integral_constant<int, 1>{}, jq + 1);
                    mfma_phase(std::integral_constant<int, 0>{}, jq);
                    bar_nowait();
                    softmax_phase(jq);
                    bar_wait();
                    if (jq + 1 > T) break;
                    load_slot(std::integral_constant<int, 0>{}, jq + 2);
                    mfma_phase(std::integral_constant<int, 1>{}, jq + 1);
                    bar_nowait();
                    softmax_phase(jq + 1);
                    bar_wait();
                }
            } else {
                bar_nowait();   // global phase 0
                for (int jq = 0; jq <= T; jq += 2) {
                    mfma_phase(std::integral_constant<int, 0>{}, jq);
                    bar_wait();
                    if (jq == T) break;
                    load_slot(std::integral_constant<int, 0>{}, jq + 2);
                    softmax_phase(jq);
                    bar_nowait();
                    mfma_phase(std::integral_constant<int, 1>{}, jq + 1);
                    bar_wait();
                    if (jq + 1 == T) break;
                    load_slot(std::integral_constant<int, 1>{}, jq + 3);
                    softmax_phase(jq + 1);
                    bar_nowait();
                }
            }
        } else {
            if (kbeg < kend) {
                const bool part = tile_part(0);
                issue_k(kbeg, 0, part, 0);
                issue_v(kbeg, 0, part);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            for (int t0 = kbeg; t0 < kend; t0 += 2 * KT) {
                tile_step(std::integral_constant<int, 0>{}, t0);
                if (t0 + KT < kend) tile_step(std::integral_constant<int, 1>{}, t0 + KT);
            }
        }

        // Finish the rows: with two key groups, the groups first merge their
        // (max, sum, O) through LDS, each then finishing half of every row's
        // columns -- group KG takes the lane's accumulator elements [KG H,
        // (KG + 1) H), H = 8 DT (whole groups of four: output column blocks)
        // and hands its other half to its partner.  Both evaluate the merge in
        // one operand order (group 0's term first), so their halves agree with
        // each other bitwise.  (The last tile step ended with a barrier and
        // issued no loads, so the tiles are free for the exchange.)  Then
        // normalise and write out/lse, or the split partial.
        const long rows_total = (long)a.B * a.Hq * a.M;
        constexpr int H = NG == 2 ? DT * 8 : DT * 16;     // elements a group finishes
        constexpr int Q4 = H / 4;                          // float4 per lane per half
        // Group KG hands the partner's half of O, and its (max, sum), to LDS.
        auto give = [&](auto kgc) {
            constexpr int KG = decltype(kgc)::value;
            constexpr int G0 = (1 - KG) * H;               // the partner's half
            float4 *dst = reinterpret_cast<float4 *>(KG == 0 ? Ks1 : Ks0) + wq * Q4 * 64;
            for (int e4 = 0; e4 < Q4; ++e4) {
                const int f = G0 + 4 * e4;
                const f32x16 &od = o[f / 16];
                dst[e4 * 64 + lane] = float4{od[f % 16], od[f % 16 + 1], od[f % 16 + 2], od[f % 16 + 3]};
            }
            ml_s[((KG * 2 + 0) * 4 + wq) * 64 + lane] = m_run;
            ml_s[((KG * 2 + 1) * 4 + wq) * 64 + lane] = l_run;
        };
        auto finish = [&](auto kgc) {
            constexpr int KG = decltype(kgc)::value;
            constexpr int E0 = KG * H, E1 = E0 + H;
            if constexpr (NG == 2) {
                const float4 *src = reinterpret_cast<const float4 *>(KG == 0 ? Ks0 : Ks1) + wq * Q4 * 64;
                const float mo = ml_s[(((1 - KG) * 2 + 0) * 4 + wq) * 64 + lane];
                const float lo = ml_s[(((1 - KG) * 2 + 1) * 4 + wq) * 64 + lane];
                const float mg0 = KG == 0 ? m_run : mo, mg1 = KG == 0 ? mo : m_run;   // group 0's, group 1's
                const float lg0 = KG == 0 ? l_run : lo, lg1 = KG == 0 ? lo : l_run;
                const float m = fmaxf(mg0, mg1);
                // a side whose max is the merged one (also both -inf) keeps scale 1
                const float a0 = mg0 == m ? 1.f : fast_exp2(mg0 - m);
                const float a1 = mg1 == m ? 1.f : fast_exp2(mg1 - m);
                for (int e4 = 0; e4 < Q4; ++e4) {
                    const float4 t = src[e4 * 64 + lane];
                    const float tv[4] = {t.x, t.y, t.z, t.w};
                    for (int c = 0; c < 4; ++c) {
                        const int f = E0 + 4 * e4 + c;
                        const float x = o[f / 16][f % 16];
                        o[f / 16][f % 16] = KG == 0 ? fmaf(x, a0, tv[c] * a1) : fmaf(tv[c], a0, x * a1);
                    }
                }
                l_run = fmaf(lg0, a0, lg1 * a1);
                m_run = m;
            }
            const float l_tot = l_run + __shfl_xor(l_run, 32);
            if (!rv) return;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const float row_lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
            const long row_flat = (long)(b * a.Hq + h) * a.M + j;
            if (ns == 1) {
                uint16_t *orow = a.out + row_flat * D;
                for (int dt = 0; dt < DT; ++dt)
                    for (int q4 = 0; q4 < 4; ++q4) {
                        if (dt * 16 + q4 * 4 < E0 || dt * 16 + q4 * 4 >= E1) continue;
                        __bf16 v4[4];
                        for (int c = 0; c < 4; ++c) v4[c] = (__bf16)(o[dt][q4 * 4 + c] * inv);
                        *reinterpret_cast<uint2 *>(orow + dt * 32 + q4 * 8 + hh * 4) =
                            *reinterpret_cast<const uint2 *>(v4);
                    }
                if (KG == 0 && hh == 0) a.lse[row_flat] = row_lse;
            } else {
                float *orow = a.ws_o + ((long)split * rows_total + row_flat) * D;
                for (int dt = 0; dt < DT; ++dt)
                    for (int q4 = 0; q4 < 4; ++q4) {
                        if (dt * 16 + q4 * 4 < E0 || dt * 16 + q4 * 4 >= E1) continue;
                        float4 v;
                        v.x = o[dt][q4 * 4 + 0] * inv;
                        v.y = o[dt][q4 * 4 + 1] * inv;
                        v.z = o[dt][q4 * 4 + 2] * inv;
                        v.w = o[dt][q4 * 4 + 3] * inv;
                        *reinterpret_cast<float4 *>(orow + dt * 32 + q4 * 8 + hh * 4) = v;
                    }
                if (KG == 0 && hh == 0) a.ws_l[(long)split * rows_total + row_flat] = row_lse;
            }
        };
        if constexpr (NG == 2) {
            if (kg == 0) give(std::integral_constant<int, 0>{});
            else give(std::integral_constant<int, 1>{});
            __syncthreads();
        }
        if (kg == 0) finish(std::integral_constant<int, 0>{});
        else if constexpr (NG == 2) finish(std::integral_constant<int, 1>{});

    __syncthreads();   // the LDS is free for the next item
    }
}

// Merge the key splits of each row in split order:
// lse = logsumexp_s lse_s, out = sum_s exp(lse_s - lse) out_s.
// One thread per 4 consecutive output elements of a row.  The lse and the
// partial outputs of the first kCombineBatch splits are loaded together
// into registers (one round trip); any further splits are read as they are
// used.  The arithmetic runs in split order either way.
constexpr int kCombineBatch = 8;

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a)
{
    constexpr int PER_ROW = D / 4;
    constexpr int RPB = 256 / PER_ROW;  // rows per block
    constexpr int NB = kCombineBatch;
    const long rows_total = (long)a.B * a.Hq * a.M;
    const int d4 = threadIdx.x % PER_ROW;
    // Merge the ns key splits of one row (fixed split order).
    auto combine_row = [&](long row, int ns) {
        const float *ls = a.ws_l + row;
        const float4 *os = reinterpret_cast<const float4 *>(a.ws_o + row * D) + d4;
        const long ostride = rows_total * PER_ROW;     // float4 between splits
        float lv[NB];
        float4 ov[NB];
        for (int s = 0; s < NB; ++s) {
            if (s < ns) {
                lv[s] = ls[s * rows_total];
                ov[s] = os[s * ostride];
            }
        }
        float m = -INFINITY;
        for (int s = 0; s < NB; ++s)
            if (s < ns) m = fmaxf(m, lv[s]);
        for (int s = NB; s < ns; ++s) m = fmaxf(m, ls[s * rows_total]);
        float4 res = {0.f, 0.f, 0.f, 0.f};
        float L = -INFINITY;
        if (m != -INFINITY) {
            float sum = 0.f;
            for (int s = 0; s < NB; ++s)
                if (s < ns) sum += fast_exp2((lv[s] - m) * kLog2e);
            for (int s = NB; s < ns; ++s) sum += fast_exp2((ls[s * rows_total] - m) * kLog2e);
            L = m + logf(sum);
            auto add = [&](float l, const float4 &v) {
                const float w = fast_exp2((l - L) * kLog2e);
                res.x = fmaf(w, v.x, res.x);
                res.y = fmaf(w, v.y, res.y);
                res.z = fmaf(w, v.z, res.z);
                res.w = fmaf(w, v.w, res.w);
            };
            for (int s = 0; s < NB; ++s)
                if (s < ns) add(lv[s], ov[s]);
            for (int s = NB; s < ns; ++s) add(ls[s * rows_total], os[s * ostride]);
        }
        __bf16 bv[4] = {(__bf16)res.x, (__bf16)res.y, (__bf16)res.z, (__bf16)res.w};
        reinterpret_cast<uint2 *>(a.out + row * D)[d4] = *reinterpret_cast<const uint2 *>(bv);
        if (d4 == 0) a.lse[row] = L;
    };
    if (!a.dyn_split) {   // planned split: one row per RPB-th of a workgroup
        const long row = (long)blockIdx.x * RPB + threadIdx.x / PER_ROW;
        if (row >= rows_total) return;
        const int b = (int)(row / ((long)a.Hq * a.M));
        if (a.m_valid && (int)(row % a.M) >= valid_rows(a, b)) return;
        const int ns = splits_for(a, b);
        if (ns > 1) combine_row(row, ns);   // with one split pass 1 wrote the row directly
        return;
    }
    // Device-decided split: a capped grid walks only the valid rows of the
    // batch entries that split (the same count pass 1 used), so the launch
    // shape stays static without a workgroup per row of the capacity.
    for (int b = 0; b < a.B; ++b) {
        const int ns = splits_for(a, b);
        const int mv = valid_rows(a, b);
        const long nb = ns > 1 ? (long)a.Hq * mv : 0;
        for (long i = (long)blockIdx.x * RPB + threadIdx.x / PER_ROW; i < nb; i += (long)gridDim.x * RPB) {
            const int h = (int)(i / mv), j = (int)(i - (long)h * mv);
            combine_row(((long)b * a.Hq + h) * a.M + j, ns);
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 2.  Workgroup = (b, kv-head g, row split, 256-key block); wave w owns
// keys [64w, 64w+64) of the block in registers for the whole pass.  It walks
// the (q-head of g, 32-row query tile) pairs of its slice of the counted rows
// as one sequence, double-buffered in LDS (tile t+1 is loaded straight into
// LDS while tile t is used), and writes one partial column sum per (q-head,
// row split).
// Rows past the slice or with lse = -inf get lse = +inf (weight 0).  Mask
// tiles: a wave whose 64 keys are hidden from every weighted row of a query
// tile skips the tile; one whose keys are visible to all of them adds
// without the predicate; otherwise the per-element predicate runs.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void colsum_kernel(AttnArgs a)
{
    constexpr int DK = D / 16;
    constexpr int ROWB = D * 2;                    // bytes per Q row
    constexpr int NQL = kCsRows * ROWB / 1024;     // 1-KB direct loads per Q tile
    constexpr int OOB = 0x7ffffff0;

    __shared__ __attribute__((aligned(1024))) uint16_t Qs0[kCsRows * D];
    __shared__ __attribute__((aligned(1024))) uint16_t Qs1[kCsRows * D];
    __shared__ __attribute__((aligned(16))) float lse2_s[2][kCsRows];
    __shared__ int qcode_s[2][kCsRows];
    __shared__ int qr_s[2][2];                     // each query tile's smallest / largest code
    __shared__ int range_s[2];
    __shared__ int grp_s[kMaxSlots];               // GROUP: slot -> group id
    __shared__ int kcs_s[kMaxSlots];               // GROUP: slot -> key code (INT_MAX: DUMMY)

    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
    if (a.kind == 2)
        for (int sl = tid; sl < a.n_slots; sl += 256) {
            const int gv = gr[sl];
            const bool dummy = st[sl] == 0;
            grp_s[sl] = gv;
            kcs_s[sl] = dummy ? INT_MAX : gv;
        }

    // Counted rows: active rows whose position lies in [cs_lo, cs_hi);
    // active_idx is ascending, so they are the index range [j_lo, j_hi).
    // Waves 0 and 1 find j_lo and j_hi with a 64-way search: each round
    // probes 64 evenly spaced entries of the remaining range at once, so
    // M <= 4096 takes two rounds of loads instead of log2(M) dependent ones.
    if (wid < 2) {
        const int target = wid == 0 ? a.cs_lo : a.cs_hi;
        int lo = 0, len = valid_rows(a, b);          // answer in [lo, lo + len]
        while (len > 0) {
            const int step = (len + 63) / 64;
            const int p = lo + lane * step;
            const bool below = p < lo + len && act[p] < target;
            const int c = __popcll(__ballot(below));   // probes below target: a prefix
            if (c == 0) {
                len = 0;
            } else {
                const int nlo = lo + (c - 1) * step + 1;
                const int nhi = min(lo + c * step, lo + len);
                lo = nlo;
                len = nhi - nlo;
            }
        }
        if (lane == 0) range_s[wid] = lo;
    }

    // This lane's two keys and their K fragments (zeros past kv_len).
    int key[2], kc[2];
    bf16x8 kf[2][DK];
    const uint16_t *kbase = a.ck + ((long)b * a.Hkv + g) * a.n_cap * D;
    const __amdgpu_buffer_rsrc_t krs = buffer_view(kbase, a.kv_len * D * 2);
    for (int ct = 0; ct < 2; ++ct) {
        key[ct] = kb * kCsKeys + wid * 64 + ct * 32 + l32;
        for (int kk = 0; kk < DK; ++kk) {
            const uint4 v = buffer_load16(krs, (key[ct] * D + kk * 16 + hh * 8) * 2);
            kf[ct][kk] = *reinterpret_cast<const bf16x8 *>(&v);
        }
    }
    const bool need_mask = a.kind != 0 && (kb + 1) * kCsKeys > a.P;
    __syncthreads();
    // the key codes from the slot table staged in LDS (no dependent global
    // loads between the K fragment loads)
    for (int ct = 0; ct < 2; ++ct) {
        const int n = key[ct];
        int c = INT_MIN;
        if (n >= a.kv_len) c = INT_MAX;
        else if (a.kind != 0 && n >= a.P) {
            const int sl = (n - a.P) / a.bs;
            c = a.kind == 1 ? sl : (sl < a.n_slots ? kcs_s[sl] : INT_MAX);
        }
        kc[ct] = c;
    }
    // This wave's key-code range (keys past kv_len are never written, so
    // they do not count): a query tile whose largest code is below it sees
    // none of the wave's keys (the wave skips the tile); one whose smallest
    // code is at least its top sees all of them (no predicate).
    int wkmin = INT_MAX, wkmax = INT_MIN;
    if (need_mask) {
        for (int ct = 0; ct < 2; ++ct)
            if (key[ct] < a.kv_len) {
                wkmin = min(wkmin, kc[ct]);
                wkmax = max(wkmax, kc[ct]);
            }
        for (int o = 32; o >= 1; o >>= 1) {
            wkmin = min(wkmin, __shfl_xor(wkmin, o));
            wkmax = max(wkmax, __shfl_xor(wkmax, o));
        }
        wkmin = __builtin_amdgcn_readfirstlane(wkmin);
        wkmax = __builtin_amdgcn_readfirstlane(wkmax);
    }
    const int j_lo = range_s[0], j_hi = range_s[1];
    const int cnt = max(0, j_hi - j_lo);
    const int per = ((cnt + a.n_rsplit - 1) / a.n_rsplit + kCsRows - 1) / kCsRows * kCsRows;
    const int r0 = min(j_hi, j_lo + rs * per);
    const int r1 = min(j_hi, r0 + per);
    const int tiles_h = (r1 - r0 + kCsRows - 1) / kCsRows;     // query tiles per q-head
    const int n_tiles = tiles_h * a.G;

    // Q tiles go straight into LDS (1-KB buffer loads with the LDS
    // destination; wave w issues loads w, w + 4, ...), with the chunk
    // swizzle of pass 1's K tiles so that the fragment reads are
    // conflict-free; rows at or past r1 read as zeros.  The per-row lse and
    // query code take the register path (threads 0-31).
    // Raw per-row values of the tile in flight (loaded when the tile is
    // issued, turned into LDS entries only after the tile's compute, so no
    // wait sits at the start of a tile).
    float lraw = -INFINITY;
    int praw = 0;
    auto tile_rows = [&](int t, int &rb, long &hrow) {
        const int hl = t / tiles_h;
        rb = r0 + (t - hl * tiles_h) * kCsRows;
        hrow = ((long)b * a.Hq + g * a.G + hl) * a.M;
    };
    // This thread's loads of a tile (load u = wid + 4 i): the tile row and
    // its byte offset within the tile, fixed for the whole pass.
    constexpr int NQW = (NQL + 3) / 4;
    int q_lr[NQW], q_goff[NQW];
    for (int i = 0; i < NQW; ++i) {
        const int byte = (wid + 4 * i) * 1024 + lane * 16;
        const int lr = byte / ROWB, lp = (byte % ROWB) / 16;
        q_lr[i] = lr;
        q_goff[i] = (lr * D + ((lp ^ k_swz<D>(lr)) * 8)) * 2;
    }
    auto issue_q = [&](int t, int buf) {
        int rb;
        long hrow;
        tile_rows(t, rb, hrow);
        const __amdgpu_buffer_rsrc_t qrs = buffer_view(a.q + hrow * D, r1 * ROWB);
        uint16_t *qs = buf ? Qs1 : Qs0;
        for (int i = 0; i < NQW; ++i) {
            const int u = wid + 4 * i;
            if (u < NQL) {
                const int off = rb + q_lr[i] < r1 ? rb * ROWB + q_goff[i] : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void *)(qs + u * 512), 16, off, 0, 0, 0);
            }
        }
        if (tid < kCsRows) {
            const int jr = rb + tid;
            lraw = jr < r1 ? a.lse[hrow + jr] : -INFINITY;
            praw = (jr < r1 && need_mask) ? act[jr] : 0;
        }
    };
    // lse in log2 units, +inf (weight 0) for a row past the slice or
    // without a visible key; the row's mask code from the staged slot table,
    // and the code range of the tile's weighted rows (wave 0; its lanes past
    // kCsRows hold no row).
    auto store_rows = [&](int buf) {
        if (wid == 0) {
            const bool ok = lraw != -INFINITY;
            int qc = 0;
            if (need_mask) {
                const int sl = (praw - a.P) / a.bs;
                qc = a.kind == 1 ? sl : (sl >= 0 && sl < a.n_slots ? grp_s[sl] : INT_MIN);
            }
            if (tid < kCsRows) {
                lse2_s[buf][tid] = ok ? lraw * kLog2e : INFINITY;
                qcode_s[buf][tid] = ok ? qc : INT_MIN;
            }
            if (need_mask) {
                int mn = ok ? qc : INT_MAX, mx = ok ? qc : INT_MIN;
                for (int o = 32; o >= 1; o >>= 1) {
                    mn = min(mn, __shfl_xor(mn, o));
                    mx = max(mx, __shfl_xor(mx, o));
                }
                if (lane == 0) {
                    qr_s[buf][0] = mn;
                    qr_s[buf][1] = mx;
                }
            }
        }
    };
    int q_rd[DK];                                        // Q chunk 2kk+hh of row l32
    for (int kk = 0; kk < DK; ++kk) q_rd[kk] = l32 * D + (((2 * kk + hh) ^ k_swz<D>(l32)) * 8);

    float acc[2] = {0.f, 0.f};
    // One query tile on LDS buffer BUF while tile t + 1 streams into the
    // other (BUF a compile-time constant: the compiler sees the reads and
    // the in-flight loads touch different arrays).
    auto tile = [&](auto bufc, int t) {
        constexpr int BUF = decltype(bufc)::value;
        const bool more = t + 1 < n_tiles;
        if (more) issue_q(t + 1, BUF ^ 1);
        const uint16_t *qs = BUF ? Qs1 : Qs0;
        bool run = true, masked = false;
        if (need_mask) {
            run = wkmin <= __builtin_amdgcn_readfirstlane(qr_s[BUF][1]);
            masked = wkmax > __builtin_amdgcn_readfirstlane(qr_s[BUF][0]);
        }
        if (run) {
            f32x16 s0 = f32x16{}, s1 = f32x16{};
            for (int kk = 0; kk < DK; ++kk) {
                const bf16x8 qa = lds_frag(qs + q_rd[kk]);
                s0 = mfma32(qa, kf[0][kk], s0);
                s1 = mfma32(qa, kf[1][kk], s1);
            }
            // element i of this lane is query row 8*(i/4) + 4*hh + i%4 of the tile
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 l2 = *reinterpret_cast<const float4 *>(&lse2_s[BUF][8 * q4 + 4 * hh]);
                const float lv[4] = {l2.x, l2.y, l2.z, l2.w};
                if (!masked) {
                    for (int e = 0; e < 4; ++e) {
                        acc[0] += fast_exp2(fmaf(s0[q4 * 4 + e], a.scale_log2, -lv[e]));
                        acc[1] += fast_exp2(fmaf(s1[q4 * 4 + e], a.scale_log2, -lv[e]));
                    }
                } else {
                    for (int e = 0; e < 4; ++e) {
                        const int qc = qcode_s[BUF][8 * q4 + 4 * hh + e];
                        const float p0 = fast_exp2(fmaf(s0[q4 * 4 + e], a.scale_log2, -lv[e]));
                        const float p1 = fast_exp2(fmaf(s1[q4 * 4 + e], a.scale_log2, -lv[e]));
                        acc[0] += kc[0] <= qc ? p0 : 0.f;
                        acc[1] += kc[1] <= qc ? p1 : 0.f;
                    }
                }
            }
        }
        if (more) store_rows(BUF ^ 1);
        if (t % tiles_h == tiles_h - 1) {
            // last tile of a q-head: write its partial column sums
            const int h = g * a.G + t / tiles_h;
            for (int ct = 0; ct < 2; ++ct) {
                const float tot = acc[ct] + __shfl_xor(acc[ct], 32);
                if (hh == 0 && key[ct] < a.kv_len)
                    a.ws_cs[(((long)b * a.Hq + h) * a.n_rsplit + rs) * a.kv_len + key[ct]] = tot;
                acc[ct] = 0.f;
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // this thread's loads of the next tile landed
        __syncthreads();
    };

    if (n_tiles > 0) {
        issue_q(0, 0);
        store_rows(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; t += 2) {
        tile(std::integral_constant<int, 0>{}, t);
        if (t + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, t + 1);
    }
    if (n_tiles == 0) {
        // no counted rows in this slice: zero partials for every q-head
        for (int hl = 0; hl < a.G; ++hl)
            for (int ct = 0; ct < 2; ++ct)
                if (hh == 0 && key[ct] < a.kv_len)
                    a.ws_cs[(((long)b * a.Hq + g * a.G + hl) * a.n_rsplit + rs) * a.kv_len + key[ct]] = 0.f;
    }
}

// colsum[b, n] = sum_h sum_rs part[b, h, rs, n] (or per head: sum_rs); with
// accumulate, added to what colsum holds.
// Workgroup = (256 / SL) consecutive columns of one (b, h-or-all) x SL
// slices; slice q sums partials s = q, q + SL, ... with eight independent
// accumulators (eight loads in flight per thread), and the slices are then
// added in a fixed tree order: the result depends on the shape only, so it
// is bitwise reproducible.  SL = 16 when there are many partials per column
// (all heads), 1 when there are few (per head).
template <int SL>
__global__ __launch_bounds__(256) void colsum_reduce_kernel(AttnArgs a)
{
    constexpr int CW = 256 / SL;             // columns per workgroup
    constexpr int U = 8;
    __shared__ float part_s[SL][CW];
    const int nblk = (a.kv_len + CW - 1) / CW;
    const int bh = blockIdx.x / nblk;        // (b, h) or b
    const int c = threadIdx.x % CW, q = threadIdx.x / CW;
    const int n = (blockIdx.x - bh * nblk) * CW + c;
    const int S = a.per_head ? a.n_rsplit : a.Hq * a.n_rsplit;
    float acc[U];
    for (int u = 0; u < U; ++u) acc[u] = 0.f;
    if (n < a.kv_len) {
        const float *p = a.ws_cs + (long)bh * S * a.kv_len + n;
        for (int s0 = q; s0 < S; s0 += U * SL) {
            float v[U];
            for (int u = 0; u < U; ++u) {
                const int s = s0 + u * SL;
                v[u] = s < S ? p[(long)s * a.kv_len] : 0.f;
            }
            for (int u = 0; u < U; ++u) acc[u] += v[u];
        }
    }
    const float mine = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    if (SL == 1) {
        if (n < a.kv_len) {
            float *c = a.colsum + (long)bh * a.kv_len + n;
            *c = a.accumulate ? *c + mine : mine;
        }
        return;
    }
    part_s[q][c] = mine;
    __syncthreads();
    if (q == 0 && n < a.kv_len) {
        float t[SL];
        for (int k = 0; k < SL; ++k) t[k] = part_s[k][c];
        for (int w = SL / 2; w >= 1; w >>= 1)
            for (int k = 0; k < w; ++k) t[k] = t[k] + t[k + w];
        float *c = a.colsum + (long)bh * a.kv_len + n;
        *c = a.accumulate ? *c + t[0] : t[0];
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, long n)
{
    long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t < n) p[t] = 0.f;
}

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, hipStream_t stream, hipEvent_t pass1_done)
{
    if (a.M > 0 && a.k != nullptr) {
        const long nblk = ((long)a.M * (D / 8) + 255) / 256 * a.B * a.Hkv;
        const long grid = nblk < kScatterWgs ? nblk : kScatterWgs;
        kv_scatter_kernel<D><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
    }
    if (a.M == 0) {
        if (pass1_done) {
            const hipError_t e = hipEventRecord(pass1_done, stream);
            if (e != hipSuccess) return e;
        }
        if (a.colsum && !a.accumulate) {
            long n = (long)a.B * (a.per_head ? a.Hq : 1) * a.kv_len;
            fill_zero_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a.colsum, n);
        }
        return hipGetLastError();
    }
    {
        long nwg = (long)a.B * a.Hkv * a.n_split * a.n_qtiles;
        if (a.dyn_split) {
            // persistent: one workgroup per CU walks the items the row counts ask for
            nwg = min(nwg, (long)kNumCU);
            if (a.n_kgroups == 2)
                attn_fwd_kernel<D, 2, 4, true><<<dim3((unsigned)nwg), dim3(512), 0, stream>>>(a);
            else
                attn_fwd_kernel<D, 1, qwaves1(D), true><<<dim3((unsigned)nwg), dim3(64 * qwaves1(D)), 0, stream>>>(a);
        } else if (a.n_kgroups == 2) {
            attn_fwd_kernel<D, 2, 4, false><<<dim3((unsigned)nwg), dim3(512), 0, stream>>>(a);
        } else {
            attn_fwd_kernel<D, 1, qwaves1(D), false><<<dim3((unsigned)nwg), dim3(64 * qwaves1(D)), 0, stream>>>(a);
        }
    }
    if (a.n_split > 1) {
        const long rows = (long)a.B * a.Hq * a.M;
        constexpr int RPB = 256 / (D / 4);
        long nblk = (rows + RPB - 1) / RPB;
        if (a.dyn_split && nblk > 2L * kNumCU) nblk = 2L * kNumCU;   // the walk covers the rest
        attn_combine_kernel<D><<<dim3((unsigned)nblk), dim3(256), 0, stream>>>(a);
    }
    if (pass1_done) {
        const hipError_t e = hipEventRecord(pass1_done, stream);
        if (e != hipSuccess) return e;
    }
    if (a.colsum) {
        long nwg = (long)a.B * a.Hkv * a.n_rsplit * a.n_kblocks;
        colsum_kernel<D><<<dim3((unsigned)nwg), dim3(256), 0, stream>>>(a);
        const long nbh = (long)a.B * (a.per_head ? a.Hq : 1);
        const int S = a.per_head ? a.n_rsplit : a.Hq * a.n_rsplit;
        if (S >= 32)
            colsum_reduce_kernel<16><<<dim3((unsigned)(nbh * ((a.kv_len + 15) / 16))), dim3(256), 0, stream>>>(a);
        else
            colsum_reduce_kernel<1><<<dim3((unsigned)(nbh * ((a.kv_len + 255) / 256))), dim3(256), 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_attn(const AttnArgs &a, hipStream_t stream, hipEvent_t pass1_done)
{
    switch (a.D) {
    case 32: return launch_attn_d<32>(a, stream, pass1_done);
    case 64: return launch_attn_d<64>(a, stream, pass1_done);
    case 128: return launch_attn_d<128>(a, stream, pass1_done);
    default: return hipErrorInvalidValue;
    }
}

AttnPlan plan_attn(int B, int Hq, int Hkv, int D, int M, int kv_len, int n_cap, bool dyn)
{
    AttnPlan p{};
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.D = D; p.M = M;
    p.kv_len = kv_len; p.n_cap = n_cap;
    p.n_qtiles = (p.G * M + kAttnRows - 1) / kAttnRows;
    long base = (long)B * Hkv * p.n_qtiles;
    // Enough query tiles for two 4-wave workgroups per CU: one key group,
    // and the two workgroups on a CU keep their own barriers (one can run
    // its softmax while the other runs MFMAs).  Fewer: two key groups per
    // workgroup (8 waves), and split the keys until there are
    // kAttnWgTarget workgroups, keeping at least 1024 keys per split:
    // shorter splits lose more to the split merge than they gain in
    // parallelism (measured on MI355X).
    p.n_kgroups = base >= 2L * kNumCU ? 1 : 2;
    // A planned launch whose two-key-group shape would split the keys (so
    // pays the split merge anyway) takes one key group of 32 * qwaves1 rows
    // with about twice the splits when that gives at least as many
    // workgroups: each K/V chunk is then read by half as many workgroups
    // (measured on MI355X: the long-prefix pass 1, 256 rows over 16640 keys,
    // 96 -> 90 us; the multi-block one, which needs no split, keeps two key
    // groups).
    if (!dyn && p.n_kgroups == 2 && qwaves1(D) != 4 && base > 0 && base < kAttnWgTarget) {
        auto wgs_for = [&](long bs, int tl) {
            const int kt = (kv_len + tl - 1) / tl;
            const long sp = min((kAttnWgTarget + bs - 1) / bs, (long)max(1, kt / (1024 / tl)));
            return bs * sp;
        };
        const long base1 = (long)B * Hkv * ((p.G * M + 32 * qwaves1(D) - 1) / (32 * qwaves1(D)));
        if (wgs_for(base1, 64) >= wgs_for(base, 128)) p.n_kgroups = 1;
    }
    // DLM_ATTN_KGROUPS=1 or 2 forces the workgroup shape (tests and tuning;
    // the workspace query must see the same setting as the call).
    if (const char *e = getenv("DLM_ATTN_KGROUPS")) {
        if (e[0] == '1' && e[1] == 0) p.n_kgroups = 1;
        if (e[0] == '2' && e[1] == 0) p.n_kgroups = 2;
    }
    if (p.n_kgroups == 1 && qwaves1(D) != 4) {   // one key group: query tiles of 32 * qwaves1 rows
        p.n_qtiles = (p.G * M + 32 * qwaves1(D) - 1) / (32 * qwaves1(D));
        base = (long)B * Hkv * p.n_qtiles;
    }
    const int tile = 64 * p.n_kgroups;
    const int key_tiles = (kv_len + tile - 1) / tile;
    int split = 1;
    if (base > 0 && base < kAttnWgTarget) {
        split = (int)((kAttnWgTarget + base - 1) / base);
        split = min(split, max(1, key_tiles / (1024 / tile)));
    }
    // With a device row count the launch is sized for the most splits a
    // batch entry may take (one key tile each, at most kMaxDynSplit) and
    // each workgroup derives its entry's count from the row count
    // (splits_for): workgroups of unused splits leave at once, so the
    // launch shape stays static (graph capture) while pass 1 follows M_t.
    p.dyn_split = dyn && split == 1 && key_tiles > 1 ? 1 : 0;
    if (p.dyn_split) split = min(key_tiles, kMaxDynSplit);
    int tiles_per = (key_tiles + split - 1) / split;
    p.split_keys = max(1, tiles_per) * tile;
    p.n_split = max(1, (kv_len + p.split_keys - 1) / p.split_keys);
    if (p.dyn_split && p.n_split == 1) p.dyn_split = 0;
    p.rows_wg = p.n_kgroups == 2 ? kAttnRows : 32 * qwaves1(D);
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
