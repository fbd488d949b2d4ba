// dlm_internal.h -- types, tile constants, launch plans and kernel-launch
// declarations shared by the HIP sources of libdlm_step.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dlm {

// MFMA operand / accumulator types (gfx950 v_mfma_f32_32x32x16_bf16).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNumCU = 256;          // MI355X: 256 CUs in 8 XCDs
constexpr int kNumXCD = 8;
constexpr int kAttnRows = 128;       // query rows per pass-1 workgroup (4 query waves x 32)
#ifndef DLM_ATTN_WG_TARGET
#define DLM_ATTN_WG_TARGET 256
#endif
constexpr long kAttnWgTarget = DLM_ATTN_WG_TARGET;  // 8-wave pass-1 workgroups wanted (1 per CU)
constexpr int kMaxDynSplit = 8;      // key splits pass 1 may take with a device row count
constexpr int kCsKeys = 256;         // keys per column-sum workgroup (4 waves x 64)
constexpr int kCsRows = 32;          // query rows per column-sum tile
constexpr int kMaxSlots = 1024;      // GROUP: slots per batch entry
constexpr int kMaxGroupRows = 1024;  // posterior selection group
constexpr int kPostThreads = 256;
constexpr int kPostVec = 4 * 4;      // floats per thread per streaming step (4 x float4)

// Launch plan of dlm_step_attn, a pure function of the shapes.
struct AttnPlan {
    int B, Hq, Hkv, G, D, M, kv_len, n_cap;
    int n_qtiles;       // query tiles of kAttnRows packed rows per (b, kv-head)
    int n_kgroups;      // key groups per pass-1 workgroup (1: 4 waves, 2: 8 waves)
    int n_split;        // key splits of pass 1 (with dyn: the most a batch entry may use)
    int dyn_split;      // 1: the split count follows the device row count
    int rows_wg;        // packed query rows per pass-1 workgroup
    int split_keys;     // keys per split (multiple of the 64 * n_kgroups key tile)
    int n_kblocks;      // column-sum key blocks of kCsKeys
    int n_rsplit;       // column-sum row splits
    size_t ws_split_o;  // bytes of split partial outputs (fp32)
    size_t ws_split_l;  // bytes of split partial lse (fp32)
    size_t ws_colsum;   // bytes of column-sum partials (fp32)
    size_t ws_total;
};
// dyn: a device row count (m_active) is given; pass 1 then plans for the
// largest key split and picks each batch entry's split count on the device.
AttnPlan plan_attn(int B, int Hq, int Hkv, int D, int M, int kv_len, int n_cap, bool dyn = false);

// Per-row partial state of the posterior stream over one vocabulary chunk
// (48 bytes: staged through LDS in 16-byte pieces).
struct PostPartial {
    float mx;   // running max of logits x
    float sx;   // sum exp(x - mx)
    float tx;   // sum exp(x - mx) * (x - y)
    float my;   // running max of previous logits y
    float sy;   // sum exp(y - my)
    float av;   // largest x seen
    float a2;   // runner-up: largest x at any other index (= av on a tie)
    float ex;   // sum exp(x - mx) * (x - mx)
    int ai;     // lowest index attaining av
    int pad[3];
};
static_assert(sizeof(PostPartial) % 16 == 0, "partials are staged in 16-byte pieces");

// A row's results handed from the workgroup that finishes the row to the
// one that runs its selection group (single-launch path).
struct PostRowRes {
    float key;  // ranking key: conf, margin or -entropy
    float conf;
    int tok;    // lowest argmax
    int lock;   // the lock decision of this step
};

struct PostPlan {
    int n_chunks;       // vocabulary chunks per row
    int chunk;          // elements per chunk (multiple of 4)
    int group_rows;     // rows per finishing workgroup
    int fused;          // 1: one launch (stream + row merge + selection)
    size_t off_part;    // workspace offset of the partials
    size_t off_rowres, off_row_cnt, off_grp_cnt;   // fused: workspace offsets
    size_t ws_total;
};
// The counter block at the start of every posterior workspace: row
// counters, then selection-group counters, kPostMaxCounters of each.
constexpr int kPostMaxCounters = 4096;
constexpr size_t kPostCounterBytes = 2 * kPostMaxCounters * sizeof(unsigned);
// live: with a device live-row list (dlm_select.live_rows); the plan then
// sizes the partials for the largest split and n_chunks is that cap.
// fused: the single-launch path when the shapes allow it (no live-row
// list, selection groups of at most 256 rows).
PostPlan plan_post(int R, int V, int mode, int group_rows, bool live = false, bool fused = false);
// Workspace bytes a call needs: enough for either path.
size_t post_ws_bytes(int R, int V, int mode, int group_rows, bool live);

struct AttnArgs {
    const uint16_t *q, *k, *v;      // bf16 bit patterns
    uint16_t *ck, *cv;
    const int32_t *active_idx;
    const uint8_t *slot_state;
    const int32_t *slot_group;
    uint16_t *out;
    float *lse, *colsum;
    float *ws_o, *ws_l, *ws_cs;
    const int32_t *m_valid;         // optional device [B]: rows of batch b that are valid
    int B, Hq, Hkv, G, D, M, n_cap, kv_len, P, bs, n_slots, kind;
    int cs_lo, cs_hi, per_head, accumulate;
    float scale_log2;               // softmax scale * log2(e)
    int n_qtiles, n_kgroups, n_split, split_keys, n_kblocks, n_rsplit;
    int dyn_split, rows_wg;         // device-decided key split (see plan_attn)
};

struct PostArgs {
    const float *x, *y;
    uint8_t *locked;
    const float *score;
    int32_t *sel;
    float *kl, *conf;
    float *margin, *entropy;        // optional outputs (nullptr: not written)
    const uint8_t *flags;           // optional [R]: bit 0 selectable, bit 1 lockable
    PostPartial *part;
    int R, V, mode, k, group_rows;
    float eps, tau, conf_gate;
    int n_chunks, chunk;
    // optional live-row list: live_rows[i] - live_offset for i < *n_live
    // are the rows that may arrive unlocked; the split of the vocabulary is
    // then chosen on the device from the count (at most nc_cap chunks)
    const int32_t *live_rows, *n_live;
    int live_offset, nc_cap;
    // single-launch path: per-row results and the arrival counters (zero
    // between calls: the last arrival resets its counter)
    PostRowRes *rowres;
    unsigned *row_cnt, *grp_cnt;
};

// Block Buffer state of a multi-step run (device arrays, see dlm_step.h).
struct BBArgs {
    uint8_t *state;
    int32_t *group;
    uint8_t *decoded;
    int32_t *tokens;
    uint8_t *locked, *skip, *flags;
    int32_t *active_idx, *m_active, *n_open;
    const int32_t *sel;             // nullptr: initialise instead of advancing
    int B, n_slots, bs, max_active, P, n_gen;
};

// One active-row product C = A W^T with its epilogue (gemm_kernels.hip).
struct GemmArgs {
    const uint16_t *a;              // A rows: see a_mode
    long a_bytes;                   // size of the A tensor (loads past it read zero)
    const int32_t *act;             // active_idx [B, M] (gather modes)
    const int32_t *m_valid;         // optional device [B] row counts
    const uint16_t *w0, *w1;        // W [N, K]; w1: the up matrix of SwiGLU (else nullptr)
    int w_packed;                   // 1: W in the fragment-packed layout of dlm_pack_weights
    uint16_t *out, *out_k, *out_v;  // outputs (QKV: q, k, v)
    const uint16_t *resid;          // residual rows (EP_RESID, EP_SCATTER)
    int a_mode;                     // 0 plain [B*M, K], 1 gather x[b, act, :], 2 heads out[b, h, j, d],
                                    // 3 packed 16-row operand fragments (at most 16 rows)
    int ep_mode;                    // 0 plain / SwiGLU, 1 QKV, 2 residual to compact rows, 3 residual scattered to x
    int resid_gather;               // residual row: 1 x[b, act[b, j]], 0 resid[b * M + j]
    int out_packed;                 // SwiGLU, at most 16 rows: write the gated rows as packed fragments
    int B, M, K, N, n_pos, Hq, Hkv, D;
    int splits, kc;                 // K splits of kc columns each (1: one pass, fused epilogue)
    float *part;                    // splits > 1: fp32 partial sums [splits, B*M, N (2N for SwiGLU)]
};
struct GemmPlan {
    int splits, kc;
    size_t part_bytes;
};
GemmPlan plan_gemm(int rows, int N, int K, bool swiglu);
bool gemm_skinny(int rows);         // rows handled by the weight-streaming kernel (a_mode 3 / out_packed)
// The A rows of a skinny product (a_mode 0-2) as packed fragments: 16 K bf16 at dst.
hipError_t launch_pack_rows(const GemmArgs &a, uint16_t *dst, hipStream_t stream);

// The right-to-left selective scan of one step (r2l_kernels.hip).
struct R2LArgs {
    const uint16_t *u, *delta, *Bm, *Cm;   // bf16 [B, L, E], [B, L, E], [B, L, N], [B, L, N]
    const float *A, *D;                    // [E, N], [E]
    float *y;                              // optional fp32 [B, L, E] out
    uint16_t *x;                           // optional bf16 [B, L, E] in/out (x += y)
    int B, L, E, N;
    float gate;
};

// Valid rows of batch entry b: all M unless a device count is given.
__device__ __forceinline__ int valid_rows(const AttnArgs &a, int b)
{
    return a.m_valid ? min(max(a.m_valid[b], 0), a.M) : a.M;
}

// Key splits pass 1 uses for batch entry b: the planned count, or with a
// device row count, enough splits (at most the planned n_split) that the
// workgroups of a batch like this one would number about kAttnWgTarget.
// Pass 1 and the split merge evaluate the same function.
__device__ __forceinline__ int splits_for(const AttnArgs &a, int b)
{
    if (!a.dyn_split) return a.n_split;
    const long wgs = (long)a.B * a.Hkv * ((a.G * valid_rows(a, b) + a.rows_wg - 1) / a.rows_wg);
    if (wgs >= kAttnWgTarget) return 1;
    return (int)min((long)a.n_split, (kAttnWgTarget + max(wgs, 1L) - 1) / max(wgs, 1L));
}

// Enqueue the kernels of one call (arguments already validated).
hipError_t launch_step_attn(const AttnArgs &a, hipStream_t stream, hipEvent_t pass1_done);
hipError_t launch_posterior(const PostArgs &a, hipStream_t stream, hipEvent_t finish_after);
hipError_t launch_block_buffer(const BBArgs &a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);
// Row-major bf16 W [N, K] -> the fragment-packed layout (N % 16 == 0, K % 32 == 0).
hipError_t launch_pack_weights(const uint16_t *w, uint16_t *packed, int N, int K, hipStream_t stream);
hipError_t launch_r2l(const R2LArgs &a, hipStream_t stream);

// ---- direct global-to-LDS loads ------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor of a byte range: base address, stride 0, size in bytes
// (16-byte loads at offsets at or past it return zeros), raw 32-bit format.
__device__ __forceinline__ i32x4 dma_view(const void *base, long bytes)
{
    const unsigned long long p = (unsigned long long)base;
    return i32x4{(int)(unsigned)p, (int)((unsigned)(p >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Each lane loads 16 bytes at byte offset voff of the view into LDS at
// lds + 16 * lane (lds the same for the whole wave).  The load is issued
// from inline assembly and has no register result: the compiler neither
// tracks it nor adds waits for it, so every wait for these loads is the
// caller's (dma_wait_barrier, or a final vmcnt(0)), and the "memory"
// clobber keeps the compiler from moving LDS accesses across the issue.
// The compiler's hazard checks do not see inside the block, so it starts
// with the wait states the hardware needs between a write of M0 (one) or a
// VALU write of an SGPR (five) and a vector memory instruction reading it.
__device__ __forceinline__ void dma16(i32x4 view, int voff, const void *lds)
{
    typedef __attribute__((address_space(3))) const void lds_cvoid;
    const int m0 = __builtin_amdgcn_readfirstlane((int)(size_t)(lds_cvoid *)lds);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(view), "{m0}"(m0)
                 : "memory");
}

// Stage boundary of a ring of LDS tiles filled by dma16: wait until at
// most N vector-memory operations of this wave are outstanding (they
// complete in issue order, so the loads of the tile about to be read have
// landed) and all its LDS operations are done, then the workgroup barrier.
// The "memory" clobber keeps the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void dma_wait_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Map a hardware workgroup id to a logical one so that logically
// consecutive workgroups (which share K/V) run on the same XCD: the
// dispatcher deals workgroups round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int hw, int n)
{
    int per = n / kNumXCD, rem = n % kNumXCD;
    int x = hw % kNumXCD, kth = hw / kNumXCD;
    return x * per + (x < rem ? x : rem) + kth;
}

}  // namespace dlm
