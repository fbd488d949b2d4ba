// loop_kernels.hip -- the Block Buffer of a multi-step denoising run on gfx950.
//
// One kernel, one workgroup of 1024 threads per batch entry, does all the
// per-step bookkeeping between two steps on the device, so that a run
// needs no host round trip and every step has the same launch shapes:
//   1. the step's results for rows of active slots: a selected row is
//      unmasked (decoded, its token stored); a row the posterior locked
//      stays locked (SureLock page, sec. 2: its computation stops);
//   2. slot transitions ("Multi-Block Diffusion Language Models" page, sec.
//      2.3): to-cache -> in-cache (the step just taken recomputed the
//      finished block and wrote its K/V), then the leading run of fully
//      decoded active slots -> to-cache, then the lowest dummy slots ->
//      active until the running set is full; noise groups: a clean slot s
//      is group s, every active slot is group n_slots;
//   3. the next step's per-row posterior inputs (skip = locked or not in an
//      active slot; flags: masked rows may be selected, decoded rows whose
//      slot was active in the step just taken may lock) and the compaction
//      of the rows it computes (unlocked rows of active and to-cache slots,
//      ascending): a block-wide prefix sum of a per-position predicate,
//      64 positions per wave and ballot, 1024 per round.
// Initialisation runs the same kernel without step 1 and with the first
// max_active slots active.
#include "dlm_internal.h"

namespace dlm {

namespace {

constexpr int kBBThreads = 1024;
constexpr uint8_t kDummy = 0, kActive = 1, kToCache = 2, kInCache = 3;
constexpr uint8_t kRowSelect = 1, kRowLock = 2;

__global__ __launch_bounds__(kBBThreads) void block_buffer_kernel(BBArgs a)
{
    __shared__ uint8_t st_s[kMaxSlots];    // slot states before this call
    __shared__ uint8_t nst_s[kMaxSlots];   // and after
    __shared__ uint8_t undone_s[kMaxSlots];
    __shared__ int wsum_s[kBBThreads / 64];

    const int b = blockIdx.x, tid = threadIdx.x;
    const bool init = a.sel == nullptr;
    const long r0 = (long)b * a.n_gen;
    const long s0 = (long)b * a.n_slots;
    for (int s = tid; s < a.n_slots; s += kBBThreads) {
        st_s[s] = init ? (s < a.max_active ? kActive : kDummy) : a.state[s0 + s];
        undone_s[s] = 0;
    }
    __syncthreads();

    // 1. results of the step for rows of active slots.  Thread tid owns
    // positions tid, tid + 1024, ... here and in step 3, so it reads back
    // its own writes.
    for (int p = tid; p < a.n_gen; p += kBBThreads) {
        const int s = p / a.bs;
        uint8_t dec = a.decoded[r0 + p];
        if (init) {
            a.locked[r0 + p] = 0;
        } else if (st_s[s] == kActive) {
            const int32_t v = a.sel[r0 + p];
            if (v >= 0) {
                dec = 1;
                a.decoded[r0 + p] = 1;
                a.tokens[r0 + p] = v;
            }
            if (a.skip[r0 + p]) a.locked[r0 + p] = 1;
        }
        if (!dec) undone_s[s] = 1;
    }
    __syncthreads();

    // 2. slot transitions, in slot order (one thread: a buffer holds few slots).
    if (tid == 0) {
        int open = 0;
        if (init) {
            for (int s = 0; s < a.n_slots; ++s) nst_s[s] = st_s[s];
        } else {
            for (int s = 0; s < a.n_slots; ++s) nst_s[s] = st_s[s] == kToCache ? kInCache : st_s[s];
            for (int s = 0; s < a.n_slots; ++s) {
                if (nst_s[s] == kToCache || nst_s[s] == kInCache) continue;
                if (nst_s[s] == kActive && !undone_s[s]) {
                    nst_s[s] = kToCache;
                    continue;
                }
                break;
            }
            int n_act = 0;
            for (int s = 0; s < a.n_slots; ++s) n_act += nst_s[s] == kActive;
            for (int s = 0; s < a.n_slots && n_act < a.max_active; ++s)
                if (nst_s[s] == kDummy) {
                    nst_s[s] = kActive;
                    ++n_act;
                }
        }
        for (int s = 0; s < a.n_slots; ++s) open += nst_s[s] != kInCache;
        a.n_open[b] = open;
    }
    __syncthreads();
    for (int s = tid; s < a.n_slots; s += kBBThreads) {
        const uint8_t ns = nst_s[s];
        a.state[s0 + s] = ns;
        a.group[s0 + s] = (ns == kToCache || ns == kInCache) ? s : a.n_slots;
    }

    // 3. the next step's posterior inputs and rows to compute.
    const int lane = tid & 63, w = tid >> 6;
    int base = 0;
    for (int c0 = 0; c0 < a.n_gen; c0 += kBBThreads) {
        const int p = c0 + tid;
        bool comp = false;
        if (p < a.n_gen) {
            const int s = p / a.bs;
            const uint8_t ns = nst_s[s];
            const uint8_t lk = a.locked[r0 + p];
            const uint8_t dec = a.decoded[r0 + p];
            a.skip[r0 + p] = (lk || ns != kActive) ? 1 : 0;
            a.flags[r0 + p] = !dec ? kRowSelect : ((!init && st_s[s] == kActive) ? kRowLock : 0);
            comp = (ns == kActive || ns == kToCache) && !lk;
        }
        const unsigned long long bal = __ballot(comp);
        if (lane == 0) wsum_s[w] = __popcll(bal);
        __syncthreads();
        int off = base, tot = 0;
        for (int i = 0; i < kBBThreads / 64; ++i) {
            off += i < w ? wsum_s[i] : 0;
            tot += wsum_s[i];
        }
        if (comp) a.active_idx[r0 + off + __popcll(bal & ((1ull << lane) - 1))] = a.P + p;
        base += tot;
        __syncthreads();   // wsum_s is rewritten by the next round
    }
    for (int j = base + tid; j < a.n_gen; j += kBBThreads) a.active_idx[r0 + j] = -1;
    if (tid == 0) a.m_active[b] = base;
}

}  // namespace

hipError_t launch_block_buffer(const BBArgs &a, hipStream_t stream)
{
    block_buffer_kernel<<<dim3((unsigned)a.B), dim3(kBBThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dlm
