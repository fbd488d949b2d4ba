/*
 * dlm_step.h -- C ABI of one masked-diffusion LM denoising step on MI355X
 * (gfx950).
 *
 * One step has two calls:
 *   dlm_step_attn  -- sparse-query attention of the active rows over the K/V
 *                     cache under a bidirectional, block-causal or
 *                     group-aware mask, plus attention column sums;
 *   dlm_posterior  -- per-row softmax posterior, confidence, the step-wise
 *                     KL(p_t || p_{t-1}) lock test and unmask selection.
 * A multi-step run adds one call between steps:
 *   dlm_block_buffer_advance -- the Block Buffer slot state machine, the
 *                     unmasking and locking of rows, and the compaction of
 *                     the rows the next step computes, all on the device
 *                     (dlm_block_buffer_init starts a run).
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers (HIP global memory) and every
 *    tensor is dense and row-major in the layout stated.  The descriptor
 *    structs themselves (dlm_kv_cache, dlm_mask_desc, dlm_select,
 *    dlm_block_buffer) live in HOST memory and are read during the call
 *    only.  A run's Block Buffer state lives in device arrays the caller
 *    owns; the library itself keeps none.
 *  - bf16 is IEEE bfloat16 stored as 16-bit words; fp32 is IEEE binary32.
 *  - The caller owns every buffer, the workspace included.  The library
 *    allocates nothing, frees nothing, keeps no state between calls and does
 *    not synchronise: all work is enqueued on `stream` and outputs are valid
 *    once that stream reaches the point of the call.
 *  - Every function returns DLM_OK (0) or a negative DLM_E_* code; the
 *    message of the last failure on the calling thread is dlm_last_error().
 *    Scalar and descriptor checks run on the host before anything is
 *    enqueued, so a failed call has enqueued no work.  The CONTENTS of device
 *    arrays (order of active_idx, slot tables) are not checked unless the
 *    environment variable DLM_VALIDATE=1 is set, in which case a host copy is
 *    checked first (this synchronises the stream); otherwise contents that
 *    break the stated rules give undefined results.
 *  - Calls on one stream are ordered; calls on different streams that share
 *    a workspace or an output race.
 *  - DLM_ATTN_KGROUPS=1 or 2 in the environment forces the shape of the
 *    pass-1 workgroups (one key group of 4 waves, or two of 4); by default
 *    it follows from the shapes.  It changes the workspace size, so
 *    dlm_step_attn_workspace_bytes and dlm_step_attn must see the same
 *    setting.  Results agree to rounding either way.
 */
#ifndef DLM_STEP_H
#define DLM_STEP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DLM_OK = 0,
    DLM_E_NULL = -1,        /* a required pointer is NULL */
    DLM_E_SHAPE = -2,       /* a size is out of range or sizes disagree */
    DLM_E_UNSUPPORTED = -3, /* valid, but not built: D not in {32,64,128}, Hq % Hkv != 0, ... */
    DLM_E_DESC = -4,        /* bad mask / selection descriptor (or DLM_VALIDATE content check) */
    DLM_E_WORKSPACE = -5,   /* workspace missing or too small */
    DLM_E_HIP = -6          /* a HIP runtime call or kernel launch failed */
};

/* Mask kinds.  Query position i (an active row), key position n:
 *  FULL          n < kv_len: bidirectional attention, every token sees the
 *                whole context ("Bifocal Diffusion Language Models", sec. 1).
 *  BLOCK_CAUSAL  n < prefix_len, or block(n) <= block(i), where
 *                block(x) = (x - prefix_len) / block_size: one noisy block
 *                sees the clean prefix and the blocks before it and itself
 *                ("Multi-Block Diffusion LMs", sec. 1, SingleBD).
 *  GROUP         n < prefix_len, or slot(n) is not DUMMY and
 *                group(slot(n)) <= group(slot(i)), slot(x) = block(x):
 *                blocks of one noise group see each other, earlier groups
 *                and completed slots are clean context, the prefix never sees
 *                the noisy blocks because it is never a query
 *                ("Multi-Block Diffusion LMs", sec. 2.2 group-aware mask,
 *                sec. 2.3 block-buffer slot states).
 * Keys at or beyond kv_len are never visible. */
enum { DLM_MASK_FULL = 0, DLM_MASK_BLOCK_CAUSAL = 1, DLM_MASK_GROUP = 2 };

/* Block-buffer slot states ("Multi-Block Diffusion LMs", sec. 2.3). */
enum { DLM_SLOT_DUMMY = 0, DLM_SLOT_ACTIVE = 1, DLM_SLOT_TO_CACHE = 2, DLM_SLOT_IN_CACHE = 3 };

/* The K/V cache of one attention layer: k and v are bf16 [B, Hkv, n_cap, D]
 * each (device).  Rows [0, kv_len) of each (b, kv-head) are meaningful. */
typedef struct {
    void *k;
    void *v;
    int32_t B, Hkv, n_cap, D;
} dlm_kv_cache;

/* Problem and mask descriptor of dlm_step_attn. */
typedef struct {
    int32_t kind;            /* DLM_MASK_* */
    int32_t Hq;              /* query heads; Hq % Hkv == 0; q-head h reads kv-head h / (Hq/Hkv) */
    int32_t M;               /* active query rows per batch entry */
    int32_t kv_len;          /* key positions [0, kv_len), kv_len <= n_cap */
    int32_t prefix_len;      /* clean prefix [0, prefix_len): never written, never a query */
    int32_t block_size;      /* BLOCK_CAUSAL / GROUP: positions per block (slot) */
    int32_t n_slots;         /* GROUP: slots per batch entry, <= 1024, and
                                kv_len <= prefix_len + n_slots * block_size */
    const uint8_t *slot_state;   /* GROUP: device uint8 [B, n_slots], DLM_SLOT_* */
    const int32_t *slot_group;   /* GROUP: device int32 [B, n_slots], noise-group id */
    int32_t cs_lo, cs_hi;    /* active rows whose POSITION lies in [cs_lo, cs_hi) feed colsum */
    int32_t colsum_per_head; /* 0: colsum is [B, kv_len] summed over q-heads; 1: [B, Hq, kv_len] */
    float scale;             /* softmax scale; 0 means 1/sqrt(D) */
    void *workspace;         /* device scratch, >= dlm_step_attn_workspace_bytes() */
    size_t workspace_bytes;
    int32_t colsum_accumulate;   /* 0: colsum = the sums of this call; 1: colsum += them,
                                    e.g. summed over the layers of a model (the
                                    Attention-Based Sampler page, sec. 4, averages the
                                    scores of all layers and heads; a sum ranks the same) */
    const int32_t *m_active;     /* optional device int32 [B] (NULL: every row is valid).
                                    Only rows j < m_active[b] (clamped to [0, M]) of batch
                                    entry b are valid: the others are not read (q, k, v,
                                    active_idx) nor written (out, lse, the cache) and add
                                    nothing to colsum.  M stays the row stride and the
                                    capacity.  With it a step whose row count is decided
                                    on the device (dlm_block_buffer_advance) keeps the
                                    same launch shapes, e.g. inside a captured HIP graph
                                    (SureLock page, sec. 2: M_t rows are computed).
                                    Pass 1 then also splits the keys by the row count, on
                                    the device, so its cost follows M_t: query the
                                    workspace with m_active set (the size depends on
                                    whether it is). */
    hipEvent_t pass1_done;       /* optional (NULL: none).  Recorded on `stream` once pass 1
                                    (and its split merge) is enqueued, before the column-sum
                                    pass: out and lse are final when it completes.  A caller
                                    can start work that does not need the column sums (the
                                    posterior's logit stream) on a second stream from this
                                    event, beside the column-sum pass. */
} dlm_mask_desc;

/*
 * dlm_step_attn -- one denoising step's attention for the active rows.
 *
 * Defines ("Stopping Computation for Converged Tokens in Masked Diffusion-LM
 * Decoding" (SureLock), sec. 2 core mechanism; "Bifocal Diffusion Language
 * Models", sec. 2 inference; "Attention-Based Sampler for Diffusion
 * Language Models", sec. 2B):
 *   1. the fresh K/V of the active rows are written into the cache at their
 *      positions: cache[b, g, active_idx[b, j], :] = k[b, g, j, :] (same for
 *      v).  Locked rows and the prefix keep their cached K/V.
 *   2. for each active row j of batch b and q-head h (kv-head g = h/(Hq/Hkv)),
 *      at position i = active_idx[b, j], over the keys n visible to i:
 *        s_n   = scale * q[b,h,j,:] . Kcache[b,g,n,:]
 *        lse   = log sum_n exp(s_n)                (natural log)
 *        out   = sum_n exp(s_n - lse) * Vcache[b,g,n,:]
 *      A row with no visible key gets out = 0 and lse = -inf.
 *   3. if colsum != NULL, the attention column sums
 *        colsum[b, n] = sum_h sum_{j : cs_lo <= active_idx[b,j] < cs_hi}
 *                       exp(s^{(b,h,j)}_n - lse_{b,h,j})   (0 where not visible)
 *      ([B, Hq, kv_len] without the sum over h if colsum_per_head).  Columns
 *      are exact (each row normalised by its full log-sum-exp), computed in a
 *      fixed order: bitwise reproducible for equal inputs.
 *
 * Arguments (device unless stated):
 *   q          bf16 [B, Hq, M, D]       queries of the active rows
 *   k, v       bf16 [B, Hkv, M, D]      fresh K/V of the active rows; both
 *                                       NULL means "already in the cache"
 *   kv_cache   host struct; cache k/v are written at active positions only
 *   active_idx int32 [B, M]             positions, strictly ascending per b,
 *                                       each in [prefix_len, kv_len)
 *   mask_desc  host struct (above)
 *   out        bf16 [B, Hq, M, D]       attention output (round to nearest even)
 *   lse        fp32 [B, Hq, M]          natural-log log-sum-exp of each row
 *   colsum     fp32 [B, kv_len] or [B, Hq, kv_len], or NULL
 *   stream     HIP stream all work is enqueued on
 * Supported: D in {32, 64, 128}; Hq % Hkv == 0; kv_len * D * 2 bytes
 * (one (batch, head) slice of K or V) below 2 GiB - 4 KiB, since the
 * kernels address a slice with 32-bit byte offsets (DLM_E_SHAPE otherwise).
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED, DLM_E_DESC,
 *         DLM_E_WORKSPACE, DLM_E_HIP.
 */
int dlm_step_attn(const void *q, const void *k, const void *v,
                  const dlm_kv_cache *kv_cache, const int32_t *active_idx,
                  const dlm_mask_desc *mask_desc, void *out, float *lse,
                  float *colsum, hipStream_t stream);

/* Workspace bytes dlm_step_attn needs for this problem (with colsum).
 * Writes *bytes; returns DLM_OK or the error dlm_step_attn would return
 * for the scalar arguments. */
int dlm_step_attn_workspace_bytes(const dlm_kv_cache *kv_cache,
                                  const dlm_mask_desc *mask_desc, size_t *bytes);

/* Unmask selection modes:
 *  NONE          lock test only.
 *  TOPK_CONF     the k most confident eligible rows of each group
 *                (confidence sampler; "Attention-Based Sampler ...", sec. 1).
 *  THRESH_CONF   eligible rows with conf > tau; if none, the most confident.
 *  ATTN_DYNAMIC  Attn-Sampler dynamic attention threshold (sec. 2B):
 *                candidates = eligible rows with conf > tau; threshold =
 *                largest score among eligible non-candidates (-inf if none);
 *                decode candidates whose score exceeds it; if none, the
 *                eligible row of highest score.
 *  TOPK_SCORE    the k eligible rows of highest score (column-sum order).
 *  TOPK_MARGIN   the k eligible rows of largest margin p(top-1) - p(top-2)
 *                (margin sampler; sec. 1 names margin among the token-level
 *                scores of the greedy samplers).
 *  TOPK_LOW_ENTROPY  the k eligible rows of lowest entropy -sum p ln p
 *                (entropy sampler; likewise sec. 1).
 * Eligible = not locked on entry and selectable (dlm_select.row_flags).
 * Order: larger key first, then lower row index.  If fewer than k rows are
 * eligible, all are taken. */
enum { DLM_SEL_NONE = 0, DLM_SEL_TOPK_CONF = 1, DLM_SEL_THRESH_CONF = 2,
       DLM_SEL_ATTN_DYNAMIC = 3, DLM_SEL_TOPK_SCORE = 4, DLM_SEL_TOPK_MARGIN = 5,
       DLM_SEL_TOPK_LOW_ENTROPY = 6 };

typedef struct {
    int32_t mode;            /* DLM_SEL_* */
    int32_t k;               /* TOPK_*: rows per group, >= 0 */
    int32_t group_rows;      /* rows per selection group (consecutive rows), 1..1024 */
    float tau;               /* THRESH_CONF / ATTN_DYNAMIC confidence threshold */
    const float *score;      /* device fp32 [R]: ATTN_DYNAMIC / TOPK_SCORE ranking key */
    void *workspace;         /* device scratch, >= dlm_posterior_workspace_bytes().
                                Zero it once when it is allocated (hipMemset): it
                                holds arrival counters that every call leaves at zero
                                again, so a workspace reused by later calls needs no
                                clearing (nor a memset node inside a captured graph).
                                Any other use of its bytes between calls breaks this. */
    size_t workspace_bytes;
    hipEvent_t score_ready;  /* optional (NULL: none).  The selection stage, the only
                                part that reads `score`, first waits for this event on
                                `stream` (hipStreamWaitEvent); the KL / confidence
                                stream over the logits does not.  A caller that records
                                an event after the dlm_step_attn producing the column
                                sums and calls dlm_posterior on a second stream thus
                                overlaps the logit stream with the attention passes. */
    float *margin;           /* optional device fp32 [R] out (NULL: not written):
                                p_t(top-1) - p_t(top-2); 0 on a tie and for rows locked
                                on entry; p_t(top-1) when V == 1 */
    float *entropy;          /* optional device fp32 [R] out (NULL: not written):
                                -sum_v p_t(v) ln p_t(v); 0 for rows locked on entry */
    const uint8_t *row_flags;    /* optional device uint8 [R] (NULL: every row both):
                                DLM_ROW_SELECT -- the row may be selected (a masked token);
                                DLM_ROW_LOCK   -- the row may lock (SureLock page, sec. 2:
                                a converged, already unmasked token stops).  A row
                                without DLM_ROW_LOCK keeps locked[r] = 0 whatever its
                                KL; its kl, conf and scores are still written. */
    float conf_gate;         /* the optional confidence gate of the lock test (SureLock
                                page, sec. 2: a peaked posterior): a row locks only if
                                also conf >= conf_gate.  0 (no gate) or any finite value. */
    const int32_t *live_rows;    /* optional device int32 [*n_live] (NULL: none): the rows
                                that may arrive unlocked, as live_rows[i] - live_offset
                                (entries outside [0, R) are ignored; a listed row that
                                arrives locked is skipped).  Every row NOT listed must
                                arrive locked: it is not read, as any locked row.  With
                                the list, the split of each row's vocabulary into chunks
                                is chosen on the device from the count, so the logit
                                stream's parallelism follows the live rows late in a
                                run (SureLock page, sec. 2: only the M_t active rows are
                                computed) while the launch shapes stay fixed for graph
                                capture.  The workspace size depends on whether a list
                                is given (set it before dlm_posterior_workspace_bytes).
                                Outputs are those of the call without the list up to
                                the fp32 summation order of the chunks. */
    const int32_t *n_live;       /* device int32 [1], required with live_rows: list length (<= R) */
    int32_t live_offset;         /* subtracted from every live_rows entry */
} dlm_select;

/* Bits of dlm_select.row_flags. */
enum { DLM_ROW_SELECT = 1, DLM_ROW_LOCK = 2 };

/*
 * dlm_posterior -- posterior, lock test and unmask selection for R rows.
 *
 * Defines (SureLock page, sec. 2 core mechanism; Attn-Sampler page,
 * sec. 1 and 2B), per row r that arrives with locked[r] == 0:
 *   p_t = softmax(logits[r]), p_{t-1} = softmax(prev_logits[r])
 *   kl[r]   = KL(p_t || p_{t-1}) = sum_v p_t(v) (log p_t(v) - log p_{t-1}(v))
 *   conf[r] = max_v p_t(v);  tok = lowest v with the largest logit
 *   locked[r] = 1 if kl[r] <= eps, the row may lock (row_flags) and
 *               conf[r] >= conf_gate (a lock is never undone)
 *   sel[r]  = tok if the row is selected (mode above), else -1.
 * A row that arrives locked is not read: kl = conf = 0, sel = -1, stays locked.
 * kl and conf are fp32; KL is computed in one pass as
 * E_p[x - y] - (logsumexp x - logsumexp y).
 * Without a live-row list or a score_ready event, and with selection groups
 * of at most 256 rows, the call is one kernel launch when its own split of
 * the rows into vocabulary chunks (about 512 workgroups in all) fits one
 * round on the GPU (1280 workgroups), or with DLM_SEL_NONE when each row
 * is one workgroup: the workgroups of a row's chunks count their arrivals
 * in the workspace, the last one merges the row, and the last row of a
 * group runs its selection.
 * Otherwise a second launch merges and selects.  Results are deterministic
 * for given shapes on either path; the two paths merge a row's chunks in
 * different fp32 orders.
 *
 * Arguments (device unless stated):
 *   logits       fp32 [R, V]   step-t logits
 *   prev_logits  fp32 [R, V]   step-(t-1) logits of the same rows
 *   locked       uint8 [R]     in/out lock flags
 *   eps          lock threshold
 *   select       host struct (above)
 *   sel          int32 [R]     out
 *   kl, conf     fp32 [R]      out
 *   R, V         rows (>= 0) and vocabulary size (>= 1)
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_DESC, DLM_E_WORKSPACE, DLM_E_HIP.
 */
int dlm_posterior(const float *logits, const float *prev_logits, uint8_t *locked,
                  float eps, const dlm_select *select, int32_t *sel, float *kl,
                  float *conf, int32_t R, int32_t V, hipStream_t stream);

/* Workspace bytes dlm_posterior needs for R x V.  Writes *bytes. */
int dlm_posterior_workspace_bytes(int32_t R, int32_t V, const dlm_select *select,
                                  size_t *bytes);

/* Largest partials area the allocation-free posterior holds (bytes). */
#define DLM_NOALLOC_SCRATCH_BYTES (8u << 20)

/* dlm_posterior without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, outputs and errors as
 * dlm_posterior; select->workspace and workspace_bytes are ignored.  The
 * per-(row, vocabulary chunk) partials and the arrival counters go to a
 * file-scope device array of DLM_NOALLOC_SCRATCH_BYTES (zero when the module
 * loads; every call leaves its counters zero), which each GPU the library
 * runs on holds from the first call on it until the process ends; its device address is
 * fetched on that first call (the only call that may load the module's
 * globals), after which no call allocates or frees anything.
 * Limit: a problem whose workspace (dlm_posterior_workspace_bytes) exceeds
 * DLM_NOALLOC_SCRATCH_BYTES returns DLM_E_WORKSPACE before any work is
 * enqueued.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and give
 * undefined results; calls ordered on one stream are safe. */
int dlm_posterior_noalloc(const float *logits, const float *prev_logits,
                          uint8_t *locked, float eps, const dlm_select *select,
                          int32_t *sel, float *kl, float *conf, int32_t R,
                          int32_t V, hipStream_t stream);

/*
 * Block Buffer of a multi-step run ("Multi-Block Diffusion Language Models"
 * page, sec. 2.3; SureLock page, sec. 2).  The generation region of each
 * batch entry is n_slots blocks of block_size positions starting at
 * absolute position prefix_len; position p (0-based in the region) is in
 * slot p / block_size.  All arrays are device memory owned by the caller;
 * n_gen = n_slots * block_size.
 *   slot_state  uint8 [B, n_slots]   DLM_SLOT_*            (written)
 *   slot_group  int32 [B, n_slots]   noise group of a slot (written): a
 *               to-cache or in-cache slot s is group s (clean, block-causal
 *               context), every active slot is group n_slots (the running
 *               noise group, mutually visible); use both as the GROUP mask's
 *               slot tables
 *   decoded     uint8 [B, n_gen]     1 once unmasked        (read, updated)
 *   tokens      int32 [B, n_gen]     token of an unmasked position (updated)
 *   locked      uint8 [B, n_gen]     1 once locked (its query stops)
 *   skip        uint8 [B, n_gen]     the next step's dlm_posterior `locked`
 *               argument: 1 for locked rows and rows outside active slots;
 *               the posterior then sets it for rows that lock
 *   row_flags   uint8 [B, n_gen]     the next step's dlm_select.row_flags:
 *               DLM_ROW_SELECT for masked rows, DLM_ROW_LOCK for unmasked
 *               rows whose slot was active in the step just taken (they
 *               have a previous-step posterior)
 *   active_idx  int32 [B, n_gen]     the next step's rows to compute: the
 *               absolute positions of unlocked rows of active and to-cache
 *               slots, ascending, then -1 (dlm_step_attn's active_idx with
 *               M = n_gen)
 *   m_active    int32 [B]            how many (dlm_mask_desc.m_active)
 *   n_open      int32 [B]            slots not yet in-cache (0: finished)
 */
typedef struct {
    int32_t B;              /* batch entries, >= 1 */
    int32_t n_slots;        /* slots per batch entry, 1..1024 */
    int32_t block_size;     /* positions per slot, >= 1 */
    int32_t max_active;     /* running-set size: most slots active at once, >= 1 */
    int32_t prefix_len;     /* absolute position of the region's first row, >= 0 */
    uint8_t *slot_state;
    int32_t *slot_group;
    uint8_t *decoded;
    int32_t *tokens;
    uint8_t *locked;
    uint8_t *skip;
    uint8_t *row_flags;
    int32_t *active_idx;
    int32_t *m_active;
    int32_t *n_open;
} dlm_block_buffer;

/* Start a run: slots 0 .. max_active-1 active, the rest dummy; locked
 * cleared; decoded and tokens kept as the caller set them (e.g. a prompt
 * inside the region starts unmasked); no row may lock in the first step.
 * Writes slot_state, slot_group, locked, skip, row_flags, active_idx,
 * m_active, n_open.  One kernel on `stream`.
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_HIP. */
int dlm_block_buffer_init(const dlm_block_buffer *bb, hipStream_t stream);

/* Between two steps: apply the step's results to rows of active slots (a
 * row with sel >= 0 becomes unmasked with that token; a row the posterior
 * locked in `skip` becomes locked), then move the slots in this order:
 * to-cache -> in-cache (the step just taken recomputed those blocks and
 * wrote their K/V into the cache); the leading run of fully unmasked active
 * slots -> to-cache (a block is committed only after every earlier one, so
 * the cached prefix stays contiguous); the lowest dummy slots -> active
 * until max_active are active.  Then derives skip, row_flags, active_idx,
 * m_active and n_open for the next step.  The next step's forward computes
 * the to-cache rows (their commit) together with the active rows (their
 * decoding), so decoding and cache writes overlap in one launch.
 *   sel  int32 [B, n_gen]  (device) the step's dlm_posterior selections
 * One kernel on `stream`.  Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_HIP. */
int dlm_block_buffer_advance(const dlm_block_buffer *bb, const int32_t *sel,
                             hipStream_t stream);

/*
 * Active-row projections and feed-forward of one layer (SureLock page,
 * sec. 2: a locked position skips its query projection and its feed-forward
 * sub-layer, so a step's dense work is O(M_t d^2) over the active rows).
 *
 * The rows are those of dlm_step_attn: row j of batch entry b is the position
 * active_idx[b, j], j < M (j < m_active[b] when m_active is given).  Weights
 * are bf16, row-major [out_features, in_features]; products accumulate in
 * fp32 and results are rounded to bf16 (nearest even).  The layer is
 *   q | k | v = x[act] W_qkv^T                       (dlm_proj_qkv)
 *   h         = x[act] + attn_out W_o^T              (dlm_proj_out)
 *   x[act]    = h + (silu(h W_gate^T) * (h W_up^T)) W_down^T   (dlm_ffn)
 * silu(z) = z / (1 + exp(-z)).  The layer's normalisations are not part of
 * these calls.  Rows of locked positions are neither read nor written.
 */
typedef struct {
    int32_t B;                  /* batch entries, >= 1 */
    int32_t n_pos;              /* positions of the hidden states x: bf16 [B, n_pos, d] */
    int32_t d;                  /* model width, a multiple of 64 */
    int32_t M;                  /* active rows per batch entry (row capacity), >= 0 */
    const int32_t *active_idx;  /* device int32 [B, M], positions in [0, n_pos) */
    const int32_t *m_active;    /* optional device int32 [B] (NULL: all M rows) */
    int32_t Hq, Hkv, D;         /* attention heads (Hq % Hkv == 0) and head width */
    int32_t F;                  /* feed-forward width, a multiple of 64 */
    int32_t weights_packed;     /* 0: every weight argument row-major as stated below;
                                   1: every one in the layout of dlm_pack_weights */
} dlm_layer_desc;

/* Repack a bf16 weight matrix for the layer calls (weights_packed = 1): the
 * same products, bit for bit, from a layout that streams from HBM faster
 * when few rows are active (each 1 KB of it is one MFMA operand).  For each
 * group of 16 rows g and each step of 32 columns s (s < K/32), 1 KB at
 * element offset (g K/32 + s) * 512 holds 64 lanes of 8 bf16: lane l has
 * row 16 g + l % 16, columns 32 s + 8 (l / 16) .. + 7.
 *   w       bf16 [N, K] row-major (device), read
 *   packed  bf16, N * K elements (device), written; must not overlap w
 * N a multiple of 16, K of 32 (every layer weight qualifies: its dimensions
 * are multiples of 64).  Done once per weight, e.g. at load time.  One
 * kernel on `stream`.  Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED,
 * DLM_E_DESC (overlap), DLM_E_HIP. */
int dlm_pack_weights(const void *w, void *packed, int32_t N, int32_t K, hipStream_t stream);

/* Every call takes a device workspace of at least dlm_layer_workspace_bytes()
 * (fp32 partial sums when a product has too few output tiles to fill the chip
 * and its K dimension is split; the gated hidden rows of dlm_ffn).  Calls that
 * share a workspace must be ordered (one stream). */
int dlm_layer_workspace_bytes(const dlm_layer_desc *layer, size_t *bytes);

/* q | k | v projection of the active rows.
 *   x      bf16 [B, n_pos, d]
 *   w_qkv  bf16 [(Hq + 2 Hkv) * D, d]: the q rows (head-major), then k, then v
 *   q      bf16 [B, Hq, M, D] out;  k, v  bf16 [B, Hkv, M, D] out
 * (the layouts dlm_step_attn reads).  Errors: DLM_E_NULL, DLM_E_SHAPE,
 * DLM_E_UNSUPPORTED, DLM_E_WORKSPACE, DLM_E_HIP. */
int dlm_proj_qkv(const dlm_layer_desc *layer, const void *x, const void *w_qkv, void *q, void *k,
                 void *v, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Output projection with the residual: h = x[act] + attn_out W_o^T.
 *   attn_out  bf16 [B, Hq, M, D] (dlm_step_attn's out); D a multiple of 64
 *   w_o       bf16 [d, Hq * D]
 *   h         bf16 [B, M, d] out
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED, DLM_E_WORKSPACE, DLM_E_HIP. */
int dlm_proj_out(const dlm_layer_desc *layer, const void *x, const void *attn_out, const void *w_o,
                 void *h, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* SwiGLU feed-forward with the residual, written back to the active rows of
 * x: x[b, active_idx[b, j], :] = h + (silu(h W_gate^T) * (h W_up^T)) W_down^T.
 *   h               bf16 [B, M, d]
 *   w_gate, w_up    bf16 [F, d];  w_down  bf16 [d, F]
 *   x               bf16 [B, n_pos, d] in/out (only active rows written)
 *   the gated hidden rows are rounded to bf16 (in the workspace) before the
 *   down projection
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED, DLM_E_WORKSPACE, DLM_E_HIP. */
int dlm_ffn(const dlm_layer_desc *layer, const void *h, const void *w_gate, const void *w_up,
            const void *w_down, void *x, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * R2LM right-to-left selective scan over the generation block ("Bifocal
 * Diffusion Language Models" page, sec. 2: the right-to-left stream flips
 * the hidden states, applies a selective scan (Mamba) and flips them back; a
 * learnable scalar gate s, 0 at initialisation, scales the correction).  Per
 * batch entry b and channel e, from a zero state at the block's last token,
 * for t = L-1 down to 0:
 *   h[e, n] = exp(delta[b,t,e] * A[e,n]) * h[e, n] + delta[b,t,e] * Bm[b,t,n] * u[b,t,e]
 *   y[b,t,e] = s * (sum_n Cm[b,t,n] * h[e, n] + D[e] * u[b,t,e])
 * in fp32 (exp as exp2 of delta * A * log2 e).
 *   u, delta  bf16 [B, L, E] (delta > 0 in use; not checked)
 *   A         fp32 [E, N];  D  fp32 [E]
 *   Bm, Cm    bf16 [B, L, N]
 *   y         fp32 [B, L, E] out, or NULL
 *   x         bf16 [B, L, E] in/out, or NULL: x = bf16(x + y), the correction
 *             joining the hidden stream
 * At least one of y and x.  u, delta, Bm, Cm and x 16-byte aligned.
 * Errors: DLM_E_NULL, DLM_E_SHAPE, DLM_E_UNSUPPORTED (N not in {8, 16, 32}, or E
 * not a multiple of 8),
 * DLM_E_DESC (gate not finite), DLM_E_HIP.
 */
typedef struct {
    int32_t B, L, E, N;     /* batch, tokens of the block, channels, states per channel */
    float gate;             /* s */
} dlm_r2l_desc;

int dlm_r2l_scan(const dlm_r2l_desc *desc, const void *u, const void *delta, const float *A,
                 const void *Bm, const void *Cm, const float *D, float *y, void *x, hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char *dlm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLM_STEP_H */
