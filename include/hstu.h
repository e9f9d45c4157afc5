/*
 * hstu.h -- C ABI of the MI355X (gfx950) HSTU jagged-attention library.
 *
 * The library computes HSTU pointwise attention over jagged user-behaviour sequences and the full
 * HSTU layer built around it.  Sources for each operation:
 *
 *   - Jagged layout: sequences are stored back to back in the token dimension and located by
 *     start offsets, as in TorchRec's KeyedJaggedTensor (page 1, "Generative recommendation:
 *     algorithm evolution to engineering", section 3.1.2).
 *   - Attention (page 1 section 2.1.2, HSTU, spatial aggregation, equation (2)): no softmax;
 *     a relative attention bias from positions and timestamps is added to the scaled scores and
 *     SiLU is applied pointwise:
 *         S_ij = alpha * <q_i, k_j> + rab_pos[h, bucket(|i - j|)] + rab_ts[h, bucket(|t_i - t_j|)]
 *         O_i  = sum_j vis(i, j) * SiLU(S_ij) / N * v_j           (N = max_seqlen)
 *   - Mask (page 2, "RecSDK supports generative recommendation", HSTU acceleration operator:
 *     composite causal + context/target mask; page 1 section 2.1.2, ranking task: candidates at
 *     the end of a sequence must not interact).  For a sequence of length n:
 *         nc = min(num_contexts, n), nt = min(num_targets[b], n - nc), nh = n - nt
 *         vis(i, j) = j < nc  or  (i < nh and j <= i)  or  (i >= nh and (j < nh or j == i))
 *   - bucket(x) = x for x < 16, else min(127, 16 + 4 (e - 4) + ((x >> (e - 2)) & 3)) with
 *     e = floor(log2 x): exact buckets for short distances, then four per octave.
 *   - Layer (page 1 section 2.1.2, equations (1)-(3)): Z = SiLU(X W1) split into U, V, Q, K
 *     (column blocks of width H*d in that order, head-major inside a block); A = attention;
 *     Y = (LayerNorm(A) * U) W2 + X, LayerNorm per token over all H*d features, biased variance,
 *     no affine parameters.
 *
 * Conventions shared by every entry point:
 *   - Tensors are caller-owned device memory.  q, k, v, u, out, dout, dq, dk, dv are "THD":
 *     element (token t, head h, channel c) sits at t * token_stride + h * head_dim + c, with
 *     token_stride = num_heads * head_dim unless args->qkv_token_stride says otherwise (q, k, v
 *     and u only; outputs are always dense).  Element type is args->dtype.
 *   - Device pointers must be 16-byte aligned and token strides a multiple of 8 elements
 *     (HSTU_ERR_MISALIGNED otherwise).  For bf16, (max_seqlen + 64) * token_stride * 2 bytes must
 *     stay below 2^31 (HSTU_ERR_UNSUPPORTED otherwise): one sequence's rows of one tensor are
 *     addressed with 32-bit offsets.
 *   - Calls validate on the host, enqueue on `stream` (a hipStream_t; NULL = default stream) and
 *     return without waiting.  Nothing is allocated during fwd/bwd/layer calls; scratch memory is
 *     the caller's `ws` of at least hstu_workspace_bytes() bytes.  Kernel faults surface at the
 *     caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into.
 *   - Every function is reentrant; a plan is read-only after creation and may serve calls on any
 *     stream of the device it was created on.
 */
#ifndef HSTU_H
#define HSTU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HSTU_OK = 0,
    HSTU_ERR_NULL_ARG = 1,             /* a required pointer is NULL */
    HSTU_ERR_BAD_SHAPE = 2,            /* sizes invalid or inconsistent with the plan */
    HSTU_ERR_BAD_OFFSETS = 3,          /* seq_offsets not 0 .. T non-decreasing, or a length > N */
    HSTU_ERR_UNSUPPORTED = 4,          /* head_dim / dtype combination not implemented */
    HSTU_ERR_MISALIGNED = 5,           /* pointer or stride alignment */
    HSTU_ERR_WORKSPACE_TOO_SMALL = 6,  /* ws_bytes < hstu_workspace_bytes() */
    HSTU_ERR_HIP = 7,                  /* a HIP runtime call failed */
    HSTU_ERR_NO_DEVICE_PLAN = 8,       /* plan was created host-only and cannot be launched */
    HSTU_ERR_SCRATCH_LIMIT = 9         /* needs more than the static scratch of _noalloc calls */
} hstu_status_t;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype_t;

/* Problem description shared by a plan and the calls that use it. */
typedef struct {
    int32_t dtype;             /* hstu_dtype_t of q, k, v, u, out, dout, dq, dk, dv, x, w1, w2, y */
    int32_t batch;             /* B >= 0 sequences */
    int32_t num_heads;         /* H >= 1 */
    int32_t head_dim;          /* d = d_qk = d_v; 32, 64 or 128 */
    int64_t total_tokens;      /* T = seq_offsets[B], < 2^31 */
    int32_t max_seqlen;        /* N >= every length; the output scale is 1/N */
    int32_t num_contexts;      /* >= 0 leading tokens of every sequence visible to all queries */
    float alpha;               /* multiplies q.k only, not the bias */
    int32_t reserved;          /* must be 0 */
    int64_t qkv_token_stride;  /* elements between tokens of q, k, v, u; 0 means H * d */
    const int64_t* timestamps; /* device [T] int64 seconds, or NULL (then rab_ts must be NULL) */
    const float* rab_pos;      /* device [H][128] fp32 position-bias table, or NULL */
    const float* rab_ts;       /* device [H][128] fp32 time-bias table, or NULL */
} hstu_attn_args_t;

typedef struct hstu_plan hstu_plan_t;

/* Summary of a plan, for throughput accounting and tests. */
typedef struct {
    int64_t visible_pairs;     /* sum over sequences of visible (i, j) pairs, all heads */
    int64_t fwd_units;         /* work items of the forward (and dQ) launch */
    int64_t bwd_units;         /* work items of the dK/dV launch */
    int64_t fwd_tiles;         /* (32-row, 64-key) tiles the forward computes, all units */
    int64_t fwd_row_block;     /* query rows per forward (and dQ) work unit */
    int64_t bwd_key_block;     /* keys per dK/dV work item */
    int64_t fwd_items;         /* items of the forward launch (bf16: row blocks, long ones split) */
    int64_t fwd_split_blocks;  /* row blocks whose key tiles are split over several items */
    int64_t bwd_stored_ds;     /* 1: given a workspace, the backward stores dS and the dQ pass reads
                                  it back; 0: the dQ pass recomputes S and dP (fp32, head_dim 32,
                                  or a sequence of 8M tokens or more) */
    int64_t bwd_ds_bytes;      /* bytes of stored dS in the op 2 workspace (0 when not stored) */
    int64_t fwd_item_rows;     /* rows per item of the forward launch: 128, or 64 for candidate
                                  scoring and for batches whose 128-row blocks fill at most half
                                  of the workgroup slots (2 per compute unit) */
} hstu_plan_info_t;

#define HSTU_PLAN_HOST_ONLY 1u /* plan_create flag: plan on the host only (inspection, tests) */

/* Build the cost-balanced work lists for one batch (page 2, HSTU acceleration operator: greedy
 * even assignment of irregular work to cores).  seq_offsets_host: host [B+1] int64 start offsets
 * (KeyedJaggedTensor offsets, page 1 section 3.1.2) with [0] = 0 and [B] = T.
 * num_targets_host: host [B] int32 candidates per sequence, or NULL for none.  Work items are
 * (sequence, head, row block) and (sequence, head, key block).  Key blocks are ordered by
 * decreasing cost, so the hardware dispatcher assigns the longest first; row blocks (and forward
 * items) are dealt to the 8 XCDs' dispatch residues one (sequence, head) at a time, longest group
 * first, so that the blocks sharing K and V run on one XCD and read them from its L2.  For bf16, a row block costing more than the average load of a workgroup slot
 * (two per compute unit of the current device, 256 units for a host-only plan) runs as several
 * forward items over disjoint key tiles whose fp32 partial outputs are summed afterwards (exact
 * up to fp32 summation order: there is no softmax normalisation).  Unless flags has
 * HSTU_PLAN_HOST_ONLY, the lists are copied into one device buffer owned by the plan, on the
 * current device, through a non-blocking stream the library keeps per device: the call returns
 * once the copy is complete and does not wait for work queued on other streams (a plan for the
 * next batch can be built while the current batch's kernels run).  *out receives the plan, or
 * NULL on error.  The caller frees it
 * with hstu_plan_destroy. */
hstu_status_t hstu_plan_create(const hstu_attn_args_t* args, const int64_t* seq_offsets_host,
                               const int32_t* num_targets_host, uint32_t flags,
                               hstu_plan_t** out);

/* Frees the plan and its device buffer.  Waits for all work queued on the plan's device (on
 * every stream) first, so it is safe whatever stream used the plan, at the cost of a device
 * synchronisation; hstu_plan_destroy_on frees without waiting.  NULL is ignored. */
void hstu_plan_destroy(hstu_plan_t* plan);

/* Frees the plan without waiting on the host: its device buffer goes back to the device's
 * stream-ordered pool in the order of `stream` (a hipStream_t of the plan's device; NULL = the
 * default stream), i.e. after the work already queued there.  Every call that used the plan must
 * be queued on `stream` already, or on a stream that `stream` waits for (an event); calls on
 * other streams must be joined into `stream` first.  Where the device has no stream-ordered pool
 * the buffer is released with hipFree, which waits for the device.  NULL is ignored. */
void hstu_plan_destroy_on(hstu_plan_t* plan, void* stream);

/* Fills *info. */
hstu_status_t hstu_plan_info(const hstu_plan_t* plan, hstu_plan_info_t* info);

/* Copies the work list of `op` (0 = forward / recomputing dQ, 1 = dK/dV, 3 = the stored-dS dQ
 * pass's 256-row blocks) to host memory as int32 quadruples {sequence, head, first row (or key),
 * cost} in launch order; op 2 gives the bf16 forward items
 * as int32 octets {sequence, head, first row, cost, first tile, end tile, partial slot or -1, 0}
 * (row blocks of fwd_item_rows rows; tiles index the row block's list of visible key tiles).  Writes at most `cap` items and
 * returns the total count through *count. */
hstu_status_t hstu_plan_units(const hstu_plan_t* plan, int32_t op, int32_t* units, int64_t cap,
                              int64_t* count);

/* Scratch bytes a call needs: op 0 = hstu_attn_fwd without u, 1 = hstu_attn_fwd with u,
 * 2 = hstu_attn_bwd, 3 = hstu_layer_fwd, 4 = hstu_layer_bwd, 5 = hstu_attn_fwd_cached (d_model
 * is the model width; it does not change the result at present).  The forward ops, and op 4,
 * include 4 * head_dim bytes per row per partial slot of split row blocks (fwd_item_rows rows:
 * 512 * head_dim bytes for 128-row items; 0 when the plan splits none).  Op 2, and op 4 when
 * larger than the partial slots, is the stored dS of the bf16 backward with head_dim 64 or 128:
 * per sequence and head, each 128-key block holds one 128 x 64 bf16 chunk per 64-query tile of
 * the queries that see it (their range rounded out to 128), about 2 bytes per visible pair plus
 * the blocks on the diagonal (0 for fp32, head_dim 32, or a sequence of 8M tokens or more),
 * followed by the dK/dV pass's bias-mode records (256 bytes per chunk of one head, rounded up to
 * 256 bytes) and the query times relative to each sequence's first (4 bytes per token, rounded
 * up to 256 bytes); op 2 puts 2 * H * 128 fp32 (rounded up to 256 bytes) between the dS and the
 * records for the bias-table gradients that pass sums. */
size_t hstu_workspace_bytes(const hstu_plan_t* plan, int32_t op, int32_t d_model);

/* Attention forward (equation (2) above).  q, k, v: THD inputs; out: dense THD output.
 * If u is non-NULL, out instead receives LayerNorm(O) * u per token over all H*d features
 * (the gating part of equation (3), without W2).  ws must hold hstu_workspace_bytes(plan, u ? 1 : 0)
 * bytes (it may be NULL when that is 0).  ln_eps is used only with u. */
hstu_status_t hstu_attn_fwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                            const void* q, const void* k, const void* v, const void* u,
                            float ln_eps, void* out, void* ws, size_t ws_bytes, void* stream);

/* hstu_attn_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and arguments,
 * without ws.  The scratch it needs (hstu_workspace_bytes(plan, u ? 1 : 0, 0): the partial sums
 * of split row blocks, and the attention output before the LayerNorm when u is given) lives in
 * a static 64 MiB device array of the library, one per device, held from the first call on that
 * device until the process ends; the call allocates nothing and returns HSTU_ERR_SCRATCH_LIMIT
 * when the plan needs more.  The current device must be the plan's (HSTU_ERR_BAD_SHAPE
 * otherwise).  All such calls on one device share the array: calls that may overlap in time on
 * one device (different streams, or hosts threads without ordering) race; calls queued on one
 * stream do not.  Nothing from an earlier call is read (the scratch is written before it is
 * read). */
hstu_status_t hstu_attn_fwd_noalloc(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                    const void* q, const void* k, const void* v, const void* u,
                                    float ln_eps, void* out, void* stream);

/* Attention backward (page 1 section 2.1.2, HSTU spatial aggregation, equation (2), through the
 * chain rule; the pages give no backward of their own).  With S, sigma = sigmoid(S) and
 * P = SiLU(S) / N on visible pairs as in hstu_attn_fwd, and dO = dout:
 *     dV_j = sum_i P_ij dO_i,      dP_ij = dO_i . v_j,     dS_ij = dP_ij sigma (1 + S (1 - sigma)) / N,
 *     dQ_i = alpha sum_j dS_ij k_j,    dK_j = alpha sum_i dS_ij q_i,
 *     d rab_pos[h, b] = sum of dS_ij over pairs with bucket(|i - j|) = b (and d rab_ts likewise
 *     over bucket(|t_i - t_j|)).
 * Writes dq, dk, dv (dense THD, args->dtype) and, when the pointers and the matching tables are
 * non-NULL, drab_pos / drab_ts ([H][128] fp32, overwritten).  Bias gradients are summed with fp32
 * atomics, so their low bits depend on scheduling.  ws must hold hstu_workspace_bytes(plan, 2, 0)
 * bytes (it may be NULL when that is 0): the dK/dV pass stores dS there (bf16, dS * max_seqlen)
 * for every pair it visits and sums the bias-table gradients from it (fp32, before rounding),
 * and the dQ pass reads dS back instead of recomputing S and dP and copies the gradients out.
 * With ws the dK/dV half is two launches: a short pass that writes the per-tile bias-mode
 * records and relative query times into ws, then the dK/dV pass that reads them.
 * Same as hstu_attn_bwd_dkdv followed by hstu_attn_bwd_dq with the same ws. */
hstu_status_t hstu_attn_bwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                            const void* q, const void* k, const void* v, const void* dout,
                            void* dq, void* dk, void* dv, float* drab_pos, float* drab_ts,
                            void* ws, size_t ws_bytes, void* stream);

/* The two halves of hstu_attn_bwd (the same passage and formulas).  _dkdv writes dk and dv; _dq writes dq and the bias gradients
 * as hstu_attn_bwd does.  With ws (at least hstu_workspace_bytes(plan, 2, 0) bytes, else
 * HSTU_ERR_WORKSPACE_TOO_SMALL) _dkdv stores dS and the bias-table gradients into it and _dq
 * reads them: call _dq after _dkdv on the same stream (or after it has finished), with the same
 * plan, args, inputs and ws.  With ws
 * NULL (or a plan whose op 2 needs 0 bytes) nothing is stored and _dq recomputes S and dP; the
 * two calls then only read the inputs and may run on different streams at once. */
hstu_status_t hstu_attn_bwd_dkdv(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                 const void* q, const void* k, const void* v, const void* dout,
                                 void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);
hstu_status_t hstu_attn_bwd_dq(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                               const void* q, const void* k, const void* v, const void* dout,
                               void* dq, float* drab_pos, float* drab_ts, void* ws,
                               size_t ws_bytes, void* stream);

/* Full HSTU layer forward (page 1 section 2.1.2, HSTU layer: equation (1) pointwise projection
 * Z = SiLU(X W1) split into U, V, Q, K; equation (2) spatial aggregation A = attention(Q, K, V)
 * as in hstu_attn_fwd; equation (3) pointwise transformation Y = (LayerNorm(A) * U) W2 + X, with
 * the residual connection the section describes between layers), bf16 only.  x: (T, d_model)
 * dense; w1: (d_model, 4*H*d) row-major; w2: (H*d, d_model) row-major; y: (T, d_model).
 * args->qkv_token_stride is ignored (Q, K, V, U are produced internally).  ws must hold
 * hstu_workspace_bytes(plan, 3, d_model). */
hstu_status_t hstu_layer_fwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                             int32_t d_model, const void* x, const void* w1, const void* w2,
                             float ln_eps, void* y, void* ws, size_t ws_bytes, void* stream);

/* Full HSTU layer backward, bf16 only: the gradients of sum(dy * Y) for Y = hstu_layer_fwd(x)
 * (page 1 section 2.1.2, equations (1)-(3), by the chain rule; the forward's intermediates are
 * recomputed, not stored).  With H = x w1, Z = SiLU(H) = [U | V | Q | K], A = attention(Q, K, V),
 * xhat = LayerNorm(A), G = xhat * U:
 *     dw2 = G^T dy,  dG = dy w2^T,  dU = dG * xhat,
 *     dA = rstd * (dG*U - mean(dG*U) - xhat * mean(dG*U*xhat))          (per token),
 *     dQ, dK, dV, drab_* = attention backward with dout = dA,
 *     dH = [dU | dV | dQ | dK] * SiLU'(H),  dw1 = x^T dH,  dx = dy + dH w1^T.
 * x, dy, dx: (T, d_model) bf16; w1: (d_model, 4*H*d), w2: (H*d, d_model) bf16 row-major, as in
 * hstu_layer_fwd.  dw1 and dw2 (same shapes, fp32) and drab_pos / drab_ts ([H][128] fp32, when
 * non-NULL and the matching table is given) are overwritten; they are summed over tokens with
 * fp32 atomics, so their low bits depend on scheduling.  H*d must be a multiple of 128 and at
 * most 4096, d_model a multiple of 128 (HSTU_ERR_UNSUPPORTED otherwise).  ws must hold
 * hstu_workspace_bytes(plan, 4, d_model) bytes.  ln_eps must equal the forward's.  With no
 * tokens only dw1 and dw2 must be non-NULL (the gradients are cleared and nothing else runs). */
hstu_status_t hstu_layer_bwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                             int32_t d_model, const void* x, const void* w1, const void* w2,
                             const void* dy, float ln_eps, void* dx, float* dw1, float* dw2,
                             float* drab_pos, float* drab_ts, void* ws, size_t ws_bytes,
                             void* stream);

/* Candidate scoring against cached history (page 2, "RecSDK supports generative
 * recommendation", HSTU acceleration operator: KV-cache support; page 1 section 2.1.2, ranking:
 * candidates appended after a user's history are all scored in one pass, each seeing the whole
 * history and itself, never another candidate).  User b has cache_off[b + 1] - cache_off[b]
 * history tokens whose keys and values were computed earlier (the cache) and
 * cand_off[b + 1] - cand_off[b] new candidates.  A candidate at index c of user b has position
 * nk + c (nk = the user's cache length) and, with S defined as for hstu_attn_fwd,
 *     O_c = sum_{j < nk} SiLU(S_cj) / N v_j + SiLU(S_cc) / N v_c,
 * i.e. exactly the candidate rows of hstu_attn_fwd over [history | candidates] with the
 * candidates as targets.  bf16 only (HSTU_ERR_UNSUPPORTED otherwise).
 *
 * hstu_plan_create_cached: args describe the candidates (total_tokens = cand_off[B]; timestamps
 * = candidate times) and max_seqlen = N must be >= nk + m for every user (HSTU_ERR_BAD_OFFSETS
 * otherwise).  num_contexts is ignored: candidates see every cached key anyway.  cand_off and
 * cache_off are host arrays of B + 1 non-decreasing offsets starting at 0.  The plan serves only
 * hstu_attn_fwd_cached (other calls return HSTU_ERR_BAD_SHAPE). */
hstu_status_t hstu_plan_create_cached(const hstu_attn_args_t* args, const int64_t* cand_off,
                                      const int64_t* cache_off, uint32_t flags,
                                      hstu_plan_t** plan);

/* Candidate scoring of the rows hstu_plan_create_cached describes (page 1 section 2.1.2, ranking:
 * candidates see the whole history and themselves; page 2, HSTU acceleration operator: KV cache).
 * q, k, v: candidate THD tensors (token stride args->qkv_token_stride or H*d); k_cache, v_cache:
 * dense THD cache (cache_off[B] rows); cache_timestamps: [cache_off[B]] int64, needed when
 * args->rab_ts is set; out: dense THD (T, H, d).  ws must hold hstu_workspace_bytes(plan, 5, 0)
 * bytes (partial sums of long caches split over several workgroups; 0 when nothing is split). */
hstu_status_t hstu_attn_fwd_cached(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                   const void* q, const void* k, const void* v,
                                   const void* k_cache, const void* v_cache,
                                   const int64_t* cache_timestamps, void* out, void* ws,
                                   size_t ws_bytes, void* stream);

/* Stochastic Length compaction (page 1 section 2.1.3, algorithm-level optimisation: each
 * training sequence is cut to a randomly drawn length before the encoder runs, which lowers the
 * cost without a visible loss in quality).  The draw is the caller's (the pages give its rule
 * only in a figure); this call moves the kept tokens on the device.  Sequence b of the jagged
 * tensor src (device offsets src_offsets[batch + 1], src_rows rows of row_bytes bytes) keeps
 * dst_offsets[b + 1] - dst_offsets[b] consecutive rows starting at row keep_start[b] of the
 * sequence (device int64[batch]; NULL keeps its last rows, the most recent tokens), and dst
 * (dst_rows = dst_offsets[batch] rows) receives them packed in sequence order.  Offsets are
 * device arrays and are not checked on the host: a window that leaves its sequence or the
 * source tensor yields zero rows there.  row_bytes must be a multiple of 8, pointers 8-byte
 * aligned (16-byte aligned rows of a multiple of 16 bytes take the wide path).  Call it once
 * per tensor (x or q / k / v / u, timestamps) with the same offsets. */
hstu_status_t hstu_jagged_select(int32_t batch, const int64_t* src_offsets, int64_t src_rows,
                                 const int64_t* dst_offsets, int64_t dst_rows,
                                 const int64_t* keep_start, int64_t row_bytes, const void* src,
                                 void* dst, void* stream);

/* Static string naming a status code. */
const char* hstu_status_str(hstu_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H */
