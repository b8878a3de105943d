/*
 * moe.h -- C ABI of the paged fused-MoE layer for MI355X (gfx950).
 *
 * One MoE layer routes each token to k experts and runs every chosen expert's
 * SwiGLU FFN, y_t = sum_j w_{t,j} * W2_e (silu(W1_e x_t) * (W3_e x_t)), reading
 * the expert weights in place: from pages of a shared pool addressed through a
 * per-expert page table, or from a slot of one of two load buffers, never from
 * a copy gathered into a contiguous weight array.
 *
 * Source: "Rimuru: Unified Memory Management for Modern LLM Serving via Elastic
 * Expert Offloading" (paper-daily.com digest), sections
 *   "One pool for data whose sizes differ by orders of magnitude" (one
 *     contiguous pool read through typed views; expert pages),
 *   "Expert weights are scattered across pages. How does the kernel read them?"
 *     (location metadata per expert: a page number when cached, a buffer slot
 *     when just copied in; W1/W3 picked by column half; the address formula
 *     addr_e(n,t) = B_P + p_e(n)*f*d + (n mod f)*d + t; two alternating load
 *     buffers),
 *   "The adjuster: when to evict an expert, and which one?" (three pages per
 *     expert: W1 gate, W3 up, W2 down; copies finish before the page table
 *     points at them, pages are reused only after the forward pass ends).
 *
 * Conventions for every entry point:
 *   - Every data pointer is caller-owned memory.  "device" means memory of the
 *     current HIP device (e.g. a torch tensor's data_ptr); "host" means plain
 *     CPU memory; "pinned host" means page-locked memory from hipHostMalloc or
 *     torch's pin_memory.  The library never frees caller memory.
 *   - bf16 means IEEE bfloat16 bit patterns (uint16), row-major, no padding.
 *     bf16 arrays, load buffers and workspaces must be 16-byte aligned
 *     (workspaces 256-byte), int32 / fp32 arrays 4-byte and int64 arrays
 *     8-byte aligned (MOE_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Work is enqueued asynchronously; no entry point synchronises
 *     the host with the device except where stated.
 *   - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     launched and moe_last_error() describes the problem.  A device fault of an
 *     earlier launch surfaces as MOE_ERR_HIP on a later call.  No exception
 *     crosses this boundary.
 *   - T = 0 tokens is a valid no-op.
 *   - Concurrency: the host state of one pool, pipeline or allocator handle is
 *     not guarded, so calls on one handle must not run at the same time from
 *     several host threads; calls on different handles may.  On the device,
 *     forwards over one pool enqueued on different streams may overlap (they
 *     only read the pool, the load buffers and the page table) when each has
 *     its own workspace and outputs; page-table uploads and load-buffer fills
 *     are ordered against them as stated at those calls.
 */
#ifndef PMOE_MOE_H
#define PMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, size out of range, bad flag */
#define MOE_ERR_PAGE_RANGE (-2)  /* a page number outside [0, num_pages) */
#define MOE_ERR_PAGE_ALIAS (-3)  /* two expert matrices on one page */
#define MOE_ERR_SLOT_RANGE (-4)  /* a load-buffer slot outside [0, loadbuf_slots) or used twice */
#define MOE_ERR_ALIGN (-5)       /* a device pointer not 16-byte aligned */
#define MOE_ERR_WORKSPACE (-6)   /* workspace or output capacity too small */
#define MOE_ERR_STATE (-7)       /* double-buffer misuse, e.g. reading a never-filled buffer */
#define MOE_ERR_HIP (-8)         /* a HIP runtime call failed */
#define MOE_ERR_UNSUPPORTED (-9) /* shape the kernels do not handle (see moe_pool_desc) */
#define MOE_ERR_NO_SPACE (-10)   /* the page pool cannot serve the request (nothing changed) */

/* kinds of one location-table entry */
#define MOE_LOC_POOL 0    /* idx = {W1 page, W3 page, W2 page} */
#define MOE_LOC_LOADBUF 1 /* idx[0] = slot in the active load buffer; idx[1], idx[2] ignored */

/* forward flags */
#define MOE_FLAG_ATOMIC_COMBINE 1u /* combine the k partial outputs with fp32 atomics
                                      (faster, summation order not reproducible);
                                      default: fixed slot order, bit-reproducible */
#define MOE_FLAG_DEFER_READ_DONE 2u /* moe_paged_forward: record no "buffer read"
                                       event on the stream (a stream marker costs
                                       the GPU ~2 us between forwards); the stream
                                       is remembered instead, and the next fill of
                                       that buffer (or moe_pool_destroy) marks it
                                       there.  The stream must stay alive until
                                       then.  Default: an event after each forward */

typedef struct moe_pool moe_pool; /* opaque handle: one MoE layer's view of the pool */

/*
 * Shape of one MoE layer and where its weights may live.
 *   pool_base       device, bf16, num_pages pages of f*d elements each.  Page p
 *                   starts at element p*f*d.  W1 and W3 pages are [f rows][d]
 *                   (row n of W1 is output column n; contiguous along d).  A W2
 *                   page is [d rows][f] (the pages do not fix the down
 *                   projection's layout; this mirrors W1/W3, contiguous along f).
 *   num_pages       >= 1.
 *   d, f            hidden and intermediate size; each a positive multiple of 64.
 *   num_experts     routed experts E, 1..1024.
 *   top_k           1..min(E, 32).
 *   num_shared      0 or 1.  A shared expert is id E, always chosen with
 *                   weight 1, appended after the k routed picks.
 *   loadbuf_slots   slots per load buffer (0 = no load buffer).  A slot holds
 *                   one expert as 3*f*d bf16: W1, W3, W2 back to back.
 *   loadbuf_base[b] device base of load buffer b (b = 0, 1); may be NULL when
 *                   loadbuf_slots == 0.  The two buffers alternate: one feeds
 *                   this layer while the other receives the next layer's experts.
 */
typedef struct {
    void *pool_base;
    int64_t num_pages;
    int32_t d, f;
    int32_t num_experts;
    int32_t top_k;
    int32_t num_shared;
    int32_t loadbuf_slots;
    void *loadbuf_base[2];
} moe_pool_desc;

/* One location-table entry (16 bytes).  See MOE_LOC_*. */
typedef struct {
    int32_t kind;
    int32_t idx[3];
} moe_expert_loc;

/*
 * Create a layer handle.  Defined by the Rimuru digest, "One pool for data
 * whose sizes differ by orders of magnitude" (one contiguous pool in which an
 * expert matrix fills one page) and "Expert weights are scattered across
 * pages. How does the kernel read them?" (the kernel is told where each expert
 * sits: a page number when it is cached, a slot of one of the two alternating
 * loading buffers when it was just copied in).  Validates desc (MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED / MOE_ERR_ALIGN), then allocates the handle's own small
 * state on the current device: the device copy of the location table
 * (E + S entries), a pinned staging copy, a "filled" hipEvent per load
 * buffer, and, as streams run forwards that read a load buffer, one "read"
 * hipEvent per such stream (reused from fill to fill).  The table starts with every expert unset; a
 * forward before moe_set_expert_locs fails with MOE_ERR_STATE.
 * *out receives the handle; destroy it with moe_pool_destroy.
 */
int moe_pool_create(const moe_pool_desc *desc, moe_pool **out);

/* Release the handle's state.  Waits for the handle's own pending work, and for
 * the work of streams that ran forwards with MOE_FLAG_DEFER_READ_DONE. NULL is a no-op. */
int moe_pool_destroy(moe_pool *pool);

/*
 * Host-only check of a location table against desc; touches no GPU.
 * locs: host array of n = num_experts + num_shared entries.  Errors:
 * MOE_ERR_INVALID_ARG (n or a kind wrong), MOE_ERR_PAGE_RANGE, MOE_ERR_PAGE_ALIAS
 * (a page used twice by any two matrices), MOE_ERR_SLOT_RANGE (slot out of
 * range, or one slot given to two experts).
 */
int moe_validate_locs(const moe_pool_desc *desc, const moe_expert_loc *locs, int32_t n);

/*
 * Point the layer's page table at new locations (the page-table update on the
 * GPU side in the digest's scheduling-round pipeline).  locs: host, n = E + S entries, validated as by
 * moe_validate_locs.  The upload is ordered on `stream`: forwards enqueued on
 * `stream` afterwards see the new table, forwards enqueued before it see the
 * old one.  The caller must order forwards on other streams itself.  The host
 * array may be reused as soon as the call returns.
 */
int moe_set_expert_locs(moe_pool *pool, const moe_expert_loc *locs, int32_t n, void *stream);

/*
 * Capacities the routing outputs need for T tokens and tile height block_m:
 *   *sorted_cap = T*(k+S) + (E+S)*(block_m-1)  entries of sorted_ids
 *   *blocks_cap = ceil(sorted_cap / block_m)   entries of block_expert
 * block_m must be one of 16, 32, 64, 128, 256.
 */
int moe_route_capacity(const moe_pool *pool, int64_t T, int32_t block_m,
                       int64_t *sorted_cap, int64_t *blocks_cap);

/* Bytes of device workspace moe_route and the forwards need for (T, block_m, flags).
 * A workspace may hold anything when a call starts: every call writes each
 * workspace byte before it reads it, and leaves nothing a later call depends
 * on.  Calls that may overlap on the device need separate workspaces. */
int moe_workspace_bytes(const moe_pool *pool, int64_t T, int32_t block_m, uint32_t flags,
                        size_t *bytes);

/*
 * Routing and token alignment, all on the device, no host synchronisation.
 * The digest's "The pipeline: what happens in one scheduling round" (step 5)
 * has the actual routing choose the experts a layer computes; it prints no
 * routing rule, so this is top-k softmax routing renormalised over the picks,
 * and the alignment is the grouping of picks by expert into GEMM-tile blocks
 * of the fused MoE kernel that "Expert weights are scattered across pages. How
 * does the kernel read them?" says the paged kernel is rewritten from.
 *   logits       device fp32 [T][E] router logits (finite values).
 *   topk_ids     device int32 [T][k+S] out: per token the k experts with the
 *                largest logits, largest first, equal logits to the lower id;
 *                then the shared expert id E when S = 1.
 *   topk_w       device fp32 [T][k+S] out: softmax of the chosen logits
 *                renormalised over the k picks; 1.0 for the shared expert.
 *   sorted_ids   device int32 [sorted_cap] out: flat indices i = t*(k+S)+j
 *                grouped by expert (ascending id), ascending i within an
 *                expert, each expert's segment padded with the sentinel T*(k+S)
 *                to a multiple of block_m.  Entries past *num_padded are
 *                unspecified.
 *   block_expert device int32 [blocks_cap] out: expert of each block_m-row block.
 *   num_padded   device int32 [1] out: total rows in sorted_ids (a multiple of block_m).
 *   workspace    device, >= moe_workspace_bytes(pool, T, block_m, 0) bytes.
 */
int moe_route(moe_pool *pool, const float *logits, int64_t T, int32_t block_m,
              int32_t *topk_ids, float *topk_w, int32_t *sorted_ids, int32_t *block_expert,
              int32_t *num_padded, void *workspace, size_t ws_bytes, void *stream);

/*
 * The layer output from the routing above, reading the weights in place.
 * Defined by the digest's "Expert weights are scattered across pages. How does
 * the kernel read them?": the weight of output column n, offset t of expert e
 * is at addr_e(n,t) = B_P + p_e(n)*f*d + (n mod f)*d + t, W1 (gate) for the
 * first half of the fused columns and W3 (up) for the second, W2 (down) as the
 * expert's third page ("The adjuster: when to evict an expert, and which
 * one?"); the page is found once per output tile, then read with fixed
 * strides; an expert just copied in is read from its load-buffer slot.
 *   x            device bf16 [T][d] hidden states.
 *   topk_ids ... num_padded: as produced by moe_route with the same block_m.
 *   active_buf   0 or 1: the load buffer the MOE_LOC_LOADBUF experts are read
 *                from.  The forward waits (on `stream`, via an event) for the
 *                last moe_loadbuf_fill of that buffer, and marks the buffer
 *                consumed when its last read is done (with
 *                MOE_FLAG_DEFER_READ_DONE: when the next fill of the buffer is
 *                enqueued, by an event on `stream` then); a fill waits for
 *                every forward that read the buffer before it was enqueued,
 *                on any number of streams.  It fails with MOE_ERR_STATE if the
 *                table names load-buffer experts and that buffer was never
 *                filled.
 *   y            device bf16 [T][d] out.
 *   workspace    device, >= moe_workspace_bytes(pool, T, block_m, flags) bytes;
 *                holds the SiLU-gated activations [sorted_cap][f] (bf16) and the
 *                combine buffer (bf16 expert output rows [T*(k+S)][d], or an
 *                fp32 [T][d] accumulator with MOE_FLAG_ATOMIC_COMBINE).  Not kept
 *                between calls.
 *   flags        0, MOE_FLAG_ATOMIC_COMBINE, MOE_FLAG_DEFER_READ_DONE, or both.
 * Gate/up GEMM: each output tile resolves its W1 and W3 page bases once and
 * fuses silu(gate) * up into its epilogue (fp32, g * rcp(1 + exp(-g)) * u with
 * the hardware exponential and reciprocal, then rounded to bf16 h); down GEMM: each tile resolves its
 * W2 page once; each expert output row is rounded to bf16, and the k+S rows of
 * a token are scaled by their routing weights and added in fp32 in slot order
 * (bit-reproducible) before the sum is rounded to bf16.  With
 * MOE_FLAG_ATOMIC_COMBINE the down tiles add weighted fp32 rows into the
 * accumulator instead (order not fixed).
 */
int moe_paged_forward(moe_pool *pool, const void *x, int64_t T, int32_t block_m,
                      const int32_t *topk_ids, const float *topk_w, const int32_t *sorted_ids,
                      const int32_t *block_expert, const int32_t *num_padded, int32_t active_buf,
                      void *y, void *workspace, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * Routing and the layer output in one call (moe_route followed by
 * moe_paged_forward, with the same arguments and the same outputs, bit for
 * bit).  For the few tokens of a decode step (T <= 4, T <= block_m, and the
 * shapes of the decode form, see moe_forward_form) the routing runs inside the
 * gate/up launch: every workgroup of it routes the tokens itself and takes its
 * expert from the result, so the step needs two launches instead of three.
 * Larger batches run the routing kernels, then the forward.
 *   logits       device fp32 [T][E] router logits (finite values).
 *   topk_ids ... num_padded: out, as moe_route writes them.
 *   x, active_buf, y, workspace, flags: as moe_paged_forward.
 * HIP graph capture: the call enqueues kernel launches only (no memset, no
 * allocation, no copy) when stage timing is off, the table reads no load
 * buffer or the active buffer's last fill has completed before the call, and
 * MOE_FLAG_DEFER_READ_DONE is set; so enqueued on a capturing stream, it
 * records the step, and replays of the graph recompute every output from the
 * inputs at the same addresses (a fill-completion check is made at capture:
 * capture in relaxed or thread-local mode).  A replay is outside the load
 * buffer's fill / read events: the caller orders fills of the active buffer
 * against replays.
 */
int moe_route_forward(moe_pool *pool, const float *logits, const void *x, int64_t T, int32_t block_m,
                      int32_t *topk_ids, float *topk_w, int32_t *sorted_ids, int32_t *block_expert,
                      int32_t *num_padded, int32_t active_buf, void *y, void *workspace,
                      size_t ws_bytes, uint32_t flags, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as moe_route_forward, same outputs bit for bit, with its workspace in a
 * static device array of the library instead of a caller's allocation.  The
 * array holds MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on every device the library
 * runs on, from the first call on that device until the process ends; the call
 * allocates no device memory.  A (T, block_m, flags) whose
 * moe_workspace_bytes exceeds it fails with MOE_ERR_WORKSPACE (256-row tiles
 * alone need 64 MiB of partial tiles: use block_m <= 128 here).  All calls on
 * one device share that device's array: calls that may overlap in time on one
 * device (other streams, other threads) race and must be ordered by the
 * caller.  Nothing in the array has to start at zero, so what an earlier call
 * left there does not matter.  Arguments and errors otherwise as
 * moe_route_forward.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_route_forward_noalloc(moe_pool *pool, const float *logits, const void *x, int64_t T, int32_t block_m,
                              int32_t *topk_ids, float *topk_w, int32_t *sorted_ids, int32_t *block_expert,
                              int32_t *num_padded, int32_t active_buf, void *y, uint32_t flags, void *stream);

/*
 * moe_route_forward with the weights in the two dense arrays of
 * moe_contiguous_forward (the contiguous baseline of the one-call step; same
 * kernels and launches, only the per-tile base address differs).
 */
int moe_route_contiguous_forward(const moe_pool *pool, const void *w13, const void *w2,
                                 const float *logits, const void *x, int64_t T, int32_t block_m,
                                 int32_t *topk_ids, float *topk_w, int32_t *sorted_ids,
                                 int32_t *block_expert, int32_t *num_padded, void *y,
                                 void *workspace, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * The same layer with the weights in two dense arrays (the contiguous
 * baseline the paged kernel is measured against, as in the last paragraph of
 * the digest's "Expert weights are scattered across pages. How does the
 * kernel read them?": the same inputs and routing through both kernels; same kernels and tile
 * schedule, only the per-tile base address differs, so results are
 * bit-identical to moe_paged_forward for the same weights).
 *   w13  device bf16 [E+S][2f][d]: rows [0,f) W1, rows [f,2f) W3 of each expert.
 *   w2   device bf16 [E+S][d][f].
 * The pool handle supplies the shape only; its page table is not read.
 */
int moe_contiguous_forward(const moe_pool *pool, const void *w13, const void *w2, const void *x,
                           int64_t T, int32_t block_m, const int32_t *topk_ids,
                           const float *topk_w, const int32_t *sorted_ids,
                           const int32_t *block_expert, const int32_t *num_padded, void *y,
                           void *workspace, size_t ws_bytes, uint32_t flags, void *stream);

/*
 * Fill slots of load buffer `buf` from pinned host memory on `copy_stream`
 * (the digest's double-buffered loading: this layer computes from one buffer
 * while the other receives the next layer's experts).
 *   slots[i]     slot to fill (host int32, n entries, distinct).
 *   host_src[i]  pinned host, 3*f*d bf16 (W1, W3, W2 back to back).
 * The copies wait for the last forward that read `buf` (write-after-read) and
 * for earlier fills of `buf`; the buffer's "filled" event is recorded after
 * them, and the next forward reading `buf` waits for it (read-after-write).
 * Forwards of `buf` run with MOE_FLAG_DEFER_READ_DONE are waited for by an
 * event recorded now on each stream they ran on, which covers everything
 * enqueued on that stream so far (never less than those forwards).
 */
int moe_loadbuf_fill(moe_pool *pool, int32_t buf, int32_t n, const int32_t *slots,
                     const void *const *host_src, void *copy_stream);

/*
 * Resolve weight addresses on the device with the same per-tile resolver the
 * GEMM kernels use, for checking against the address formula of the digest's
 * "Expert weights are scattered across pages. How does the kernel read them?",
 * addr_e(n,t) = B_P + p_e(n)*f*d + (n mod f)*d + t, p_e(n) the W1 page for
 * n < f and the W3 page otherwise (W2: the reading stated at moe_pool_desc;
 * load-buffer slots: the same formula from the buffer base with page 3s + m).
 *   e, which, row, col  device int32/int32/int64/int64 [n] queries:
 *       which 0: gate/up operand, row = output column n in [0, 2f), col = t in [0, d)
 *       which 1: down projection, row in [0, d), col in [0, f)
 *   off   device int64 [n] out: element offset from the base below
 *   base  device int32 [n] out: 0 = pool_base, 1 + b = loadbuf_base[b]; -1 for
 *         a query out of range (off = -1)
 *   active_buf selects the load buffer for MOE_LOC_LOADBUF experts.
 */
int moe_resolve_addrs(moe_pool *pool, int32_t active_buf, int64_t n, const int32_t *e,
                      const int32_t *which, const int64_t *row, const int64_t *col,
                      int64_t *off, int32_t *base, void *stream);

/*
 * A block_m for T tokens: the tile height that covers the expected rows per
 * active expert ((T*(k+S)) / min(T*(k+S), E+S)) in few tiles without mostly
 * padding: 16, 32 or 64 up to that many rows, 256 from 512 rows on (when d is
 * a multiple of 256 and f of 128), else 128.  Any of 16, 32, 64, 128, 256 is
 * valid for every entry point.
 */
int32_t moe_suggest_block_m(const moe_pool *pool, int64_t T);

/*
 * Which form of the two GEMMs a forward of T tokens takes (the same for every
 * block_m and for paged and contiguous weights):
 *   MOE_FORM_TILES   MFMA tiles over the aligned blocks, then the combine;
 *   MOE_FORM_DECODE  for 1..8 tokens with d <= 4096 and f <= 2048 (and at most
 *                    64 picks per token): each weight row is read once
 *                    and dotted on the vector ALUs with the x rows of the picks
 *                    of its expert block; the down projection adds the token's
 *                    picks in slot order and writes y directly (no combine
 *                    pass; MOE_FLAG_ATOMIC_COMBINE has no effect).
 * MOE_ERR_INVALID_ARG for a NULL pool or T < 0.
 */
#define MOE_FORM_TILES 0
#define MOE_FORM_DECODE 1
int32_t moe_forward_form(const moe_pool *pool, int64_t T);

/*
 * Which launches moe_route_forward makes for T tokens: MOE_FORM_DECODE_ROUTED
 * when the routing runs inside the decode form's gate/up launch (two launches
 * in all), else the form of moe_forward_form, after the routing kernels.
 * MOE_ERR_INVALID_ARG for a NULL pool or T < 0.
 */
#define MOE_FORM_DECODE_ROUTED 2
int32_t moe_route_forward_form(const moe_pool *pool, int64_t T);

/*
 * Stage timing of paged forwards, for measurement.  With enable != 0 every
 * moe_paged_forward of this handle records four hipEvents on its stream:
 * before the gate/up GEMM, after it, after the down GEMM and after the
 * combine (at most 1024 forwards are recorded; later ones run untimed).
 * moe_stage_times waits for the recorded forwards, writes the summed
 * milliseconds of the three stages to ms[0..2] (gate/up, down, combine) and
 * their number to *count, and starts a new recording.  enable = 0 stops
 * recording.  The events add a marker between kernels; time the whole
 * forward with recording off.
 */
int moe_stage_timing(moe_pool *pool, int32_t enable);
int moe_stage_times(moe_pool *pool, float *ms, int32_t *count);

/* ---------------------------------------------------------------- adjuster
 * Host-side policy of the digest's section "The adjuster: when to evict an
 * expert, and which one?", run once per scheduling round after the scheduler
 * has placed requests.  All pointers are host memory; nothing touches the
 * GPU.
 */

/*
 * How many experts to evict or add in this scheduling round.  short_pages: expert pages the
 * scheduler is short of (R_b); free_pages: free expert pages (F_b).  An expert
 * holds 3 expert pages.  R_b > 0: *n_evict = ceil((R_b + 1) / 3).  Else
 * F_b < 2: *n_evict = 1.  Else F_b > 9: *n_add = min(5, floor((F_b - 9) / 3)).
 * Else both 0.  MOE_ERR_INVALID_ARG for negative counts or null outputs.
 */
int moe_adjust_amounts(int32_t short_pages, int32_t free_pages, int32_t *n_evict, int32_t *n_add);

/*
 * Offline hot-expert ranking of one layer from sample routing.  topk_ids
 * [T][k] (as written by moe_route, k = top_k + num_shared); ids outside
 * [0, E) (the shared expert) are not ranked.  ranking[E] receives the expert
 * ids by descending routing probability (count / T; ties to the lower id),
 * prob[E] the probabilities in the same order.
 */
int moe_rank_experts(const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t *ranking, float *prob);

/*
 * Which experts: the change list of one round.  ranking / prob: [L][E] per-layer
 * rankings and their probabilities (rows of moe_rank_experts); resident[L]:
 * the number of top-ranked experts each layer keeps on the GPU, updated in
 * place.  offload_limit: a layer that already offloads this many experts
 * (E - resident[l] >= offload_limit) is left out of shrinking.  Exactly one of
 * n_evict, n_add may be > 0 (a round shrinks or grows).  Experts are decided
 * one at a time: growing, each layer nominates ranking[l][resident[l]] and the
 * highest probability wins; shrinking, each layer nominates
 * ranking[l][resident[l] - 1] and the lowest wins; ties go to the lower layer.
 * out_layer / out_expert / out_add (1 add, 0 evict) receive the decisions in
 * order (capacity n_evict + n_add), *n_out their number (fewer when no layer
 * can nominate).  MOE_ERR_INVALID_ARG for bad sizes, a ranking row that is not
 * a permutation of [0, E), or resident[l] outside [0, E].
 */
int moe_adjust_select(int32_t L, int32_t E, const int32_t *ranking, const float *prob, int32_t *resident,
                      int32_t offload_limit, int32_t n_evict, int32_t n_add, int32_t *out_layer,
                      int32_t *out_expert, int32_t *out_add, int32_t *n_out);

/* ---------------------------------------------------------------- multi-layer pipeline
 * One forward pass over L MoE layers, following the digest's sections "The
 * pipeline: what happens in one scheduling round" (two loading buffers that
 * alternate between layers) and the ordering rules at the end of "The
 * adjuster: when to evict an expert, and which one?" (copy before the page
 * table changes; compute before pages are reclaimed).
 *
 * The layers are moe_pool handles over ONE pool (same pool_base, num_pages,
 * d, f, loadbuf_slots and load buffers), each with its table set and no two
 * tables naming one page.  Layer l reads load buffer l % 2, so the fill for
 * layer l + 1 overlaps the forward of layer l.  The pipeline does not own the
 * handles: destroy it before them, and change their tables only through
 * moe_pipeline_stage_table while it exists.  All forwards run on one stream
 * (the first forward fixes it); fills, page copies and table uploads run on
 * copy_stream.  Each layer gets a second device table (16 bytes per expert)
 * and a pinned staging copy: a staged table is uploaded into the second one
 * with its page copies, and the switch exchanges the two.
 */
typedef struct moe_pipeline moe_pipeline;

/* MOE_ERR_INVALID_ARG (handles null, repeated, on other devices or over other
 * pools / buffers), MOE_ERR_STATE (a handle without a table),
 * MOE_ERR_PAGE_ALIAS (two tables share a page). */
int moe_pipeline_create(int32_t L, moe_pool *const *layers, void *copy_stream, moe_pipeline **out);

/* Waits for the pipeline's pending copies and reads, then frees it.  NULL is a no-op. */
int moe_pipeline_destroy(moe_pipeline *pipe);

/*
 * Stage one change of layer `layer`'s table: locs (host, n = E + S entries,
 * validated as by moe_validate_locs) replaces the table at the layer's next
 * moe_pipeline_forward.  copy_expert[i] (host, n_copy entries, distinct) is
 * an expert the new table places in pool pages that it newly receives;
 * copy_src[i] (pinned host, 3*f*d bf16: W1, W3, W2 back to back) is copied
 * into those three pages now, on copy_stream, after the upload of the table
 * itself; the forward that switches tables waits for all of them first.  The
 * call blocks the host only while this layer's previous change is still
 * being uploaded.  Pages the current table names but
 * the new one does not are dropped: moe_pipeline_reclaim reports them once
 * every forward enqueued before the switch has finished.
 * Errors: MOE_ERR_STATE (the layer already has a change waiting);
 * MOE_ERR_PAGE_ALIAS (a copy target the current table reads; a page another
 * layer's current or staged table names; a dropped page not yet reclaimable);
 * MOE_ERR_INVALID_ARG (a copied expert not placed in the pool by locs, listed
 * twice, or a source that is not pinned host memory).  Nothing is enqueued
 * on an error.
 */
int moe_pipeline_stage_table(moe_pipeline *pipe, int32_t layer, const moe_expert_loc *locs, int32_t n,
                             int32_t n_copy, const int32_t *copy_expert, const void *const *copy_src);

/*
 * Fill slots of load buffer layer % 2 for layer `layer` (as moe_loadbuf_fill:
 * slots distinct, host_src pinned, 3*f*d bf16 each).  The copies wait on
 * copy_stream for the last forward that read the buffer.  MOE_ERR_STATE if
 * the buffer still holds experts filled for another layer that has not run
 * since.
 */
int moe_pipeline_prefetch(moe_pipeline *pipe, int32_t layer, int32_t n, const int32_t *slots,
                          const void *const *host_src);

/*
 * The paged forward of layer `layer` (arguments as moe_paged_forward, the
 * load buffer being layer % 2).  Applies a staged table first: the stream
 * waits for its upload and page copies, then the layer reads the new table
 * (no copy on the forward stream).  MOE_ERR_STATE if
 * the table reads the load buffer and the buffer's last fill was for another
 * layer; MOE_ERR_INVALID_ARG for a stream other than the pipeline's.
 */
int moe_pipeline_forward(moe_pipeline *pipe, int32_t layer, const void *x, int64_t T, int32_t block_m,
                         const int32_t *topk_ids, const float *topk_w, const int32_t *sorted_ids,
                         const int32_t *block_expert, const int32_t *num_padded, void *y, void *ws,
                         size_t ws_bytes, uint32_t flags, void *stream);

/*
 * Non-blocking: writes up to cap dropped pages that may be reused (every
 * forward that could read them has finished) to pages[] and their number to
 * *n; pages beyond cap are reported by the next call.
 */
int moe_pipeline_reclaim(moe_pipeline *pipe, int32_t *pages, int32_t cap, int32_t *n);

/* ---------------------------------------------------------------- three-tier page pool
 * Host-side allocator of the digest's section "One pool for data whose sizes
 * differ by orders of magnitude".  The pool is one byte range seen through a
 * view per page kind: page i of a kind of B bytes covers bytes [i*B, (i+1)*B),
 * so an expert page index is the page number moe_expert_loc takes (with
 * expert_page_bytes = f*d*2) and a KV page index addresses the KV cache view
 * of the same bytes.
 *
 * Tiers: huge pages of lcm(expert, SSM) bytes (the expert page without SSM
 * layers) split into expert or SSM pages; an expert page splits into KV or
 * convolution-state pages (small pages are carved from expert pages only, so
 * their sizes must divide the expert page).  A small-page request takes, in
 * order: a free slot of an expert page that already holds pages of the same
 * request (same-request packing; off with MOE_ALLOC_NO_PACKING), a free slot
 * of any split page of that kind, a free expert page split now, a free huge
 * page split into expert pages now.  Expert and SSM requests take a free page
 * of their kind, else split a free huge page.  Among equals the lowest index
 * wins.  Frees merge upward at once: an expert page whose small pages are all
 * free becomes a free expert page, and a huge page whose pages are all free
 * returns to the pool.  Requests for n pages are all or nothing
 * (MOE_ERR_NO_SPACE leaves the pool unchanged).  Not thread-safe: one caller
 * at a time per allocator.  No call touches the GPU.
 */
typedef struct moe_alloc moe_alloc;

#define MOE_PAGE_KV 0
#define MOE_PAGE_CONV 1
#define MOE_ALLOC_NO_PACKING 1u

typedef struct {
    int64_t pool_bytes;        /* a whole number of huge pages */
    int64_t expert_page_bytes; /* > 0 */
    int64_t ssm_page_bytes;    /* 0: no SSM pages */
    int64_t kv_page_bytes;     /* > 0, divides expert_page_bytes */
    int64_t conv_page_bytes;   /* 0: no convolution-state pages; else divides expert_page_bytes */
    uint32_t flags;            /* MOE_ALLOC_NO_PACKING */
} moe_alloc_desc;

typedef struct {
    int64_t huge_bytes, n_huge;
    int64_t free_huge;                    /* whole huge pages */
    int64_t free_expert, used_expert;     /* expert pages of split huge pages */
    int64_t free_ssm, used_ssm;
    int64_t split[2];                     /* expert pages split into KV / conv pages */
    int64_t used_small[2], free_small[2]; /* small pages inside those split pages */
    int64_t expert_available;             /* free_expert + free_huge * (huge / expert page) */
    int64_t trapped_bytes;                /* free small pages that cannot hold an expert yet */
} moe_alloc_stats;

/* MOE_ERR_INVALID_ARG for sizes that break the rules above or unknown flags. */
int moe_alloc_create(const moe_alloc_desc *desc, moe_alloc **out);
int moe_alloc_destroy(moe_alloc *a); /* NULL is a no-op */

/* n pages into pages[n] (host).  Frees take distinct allocated pages of that
 * kind (MOE_ERR_INVALID_ARG otherwise, with nothing freed). */
int moe_alloc_expert_pages(moe_alloc *a, int32_t n, int64_t *pages);
int moe_free_expert_pages(moe_alloc *a, int32_t n, const int64_t *pages);
int moe_alloc_ssm_pages(moe_alloc *a, int32_t n, int64_t *pages);
int moe_free_ssm_pages(moe_alloc *a, int32_t n, const int64_t *pages);

/* kind: MOE_PAGE_KV or MOE_PAGE_CONV; request >= 0 names the owner (packing). */
int moe_alloc_small_pages(moe_alloc *a, int32_t kind, int64_t request, int32_t n, int64_t *pages);
int moe_free_small_pages(moe_alloc *a, int32_t kind, int32_t n, const int64_t *pages);

/* Free every small page of one request (KV, then conv, ascending). */
int moe_free_request(moe_alloc *a, int64_t request, int64_t *n_freed);

int moe_alloc_get_stats(const moe_alloc *a, moe_alloc_stats *stats);

/* ---------------------------------------------------------------- remapped expert views
 * The PagedTensor alternative of the wiki page "FluxMoE: Decoupling Expert
 * Residency for High-Performance MoE Serving" (core method): instead of a page
 * lookup inside the kernel, every expert matrix gets a fixed virtual address
 * and the GPU's page tables point it at whichever physical page holds the
 * matrix, so the contiguous kernels run unchanged.
 *
 * moe_vmm_create makes num_pages + 6*loadbuf_slots physical allocations of
 * page_bytes (= f*d*2; must be a multiple of the device's mapping
 * granularity, else MOE_ERR_UNSUPPORTED, as is a device without virtual memory
 * management) and maps each into a contiguous view: the pool (page p at
 * p*page_bytes) and two load buffers (slot s holds W1, W3, W2 at
 * (3s + m)*page_bytes).  Those views are ordinary device memory for every entry
 * point above: use them as moe_pool_desc.pool_base and loadbuf_base[b].  It
 * also reserves the expert views w13 [E+S][2f][d] and w2 [E+S][d][f], which
 * stay unmapped until moe_vmm_map_experts.
 */
typedef struct moe_vmm moe_vmm;

int moe_vmm_create(int64_t page_bytes, int64_t num_pages, int32_t loadbuf_slots, int32_t n_experts_total,
                   moe_vmm **out);

/* Waits for the whole device, unmaps and frees everything.  NULL is a no-op. */
int moe_vmm_destroy(moe_vmm *vmm);

/* Device addresses of the views (any output may be NULL).  w13 and w2 are NULL
 * until a moe_vmm_map_experts call has succeeded. */
int moe_vmm_views(const moe_vmm *vmm, void **pool_base, void **loadbuf0, void **loadbuf1, void **w13,
                  void **w2);

/* The device's minimum mapping granularity (page_bytes is a multiple of it)
 * and the recommended one (the alignment of every view). */
int moe_vmm_granularity(const moe_vmm *vmm, int64_t *minimum, int64_t *recommended);

/*
 * Point the expert views at the pages a location table names (host, all
 * n = E + S experts; load-buffer experts at the slots of buffer active_buf).
 * Validation as moe_validate_locs, before anything changes.  The call first
 * synchronises `stream`: every forward that reads the views must run on it
 * (or have finished), because a view page is re-pointed in place.  Only view
 * pages whose physical page changes are remapped; *n_remapped (may be NULL)
 * receives their number.  MOE_ERR_HIP from a mapping call leaves the views
 * unusable (MOE_ERR_STATE afterwards): destroy the object.
 */
int moe_vmm_map_experts(moe_vmm *vmm, const moe_expert_loc *locs, int32_t n, int32_t active_buf, void *stream,
                        int32_t *n_remapped);

/* The contiguous forward over the expert views (arguments as
 * moe_contiguous_forward).  MOE_ERR_STATE until the views are fully mapped;
 * MOE_ERR_INVALID_ARG if the layer handle's E + S or f*d*2 differ.
 * When the mapped table places experts in load buffer b (the active_buf of the
 * last moe_vmm_map_experts), `pool` must be the layer handle whose load buffers
 * are this object's views (its fills write them, MOE_ERR_INVALID_ARG
 * otherwise), and the forward keeps that handle's double-buffer protocol as
 * moe_paged_forward does: it waits on `stream` for the last moe_loadbuf_fill
 * of buffer b (MOE_ERR_STATE if b was never filled) and marks b read after its
 * kernels, so the next fill of b waits for it; flags as moe_paged_forward
 * (MOE_FLAG_ATOMIC_COMBINE, MOE_FLAG_DEFER_READ_DONE). */
int moe_vmm_forward(const moe_vmm *vmm, moe_pool *pool, const void *x, int64_t T, int32_t block_m,
                    const int32_t *topk_ids, const float *topk_w, const int32_t *sorted_ids,
                    const int32_t *block_expert, const int32_t *num_padded, void *y, void *ws,
                    size_t ws_bytes, uint32_t flags, void *stream);

/* Message for the last non-zero return on this thread ("" if none). */
const char *moe_last_error(void);

/* ABI version (major*100 + minor). */
int moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PMOE_MOE_H */
