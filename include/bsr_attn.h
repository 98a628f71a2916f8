/*
 * bsr_attn.h — C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * The operation is softmax attention restricted by a block-sparse-row (BSR)
 * mask of 128 x 128 tiles, forward and backward:
 *
 *   forward   S = scale * Q K^T on the stored blocks only; an online (running
 *             max / running sum) softmax per query row; O = P V. Returns O and
 *             the fp32 row statistics row_max (max of the scaled scores of the
 *             row) and row_denom (sum over the row of exp(score - row_max)),
 *             so that P = exp(S - row_max) / row_denom.
 *             Pages: "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0 (one launch,
 *             statistics kept on chip, no host reduction) and 0.9.0 (bf16
 *             operands with fp32 accumulation, fp32 statistics);
 *             "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.4.3/0.4.4 (per-row max
 *             and sum of exponentials, stable softmax) and 0.5.1
 *             (return_stats returns (out, row_max, row_denom)).
 *   backward  D = rowsum(dO * O) (the delta identity, CHANGELOG 0.5.0);
 *             dQ row-first: dQ_I += scale * dS K_J over the stored blocks of
 *             block row I; dK/dV column-first over the transposed (BSC)
 *             structure: dK_J += scale * dS^T Q_I, dV_J += P^T dO_I over the
 *             block rows I that store block column J (CHANGELOG 0.5.1), with
 *             the forward's row statistics reused instead of recomputed.
 *             Every output tile has exactly one writer; no atomics.
 *   head_dim above 128 is tiled in chunks of the contraction
 *             ("trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.6.0); at head_dim
 *             512 the forward runs in two passes (statistics, then output)
 *             and the backward materialises its P and dS blocks in the
 *             workspace and runs its products over the stored blocks.
 *
 * The mask is block-granular: every element of a stored block is attended
 * (the pages' benchmark expands the block mask by the block size on both
 * axes). One structure is shared by every (batch, head).
 *
 * Conventions
 *   - Dense tensors are contiguous row-major [batch, heads, seq_len, head_dim]
 *     in device memory; row statistics are [batch, heads, seq_len] fp32.
 *   - All dense operands of one call have the same dtype (fp32, bf16 or
 *     fp16; the pages run bf16 and fp16 operands with fp32 statistics,
 *     "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.9.0).
 *     bf16 runs bf16 matrix products with fp32 accumulation; softmax and the
 *     statistics are fp32; O, dQ, dK, dV are written in the operand dtype.
 *   - The caller owns every device buffer (operands, outputs, the device copy
 *     of the plan, the workspace). The library never allocates device memory
 *     and never synchronises: fwd/bwd enqueue kernels on `stream` (a
 *     hipStream_t, NULL = the default stream) and return.
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error has launched nothing.
 *   - Errors are status codes; bsr_attn_last_error() describes the last
 *     failure of the calling thread.
 */
#ifndef BSR_ATTN_H
#define BSR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSR_ATTN_OK = 0,
    BSR_ATTN_ERR_INVALID_ARGUMENT = 1, /* malformed structure, null pointer, bad size */
    BSR_ATTN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head_dim 40) */
    BSR_ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
    BSR_ATTN_ERR_HIP = 4,              /* a HIP launch failed; see bsr_attn_last_error */
    BSR_ATTN_ERR_HOST_ALLOC = 5
} bsr_attn_status;

typedef enum { BSR_ATTN_F32 = 0, BSR_ATTN_BF16 = 1, BSR_ATTN_F16 = 2 } bsr_attn_dtype;

/* Host-side; its plan is immutable after build and it may be shared between
 * threads and streams (binding device plans is internally synchronised). */
typedef struct bsr_attn_structure bsr_attn_structure;

typedef struct {
    int32_t batch, heads, seq_len, head_dim;
    int32_t dtype;  /* bsr_attn_dtype */
    float scale;    /* softmax scale, finite and > 0 (1/sqrt(head_dim) is usual) */
} bsr_attn_problem;

/* Summary of a built structure (for callers and tests). */
typedef struct {
    int32_t n_block_rows;   /* nb; seq_len must be nb * block_size */
    int32_t nnzb;           /* stored blocks */
    int32_t split_threshold;/* longest work item, in stored blocks */
    int32_t n_row_items;    /* forward / dQ work items (row segments, incl. empty rows) */
    int32_t n_col_items;    /* dK/dV work items (column segments, incl. empty columns) */
    int32_t n_row_merges;   /* block rows split into more than one segment */
    int32_t n_col_merges;   /* block columns split into more than one segment */
    int32_t n_row_slots;    /* partial-result slots for split rows */
    int32_t n_col_slots;    /* partial-result slots for split columns */
    int32_t max_row_blocks; /* longest block row */
    int32_t max_col_blocks; /* longest block column */
    int32_t fine_split_threshold; /* the finer split's threshold (0: none; see bsr_attn_fwd) */
    int32_t fine_n_row_items;     /* the finer split's forward / dQ work items (0: none) */
} bsr_attn_structure_info;

/*
 * Validate a BSR block structure and build the work plan.
 *
 *   n_block_rows    nb >= 1 (square: nb block rows and nb block columns).
 *   row_ptr         host int32[nb + 1]: row_ptr[0] == 0, non-decreasing,
 *                   row_ptr[nb] == nnzb.
 *   col_idx         host int32[nnzb]: block column of each stored block,
 *                   in [0, nb), strictly ascending within each block row.
 *                   May be NULL when nnzb == 0.
 *   block_size      must be 128.
 *   split_threshold a block row (column) with more stored blocks than this is
 *                   processed as several segments of at most this many blocks
 *                   whose fp32 partial results are merged (log-sum-exp merge
 *                   in the forward, fixed-order sums in the backward), so that
 *                   one long row cannot serialise the launch. 0 = automatic:
 *                   max(4, ceil(1.5 * ceil(nnzb / nb))), raised to the
 *                   longest line when that is at most one block longer (so
 *                   such a structure has no split at all). With 0 the
 *                   structure also carries a finer split, at threshold
 *                   max(1, ceil(nnzb / 256)) when that is smaller, which
 *                   launches over few (batch, head) pairs use: those whose
 *                   batch * heads * (forward work items of the automatic
 *                   split) is at most 64, e.g. one head of four block rows.
 *                   The choice depends only on the structure and batch *
 *                   heads; results differ only by summation order.
 *   out             receives the new structure (owned by the caller; free it
 *                   with bsr_attn_destroy_structure).
 *
 * Host only: no HIP call. Source of the structure's form: the pages' BSR
 * matrix (block_row_ptrs, block_col_indices, 128-blocks) built from a boolean
 * block mask ("trnsparse 0.7.0 -> 0.9.0", benchmarks/bench_native_trn2.py);
 * the host-side transpose (BSC) of "trnsparse 0.4.1 -> 0.6.0" CHANGELOG 0.5.1;
 * the split balanced by stored blocks with one writer per output tile of
 * "trnsparse 0.7.0 -> 0.9.0" CHANGELOG 0.9.0.
 */
bsr_attn_status bsr_attn_build_structure(int32_t n_block_rows, const int32_t *row_ptr,
                                         const int32_t *col_idx, int32_t block_size,
                                         int32_t split_threshold, bsr_attn_structure **out);

void bsr_attn_destroy_structure(bsr_attn_structure *s);

bsr_attn_status bsr_attn_structure_get_info(const bsr_attn_structure *s,
                                            bsr_attn_structure_info *info);

/*
 * The plan: an int32 array the kernels read. The caller copies the packed
 * bytes to device memory once (e.g. into a torch tensor), binds that device
 * copy to the structure (bsr_attn_structure_bind_plan), and passes it as
 * `d_plan` to fwd/bwd together with the same structure.
 * Layout (all int32, offsets in int32 units from the start):
 *   [0..23]  header: magic 0x42535241, version 5, nb, nnzb, n_row_items,
 *            n_col_items, n_row_merges, n_col_merges, n_row_slots,
 *            n_col_slots, off_col_idx, off_row_idx, off_row_items,
 *            off_col_items, off_row_merges, off_col_merges, off_row_ptr,
 *            off_col_ptr, off_row_queues, off_col_queues, off_bsc_block,
 *            off_fine_plan, then 2 zeros
 *   col_idx[nnzb]           the BSR block columns, row by row
 *   row_idx[nnzb]           the BSC block rows, column by column (ascending)
 *   row_items[n_row_items][4]  {block row, first, end (into col_idx), slot}
 *   col_items[n_col_items][4]  {block col, first, end (into row_idx), slot}
 *                           slot -1 = write the output directly; otherwise
 *                           the partial-result slot of this segment.
 *                           Items are ordered longest first.
 *   row_merges[n_row_merges][4] {block row, first slot, slot count, 0}
 *   col_merges[n_col_merges][4] {block col, first slot, slot count, 0}
 *   row_ptr[nb + 1]         the BSR row pointers
 *   col_ptr[nb + 1]         the BSC column pointers
 *   row_queues[8], col_queues[8]  offsets of 7 work-queue schedules of the
 *                           row (column) items of one head, for n = 1, 2, 4,
 *                           ..., 64 queues; 8th entry 0. Schedule for n
 *                           queues: n + 1 offsets, then the item indices
 *                           queue by queue (queue q holds entries
 *                           [off[q], off[q+1]) of that list). Items go, in
 *                           order, to the queue with the least work so far.
 *   bsc_block[nnzb]         for each BSC entry, the position of the same
 *                           block in col_idx (its BSR index)
 *   the finer split's plan  at off_fine_plan when there is one (0 = none):
 *                           a complete plan of this layout, offsets relative
 *                           to its own start, whose own off_fine_plan is 0
 *   Every array starts at a multiple of 4 int32 (16 bytes).
 */
size_t bsr_attn_structure_plan_bytes(const bsr_attn_structure *s);
bsr_attn_status bsr_attn_structure_pack(const bsr_attn_structure *s, void *host_dst, size_t bytes);

/*
 * Bind a device copy of the packed plan to its structure. fwd, bwd, their
 * variants and bsr_spmm take as d_plan only a pointer bound to the structure
 * they are given, and otherwise return BSR_ATTN_ERR_INVALID_ARGUMENT before
 * anything is enqueued, so that a plan packed from another structure (whose
 * offsets the kernels would follow out of bounds) is never read.
 *   d_plan  device pointer, 16-byte aligned, holding the
 *           bsr_attn_structure_plan_bytes(s) bytes bsr_attn_structure_pack
 *           wrote (the library cannot read device memory to check them; the
 *           caller copies them before the first call that uses d_plan).
 *   bytes   must equal bsr_attn_structure_plan_bytes(s).
 * Host bookkeeping only (no HIP call). Several copies may be bound (one per
 * device, at most 64); binding a bound pointer again is a no-op. Unbind a
 * copy before freeing its memory: a later allocation at the same address
 * would otherwise be accepted. Thread-safe.
 */
bsr_attn_status bsr_attn_structure_bind_plan(bsr_attn_structure *s, const void *d_plan, size_t bytes);
bsr_attn_status bsr_attn_structure_unbind_plan(bsr_attn_structure *s, const void *d_plan);

/*
 * Device workspace (bytes) fwd (backward = 0), bwd (backward = 1) or bwd_ds
 * (backward = 2) needs for this structure and problem (for the split the
 * problem's batch * heads runs on); 0 if none. Returns 0
 * for an invalid problem. bwd_ds adds, after bwd's own, the stored dS:
 * [B*H][nnzb][128][128] in p->dtype (0 for fp32, which it does not take).
 * At head_dim 512 (and the widths padded to it) the forward needs what it
 * needs at the other widths, and the backward materialises its gradient
 * blocks: P and dS in p->dtype, each [B*H][nnzb][128][128], fp32 delta and
 * lse2 per row, and fp32 partials of split rows and columns; bwd and bwd_ds
 * then need the same workspace.
 * Forward: fp32 partial (O, reference max, sum, row max) per split-row
 * slot. Backward: fp32
 * delta and log-sum-exp per row, plus fp32 partial dQ / dK / dV per slot.
 * A head dim that runs padded (see bsr_attn_fwd) adds, after those, its
 * zero-padded operand copies: [B*H*S, width] each, 4 for the forward
 * (Q, K, V, O) and 8 for the backward (Q, K, V, O, dO, dQ, dK, dV).
 */
size_t bsr_attn_workspace_bytes(const bsr_attn_structure *s, const bsr_attn_problem *p,
                                int backward);

/*
 * Forward. q, k, v: device [B, H, S, D] in p->dtype. Writes o (same shape and
 * dtype), row_max and row_denom (device fp32 [B, H, S]). A query row whose
 * block row stores no block gets o = 0, row_max = -inf, row_denom = 0.
 * workspace: device, at least bsr_attn_workspace_bytes(s, p, 0) bytes (may be
 * NULL if that is 0). Supported: head_dim any multiple of 16 up to 512 (bf16,
 * fp16) or 128 (fp32); anything else returns BSR_ATTN_ERR_UNSUPPORTED. The
 * kernels are built for head_dim 32, 64, 128, 256 and 512 (fp32: up to 128); any
 * other supported head_dim runs at the next of those widths on copies of the
 * operands with zero-filled columns (in the workspace), and only the real
 * columns of the outputs are written back. The zero columns add nothing to
 * any score and give zero output columns, so the result is that of the
 * unpadded problem; the cost is the wider matrix work and the copies. At
 * head_dim 512 (16-bit) this entry point runs the two-pass form below: its
 * output accumulator then takes every matrix register of a wave and is never
 * rescaled.
 */
bsr_attn_status bsr_attn_fwd(const bsr_attn_structure *s, const void *d_plan,
                             const bsr_attn_problem *p, const void *q, const void *k,
                             const void *v, void *o, float *row_max, float *row_denom,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same forward as the pages' two-pass form ("trnsparse 0.4.1 -> 0.6.0",
 * CHANGELOG 0.4.3 and 0.4.4): a statistics pass over the stored blocks (row
 * max and sum of exponentials, no V), then an output pass that recomputes
 * the scores and accumulates P V with P normalised by those statistics.
 * Arguments, outputs, workspace and errors as bsr_attn_fwd; results agree
 * with it up to rounding. It does about 1.5x the forward's matrix work and is
 * kept for comparison with the one-pass online softmax (at head_dim 512 the
 * two entry points run the same kernels).
 */
bsr_attn_status bsr_attn_fwd_two_pass(const bsr_attn_structure *s, const void *d_plan,
                                      const bsr_attn_problem *p, const void *q, const void *k,
                                      const void *v, void *o, float *row_max, float *row_denom,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward for the loss <O, dO>. Inputs: q, k, v, o (the forward's output),
 * d_o, and the forward's row_max / row_denom. Writes dq, dk, dv (device
 * [B, H, S, D] in p->dtype). Query rows with no stored block get dq = 0;
 * keys that no query attends get dk = dv = 0.
 */
bsr_attn_status bsr_attn_bwd(const bsr_attn_structure *s, const void *d_plan,
                             const bsr_attn_problem *p, const void *q, const void *k,
                             const void *v, const void *o, const void *d_o,
                             const float *row_max, const float *row_denom, void *dq,
                             void *dk, void *dv, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * bsr_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Its workspace is a 32 MiB device array
 * inside the library (one per GPU, held until the process ends), enough for
 * the backward of every benchmark workload of head_dim up to 256 (the
 * 16-head, 8192-token global mask needs 25 MiB); a problem needing more
 * returns BSR_ATTN_ERR_WORKSPACE_TOO_SMALL and launches nothing. It calls no
 * allocating routine; its first call on a device looks up that device's copy
 * of the array. Every call on one GPU shares the array: calls that overlap on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller. Nothing in it needs to start at zero (every value the kernels read
 * is written earlier in the same call). Arguments, outputs, results and other
 * errors as bsr_attn_bwd, whose kernels it runs.
 */
bsr_attn_status bsr_attn_bwd_noalloc(const bsr_attn_structure *s, const void *d_plan,
                                     const bsr_attn_problem *p, const void *q, const void *k,
                                     const void *v, const void *o, const void *d_o,
                                     const float *row_max, const float *row_denom, void *dq,
                                     void *dk, void *dv, void *stream);

/*
 * The same backward in the other schedule the design weighs against
 * recomputation ("trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.0/0.5.1: dS =
 * P (dP - D) feeds both dQ = dS K and dK = dS^T Q): the row terms (delta,
 * log-sum-exp) in one pass; the column-first dK/dV pass, which also writes
 * its dS (rounded to p->dtype, as used for dK) into the workspace; then
 * dQ = scale * dS K row-first from the stored dS, a block-sparse product
 * that recomputes no scores. Fewer matrix products (5 per stored block
 * instead of 7), 2 * 128 * 128 * sizeof(dtype) more bytes per stored block
 * per (batch, head) through HBM. bf16 and fp16 only (fp32 returns
 * BSR_ATTN_ERR_UNSUPPORTED); workspace from bsr_attn_workspace_bytes(s, p, 2);
 * otherwise arguments, outputs and errors as bsr_attn_bwd, and results agree
 * with it up to rounding.
 */
bsr_attn_status bsr_attn_bwd_ds(const bsr_attn_structure *s, const void *d_plan,
                                const bsr_attn_problem *p, const void *q, const void *k,
                                const void *v, const void *o, const void *d_o,
                                const float *row_max, const float *row_denom, void *dq,
                                void *dk, void *dv, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Block-sparse times dense on the same structure and plan: C = A B, where A
 * is the block-sparse matrix whose stored 128 x 128 blocks are given
 * (values, unlike attention's mask) and B, C are dense (page
 * "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: bsr_spmm visits exactly the
 * stored blocks and addresses B by block column; 0.9.0: output tiles
 * balanced by stored blocks, one writer each).
 *   blocks: device [nnzb, 128, 128] in BSR order (the block at block row I,
 *           block column col_idx[p] is blocks[p]), row-major within a block;
 *           may be NULL when nnzb = 0.
 *   b:      device [nb*128, n_cols] row-major; c: device [nb*128, n_cols].
 *   dtype:  bsr_attn_dtype of blocks, b and c (bf16 / fp16 run 16-bit matrix
 *           products with fp32 accumulation); n_cols a positive multiple of
 *           128 (others: BSR_ATTN_ERR_UNSUPPORTED).
 *   workspace: device, at least bsr_spmm_workspace_bytes(s, n_cols) bytes
 *           (fp32 shares of split block rows; 0 when no row is split).
 * Rows of a block row with no stored block are set to zero. Validation and
 * errors as for bsr_attn_fwd; asynchronous on `stream`.
 */
size_t bsr_spmm_workspace_bytes(const bsr_attn_structure *s, int32_t n_cols);
bsr_attn_status bsr_spmm(const bsr_attn_structure *s, const void *d_plan, int32_t dtype,
                         int32_t n_cols, const void *blocks, const void *b, void *c,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Optional per-kernel timing, for benchmarks and profiling. Between
 * bsr_attn_timing_begin() and bsr_attn_timing_end() on the calling thread,
 * fwd/bwd record a pair of hipEvents on their stream around every kernel they
 * launch. bsr_attn_timing_end() waits for those events, writes one entry per
 * distinct kernel (launch count and summed duration in milliseconds) to
 * `out` (at most max_entries) and returns the number of distinct kernels, or
 * -1 on a HIP error. Timing is off by default and costs nothing when off.
 * The events skip the system-scope fence a default event performs on
 * completion (hipEventDisableSystemFence), so the caches are not written back
 * and invalidated between the timed kernels.
 */
typedef struct {
    char name[64];      /* kernel role and instance, e.g. "dkdv<bf16,128>" */
    int32_t launches;
    double total_ms;
} bsr_attn_kernel_time;

bsr_attn_status bsr_attn_timing_begin(void);
/*
 * MFMA-loop probe, for the benchmark's measured peak: enqueues on `stream` a
 * kernel in which every wave (two per SIMD on every CU) runs `iters` rounds
 * of four independent 32x32 MFMA products (bf16/fp16: 32x32x16; fp32:
 * 32x32x2) on register operands drawn uniformly from (-1, 1), reading no
 * memory. *flops (host) receives its matrix work; time it with events on
 * the same stream. sink: device float[1], written only if the products'
 * sum equals a value it does not take (it keeps the work from being
 * removed). Errors: invalid dtype, iters < 1 or NULL pointers.
 */
bsr_attn_status bsr_attn_mfma_probe(int32_t dtype, int32_t iters, float *sink, void *stream,
                                    double *flops);
int bsr_attn_timing_end(bsr_attn_kernel_time *out, int max_entries);

/* Thread-local description of the calling thread's last failure ("" if none). */
const char *bsr_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSR_ATTN_H */
