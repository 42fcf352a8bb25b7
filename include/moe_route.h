/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE routing, dispatch and combine library.
 *
 * The operations are those of Perplexity, "Enabling trillion-parameter models on AWS EFA":
 *   - routing: a small linear router decides which experts multiply each token ("Introductie");
 *   - dispatch: receives the tokens and their per-token experts and sends every token to the
 *     ranks hosting those experts ("Introductie", "MoE all-to-all over EFA"). It counts tokens per
 *     expert, turns the counts into offsets with a cumulative sum and packs the tokens into
 *     contiguous per-destination buffers ("Verzend- en ontvangstbuffers", "Dispatch en Combine"),
 *     optionally as block-scaled fp8 ("Evaluatie / Dispatch/Combine-latentie");
 *   - combine: brings the processed rows back to their tokens and accumulates their weighted
 *     average into the output tensor ("Dispatch en Combine").
 * Here the destination ranks are disjoint row ranges of one receive buffer on one GPU.
 *
 * Conventions for every entry point:
 *   - Every pointer argument is a DEVICE pointer, except `out` of the dispatch calls, which is a
 *     HOST pointer to a struct of device pointers. The caller allocates and owns every buffer; the
 *     library allocates nothing and keeps no state between calls (the one exception,
 *     moe_route_dispatch_noalloc, keeps a fixed workspace array per device; see there).
 *   - Work is enqueued on `stream` (0 = the null stream); calls return without synchronising.
 *   - All arguments are validated before any launch. On an error status nothing is enqueued and
 *     no output is written. MOE_ERR_HIP means a launch failed (hipGetLastError after the launch).
 *   - Matrices are row-major and dense: [T, E] means T rows of E elements with no padding.
 *   - Sizes are int32; T * k must stay below 2^31.
 *   - Kernels never read or write outside the buffers described below, whatever the values in
 *     topk_idx / token_row: an expert id outside [0, E) or a row outside [0, T*k) is skipped
 *     (its row is not written, or it contributes nothing). Such inputs break the preconditions
 *     and leave the affected outputs unspecified.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* bad size, null pointer, inconsistent arguments */
    MOE_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels handle (dtype, alignment, E) */
    MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_dispatch_workspace_bytes() */
    MOE_ERR_HIP = 4          /* a kernel launch failed */
} moe_status_t;

typedef enum {
    MOE_F32 = 0,       /* IEEE-754 binary32 */
    MOE_BF16 = 1,      /* bfloat16 */
    MOE_FP8_E4M3 = 2   /* OCP e4m3fn (max 448, no infinities), one byte per element */
} moe_dtype_t;

/* Largest expert count and largest top-k the kernels handle. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 64

/*
 * moe_route_topk -- top-k expert selection with renormalised softmax weights ("Introductie": the
 * router picks the experts of every token; the softmax and its renormalisation over the kept
 * experts are the reading used where the page names no scoring function).
 *   logits   [T, E] fp32, finite.
 *   topk_idx [T, k] int32 out: expert ids, largest logit first; equal logits go to the lower id
 *            (-0.0 and +0.0 are equal).
 *   topk_w   [T, k] fp32 out: exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k kept experts,
 *            evaluated in double and rounded once to fp32; they sum to 1 within k * 2^-24.
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), 1 <= E <= MOE_MAX_EXPERTS (else MOE_ERR_UNSUPPORTED
 * for E or k beyond the maxima, MOE_ERR_INVALID otherwise). T = 0 enqueues nothing.
 */
moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream);

/*
 * Bytes of device workspace that moe_dispatch, moe_dispatch_layout and moe_route_dispatch need for
 * (T, E, k): per-block expert histograms, their in-expert prefixes, expert totals and per-item
 * ranks. Returns 0 for invalid sizes.
 * The workspace needs no initialisation and holds nothing the caller uses afterwards. Two calls
 * that may run at the same time (different streams) must not share a workspace.
 */
size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k);

/* Dispatch outputs: device pointers, all allocated by the caller. R = T * k. */
typedef struct {
    void* recv;              /* [R, H] payload rows (x's format, or e4m3 codes for FP8) */
    float* recv_scales;      /* [R, H/128] fp32 block scales when the payload is FP8, else NULL */
    int32_t* expert_counts;  /* [E]   rows routed to each expert */
    int32_t* expert_offsets; /* [E+1] exclusive cumulative sum of expert_counts; [E] = R */
    int32_t* rank_counts;    /* [N]   rows received by each destination rank */
    int32_t* rank_offsets;   /* [N+1] first row of each rank; [N] = R */
    int32_t* token_row;      /* [R]   row holding (token t, slot j), at index t*k + j */
    int32_t* row_token;      /* [R]   source token of each row */
} moe_dispatch_out_t;

/*
 * moe_dispatch_layout -- the counting half of dispatch ("Verzend- en ontvangstbuffers": every
 * sender knows all per-expert counts before writing, so writes are contiguous per destination;
 * "Dispatch en Combine": per-expert token counts, then their cumulative sum gives the offsets).
 *   topk_idx [T, k] int32 expert ids in [0, E), normally distinct within a token (a repeated id
 *            is two separate rows).
 *   n_ranks  N destination ranks; rank r hosts the experts [r*E/N, (r+1)*E/N) (E % N == 0).
 *   Writes expert_counts, expert_offsets, rank_counts, rank_offsets, token_row and row_token of
 *   `out` (recv / recv_scales are ignored). Rows are ordered by (rank, expert, token, slot): each
 *   rank's rows are contiguous, grouped by expert, tokens ascending inside an expert. The result
 *   is deterministic (no atomics decide a position).
 *   workspace: device memory of at least moe_dispatch_workspace_bytes(T, E, k) bytes.
 * Requires 1 <= k <= MOE_MAX_TOPK and E <= MOE_MAX_EXPERTS (else MOE_ERR_UNSUPPORTED); this limit
 * on k also holds for moe_dispatch, moe_route_dispatch and moe_ep_send.
 * T = 0 writes zero counts and offsets.
 */
moe_status_t moe_dispatch_layout(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                 int32_t n_ranks, const moe_dispatch_out_t* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_pack -- the packing half of dispatch ("Dispatch en Combine": once the offsets are
 * known every token is packed into the send buffers; the receiver's copy into the grouped-GEMM
 * input is merged into the same write here).
 *   x          [T, H] tokens, x_dtype MOE_F32 or MOE_BF16, 16-byte aligned, H * elem % 16 == 0.
 *   token_row  [T * k] as written by moe_dispatch_layout.
 *   payload_dtype == x_dtype: recv[token_row[t*k+j], :] = x[t, :], bytes unchanged.
 *   payload_dtype == MOE_FP8_E4M3 ("block-scaled fp8-dispatch", read as 1 x 128 blocks): for every
 *     token and block b of 128 elements, amax = max |x| over the elements that are not NaN,
 *     s = amax / 448 in fp32 (1 when amax = 0), code = e4m3 of the fp32 quotient x / s rounded to
 *     nearest even and saturated to +-448; a NaN quotient gives the NaN code 0x7F with the sign of
 *     x (a NaN element, or an infinite one in a block whose s is infinite);
 *     recv [R, H] uint8 codes, recv_scales [R, H/128] fp32 s. Requires H % 128 == 0.
 *   recv 16-byte aligned, recv_scales 4-byte aligned.
 */
moe_status_t moe_dispatch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                               int32_t k, const int32_t* token_row, moe_dtype_t payload_dtype,
                               void* recv, float* recv_scales, hipStream_t stream);

/*
 * moe_dispatch -- moe_dispatch_layout followed by moe_dispatch_pack on the same stream, with the
 * arguments described there; `out` supplies recv / recv_scales as well.
 */
moe_status_t moe_dispatch(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                          const int32_t* topk_idx, int32_t k, int32_t E, int32_t n_ranks,
                          moe_dtype_t payload_dtype, const moe_dispatch_out_t* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_dispatch -- moe_route_topk followed by moe_dispatch on the same stream: the router's
 * choice ("Introductie") and the dispatch of every token to its experts' rows ("Dispatch en
 * Combine"), with the counting of each group of tokens done in the same launch as their routing.
 *   logits [T, E] fp32 as for moe_route_topk; topk_idx [T, k] and topk_w [T, k] are written as
 *   moe_route_topk writes them; x, x_dtype, H, n_ranks, payload_dtype, out and the workspace are
 *   as for moe_dispatch. Every output equals what the two calls write.
 * Argument errors are those of the two calls.
 */
moe_status_t moe_route_dispatch(const float* logits, const void* x, moe_dtype_t x_dtype,
                                int32_t T, int32_t H, int32_t E, int32_t k, int32_t n_ranks,
                                moe_dtype_t payload_dtype, int32_t* topk_idx, float* topk_w,
                                const moe_dispatch_out_t* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_dispatch_noalloc -- moe_route_dispatch without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). It allocates nothing: its workspace is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per device, held until the
 * process ends (its address on a device is looked up on the first call there).
 *   Arguments, outputs and argument errors are those of moe_route_dispatch; every output equals
 *   what moe_route_dispatch writes. A call that needs more than MOE_NOALLOC_SCRATCH_BYTES of
 *   workspace (moe_dispatch_workspace_bytes(T, E, k) > MOE_NOALLOC_SCRATCH_BYTES) returns
 *   MOE_ERR_WORKSPACE before anything is enqueued; MOE_ERR_HIP if the array's address cannot be
 *   had on the stream's device.
 *   All calls on one device share that device's array, and a call leaves its contents behind (no
 *   call reads what another wrote before writing it itself). Calls on one device whose work may
 *   overlap in time (different streams without ordering between them) race on the array and give
 *   undefined results: order them on one stream, or use moe_route_dispatch with a workspace each.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

moe_status_t moe_route_dispatch_noalloc(const float* logits, const void* x, moe_dtype_t x_dtype,
                                        int32_t T, int32_t H, int32_t E, int32_t k,
                                        int32_t n_ranks, moe_dtype_t payload_dtype,
                                        int32_t* topk_idx, float* topk_w,
                                        const moe_dispatch_out_t* out, hipStream_t stream);

/*
 * moe_combine -- weighted sum of the returned rows of every token ("Dispatch en Combine": the
 * receiver accumulates the rows from its receive buffer into the output tensor; "Introductie":
 * combine forms their weighted average -- with renormalised weights that is this sum).
 *   y         [T * k, H] expert outputs, y_dtype MOE_F32 or MOE_BF16, 16-byte aligned.
 *   token_row [T * k] row of (t, j); topk_w [T, k] fp32 weights.
 *   out       [T, H] out_dtype MOE_F32 or MOE_BF16, 16-byte aligned:
 *             out[t, h] = sum_{j<k} w[t, j] * y[token_row[t*k+j], h], accumulated in fp32 in
 *             slot order (fused multiply-add), rounded to nearest even for bf16.
 * Requires H % 8 == 0. T = 0 enqueues nothing.
 */
moe_status_t moe_combine(const void* y, moe_dtype_t y_dtype, int32_t T, int32_t H, int32_t k,
                         const int32_t* token_row, const float* topk_w, void* out,
                         moe_dtype_t out_dtype, hipStream_t stream);

/*
 * Expert parallelism over several devices, emulated on one GPU. The pages split dispatch and
 * combine into a sender half and a receiver half ("MoE all-to-all over EFA"), size each receive
 * buffer for the worst case before any row is written and let every sender write its rows
 * straight into the receiver's buffer ("Verzend- en ontvangstbuffers"); the receiver then copies
 * the rows into the input of its grouped GEMM, and combine returns the expert outputs to their
 * senders ("Dispatch en Combine"). Here S sources (the devices that own tokens) send to N ranks
 * (rank r hosts the L = E/N experts [r*L, (r+1)*L)), all in device memory of one GPU:
 *   - the region array [N*S*cap, H] holds one region of `cap` rows per (rank r, source s), at rows
 *     [(r*S + s)*cap, (r*S + s + 1)*cap); `cap` >= moe_ep_capacity(T, E, k, N);
 *   - region_counts [N, S, L] int32: rows source s wrote for expert r*L + l, at (r*S + s)*L + l.
 * One step: moe_ep_send for every source, moe_ep_recv for every rank, the experts, moe_ep_return
 * for every rank, moe_ep_combine for every source. Calls for different sources (or ranks) write
 * disjoint memory.
 */

/* Rows of one (rank, source) region: T * min(k, E/N), the most one source can send to one rank
 * (each token at most once per hosted expert). Returns 0 for invalid sizes. */
int64_t moe_ep_capacity(int32_t T, int32_t E, int32_t k, int32_t n_ranks);

/*
 * moe_ep_send -- sender half of dispatch for source `source` (0 <= source < n_sources).
 *   x [T, H] (MOE_F32 or MOE_BF16, 16-byte aligned rows), topk_idx [T, k] ids in [0, E).
 *   Writes into `regions` (x's format; only this source's regions) the rows of every (token, slot):
 *   region (r, source) holds its rows to rank r ordered by (expert, token, slot); writes
 *   region_counts[(r*S + source)*L + l] for every r, l, and send_row[t*k + j] = the region-array row
 *   of (t, j). Uses a workspace of moe_dispatch_workspace_bytes(T, E, k) bytes.
 * Requires cap >= moe_ep_capacity(T, E, k, n_ranks) and N*S*cap < 2^31 (else MOE_ERR_INVALID),
 * and k <= MOE_MAX_TOPK (else MOE_ERR_UNSUPPORTED).
 */
moe_status_t moe_ep_send(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                         const int32_t* topk_idx, int32_t k, int32_t E, int32_t n_ranks,
                         int32_t source, int32_t n_sources, int32_t cap, void* regions,
                         int32_t* region_counts, int32_t* send_row, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * moe_ep_recv -- receiver half of dispatch for rank `rank`: copies the rows of its S regions into
 * `grouped` [S*cap, H] ordered by (local expert, source, token, slot), writes expert_counts [L],
 * expert_offsets [L+1] (offsets in `grouped`; [L] = rows received) and grouped_src [S*cap]: the
 * region-array row of each grouped row (-1 past the last one). Reads region_counts (all sources'
 * sends to this rank must be complete, i.e. enqueued earlier on the same stream).
 * Requires S*L <= 4096 (else MOE_ERR_UNSUPPORTED).
 */
moe_status_t moe_ep_recv(const void* regions, moe_dtype_t dtype, int32_t H, int32_t E,
                         int32_t n_ranks, int32_t rank, int32_t n_sources, int32_t cap,
                         const int32_t* region_counts, void* grouped, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* grouped_src, hipStream_t stream);

/*
 * moe_ep_return -- receiver half of combine: every grouped row of expert output y_grouped
 * [S*cap, H] goes back to its region row, returns[grouped_src[g]] = y_grouped[g], for
 * g < expert_offsets[L] (both from moe_ep_recv). `returns` has the region array's layout.
 */
moe_status_t moe_ep_return(const void* y_grouped, moe_dtype_t dtype, int32_t H, int32_t E,
                           int32_t n_ranks, int32_t n_sources, int32_t cap,
                           const int32_t* grouped_src, const int32_t* expert_offsets,
                           void* returns, hipStream_t stream);

/*
 * moe_ep_combine -- sender half of combine for one source: moe_combine over the returned rows,
 * out[t, h] = sum_j w[t, j] * returns[send_row[t*k + j], h] (fp32 accumulation in slot order).
 *   region_rows = N*S*cap, the rows of `returns`; a send_row outside [0, region_rows) is skipped.
 */
moe_status_t moe_ep_combine(const void* returns, moe_dtype_t y_dtype, int32_t T, int32_t H,
                            int32_t k, const int32_t* send_row, const float* topk_w,
                            int32_t region_rows, void* out, moe_dtype_t out_dtype,
                            hipStream_t stream);

/*
 * Combine with pre-reduction on the expert side. The pages accumulate only on the receiver and
 * name that as the reason they lag at prefill ("Evaluatie / Dispatch/Combine-latentie"). Here rank
 * r first sums, for every token that has experts on r, the weighted outputs of those experts into
 * one partial row (fp32 multiply-adds in slot order, rounded once to the partial format); only the
 * partial rows travel back, and the source adds a token's partial rows in rank order (fp32,
 * rounded once). One row per (token, rank) instead of one per (token, slot) travels back, at the
 * cost of a second rounding.
 *   - Partial array [N*S*pcap, H], pcap >= T: the partial rows of (rank r, source s) sit at rows
 *     [(r*S + s)*pcap, ...) in token order; part_row [T, N] of a source names the row of (t, r),
 *     -1 when t has no expert on r.
 */

/* Partial-row layout of source `source`: part_row [T, N] and part_counts[r*S + source] (the rows
 * it receives from rank r). */
moe_status_t moe_ep_partial_rows(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                 int32_t n_ranks, int32_t source, int32_t n_sources, int32_t pcap,
                                 int32_t* part_row, int32_t* part_counts, hipStream_t stream);

/* Bytes of workspace moe_ep_reduce needs (the grouped row of every region row of the rank). */
size_t moe_ep_reduce_workspace_bytes(int32_t n_sources, int32_t cap);

/*
 * moe_ep_reduce -- expert side: the partial rows that rank `rank` returns to every source.
 *   y_grouped [S*cap, H] expert outputs in the rank's grouped layout, grouped_src from
 *   moe_ep_recv; topk_idx / topk_w [S*T, k], send_row [S*T*k] and part_row [S*T, N] are the
 *   sources' tables stacked (source s owns tokens [s*T, (s+1)*T)); in a deployment they travel
 *   with the dispatched rows. Writes partials[part_row[(s*T + t)*N + rank], :] for every token with
 *   experts on the rank. H % 8 == 0.
 */
moe_status_t moe_ep_reduce(const void* y_grouped, moe_dtype_t dtype, int32_t H, int32_t E,
                           int32_t n_ranks, int32_t rank, int32_t n_sources, int32_t cap,
                           const int32_t* grouped_src, int32_t T, int32_t k,
                           const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                           const int32_t* part_row, int32_t pcap, void* partials, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * moe_ep_combine_reduced -- source side: out[t, :] = sum over r of partials[part_row[t*N + r], :]
 * (rows with part_row -1 or outside [0, partial_rows) skipped), fp32 in rank order, rounded once.
 */
moe_status_t moe_ep_combine_reduced(const void* partials, moe_dtype_t dtype, int32_t T, int32_t H,
                                    int32_t n_ranks, const int32_t* part_row,
                                    int32_t partial_rows, void* out, moe_dtype_t out_dtype,
                                    hipStream_t stream);

/*
 * moe_check_topk -- check of what dispatch takes for granted about the expert ids it is handed
 * ("MoE all-to-all over EFA": dispatch receives every token with its experts; "Introductie": the
 * router picks k of the E experts of each token). For ids that do not come from the router.
 *   topk_idx [T, k] int32 (device), counts [2] int32 (device) out:
 *   counts[0] = slots (t, j) whose id lies outside [0, E);
 *   counts[1] = slots whose id lies in [0, E) and equals the id of an earlier slot of the same
 *               token (a token naming one expert three times counts 2).
 * The dispatch calls skip out-of-range ids (their token_row is -1) and order repeated ids by
 * (expert, token, slot); this call tells a caller that either happened. Enqueued on `stream`
 * like every other call: read counts after the stream has finished. Requires k >= 1, E >= 1,
 * T * k <= INT32_MAX (else MOE_ERR_INVALID). T = 0 writes two zeros.
 */
moe_status_t moe_check_topk(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                            int32_t* counts, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* moe_status_str(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
