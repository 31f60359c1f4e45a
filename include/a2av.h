/*
 * a2av.h -- MoE token dispatch and combine over an all-to-allv whose per-destination
 * counts are produced and consumed on the GPU (gfx950 / MI355X).
 *
 * The operation is the pages' AllToAllvDynamic as used by a mixture-of-experts layer:
 *   [abhik.ai "Collective Communication for 100k+ GPUs", section "Inference: small
 *    messages, unknown sizes", Figure 13]  a router picks experts for every token, the
 *    tokens are sorted by expert into a send buffer, and an all-to-allv sends each row
 *    to the GPU that holds its expert.  The per-peer counts live in GPU memory, are
 *    read when the exchange executes (so they may change up to that moment) and the
 *    counts each rank received are returned to the caller;
 *   [hungchun0201.github.io "sigcomm26-ncclx" digest, section 3.3 and its terms list]
 *    under a captured graph a host-side all-to-allv must pad every count to the worst
 *    case; the dynamic one sends only real rows;
 *   [qiguanping.github.io "NCCLX", section 7, figures 13-18]  dispatch and combine,
 *    metadata resident on the GPU and consumed directly by kernels, exchanged between
 *    ranks without a CPU relay.
 *
 * R "virtual ranks" are modelled on one GPU as disjoint regions of rank-major device
 * tensors: rank r owns slice r of every [R][...] argument.  Expert e lives on rank
 * e / experts_per_rank.
 *
 * Conventions for every entry point:
 *   - Pointers marked (device) are device pointers of the GPU that was current when
 *     the handle was created; that GPU must be current at every call.  (host) marks
 *     host pointers.  A pointer to an array of zero elements (no tokens, or a
 *     receive capacity of 0) may be null.
 *   - `stream` is a hipStream_t passed as void* (so that this header needs no HIP
 *     header and plain C callers can include it); NULL is the null stream.  All GPU work
 *     is enqueued on it.  dispatch, combine and the harness calls never allocate,
 *     never synchronise and never copy to the host, so they can be captured in a
 *     hipGraph and replayed with routing that changes on the device.
 *   - Return value: A2AV_OK, or a negative A2AV_ERR_* code.  On a negative code nothing
 *     was enqueued (A2AV_ERR_HIP: a launch failed; work before it may have been
 *     enqueued).
 *   - Problems only the GPU can see (an expert id outside [0, E), a rank receiving
 *     more rows than its capacity) OR bits into the caller's device word `*status`
 *     (sticky; the library never clears or reads it; it must be 4-byte aligned).  No
 *     write ever goes out of bounds: a dropped assignment is not sent, a row past the
 *     capacity is not written, and either adds zero to the combine.  Counts stay true.
 *   - A handle serves one dispatch/combine pair at a time: combine uses the routing
 *     of the most recent dispatch on the same handle, in stream order.  Handles are
 *     not thread-safe.
 *
 * Layouts (all contiguous, row-major):
 *   x, y          [R][T][H]       dtype     token rows, one slice per rank
 *   topk_ids      [R][T][k]       int32     expert ids from the router
 *   gates         [R][T][k]       float32   combine weights
 *   recv, expert_out [R][cap][H]  dtype     receive rows.  Source-major layout: rank d's
 *                                           rows from source s are rows recv_offsets[d][s]
 *                                           .. recv_offsets[d][s+1]-1 of slice d, sorted
 *                                           by (expert, token, slot) as sent.  Expert-major
 *                                           layout: rows of d's local expert le are rows
 *                                           recv_expert_offsets[d][le] .. [le+1]-1, source
 *                                           ascending, each source in its sent order
 *   recv_expert_offsets [R][epr+1] int32    expert-major group starts ([d][epr] = total)
 *   split         [R][E]          int32     rows rank s sends to expert e
 *   recv_counts   [R][R]          int32     [dst][src] rows received
 *   recv_offsets  [R][R+1]        int32     [dst][src] exclusive prefix over src;
 *                                           [dst][R] = rows rank dst received (with the
 *                                           expert-major layout these are counts, not
 *                                           places)
 *   positions     [R][T][k]       int32     place of (t, slot) in rank s's expert-
 *                                           sorted send order, -1 if the id was invalid
 * Counts and offsets are in rows; byte addresses are formed in 64 bits.
 */
#ifndef A2AV_H
#define A2AV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct a2av_context* a2av_handle_t;

/* element types of x, recv, expert_out and y */
#define A2AV_F32  0
#define A2AV_BF16 1

/* return codes */
#define A2AV_OK           0
#define A2AV_ERR_INVALID (-1)   /* argument or configuration rejected */
#define A2AV_ERR_NOMEM   (-2)   /* allocation failed (create; timing_begin on the host) */
#define A2AV_ERR_HIP     (-3)   /* a HIP runtime call or launch failed */
#define A2AV_ERR_SCRATCH (-4)   /* a2av_alltoallv_noalloc: the shape needs more scratch than
                                   the library's fixed device array holds */

/* device status bits, OR-ed into *status */
#define A2AV_ST_EXPERT_RANGE  1u  /* an expert id was outside [0, E): that slot is dropped */
#define A2AV_ST_RECV_OVERFLOW 2u  /* a rank received more rows than recv_capacity_rows */
#define A2AV_ST_BOUNDS        4u  /* debug build only (liba2av_debug.so, compiled with
                                     A2AV_DEBUG=1): a device-side bounds check on a row
                                     index or a table value failed and that access was
                                     skipped.  The release library has the same exports
                                     and results and never sets it. */

/* data paths (a2av_config_t.path) */
#define A2AV_PATH_STAGED 0        /* pack into send segments, exchange, return, combine */
#define A2AV_PATH_DIRECT 1        /* pack straight into the receivers' buffers; combine
                                     gathers the expert outputs where they are */

/* receive layouts (a2av_config_t.recv_layout) */
#define A2AV_LAYOUT_SOURCE_MAJOR 0  /* rows from source 0 first, each source's rows in its
                                       sorted order (a plain all-to-allv) */
#define A2AV_LAYOUT_EXPERT_MAJOR 1  /* rows grouped by the receiver's local expert, then by
                                       source, then in the source's order: each expert's
                                       rows contiguous, ready for a grouped expert GEMM */

/* expert stand-ins of the harness call a2av_expert_apply */
#define A2AV_EXPERT_IDENTITY 0    /* out = in */
#define A2AV_EXPERT_SCALE    1    /* out = round(in * (1 + e/256)), e = the row's expert */

typedef struct {
    int32_t num_ranks;          /* R, 1 .. 1024 */
    int32_t tokens_per_rank;    /* T, >= 0 */
    int32_t hidden;             /* H, >= 1 elements per row */
    int32_t dtype;              /* A2AV_F32 or A2AV_BF16 */
    int32_t experts_per_rank;   /* E = R * experts_per_rank, 1 <= E <= 4096 */
    int32_t top_k;              /* k, 1 .. min(E, 64) */
    int64_t recv_capacity_rows; /* rows per rank's receive slice; 0 = worst case
                                   R * T * min(k, experts_per_rank).  This is an
                                   allocation size, never a transfer size. */
    int32_t path;               /* A2AV_PATH_STAGED or A2AV_PATH_DIRECT; both give the
                                   same receive rows, tables and combine results */
    int32_t recv_layout;        /* A2AV_LAYOUT_SOURCE_MAJOR or A2AV_LAYOUT_EXPERT_MAJOR */
} a2av_config_t;

/* Set-up, once per shape.  Under graph capture the buffers a collective touches are set
 * up once, when the graph is captured, and must stay the same across replays, while the
 * counts change inside them [abhik.ai page, section "Inference: small messages, unknown
 * sizes"; qiguanping.github.io "NCCLX", section 7, figure 14]; so every device buffer
 * the library itself needs is allocated here, at fixed addresses for the handle's life,
 * and dispatch and combine allocate nothing.
 *
 * a2av_create: validate cfg (host) and allocate the handle's device workspace on the
 * current GPU: the send buffer (reused as the return buffer; staged path only), the
 * position table and the count/offset tables, zeroed.  *out (host) receives the handle
 * (NULL on failure; nothing is left allocated).  The workspace size is
 * a2av_workspace_bytes(cfg).  Errors: A2AV_ERR_INVALID (null pointer or a config outside
 * the documented ranges), A2AV_ERR_NOMEM (device allocation failed), A2AV_ERR_HIP. */
int a2av_create(const a2av_config_t* cfg, a2av_handle_t* out);

/* Free the handle and its workspace (the end of the set-up's lifetime).  The caller must
 * have synchronised the streams that used it; work still in flight on it is undefined
 * behaviour.  NULL is accepted (A2AV_OK).  Errors: A2AV_ERR_HIP if a free failed (the
 * handle is released anyway). */
int a2av_destroy(a2av_handle_t h);

/* Device bytes a2av_create allocates for cfg (host), or -1 if cfg is invalid or null.
 * Host-only: touches no GPU. */
int64_t a2av_workspace_bytes(const a2av_config_t* cfg);

/* Dispatch (the token sort and the all-to-allv, abhik.ai page, Figure 13):
 *   1. histogram: rows per (rank, expert), from topk_ids, on the GPU;
 *   2. scans: per-rank expert and destination offsets; the received counts and
 *      offsets of every rank, formed from every sender's offsets on the GPU;
 *   3. pack: every (token, slot) row of x copied to its place in the sender's send
 *      segments, stable by (expert, token, slot);
 *   4. exchange: every segment copied into the receiving rank's slice of recv at the
 *      offset the device tables give.
 * The direct path fuses 3 and 4: each row goes from x straight to its receive place
 * (the pages' zero-copy transfer, user buffer to peer user buffer).  Steps of at most
 * 1024 experts and 1024 assignments per rank run 1-3 as a single launch when they hold
 * at most 2048 assignments, or at most 4096 on the staged path or with rows of at least
 * 8 KiB: every row finds its place by counting, over topk_ids, the assignments before
 * it in its destination's order (the same place the scans give).  The results are
 * identical.
 * x (device) [R][T][H] dtype; topk_ids (device) [R][T][k].  recv (device, caller
 * owned) [R][cap][H]: only the first min(recv_offsets[d][R], cap) rows of slice d are
 * written.  split, recv_counts, recv_offsets (device, optional: NULL = not wanted)
 * receive copies of the tables.  status (device, required) is OR-ed.
 * Errors: A2AV_ERR_INVALID (null x/topk_ids/recv/status, wrong device), A2AV_ERR_HIP. */
int a2av_dispatch(a2av_handle_t h, const void* x, const int32_t* topk_ids, void* recv,
                  int32_t* split, int32_t* recv_counts, int32_t* recv_offsets,
                  uint32_t* status, void* stream);

/* Combine (the return all-to-all and the merge, qiguanping.github.io page, section 7,
 * figure 13): every expert-output row goes back to the place its input row had in the
 * sender's send segments (the direct path reads it where it is instead), then every
 * token's output is
 *   y[s][t] = round_to_dtype( sum_{j<k} gates[s][t][j] * out_j ),
 * summed in float32 with one fused multiply-add per slot in slot order, rounded once
 * (nearest, ties to even).  expert_out (device) [R][cap][H] in the receive layout of
 * the latest dispatch (may be recv itself); gates (device) [R][T][k]; y (device)
 * [R][T][H].  Errors: A2AV_ERR_INVALID, A2AV_ERR_HIP. */
int a2av_combine(a2av_handle_t h, const void* expert_out, const float* gates, void* y,
                 uint32_t* status, void* stream);

/* The bare collective, for callers that sort their own send buffers (the pages'
 * AllToAllvDynamic on its own): rank s holds send (device) [R][T*k][H], whose rows for
 * rank d are the contiguous block starting at the exclusive prefix of
 * send_counts[s][0..d-1]; send_counts (device) [R][R] ([src][dst]) is read when the
 * kernels run, so it may be written by earlier work on the stream.  Rows land in recv
 * (device) [R][cap][H] source-major; recv_counts / recv_offsets (device, optional) as
 * for dispatch (always source-major).  A negative count, or counts of one sender
 * summing past T*k, set A2AV_ST_EXPERT_RANGE and that sender's counts are taken as 0.
 * It replaces the handle's routing state: a2av_combine and a2av_expert_apply after it
 * return A2AV_ERR_INVALID until the next a2av_dispatch.
 * Errors: A2AV_ERR_INVALID, A2AV_ERR_HIP. */
int a2av_alltoallv(a2av_handle_t h, const void* send, const int32_t* send_counts, void* recv,
                   int32_t* recv_counts, int32_t* recv_offsets, uint32_t* status, void* stream);

/* The bare collective of a2av_alltoallv with no handle and no allocation, for callers
 * that cannot allocate device memory: code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The three tables the collective works with (send
 * offsets [R][R+1], receive counts [R][R] and receive offsets [R][R+1]) live in one
 * fixed array of A2AV_NOALLOC_SCRATCH_BYTES device bytes that the library holds on every
 * GPU it runs on until the process ends; nothing else is used beyond the caller's
 * buffers, and the call allocates nothing (no hipMalloc, no allocating library routine).
 * cfg (host) gives the shape as for a2av_create: num_ranks R (at most
 * A2AV_NOALLOC_MAX_RANKS), tokens_per_rank * top_k send rows per rank, hidden, dtype,
 * recv_capacity_rows (0 = the worst case R * T * min(k, experts_per_rank));
 * experts_per_rank and top_k are validated as for a2av_create; path and recv_layout
 * are not used (the collective is always source-major).  send, send_counts, recv,
 * recv_counts, recv_offsets, status and stream are as for a2av_alltoallv, and the
 * results are identical to it.  The first call on a GPU looks up the array's device
 * address (a runtime query); make that first call outside graph capture.  Every call
 * on one GPU uses that GPU's one array: calls that overlap on one GPU (on different
 * streams, or from different threads without stream order between them) race and give
 * unspecified results.  Each call writes every table entry it reads, so nothing has to
 * be cleared between calls.
 * Errors: A2AV_ERR_INVALID (bad cfg or pointers), A2AV_ERR_SCRATCH (R over
 * A2AV_NOALLOC_MAX_RANKS), A2AV_ERR_HIP; nothing is enqueued on an error. */
#define A2AV_NOALLOC_MAX_RANKS 256
#define A2AV_NOALLOC_SCRATCH_BYTES (1 << 20)
int a2av_alltoallv_noalloc(const a2av_config_t* cfg, const void* send, const int32_t* send_counts, void* recv,
                           int32_t* recv_counts, int32_t* recv_offsets, uint32_t* status, void* stream);

/* Copy the position table of the latest dispatch into pos (device) [R][T][k]. */
int a2av_copy_positions(a2av_handle_t h, int32_t* pos, void* stream);

/* Copy where each local expert's rows start in the expert-major receive layout into
 * recv_expert_offsets (device) [R][epr+1] ([d][epr] = rows d received).  Only for a
 * handle created with A2AV_LAYOUT_EXPERT_MAJOR (else A2AV_ERR_INVALID). */
int a2av_copy_recv_expert_offsets(a2av_handle_t h, int32_t* recv_expert_offsets, void* stream);

/* Copy the send offsets of the latest dispatch into send_offsets (device) [R][R+1]:
 * [s][d] = first row of s's segment for d, [s][R] = rows s sent. */
int a2av_copy_send_offsets(a2av_handle_t h, int32_t* send_offsets, void* stream);

/* ---- harness calls (stand-ins for the model around the collective) ---------------- */

/* Expert stand-in over the received rows of the latest dispatch: for every received
 * row, out = in (A2AV_EXPERT_IDENTITY) or round(in * (1 + e/256)) in float32 with one
 * rounding to dtype (A2AV_EXPERT_SCALE), e being the row's expert.  in, out (device)
 * [R][cap][H]; in == out is allowed. */
int a2av_expert_apply(a2av_handle_t h, const void* in, void* out, int32_t mode, void* stream);

/* Router stand-in for replayed decode steps: copies step (*counter % steps) of the
 * tables ids_table (device) [steps][n] and gates_table (device) [steps][n] into
 * ids (device) [n] and gates (device) [n], then increments *counter (device int32).
 * One workgroup; meant for n of a decode batch. */
int a2av_route_step(const int32_t* ids_table, const float* gates_table, int32_t steps, int64_t n,
                    int32_t* counter, int32_t* ids, float* gates, void* stream);

/* ---- measurement ----------------------------------------------------------------- */

/* Reference row copy: dst[r] = src[r] for rows rows of row_bytes bytes (a multiple of
 * 16; src, dst 16-byte aligned device pointers), moved exactly as the path's kernels move
 * rows (16-byte vectors, one wavefront per row or per chunk, non-temporal when large).
 * It measures the achievable copy bandwidth that the path's kernels are compared with.
 * Errors: A2AV_ERR_INVALID, A2AV_ERR_HIP. */
int a2av_copy_reference(const void* src, void* dst, int64_t rows, int64_t row_bytes, void* stream);

/* Plain one-direction streams, for the bandwidth ceilings the path's kernels are read
 * against (a kernel reading r bytes and writing w bytes cannot beat
 * (r + w) / (r / read_bw + w / write_bw)).  bytes is a multiple of 16; pointers are
 * 16-byte aligned device pointers.
 *   A2AV_STREAM_READ: reads every byte of src once; dst receives
 *     A2AV_STREAM_READ_OUT_BYTES bytes of 32-bit words whose XOR is the XOR of all of
 *     src's 32-bit words (dst must hold that many bytes).
 *   A2AV_STREAM_WRITE: writes all of dst: 16-byte vector i becomes the words
 *     {i, i >> 32, 0x5A5A5A5A, ~i}; src is not used.
 * Errors: A2AV_ERR_INVALID, A2AV_ERR_HIP. */
#define A2AV_STREAM_READ  0
#define A2AV_STREAM_WRITE 1
#define A2AV_STREAM_READ_OUT_BYTES (1 << 20)
int a2av_stream_reference(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream);

/* Stage timing with HIP events recorded between the library's kernels on the call's
 * stream.  a2av_timing_begin(h, max_calls), 1 <= max_calls <= A2AV_TIMING_MAX_CALLS,
 * creates events for up to max_calls dispatch and max_calls combine calls (host-side
 * event objects only; no device memory); later calls record until the budget is used.
 * a2av_timing_end waits for the recorded events, writes per-stage sums of
 * milliseconds into ms_sum (host)
 * [A2AV_STAGES] and the number of timed launches per stage into launches (host)
 * [A2AV_STAGES], and releases the events.  Stages: 0 plan (histogram + scans), 1 pack,
 * 2 exchange, 3 return exchange, 4 combine (the direct path has no 2 and 3; a
 * dispatch that runs as one launch counts it as stage 1 and has no stage 0).  Events
 * recorded between kernels add a little time to each step while timing is on.
 * a2av_timing_begin returns A2AV_ERR_NOMEM if the host cannot hold the events. */
#define A2AV_STAGES 5
#define A2AV_TIMING_MAX_CALLS (1 << 20)
int a2av_timing_begin(a2av_handle_t h, int32_t max_calls);
int a2av_timing_end(a2av_handle_t h, double* ms_sum, int32_t* launches);

/* Static string for a return code. */
const char* a2av_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* A2AV_H */
