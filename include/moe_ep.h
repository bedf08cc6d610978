/*
 * moe_ep.h -- C ABI of the MoE expert-parallel dispatch/combine library for
 * AMD Instinct MI355X (gfx950).
 *
 * Pages the calls follow:
 *   [EPMC] "Efficient and portable Mixture-of-Experts communication" (Perplexity)
 *   [EFA]  "Enabling trillion-parameter models on AWS EFA" (Perplexity)
 *
 * The group.  An expert-parallel group of N ranks, each holding T tokens of H
 * elements and routing every token to K of E experts; rank d owns experts
 * [d*L, (d+1)*L), L = E/N ([EPMC] "Sharding and parallelism").  All N ranks
 * are logical: their send and receive buffers live in the one GPU's memory and
 * the network transfer is a device-local copy.  Dispatch and combine are each
 * split into a send half and a receive half so other work can overlap the
 * transfer ([EPMC] "Portable kernels"; [EFA] "MoE all-to-all over EFA").
 *
 * Conventions for every call below.
 *  - Return value: MOE_OK (0) or a negative moe_status.  Calls never throw and
 *    never abort the process.
 *  - Pointers named as device pointers are device memory of the current HIP
 *    device, 16-byte aligned (MOE_ERR_INVALID otherwise).  Tensors are dense,
 *    row-major, with the shapes given; bf16 data is passed as raw 16-bit
 *    patterns.
 *  - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *    the caller keeps inputs unchanged and outputs unread until the call's
 *    work completes in stream order.  The halves may run on different streams
 *    if the caller orders them with events.
 *  - Order: create -> (dispatch_send -> dispatch_recv -> combine_send ->
 *    combine_recv)* -> destroy.  A call out of this order returns
 *    MOE_ERR_STATE and enqueues nothing; combine_recv ends the cycle, like the
 *    pages' barrier that keeps a rank from starting the next dispatch while
 *    peers still read ([EPMC] "Portable kernels").
 *  - Routing errors (an expert id outside [0,E)) are found on the device; the
 *    kernels then write none of the row buffers or outputs of that cycle
 *    (only that cycle: the next dispatch_send starts with a clean cycle
 *    word), and moe_group_status() reports MOE_ERR_ROUTING.  The four calls
 *    never synchronise with the device, so they cannot return an error the
 *    device finds later; the status call is where device errors surface.
 *  - One host thread at a time per group.
 *  - Tracing: each of the four calls is a ROCTX range named after it
 *    (rocprofv3 --marker-trace shows them).
 *  - Debug mode: with MOE_EP_DEBUG=1 in the environment when a group is
 *    created, every call first fills (on its stream, with a kernel) each
 *    buffer its kernels must rewrite with 0xFF bytes -- bf16 NaN, int32 -1:
 *    dispatch_send the group's row pools, planes, plan tables and row maps;
 *    dispatch_recv the expert-order metadata and the caller's expert rows,
 *    scales and offsets of this cycle; combine_send both row pools;
 *    combine_recv the caller's output of this cycle -- so a stale or unwritten
 *    read shows as NaN or as an index error.  Outputs are unchanged; each
 *    call costs a few extra passes over its buffers.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID = -1,   /* bad argument: null/misaligned pointer, size out of range */
    MOE_ERR_HIP = -2,       /* a HIP runtime call failed */
    MOE_ERR_OOM = -3,       /* device allocation failed at create */
    MOE_ERR_STATE = -4,     /* call out of the dispatch/combine order */
    MOE_ERR_ROUTING = -5,   /* device saw an expert id outside [0, E) */
    MOE_ERR_CAPACITY = -6,  /* a receive count exceeded the page's bound (never expected) */
    MOE_ERR_INTERNAL = -7,  /* a device-side index check failed; the offending writes were skipped */
    MOE_ERR_SCRATCH = -8    /* moe_group_create_static: the group does not fit MOE_SCRATCH_BYTES */
} moe_status;

typedef enum moe_dtype {
    MOE_BF16 = 0,           /* dispatch payload: bf16 rows, 2H bytes */
    MOE_FP8_E4M3 = 1        /* dispatch payload: OCP e4m3 rows (H bytes) + fp32 scale per 128 elements */
} moe_dtype;

/* How rows reach the peer (same four calls and results either way, as the
 * pages keep one interface across transports -- [EFA] "MoE all-to-all over
 * EFA"):
 *   MOE_TRANSPORT_STAGED  pack into a contiguous per-peer send buffer, then a
 *                         transfer copies each (sender -> receiver) segment
 *                         into the receive buffer; combine mirrors it.  This
 *                         is the network model: one write per peer from a
 *                         send buffer ([EFA] "Dispatch and combine").
 *   MOE_TRANSPORT_DIRECT  pack writes each row straight into the receiver's
 *                         receive region and combine writes each expert
 *                         output straight back into the token owner's return
 *                         rows, like the pages' intra-node push into peers'
 *                         buffers ([EFA] "Dispatch and combine") and their
 *                         shared-buffer idea ([EPMC] "Further improvements").
 *                         No send buffer: two fewer row passes per stage. */
typedef enum moe_transport {
    MOE_TRANSPORT_STAGED = 0,
    MOE_TRANSPORT_DIRECT = 1
} moe_transport;

/* Where combine sums the weighted expert outputs:
 *   MOE_COMBINE_RECEIVER  every expert output returns to the token's owner,
 *                         which forms the weighted sum of its K rows ([EPMC]
 *                         "Combine": the receiver computes the weighted
 *                         average locally).  One fp32 fma chain per token.
 *   MOE_COMBINE_PARTIAL   each expert owner first sums the outputs of the
 *                         token's experts it holds and returns one row per
 *                         (token, rank), fewer bytes at some cost in
 *                         precision ([EFA] "Dispatch/combine latency": the
 *                         send-side accumulation of prefill kernels).  The
 *                         router weights are then given to dispatch_send and
 *                         travel with the rows.  Rounding: a bf16 partial per
 *                         (token, rank) (fp32 fma chain, k ascending, from
 *                         +0), then an fp32 sum of the partials, rank
 *                         ascending, from +0, rounded to bf16. */
typedef enum moe_combine_mode {
    MOE_COMBINE_RECEIVER = 0,
    MOE_COMBINE_PARTIAL = 1
} moe_combine_mode;

/* Layout of the receive buffers:
 *   MOE_LAYOUT_PACKED      rank d's receive rows are contiguous at bases
 *                          computed from the exchanged counts, sources
 *                          ascending ([EFA] "Send and receive buffers").
 *   MOE_LAYOUT_FIXED_SLOT  rank d holds, for each of its experts
 *                          e = d*L + j, an area of max_tokens slot planes of
 *                          N rows; a sender s writes its i-th row for expert
 *                          e to row (e*max_tokens + i)*N + s, an address it
 *                          knows from its own counts ([EPMC]
 *                          "Portable kernels": the fixed token maximum bounds
 *                          each (source, local expert) share).  The receive
 *                          buffers then have N*E*max_tokens rows.  A sender
 *                          with more than max_tokens rows for one expert
 *                          (only possible when a token names an expert twice)
 *                          raises MOE_ERR_CAPACITY and the cycle writes
 *                          nothing.  dispatch_recv's outputs are the same as
 *                          with MOE_LAYOUT_PACKED. */
typedef enum moe_layout {
    MOE_LAYOUT_PACKED = 0,
    MOE_LAYOUT_FIXED_SLOT = 1
} moe_layout;

/* Sizes fixed at creation ([EPMC] "Portable kernels": the maximum number of
 * tokens a rank may dispatch is fixed for the group, and the buffers are
 * reused by every layer).  Limits: 1 <= num_ranks <= 1024; num_experts a
 * multiple of num_ranks, <= 1024; 1 <= top_k <= 64; hidden a multiple of 8
 * (of 128 for MOE_FP8_E4M3), <= 65536; 0 <= max_tokens and
 * num_ranks*max_tokens*top_k < 2^31 (with MOE_LAYOUT_FIXED_SLOT also
 * num_ranks*num_experts*max_tokens < 2^31). */
typedef struct moe_group_desc {
    int32_t num_ranks;      /* N */
    int32_t num_experts;    /* E */
    int32_t top_k;          /* K */
    int32_t hidden;         /* H */
    int32_t max_tokens;     /* T_max per rank */
    int32_t dispatch_dtype; /* moe_dtype */
    int32_t transport;      /* moe_transport */
    int32_t combine_mode;   /* moe_combine_mode */
    int32_t layout;         /* moe_layout */
} moe_group_desc;

typedef struct moe_group_s* moe_group_t;

/* Create a group: validates `desc`, allocates every internal buffer on the
 * current HIP device (two pooled row buffers of N*T_max*K rows of
 * max(payload, 2H) bytes -- the receive one N*E*T_max rows with
 * MOE_LAYOUT_FIXED_SLOT -- used by dispatch and again by combine, as the
 * pages reuse them between the two -- [EFA] "Dispatch and combine" -- plus
 * counts, offsets and metadata).  On success *out owns them.  Errors: MOE_ERR_INVALID,
 * MOE_ERR_OOM, MOE_ERR_HIP; *out is untouched on error. */
int moe_group_create(const moe_group_desc* desc, moe_group_t* out);

/* For callers that cannot allocate device memory (code that must not call
 * hipMalloc: a serving loop, a harness that forbids allocation, setup next to
 * code under graph capture): the same group as moe_group_create, with every
 * internal buffer placed in a static device array of MOE_SCRATCH_BYTES
 * (64 MiB) that the library holds on each device it runs on until the process
 * ends.  No hipMalloc, hipFree or other allocation, on the device or the
 * host.  Enough for, e.g., the Mixtral-8x7B decode shape (8 ranks x 128
 * tokens x hidden 4096, top-2 of 8; ~35 MB); not for the DeepSeek-R1 shapes.
 *  - One such group per device at a time: while one is live (until
 *    moe_group_destroy), another returns MOE_ERR_STATE.  The area keeps the
 *    last group's contents; creation clears what must start at zero (error
 *    words, counters, offsets).  Not safe to call from two host threads at
 *    once; two groups' calls cannot overlap on one device since only one
 *    exists, and the four calls of that group race with each other only as
 *    any group's do (order them on one stream, or with events).
 *  - Errors: MOE_ERR_INVALID (bad desc, or a device index >= 64),
 *    MOE_ERR_SCRATCH (the group needs more than MOE_SCRATCH_BYTES),
 *    MOE_ERR_STATE, MOE_ERR_HIP.  *out is untouched on error.
 *  - It synchronises the device once (clearing the words); call it outside
 *    graph capture.  The group's four calls enqueue kernels only, as for any
 *    group; moe_group_destroy releases the area (it frees nothing). */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
int moe_group_create_static(const moe_group_desc* desc, moe_group_t* out);

/* Synchronise the device, free every buffer of the group and the handle (a
 * group of moe_group_create_static releases the static area instead).
 * NULL is accepted and ignored. */
int moe_group_destroy(moe_group_t g);

/* Dispatch, send half ([EFA] "Dispatch and combine": per-expert counts by
 * atomic adds in one block, a cumulative sum for the offsets, rows packed into
 * contiguous per-peer send buffers, then one write per peer; [EPMC] "Dispatch":
 * activations, block scales and the token's index packed together).
 *   num_tokens    T, 0 <= T <= max_tokens (same T on every logical rank)
 *   x             device, bf16 [N][T][H]
 *   topk_idx      device, int32 [N][T][K], expert ids in [0, E)
 *   topk_weights  device, fp32 [N][T][K] with MOE_COMBINE_PARTIAL (carried
 *                 to the expert owners with the rows); ignored, may be
 *                 NULL, with MOE_COMBINE_RECEIVER
 * Enqueues: route plan (counts, stable positions, send offsets; the group
 * offsets too where the pack or the partial combine needs them before
 * dispatch_recv; with MOE_COMBINE_PARTIAL also the partial-row plan), pack
 * (+ e4m3 encode) and, with the staged transport, the transfer into the
 * receive buffers.  Reads x, topk_idx and topk_weights only. */
int moe_dispatch_send(moe_group_t g, int32_t num_tokens, const void* x,
                      const int32_t* topk_idx, const float* topk_weights,
                      hipStream_t stream);

/* Dispatch, receive half ([EPMC] "Dispatch": received tokens are copied into
 * contiguous buffers for the grouped GEMM and the source rank, expert and
 * token index are stored for combine; [EFA] "Dispatch and combine": shuffle
 * from the receive buffer into the grouped-GEMM tensor).
 *   expert_x        device, [N*T*K] rows: bf16 [..][H] or e4m3 bytes [..][H];
 *                   rows sorted by (expert, source rank, token, k)
 *   expert_scale    device, fp32 [N*T*K][H/128] for MOE_FP8_E4M3, else NULL
 *   expert_offsets  device, int32 [E+1]: expert e's rows are
 *                   [expert_offsets[e], expert_offsets[e+1]); rank d's GEMM
 *                   input is rows [expert_offsets[d*L], expert_offsets[(d+1)*L])
 * Enqueues: the receiver's group offsets and row maps from the exchanged
 * counts and send offsets, then the shuffle.  The back-routing metadata
 * stays in the group. */
int moe_dispatch_recv(moe_group_t g, void* expert_x, float* expert_scale,
                      int32_t* expert_offsets, hipStream_t stream);

/* Combine, send half ([EPMC] "Combine": unquantised 16-bit expert outputs are
 * sent back, each to the rank and token slot it came from; [EFA] "Dispatch and
 * combine": routing is already known, rows go one write per peer).
 *   expert_y  device, bf16 [N*T*K][H], rows in the order of expert_x
 * Enqueues (staged): inverse shuffle into the per-peer layout, transfer back;
 * (direct): one kernel writing each output into its return row.  With
 * MOE_COMBINE_PARTIAL: one kernel forming the bf16 partial row of every
 * (token, rank) from the expert outputs and the carried weights, into the
 * ranks' return rows (staged) or straight into the token owner's rows
 * (direct); staged adds the transfer of the partial rows. */
int moe_combine_send(moe_group_t g, const void* expert_y, hipStream_t stream);

/* Combine, receive half ([EPMC] "Introduction": the output is the sum of the
 * K expert outputs weighted by the router; [EPMC] "Combine": the receiver
 * computes it locally into an externally allocated tensor).
 *   topk_weights  device, fp32 [N][T][K] (MOE_COMBINE_RECEIVER); ignored,
 *                 may be NULL, with MOE_COMBINE_PARTIAL
 *   out           device, bf16 [N][T][H]
 * MOE_COMBINE_RECEIVER: out[s][t][h] = bf16_rne(acc) with acc = +0 and, for
 * k = 0..K-1 in order, acc = fma(w[s][t][k], y_k[h], acc) in fp32, y_k the
 * expert output of (s,t,k).
 * MOE_COMBINE_PARTIAL: out[s][t][h] = bf16_rne(sum over the ranks d the
 * token visited, d ascending, from +0, in fp32, of its partial row's value);
 * partial(s,t,d) = bf16_rne(fp32 fma chain from +0 over the k with
 * topk_idx / L == d, k ascending, of w * y_k). */
int moe_combine_recv(moe_group_t g, const float* topk_weights, void* out,
                     hipStream_t stream);

/* Device pointers of the group's internal buffers, for checking only.  The
 * pooled send buffer holds send_x during dispatch and comb_send during
 * combine; the pooled receive buffer holds recv_x, then comb_recv.  Layouts:
 * send rows of sender s are rows [s*T*K, (s+1)*T*K); receive rows of rank d
 * are rows [recv_base[d], recv_base[d+1]).  With the direct transport there
 * is no send buffer: send_x, send_scale, send_meta and comb_send are NULL.
 * With MOE_LAYOUT_FIXED_SLOT the receive planes have recv_rows rows, the
 * slots first (slots no row names hold stale data), recv_off and recv_base still
 * give the packed order the kernels walk, and with the staged transport the
 * two pools swap roles in combine: comb_send (slot layout) is in the
 * receive pool, comb_recv (send layout) in the send pool.
 * With MOE_COMBINE_PARTIAL the first P = part_base[N] rows of comb_send hold
 * the partial rows in owner layout (rank d, then sender s, then token t; rank
 * d's rows start at part_owner_base[d]) and those of comb_recv in token layout
 * (sender s, then rank d, then token t; row part_base[s] + part_pos[s][t][k]
 * for the first k of the token on rank d).  The part_* fields and the weight
 * planes are NULL with MOE_COMBINE_RECEIVER (send_w also with direct). */
typedef struct moe_group_view {
    moe_group_desc desc;
    int32_t num_tokens;          /* T of the current cycle */
    int64_t rows;                /* N*T*K */
    int64_t payload_row_bytes;   /* 2H (bf16) or H (e4m3) */
    int64_t combine_row_bytes;   /* 2H */
    int32_t scale_blocks;        /* H/128 for e4m3, else 0 */
    int32_t* cnt;                /* [N][E]     tokens of sender s for expert e */
    int32_t* pos;                /* [N][T][K]  row of (t,k) in its sender's rows */
    int32_t* send_off;           /* [N][E+1]   first row of expert e in sender s's rows */
    int32_t* recv_off;           /* [N][N+1]   first row from sender s in receiver d's rows */
    int32_t* recv_base;          /* [N+1]      first pooled receive row of rank d */
    int32_t* expert_off;         /* [E+1]      first expert-order row of expert e */
    void* send_x;                /* [rows][payload_row_bytes] */
    float* send_scale;           /* [rows][scale_blocks] or NULL */
    int32_t* send_meta;          /* [rows] t*K+k */
    void* recv_x;
    float* recv_scale;
    int32_t* recv_meta;
    int32_t* expert_src_rank;    /* [rows] source rank of each expert-order row */
    int32_t* expert_src_slot;    /* [rows] t*K+k on the source rank */
    void* comb_send;             /* [rows][combine_row_bytes], receive layout */
    void* comb_recv;             /* [rows][combine_row_bytes], send layout */
    float* send_w;               /* [rows] router weight of each send row */
    float* recv_w;               /* [rows] router weight of each receive row */
    int32_t* part_dst;           /* [N][T][K]  destination rank of item (s,t,k) */
    int32_t* part_pos;           /* [N][T][K]  row of (s,t,rank) among sender s's partial
                                    rows for the rank's first k of the token, else -1 */
    int32_t* part_send_off;      /* [N][N+1]   first partial row of rank d among sender s's */
    int32_t* part_base;          /* [N+1]      first token-layout partial row of sender s */
    int32_t* part_owner_base;    /* [N+1]      first owner-layout partial row of rank d */
    int64_t recv_rows;           /* rows of the receive planes: N*T_max*K, or with
                                    MOE_LAYOUT_FIXED_SLOT max(N*E*T_max, N*T_max*K) */
} moe_group_view;

int moe_group_view_get(moe_group_t g, moe_group_view* out);

/* Synchronise `stream`, then return and clear the device-side errors of
 * every cycle since the previous status call: MOE_OK, MOE_ERR_ROUTING,
 * MOE_ERR_CAPACITY or MOE_ERR_INTERNAL (in that order of precedence when
 * several bits are set).  Only `stream` is synchronised: when the group's
 * calls ran on several streams, synchronise the others first (or pass the
 * stream that was ordered after them), or a bit set by work still running on
 * another stream can be missed. */
int moe_group_status(moe_group_t g, hipStream_t stream);

/* Per-kernel timing, for measurement.  kernel_mask selects the kernels to
 * time (bit k = moe_kernel_id k; 0 = off; MOE_KERNEL_ALL = every kernel).  A
 * timed launch carries a pair of HIP events attached to its dispatch
 * (recorded at the kernel's start and end on the launch stream); each timed
 * kernel costs a few microseconds of extra gap, so time only what is needed.
 * Reading synchronises on the events, returns the summed milliseconds and
 * launch counts per kernel (arrays of MOE_KERNEL_COUNT) and resets them. */
typedef enum moe_kernel_id {
    MOE_KERNEL_ROUTE_PLAN = 0,      /* counts, stable positions, all offsets */
    MOE_KERNEL_PACK = 1,
    MOE_KERNEL_TRANSFER = 2,
    MOE_KERNEL_SHUFFLE = 3,
    MOE_KERNEL_COMBINE_PACK = 4,
    MOE_KERNEL_TRANSFER_BACK = 5,
    MOE_KERNEL_COMBINE_REDUCE = 6,
    MOE_KERNEL_COMBINE_PUSH = 7,    /* direct transport: replaces combine pack + transfer back */
    MOE_KERNEL_PARTIAL_SEND = 8,    /* MOE_COMBINE_PARTIAL: the expert-side partial sums */
    MOE_KERNEL_PARTIAL_TRANSFER = 9,
    MOE_KERNEL_PARTIAL_REDUCE = 10,
    MOE_KERNEL_RECV_MAP = 11,       /* dispatch_recv: the receiver's group offsets and row maps from the exchanged counts */
    MOE_KERNEL_COUNT = 12
} moe_kernel_id;

typedef enum moe_kernel_mask { MOE_KERNEL_ALL = (1 << MOE_KERNEL_COUNT) - 1 } moe_kernel_mask;

int moe_group_timing_enable(moe_group_t g, int kernel_mask);
int moe_group_timing_read(moe_group_t g, double* total_ms, int64_t* launches);

/* MEASUREMENT-ONLY EXPORT, not one of the method's calls (the benchmark uses
 * it to measure the copy ceiling the row movers are compared against).
 * Streaming kernels with the row
 * movers' access style (16-byte nontemporal vectors, all loads of a lane in
 * flight before its stores), to measure what HBM delivers for each traffic
 * mix on this device.  kind: MOE_PROBE_COPY (read src, write dst),
 * MOE_PROBE_READ (read src; dst receives at most one 4-byte word),
 * MOE_PROBE_WRITE (write dst).  bytes: a multiple of 16, > 0; device
 * pointers 16-byte aligned.  Errors: MOE_ERR_INVALID, MOE_ERR_HIP. */
typedef enum moe_probe_kind {
    MOE_PROBE_COPY = 0,
    MOE_PROBE_READ = 1,
    MOE_PROBE_WRITE = 2
} moe_probe_kind;

int moe_hbm_probe(int kind, void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* moe_strerror(int status);

/* Name of a kernel id (as listed in profiler traces); "" if out of range. */
const char* moe_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
