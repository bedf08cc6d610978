// Internal launch interface between the host planner (moe_ep.hip) and the
// device kernels (moe_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Bits of the device-side error word.
constexpr int32_t ERR_BIT_ROUTING = 1;
constexpr int32_t ERR_BIT_CAPACITY = 2;
constexpr int32_t ERR_BIT_INTERNAL = 4;   // a device-side index check failed

// Limits the kernels are written for (checked by the host before launch).
constexpr int MAX_EXPERTS = 1024;
constexpr int MAX_RANKS = 1024;
constexpr int MAX_TOPK = 64;

struct Shape {
    int N, E, K, L, H, T;
    int fp8;              // payload is e4m3 + fp32 block scales
    int direct;           // direct transport: pack and combine write the peer's rows
    int partial;          // combine sums on the expert side, one row per (token, rank)
    int fixed;            // fixed-slot receive layout: T_max slots per (source, expert),
                          // each expert's area slot-major
    int sender_only;      // fixed slots with the receiver-side combine: dispatch_send's
                          // kernels use only each sender's own plan
    int plan_offsets;     // the route plan's last workgroup forms the group offsets
                          // (plan_offsets_needed); else the receiver's map kernel does
    int slots;            // T_max (fixed-slot layout)
    int64_t recv_rows;    // rows of the receive planes: rows, or N*E*slots (fixed-slot)
    int64_t rows;         // N*T*K
    int payload_vecs;     // 16-byte vectors per payload row (2H/16 or H/16)
    int comb_vecs;        // 16-byte vectors per combine row (2H/16)
    int scale_blocks;     // H/128 (fp8) or 0
};

// Whether the pack runs in send-row order (each row's item then comes from
// the route plan): when one sender's tokens fit well within an XCD's 4 MiB
// L2, so that the K reads of each token after the first hit it.  DeepSeek-R1 decode (1.75 MiB per sender, one sender per XCD
// run), staged: pack 86.9 -> 74.5 us warm, 115 -> 99 MALL-flushed; on the
// prefill (28 MiB per sender) the row order re-reads every token from HBM or
// the MALL and took 4.9-5.0 ms against 1.87 in token order.  With the
// partial combine, whose records are made per token, the same launch runs a
// block per sender for them ahead of the row blocks.
constexpr int64_t PACK_ROWS_MAX_SENDER_BYTES = 2 << 20;

inline bool pack_in_row_order(const Shape& sh)
{
    return (int64_t)sh.T * sh.H * 2 <= PACK_ROWS_MAX_SENDER_BYTES;
}

// With the partial combine and the send-row-order pack, each block of the
// pack's token records forms its sender's bases itself: E + 2N + 2 sums of N
// terms over the senders' send offsets (the first expert row of each of its
// experts, the first receive row and the first owner-layout partial row on
// each rank, its first token-layout partial row and the total).  Up to this
// many terms per block; past it the route plan's last workgroup forms the
// group tables once and the blocks read them.  Partial combine, route plan
// with the tables -> without, warm: Mixtral decode 11.8 -> 6.6 us, DeepSeek-R1
// decode 19.7 -> 11.0, Kimi-K2 decode 26.6 -> 11.4; staged step, warm /
// MALL-flushed: Mixtral 62.6 -> 57.0 / 67.2 -> 62.1 (direct 48.3 -> 43.7 /
// 52.0 -> 46.0), DeepSeek-R1 754 -> 752 / 779 -> 772, Kimi-K2 1359 -> 1364 /
// 1407 -> 1394 (the direct pack forms each row's receive base from the send
// offsets and takes back 5-8 us of the plan's gain there).
constexpr int64_t RECORD_SUMS_MAX = 1 << 16;

inline bool record_sums(const Shape& sh)
{
    return (int64_t)(sh.E + 2 * sh.N + 2) * sh.N <= RECORD_SUMS_MAX;
}

// Whether the route plan forms the group offsets in its last workgroup: for
// the kernels that need them before dispatch_recv -- the packed layout's
// token-order pack (its rows' receive rows), the partial combine's records
// in the token-order pack, and those of the send-row-order pack past
// RECORD_SUMS_MAX.  Otherwise (the send-row-order pack, which derives its
// receive rows or transfer map, and its records, from the send offsets, and
// fixed slots with the receiver-side combine) the route plan ends when its
// ranks do, and the receiver's map kernel forms them from the exchanged
// counts.  Route plan, warm: Mixtral decode 7.3 -> 5.1 us (staged) and
// 8.7 -> 6.6 (direct); DeepSeek-R1 decode 11.2 -> 6.3 and 11.6 -> 6.1;
// Kimi-K2 decode 15.2 -> 6.6 and 15.3 -> 6.8, the pack and the receive map
// taking back 0.5-7 us of it.
inline bool plan_offsets_needed(const Shape& sh)
{
    if (!pack_in_row_order(sh))
        return sh.partial || !sh.fixed;
    return sh.partial && !record_sums(sh);
}

struct Plan {              // device pointers owned by the group
    // Errors.  err is the current cycle's word and err_next the next cycle's
    // (the group alternates two words): every route-plan workgroup ORs its
    // sender's bits into err, and one clears err_next for the next cycle, so
    // an error stops only the kernels of its own cycle; every later kernel of
    // the cycle writes nothing while err is set.  err_sticky collects every
    // cycle's bits until moe_group_status reads and clears it.
    int32_t* err;
    int32_t* err_next;
    int32_t* err_rank;     // [N]  routing/capacity bits of each sender, this cycle
    int32_t* err_sticky;
    int32_t* ticket;       // arrival counter of the route-plan workgroups (0 between launches)
    int32_t* cnt;          // [N][E]
    int32_t* pos;          // [N][T][K]
    int32_t* soff;         // [N][E+1]
    int32_t* soff_col;     // [E+1][N]  soff transposed, for sums over the senders
    int32_t* roff;         // [N][N+1]
    int32_t* rbase;        // [N+1]
    int32_t* eoff;         // [E+1]
    // Receive rows are numbered in the packed order q (rank, source, expert,
    // t, k); with the fixed-slot layout a row's place in the receive planes
    // is slot_of[q], otherwise q itself.  The sender's pack writes the maps its
    // own transfer follows (xfer_src, send_slot); the receiver's map kernel
    // writes the rest from the exchanged counts and offsets.
    int32_t* xfer_src;     // [rows]  packed receive row q <- send row xfer_src[q] (sender)
    int32_t* send_slot;    // [rows]  send row -> its slot (fixed-slot layout; sender)
    int2* xfer_dst;        // [rows]  send row -> (its receive-plane row, its expert row)
    int2* shuf_map;        // [rows]  expert row r <- (receive-plane row, source rank)
    int32_t* shuf_inv;     // [rows]  packed receive row -> its expert row
    int32_t* send_item;    // [rows]  send row -> its item t*K+k, for the direct transport's
                           //         send-row-order pack (staged: the send meta words)
    // combine with expert-side partial sums (null unless Shape::partial)
    int32_t* pdst;         // [N][T][K]  destination rank of item (s,t,k)
    int32_t* ppos;         // [N][T][K]  first k of its rank in the token: row among sender
                           //            s's partial rows (rank-major, then t); else -1
    int32_t* psoff;        // [N][N+1]   first partial row of (sender s, rank d) among s's
    int32_t* psoff_col;    // [N+1][N]   psoff transposed, for sums over the senders
    int32_t* sbase;        // [N][E+2N+2] each sender's bases, formed by the route plan's
                           //            last workgroup (Shape::plan_offsets): its first
                           //            expert row of each expert, first receive row and
                           //            first owner-layout partial row on each rank, first
                           //            token-layout partial row, and P
    int32_t* qoff;         // [N][N+1]   first owner-layout row of sender s among rank d's
    int32_t* qbase;        // [N+1]      first owner-layout row of rank d (qbase[N] = P)
    int32_t* pbase;        // [N+1]      first token-layout row of sender s (pbase[N] = P)
    int32_t* pmap;         // [rows]     token-layout row -> owner-layout row (staged)
    int4* phead;           // [rows][2]  partial row the expert side writes (owner layout when
                           //            staged, token layout when direct) -> (expert row,
                           //            receive-plane row of its first item, the same of its
                           //            second), (token, item count, mask of the token's
                           //            items on that rank: low word, high word)
    int2* pitem;           // [N][T][K]  item (s,t,k) -> (its expert row, its receive-plane row)
    int32_t* slot_of;      // [rows]     packed receive row -> its slot (fixed-slot layout)
};

struct Rows {              // pooled row buffers
    void* send_x;          // payload, send layout
    float* send_scale;
    int32_t* send_meta;
    void* recv_x;          // payload, receive layout
    float* recv_scale;
    int32_t* recv_meta;
    int32_t* src_rank;     // expert-order metadata
    int32_t* src_slot;
    void* comb_send;       // combine rows, receive layout (aliases send_x storage)
    void* comb_recv;       // combine rows, send layout (aliases recv_x storage)
    float* send_w;         // router weight of each send row (partial combine, staged)
    float* recv_w;         // router weight of each receive row (partial combine)
};

// Where and how a kernel is launched: the caller's stream, and optionally a
// pair of events attached to the dispatch itself (they time the kernel
// without adding packets to the stream).
struct Launch {
    hipStream_t stream;
    hipEvent_t start;
    hipEvent_t stop;
};

hipError_t launch_route_plan(const Shape& sh, const int32_t* idx, const Plan& p, const Rows& r,
                             const Launch& L);
hipError_t launch_pack(const Shape& sh, const void* x, const int32_t* idx, const float* w,
                       const Plan& p, const Rows& r, const Launch& L);
hipError_t launch_transfer(const Shape& sh, const Plan& p, const Rows& r, const Launch& L);
// The receiver's group offsets and row maps from the exchanged counts and
// send offsets.
hipError_t launch_recv_map(const Shape& sh, const Plan& p, const Launch& L);
hipError_t launch_shuffle(const Shape& sh, const Plan& p, const Rows& r, void* expert_x,
                          float* expert_scale, int32_t* expert_offsets, const Launch& L);
hipError_t launch_combine_pack(const Shape& sh, const Plan& p, const Rows& r,
                               const void* expert_y, const Launch& L);
hipError_t launch_transfer_back(const Shape& sh, const Plan& p, const Rows& r, const Launch& L);
hipError_t launch_combine_push(const Shape& sh, const Plan& p, const Rows& r,
                               const void* expert_y, const Launch& L);
hipError_t launch_combine_reduce(const Shape& sh, const Plan& p, const Rows& r, const float* w,
                                 void* out, const Launch& L);
hipError_t launch_partial_send(const Shape& sh, const Plan& p, const Rows& r, const void* expert_y,
                               const Launch& L);
hipError_t launch_partial_transfer(const Shape& sh, const Plan& p, const Rows& r, const Launch& L);
hipError_t launch_partial_reduce(const Shape& sh, const Plan& p, const Rows& r, void* out,
                                 const Launch& L);
// Fill `bytes` bytes (a multiple of 4, p 16-byte aligned) with a repeated
// 32-bit pattern: the debug mode's poisoning of buffers a call must rewrite.
hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream);
// Streaming probes (kind: 0 copy, 1 read, 2 write) over `vecs` 16-byte vectors.
hipError_t launch_hbm_probe(int kind, void* dst, const void* src, int64_t vecs, hipStream_t stream);

}  // namespace moe
