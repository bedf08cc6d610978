// Host side of the C ABI declared in include/moe_ep.h: argument validation,
// the group's memory plan, the call-order state machine, and kernel launches
// on the caller's stream.
//
// Pages cited:
//   [EPMC] "Efficient and portable Mixture-of-Experts communication"
//   [EFA]  "Enabling trillion-parameter models on AWS EFA"
//
// Memory plan.  The pages size every rank's receive space for the worst case
// (a rank receives at most N*T*max(K, E/N) rows -- [EFA] "Send and receive
// buffers").  Here all N logical ranks share one device, and together they
// always hold exactly N*T*K rows per stage, so the send and receive buffers are
// each ONE pooled array of N*T_max*K rows: sender s owns rows
// [s*T*K, (s+1)*T*K) of the send pool, receiver d owns rows
// [rbase[d], rbase[d+1]) of the receive pool, bases computed on the device from
// the exchanged counts.  The same two pools carry the combine rows, as the
// pages reuse buffers between dispatch and combine ([EFA] "Dispatch and
// combine").  Row size of a pool = max(payload row, 2H) = 2H bytes.
//
// With the fixed-slot layout ([EPMC] "Portable kernels") the receive pool and
// its planes instead hold T_max slots per (source, expert), each expert's
// area slot-major (row (e*T_max + i)*N + s): N*E*T_max rows.  The direct transport has no send pool; the
// partial combine's rows (at most N*T*K) reuse whichever pools combine uses.
#include <hip/hip_runtime.h>

#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "moe_ep.h"
#include "moe_kernels.h"

namespace {

enum class State { Idle, Sent, Received, CombineSent };

struct EventPair {
    hipEvent_t start = nullptr, stop = nullptr;
    int kernel = 0;
};

}  // namespace

struct moe_group_s {
    moe_group_desc desc{};
    int device = 0;
    int L = 0;
    int64_t rows_max = 0;
    int64_t recv_rows_max = 0;  // rows of the receive planes
    int payload_bytes = 0;   // per row
    int comb_bytes = 0;
    int scale_blocks = 0;

    moe::Plan plan{};
    void* pool_send = nullptr;
    void* pool_recv = nullptr;
    float* send_scale = nullptr;
    float* recv_scale = nullptr;
    int32_t* send_meta = nullptr;
    int32_t* recv_meta = nullptr;
    int32_t* src_rank = nullptr;
    int32_t* src_slot = nullptr;
    float* send_w = nullptr;     // partial combine: router weights beside the rows
    float* recv_w = nullptr;

    State state = State::Idle;
    int32_t T = 0;
    uint32_t cycle = 0;          // dispatch_send calls so far: picks the cycle's error word
    int32_t* err_words = nullptr;  // the two alternating cycle words

    int timing_mask = 0;
    std::vector<EventPair> events;
    size_t events_used = 0;

    std::vector<void*> allocations;
    bool in_scratch = false;     // buffers carved from the device's static scratch area
    bool debug = false;          // MOE_EP_DEBUG: poison what each call must rewrite
};

namespace {

const char* const kKernelNames[MOE_KERNEL_COUNT] = {
    "route_plan_kernel",   "pack_kernel",          "transfer_kernel",       "shuffle_kernel",
    "combine_pack_kernel", "transfer_back_kernel", "combine_reduce_kernel", "combine_push_kernel",
    "partial_send_kernel", "partial_transfer_kernel", "partial_reduce_kernel",
    "recv_map_kernel",
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int validate_desc(const moe_group_desc* d)
{
    if (!d)
        return MOE_ERR_INVALID;
    if (d->num_ranks < 1 || d->num_ranks > moe::MAX_RANKS)
        return MOE_ERR_INVALID;
    if (d->num_experts < d->num_ranks || d->num_experts > moe::MAX_EXPERTS ||
        d->num_experts % d->num_ranks != 0)
        return MOE_ERR_INVALID;
    if (d->top_k < 1 || d->top_k > moe::MAX_TOPK)
        return MOE_ERR_INVALID;
    if (d->hidden < 8 || d->hidden > 65536 || d->hidden % 8 != 0)
        return MOE_ERR_INVALID;
    if (d->dispatch_dtype != MOE_BF16 && d->dispatch_dtype != MOE_FP8_E4M3)
        return MOE_ERR_INVALID;
    if (d->dispatch_dtype == MOE_FP8_E4M3 && d->hidden % 128 != 0)
        return MOE_ERR_INVALID;
    if (d->max_tokens < 0)
        return MOE_ERR_INVALID;
    if (d->transport != MOE_TRANSPORT_STAGED && d->transport != MOE_TRANSPORT_DIRECT)
        return MOE_ERR_INVALID;
    if (d->combine_mode != MOE_COMBINE_RECEIVER && d->combine_mode != MOE_COMBINE_PARTIAL)
        return MOE_ERR_INVALID;
    if (d->layout != MOE_LAYOUT_PACKED && d->layout != MOE_LAYOUT_FIXED_SLOT)
        return MOE_ERR_INVALID;
    const int64_t rows = (int64_t)d->num_ranks * d->max_tokens * d->top_k;
    if (rows >= ((int64_t)1 << 31))
        return MOE_ERR_INVALID;
    const int64_t slots = (int64_t)d->num_ranks * d->num_experts * d->max_tokens;
    if (d->layout == MOE_LAYOUT_FIXED_SLOT && slots >= ((int64_t)1 << 31))
        return MOE_ERR_INVALID;
    return MOE_OK;
}

moe::Shape shape_of(const moe_group_s* g, int T)
{
    moe::Shape sh{};
    sh.N = g->desc.num_ranks;
    sh.E = g->desc.num_experts;
    sh.K = g->desc.top_k;
    sh.L = g->L;
    sh.H = g->desc.hidden;
    sh.T = T;
    sh.fp8 = g->desc.dispatch_dtype == MOE_FP8_E4M3;
    sh.direct = g->desc.transport == MOE_TRANSPORT_DIRECT;
    sh.partial = g->desc.combine_mode == MOE_COMBINE_PARTIAL;
    sh.fixed = g->desc.layout == MOE_LAYOUT_FIXED_SLOT;
    sh.sender_only = sh.fixed && !sh.partial;
    sh.slots = g->desc.max_tokens;
    sh.rows = (int64_t)sh.N * T * sh.K;
    sh.recv_rows = sh.fixed ? g->recv_rows_max : sh.rows;
    sh.payload_vecs = g->payload_bytes / 16;
    sh.comb_vecs = g->comb_bytes / 16;
    sh.scale_blocks = g->scale_blocks;
    sh.plan_offsets = moe::plan_offsets_needed(sh);
    return sh;
}

moe::Rows rows_of(const moe_group_s* g)
{
    moe::Rows r{};
    r.send_x = g->pool_send;
    r.send_scale = g->send_scale;
    r.send_meta = g->send_meta;
    r.recv_x = g->pool_recv;
    r.recv_scale = g->recv_scale;
    r.recv_meta = g->recv_meta;
    r.src_rank = g->src_rank;
    r.src_slot = g->src_slot;
    // combine rows: the receive layout in the send pool and the send layout
    // in the receive pool; the fixed-slot receive layout is larger than the
    // send pool, so with it the two swap (direct push has no send pool)
    const bool swap = g->desc.layout == MOE_LAYOUT_FIXED_SLOT &&
                      g->desc.transport == MOE_TRANSPORT_STAGED;
    r.comb_send = swap ? g->pool_recv : g->pool_send;
    r.comb_recv = swap ? g->pool_send : g->pool_recv;
    r.send_w = g->send_w;
    r.recv_w = g->recv_w;
    return r;
}

void free_all(moe_group_s* g)
{
    for (void* p : g->allocations)
        (void)hipFree(p);
    g->allocations.clear();
    for (auto& e : g->events) {
        if (e.start) (void)hipEventDestroy(e.start);
        if (e.stop) (void)hipEventDestroy(e.stop);
    }
    g->events.clear();
}

// Where a group's device buffers go: each its own hipMalloc allocation, or
// (region mode) consecutive 256-byte aligned pieces of one region starting
// at `base`; with a null base the region mode only counts the bytes.  Every
// buffer takes at least 256 bytes either way.
struct Placer {
    moe_group_s* g;
    bool region = false;
    uintptr_t base = 0;
    size_t used = 0;

    template <typename T>
    int operator()(T** out, size_t count)
    {
        const size_t bytes = std::max<size_t>(count * sizeof(T), 256);
        if (region) {
            *out = reinterpret_cast<T*>(base + used);
            used += (bytes + 255) / 256 * 256;
            return MOE_OK;
        }
        void* p = nullptr;
        const hipError_t e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation ? MOE_ERR_OOM
                                                                             : MOE_ERR_HIP;
        }
        g->allocations.push_back(p);
        *out = static_cast<T*>(p);
        return MOE_OK;
    }
};

// Sizes of a group from its (validated) descriptor.
void init_sizes(moe_group_s* g)
{
    const moe_group_desc* desc = &g->desc;
    const int N = desc->num_ranks, E = desc->num_experts, K = desc->top_k, H = desc->hidden;
    const int T = desc->max_tokens;
    g->L = E / N;
    g->rows_max = (int64_t)N * T * K;
    const bool fixed = desc->layout == MOE_LAYOUT_FIXED_SLOT;
    // the receive pool also takes combine's send-layout rows (direct push),
    // and N*E*T_max < N*T_max*K when K > E
    g->recv_rows_max = fixed ? std::max((int64_t)N * E * T, g->rows_max) : g->rows_max;
    const bool fp8 = desc->dispatch_dtype == MOE_FP8_E4M3;
    g->payload_bytes = fp8 ? H : 2 * H;
    g->comb_bytes = 2 * H;
    g->scale_blocks = fp8 ? H / 128 : 0;
}

// Every device buffer of a group, placed by `take`.
int place_buffers(moe_group_s* g, Placer& take)
{
    const moe_group_desc* desc = &g->desc;
    const int N = desc->num_ranks, E = desc->num_experts, K = desc->top_k;
    const int T = desc->max_tokens;
    const size_t R = (size_t)g->rows_max;
    const size_t RQ = (size_t)g->recv_rows_max;
    const size_t row_bytes = (size_t)std::max(g->payload_bytes, g->comb_bytes);
    const bool fp8 = desc->dispatch_dtype == MOE_FP8_E4M3;
    const bool fixed = desc->layout == MOE_LAYOUT_FIXED_SLOT;
    const bool staged = desc->transport == MOE_TRANSPORT_STAGED;   // direct: no send buffer
    const bool partial = desc->combine_mode == MOE_COMBINE_PARTIAL;
    moe::Plan& p = g->plan;
    uint8_t* pool_send = nullptr;
    uint8_t* pool_recv = nullptr;
    int rc;
    if ((rc = take(&p.err, 2)) || (rc = take(&p.err_sticky, 1)) ||
        (rc = take(&p.err_rank, (size_t)N)) || (rc = take(&p.ticket, 1)) ||
        (rc = take(&p.cnt, (size_t)N * E)) ||
        (rc = take(&p.pos, (size_t)N * T * K)) || (rc = take(&p.soff, (size_t)N * (E + 1))) ||
        (rc = take(&p.soff_col, (size_t)N * (E + 1))) ||
        (rc = take(&p.roff, (size_t)N * (N + 1))) || (rc = take(&p.rbase, (size_t)N + 1)) ||
        (rc = take(&p.eoff, (size_t)E + 1)) ||
        (rc = take(&p.xfer_src, R)) || (rc = take(&p.xfer_dst, R)) ||
        (rc = take(&p.shuf_map, R)) || (rc = take(&p.shuf_inv, R)) ||
        (staged && (rc = take(&pool_send, R * row_bytes))) ||
        (rc = take(&pool_recv, RQ * row_bytes)) ||
        (staged && (rc = take(&g->send_meta, R))) || (rc = take(&g->recv_meta, RQ)) ||
        (rc = take(&g->src_rank, R)) || (rc = take(&g->src_slot, R)) ||
        (fp8 && staged && (rc = take(&g->send_scale, R * g->scale_blocks))) ||
        (fp8 && (rc = take(&g->recv_scale, RQ * g->scale_blocks))) ||
        (fixed && ((rc = take(&p.slot_of, R)) || (rc = take(&p.send_slot, R)))) ||
        (!staged && (rc = take(&p.send_item, R))) ||
        (partial && ((rc = take(&p.pdst, R)) || (rc = take(&p.ppos, R)) ||
                     (rc = take(&p.psoff, (size_t)N * (N + 1))) ||
                     (rc = take(&p.psoff_col, (size_t)N * (N + 1))) ||
                     (rc = take(&p.sbase, (size_t)N * (E + 2 * N + 2))) ||
                     (rc = take(&p.qoff, (size_t)N * (N + 1))) ||
                     (rc = take(&p.qbase, (size_t)N + 1)) ||
                     (rc = take(&p.pbase, (size_t)N + 1)) ||
                     (rc = take(&g->recv_w, RQ)) ||
                     (rc = take(&p.phead, 2 * R)) || (rc = take(&p.pitem, R)) ||
                     (staged && ((rc = take(&p.pmap, R)) || (rc = take(&g->send_w, R)))))))
        return rc;
    g->pool_send = pool_send;
    g->pool_recv = pool_recv;
    g->err_words = p.err;
    p.err_next = p.err + 1;
    return MOE_OK;
}

// The error words and the ticket counter start at zero; the offsets start
// valid for an empty cycle.
int zero_words(moe_group_s* g)
{
    const moe::Plan& p = g->plan;
    if (hipMemset(g->err_words, 0, 2 * sizeof(int32_t)) != hipSuccess ||
        hipMemset(p.err_sticky, 0, sizeof(int32_t)) != hipSuccess ||
        hipMemset(p.ticket, 0, sizeof(int32_t)) != hipSuccess ||
        hipMemset(p.eoff, 0, sizeof(int32_t) * (g->desc.num_experts + 1)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

// Run one kernel launch; with timing enabled, a pair of events is attached to
// the dispatch (recorded by the kernel's own start and end).  `launches` is
// false when the call has nothing to do and enqueues no kernel.
template <typename F>
int timed_launch(moe_group_s* g, int kernel, hipStream_t st, bool launches, F&& launch)
{
    moe::Launch L{st, nullptr, nullptr};
    if (((g->timing_mask >> kernel) & 1) && launches) {
        if (g->events_used == g->events.size()) {
            EventPair e;
            if (hipEventCreate(&e.start) != hipSuccess || hipEventCreate(&e.stop) != hipSuccess)
                return MOE_ERR_HIP;
            g->events.push_back(e);
        }
        EventPair* ev = &g->events[g->events_used++];
        ev->kernel = kernel;
        L.start = ev->start;
        L.stop = ev->stop;
    }
    return launch(L) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// A ROCTX range around one call of the C ABI (shown by rocprofv3
// --marker-trace; a few tens of nanoseconds when no tool listens).
struct CallRange {
    explicit CallRange(const char* name) { roctxRangePushA(name); }
    ~CallRange() { roctxRangePop(); }
    CallRange(const CallRange&) = delete;
    CallRange& operator=(const CallRange&) = delete;
};

bool debug_from_env()
{
    const char* v = std::getenv("MOE_EP_DEBUG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

// Debug mode: fill a buffer with 0xFF bytes (bf16 NaN, int32 -1) on the
// call's stream, so a kernel reading a row or entry its call did not write
// sees NaN or an out-of-range index instead of last cycle's value.
int poison(hipStream_t st, const void* p, size_t bytes)
{
    if (!p || bytes < 4)
        return MOE_OK;
    return from_hip(moe::launch_fill(const_cast<void*>(p), bytes, 0xFFFFFFFFu, st));
}

// Everything dispatch_send's kernels write: the row pools and planes, the
// plan tables and the row maps (not the error words or the ticket counter).
int poison_dispatch_send(const moe_group_s* g, hipStream_t st)
{
    const moe::Plan& p = g->plan;
    const size_t N = g->desc.num_ranks, E = g->desc.num_experts;
    const size_t R = (size_t)g->rows_max, RQ = (size_t)g->recv_rows_max;
    const size_t row = (size_t)std::max(g->payload_bytes, g->comb_bytes);
    const size_t sb = (size_t)g->scale_blocks * 4;
    int rc;
    if ((rc = poison(st, g->pool_send, R * row)) || (rc = poison(st, g->pool_recv, RQ * row)) ||
        (rc = poison(st, g->send_scale, R * sb)) || (rc = poison(st, g->recv_scale, RQ * sb)) ||
        (rc = poison(st, g->send_meta, R * 4)) || (rc = poison(st, g->recv_meta, RQ * 4)) ||
        (rc = poison(st, g->send_w, R * 4)) || (rc = poison(st, g->recv_w, RQ * 4)) ||
        (rc = poison(st, p.cnt, N * E * 4)) || (rc = poison(st, p.pos, R * 4)) ||
        (rc = poison(st, p.soff, N * (E + 1) * 4)) || (rc = poison(st, p.soff_col, N * (E + 1) * 4)) || (rc = poison(st, p.roff, N * (N + 1) * 4)) ||
        (rc = poison(st, p.rbase, (N + 1) * 4)) || (rc = poison(st, p.eoff, (E + 1) * 4)) ||
        (rc = poison(st, p.sbase, N * (E + 2 * N + 2) * 4)) || (rc = poison(st, p.xfer_src, R * 4)) ||
        (rc = poison(st, p.xfer_dst, R * 8)) || (rc = poison(st, p.shuf_map, R * 8)) ||
        (rc = poison(st, p.shuf_inv, R * 4)) || (rc = poison(st, p.slot_of, R * 4)) ||
        (rc = poison(st, p.send_slot, R * 4)) || (rc = poison(st, p.send_item, R * 4)) ||
        (rc = poison(st, p.pdst, R * 4)) || (rc = poison(st, p.ppos, R * 4)) ||
        (rc = poison(st, p.psoff, N * (N + 1) * 4)) || (rc = poison(st, p.psoff_col, N * (N + 1) * 4)) ||
        (rc = poison(st, p.qoff, N * (N + 1) * 4)) ||
        (rc = poison(st, p.qbase, (N + 1) * 4)) || (rc = poison(st, p.pbase, (N + 1) * 4)) ||
        (rc = poison(st, p.pmap, R * 4)) || (rc = poison(st, p.phead, 2 * R * 16)) ||
        (rc = poison(st, p.pitem, R * 8)))
        return rc;
    return MOE_OK;
}

int check_device(const moe_group_s* g)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_ERR_HIP;
    return dev == g->device ? MOE_OK : MOE_ERR_INVALID;
}

// The static scratch area of groups made by moe_group_create_static: one per
// device (each GPU the library runs on holds its own copy from the library's
// first use on it until the process ends).  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is used.
__device__ __align__(256) static uint8_t scratch[MOE_SCRATCH_BYTES];

constexpr int MAX_SCRATCH_DEVICES = 64;

struct ScratchSlot {
    bool resolved = false;
    bool in_use = false;           // a live group holds the area
    uint8_t* ptr = nullptr;        // device address of this device's scratch
    moe_group_s group;             // the handle moe_group_create_static returns
};

ScratchSlot g_scratch[MAX_SCRATCH_DEVICES];

// The device address of the current device `dev`'s scratch area, looked up on
// first use.
int scratch_address(int dev)
{
    ScratchSlot& slot = g_scratch[dev];
    if (slot.resolved)
        return MOE_OK;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    slot.ptr = static_cast<uint8_t*>(ptr);
    slot.resolved = true;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_strerror(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_OOM: return "out of device memory";
    case MOE_ERR_STATE: return "call out of the dispatch/combine order";
    case MOE_ERR_ROUTING: return "expert id outside [0, num_experts)";
    case MOE_ERR_CAPACITY: return "receive count above the group's bound";
    case MOE_ERR_INTERNAL: return "device-side index check failed";
    case MOE_ERR_SCRATCH: return "group larger than the static scratch area (MOE_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

const char* moe_kernel_name(int kernel_id)
{
    if (kernel_id < 0 || kernel_id >= MOE_KERNEL_COUNT)
        return "";
    return kKernelNames[kernel_id];
}

int moe_group_create(const moe_group_desc* desc, moe_group_t* out)
{
    if (!out)
        return MOE_ERR_INVALID;
    int rc = validate_desc(desc);
    if (rc != MOE_OK)
        return rc;
    moe_group_s* g = new (std::nothrow) moe_group_s();
    if (!g)
        return MOE_ERR_OOM;
    g->desc = *desc;
    if (hipGetDevice(&g->device) != hipSuccess) {
        delete g;
        return MOE_ERR_HIP;
    }
    init_sizes(g);
    g->debug = debug_from_env();
    Placer take{g};
    if ((rc = place_buffers(g, take)) || (rc = zero_words(g))) {
        free_all(g);
        delete g;
        return rc;
    }
    *out = g;
    return MOE_OK;
}

int moe_group_create_static(const moe_group_desc* desc, moe_group_t* out)
{
    if (!out)
        return MOE_ERR_INVALID;
    int rc = validate_desc(desc);
    if (rc != MOE_OK)
        return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOE_ERR_HIP;
    if (dev < 0 || dev >= MAX_SCRATCH_DEVICES)
        return MOE_ERR_INVALID;
    ScratchSlot& slot = g_scratch[dev];
    if (slot.in_use)
        return MOE_ERR_STATE;
    if ((rc = scratch_address(dev)) != MOE_OK)
        return rc;
    moe_group_s* g = &slot.group;
    *g = moe_group_s{};
    g->desc = *desc;
    g->device = dev;
    g->in_scratch = true;
    init_sizes(g);
    g->debug = debug_from_env();
    Placer count{g, true, 0, 0};
    if ((rc = place_buffers(g, count)) != MOE_OK)
        return rc;
    if (count.used > MOE_SCRATCH_BYTES) {
        *g = moe_group_s{};
        return MOE_ERR_SCRATCH;
    }
    Placer carve{g, true, reinterpret_cast<uintptr_t>(slot.ptr), 0};
    if ((rc = place_buffers(g, carve)) || (rc = zero_words(g))) {
        *g = moe_group_s{};
        return rc;
    }
    slot.in_use = true;
    *out = g;
    return MOE_OK;
}

int moe_group_destroy(moe_group_t g)
{
    if (!g)
        return MOE_OK;
    int rc = MOE_OK;
    if (hipDeviceSynchronize() != hipSuccess)
        rc = MOE_ERR_HIP;
    free_all(g);
    if (g->in_scratch) {
        // the buffers stay in the device's scratch area; the slot is free again
        g_scratch[g->device].in_use = false;
        return rc;
    }
    delete g;
    return rc;
}

int moe_dispatch_send(moe_group_t g, int32_t num_tokens, const void* x, const int32_t* topk_idx,
                      const float* topk_weights, hipStream_t stream)
{
    CallRange range("moe_dispatch_send");
    if (!g)
        return MOE_ERR_INVALID;
    if (g->state != State::Idle)
        return MOE_ERR_STATE;
    if (num_tokens < 0 || num_tokens > g->desc.max_tokens)
        return MOE_ERR_INVALID;
    if (num_tokens > 0 && (!x || !topk_idx || !aligned16(x) || !aligned16(topk_idx)))
        return MOE_ERR_INVALID;
    const bool partial = g->desc.combine_mode == MOE_COMBINE_PARTIAL;
    if (partial && num_tokens > 0 && (!topk_weights || !aligned16(topk_weights)))
        return MOE_ERR_INVALID;
    int rc = check_device(g);
    if (rc != MOE_OK)
        return rc;
    const moe::Shape sh = shape_of(g, num_tokens);
    const moe::Rows rows = rows_of(g);
    const bool any = sh.rows > 0;
    using moe::Launch;
    if (g->debug && (rc = poison_dispatch_send(g, stream)))
        return rc;
    // this cycle's error word, and the next cycle's, which the route plan clears
    g->plan.err = g->err_words + (g->cycle & 1);
    g->plan.err_next = g->err_words + ((g->cycle + 1) & 1);
    if ((rc = timed_launch(g, MOE_KERNEL_ROUTE_PLAN, stream, true, [&](const Launch& L) {
             return moe::launch_route_plan(sh, topk_idx, g->plan, rows, L);
         })) ||
        (rc = timed_launch(g, MOE_KERNEL_PACK, stream, any, [&](const Launch& L) {
             return moe::launch_pack(sh, x, topk_idx, partial ? topk_weights : nullptr, g->plan,
                                     rows, L);
         })) ||
        (!sh.direct && (rc = timed_launch(g, MOE_KERNEL_TRANSFER, stream, any, [&](const Launch& L) {
             return moe::launch_transfer(sh, g->plan, rows, L);
         }))))
        return rc;
    g->cycle++;
    g->T = num_tokens;
    g->state = State::Sent;
    return MOE_OK;
}

int moe_dispatch_recv(moe_group_t g, void* expert_x, float* expert_scale, int32_t* expert_offsets,
                      hipStream_t stream)
{
    CallRange range("moe_dispatch_recv");
    if (!g)
        return MOE_ERR_INVALID;
    if (g->state != State::Sent)
        return MOE_ERR_STATE;
    const bool fp8 = g->desc.dispatch_dtype == MOE_FP8_E4M3;
    const bool any_rows = g->T > 0;
    if (!expert_offsets || !aligned16(expert_offsets))
        return MOE_ERR_INVALID;
    if (any_rows && (!expert_x || !aligned16(expert_x)))
        return MOE_ERR_INVALID;
    if (fp8 && any_rows && (!expert_scale || !aligned16(expert_scale)))
        return MOE_ERR_INVALID;
    if (!fp8 && expert_scale)
        return MOE_ERR_INVALID;
    int rc = check_device(g);
    if (rc != MOE_OK)
        return rc;
    const moe::Shape sh = shape_of(g, g->T);
    const moe::Rows rows = rows_of(g);
    // debug: the expert-order metadata and the caller's outputs, all of which
    // the shuffle must write
    if (g->debug &&
        ((rc = poison(stream, g->src_rank, (size_t)g->rows_max * 4)) ||
         (rc = poison(stream, g->src_slot, (size_t)g->rows_max * 4)) ||
         (rc = poison(stream, expert_x, (size_t)sh.rows * g->payload_bytes)) ||
         (rc = poison(stream, expert_scale, (size_t)sh.rows * g->scale_blocks * 4)) ||
         (rc = poison(stream, expert_offsets, (size_t)(sh.E + 1) * 4))))
        return rc;
    // the receiver's side of the plan: the group offsets and row maps from
    // the exchanged counts (also for an empty cycle, whose offsets are all
    // zero), then the shuffle
    if ((rc = timed_launch(g, MOE_KERNEL_RECV_MAP, stream, true, [&](const moe::Launch& L) {
             return moe::launch_recv_map(sh, g->plan, L);
         })) ||
        (rc = timed_launch(g, MOE_KERNEL_SHUFFLE, stream, true, [&](const moe::Launch& L) {
             return moe::launch_shuffle(sh, g->plan, rows, expert_x, expert_scale, expert_offsets,
                                        L);
         })))
        return rc;
    g->state = State::Received;
    return MOE_OK;
}

int moe_combine_send(moe_group_t g, const void* expert_y, hipStream_t stream)
{
    CallRange range("moe_combine_send");
    if (!g)
        return MOE_ERR_INVALID;
    if (g->state != State::Received)
        return MOE_ERR_STATE;
    if (g->T > 0 && (!expert_y || !aligned16(expert_y)))
        return MOE_ERR_INVALID;
    int rc = check_device(g);
    if (rc != MOE_OK)
        return rc;
    const moe::Shape sh = shape_of(g, g->T);
    const moe::Rows rows = rows_of(g);
    const bool any = sh.rows > 0;
    // debug: both row pools (their dispatch rows are consumed; combine's
    // kernels rewrite every row they later read)
    if (g->debug &&
        ((rc = poison(stream, g->pool_send,
                      (size_t)g->rows_max * std::max(g->payload_bytes, g->comb_bytes))) ||
         (rc = poison(stream, g->pool_recv,
                      (size_t)g->recv_rows_max * std::max(g->payload_bytes, g->comb_bytes)))))
        return rc;
    if (sh.partial) {
        if ((rc = timed_launch(g, MOE_KERNEL_PARTIAL_SEND, stream, any, [&](const moe::Launch& L) {
                 return moe::launch_partial_send(sh, g->plan, rows, expert_y, L);
             })) ||
            (!sh.direct &&
             (rc = timed_launch(g, MOE_KERNEL_PARTIAL_TRANSFER, stream, any, [&](const moe::Launch& L) {
                  return moe::launch_partial_transfer(sh, g->plan, rows, L);
              }))))
            return rc;
    } else if (sh.direct) {
        if ((rc = timed_launch(g, MOE_KERNEL_COMBINE_PUSH, stream, any, [&](const moe::Launch& L) {
                 return moe::launch_combine_push(sh, g->plan, rows, expert_y, L);
             })))
            return rc;
    } else if ((rc = timed_launch(g, MOE_KERNEL_COMBINE_PACK, stream, any, [&](const moe::Launch& L) {
                    return moe::launch_combine_pack(sh, g->plan, rows, expert_y, L);
                })) ||
               (rc = timed_launch(g, MOE_KERNEL_TRANSFER_BACK, stream, any, [&](const moe::Launch& L) {
                    return moe::launch_transfer_back(sh, g->plan, rows, L);
                }))) {
        return rc;
    }
    g->state = State::CombineSent;
    return MOE_OK;
}

int moe_combine_recv(moe_group_t g, const float* topk_weights, void* out, hipStream_t stream)
{
    CallRange range("moe_combine_recv");
    if (!g)
        return MOE_ERR_INVALID;
    if (g->state != State::CombineSent)
        return MOE_ERR_STATE;
    // with the partial combine the weights were applied on the expert side
    const bool partial = g->desc.combine_mode == MOE_COMBINE_PARTIAL;
    if (g->T > 0 && (!out || !aligned16(out)))
        return MOE_ERR_INVALID;
    if (!partial && g->T > 0 && (!topk_weights || !aligned16(topk_weights)))
        return MOE_ERR_INVALID;
    int rc = check_device(g);
    if (rc != MOE_OK)
        return rc;
    const moe::Shape sh = shape_of(g, g->T);
    const moe::Rows rows = rows_of(g);
    if (g->debug && (rc = poison(stream, out, (size_t)sh.N * sh.T * sh.H * 2)))
        return rc;
    if (partial) {
        if ((rc = timed_launch(g, MOE_KERNEL_PARTIAL_REDUCE, stream, sh.rows > 0,
                               [&](const moe::Launch& L) {
                                   return moe::launch_partial_reduce(sh, g->plan, rows, out, L);
                               })))
            return rc;
    } else if ((rc = timed_launch(g, MOE_KERNEL_COMBINE_REDUCE, stream, sh.rows > 0,
                                  [&](const moe::Launch& L) {
                                      return moe::launch_combine_reduce(sh, g->plan, rows,
                                                                        topk_weights, out, L);
                                  }))) {
        return rc;
    }
    g->state = State::Idle;
    return MOE_OK;
}

int moe_group_view_get(moe_group_t g, moe_group_view* v)
{
    if (!g || !v)
        return MOE_ERR_INVALID;
    std::memset(v, 0, sizeof(*v));
    v->desc = g->desc;
    v->num_tokens = g->T;
    v->rows = (int64_t)g->desc.num_ranks * g->T * g->desc.top_k;
    v->payload_row_bytes = g->payload_bytes;
    v->combine_row_bytes = g->comb_bytes;
    v->scale_blocks = g->scale_blocks;
    v->cnt = g->plan.cnt;
    v->pos = g->plan.pos;
    v->send_off = g->plan.soff;
    v->recv_off = g->plan.roff;
    v->recv_base = g->plan.rbase;
    v->expert_off = g->plan.eoff;
    v->send_x = g->pool_send;
    v->send_scale = g->send_scale;
    v->send_meta = g->send_meta;
    v->recv_x = g->pool_recv;
    v->recv_scale = g->recv_scale;
    v->recv_meta = g->recv_meta;
    v->expert_src_rank = g->src_rank;
    v->expert_src_slot = g->src_slot;
    const moe::Rows r = rows_of(g);
    v->comb_send = r.comb_send;
    v->comb_recv = r.comb_recv;
    v->recv_rows = g->recv_rows_max;
    v->send_w = g->send_w;
    v->recv_w = g->recv_w;
    v->part_dst = g->plan.pdst;
    v->part_pos = g->plan.ppos;
    v->part_send_off = g->plan.psoff;
    v->part_base = g->plan.pbase;
    v->part_owner_base = g->plan.qbase;
    return MOE_OK;
}

int moe_group_status(moe_group_t g, hipStream_t stream)
{
    if (!g)
        return MOE_ERR_INVALID;
    int rc = check_device(g);
    if (rc != MOE_OK)
        return rc;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return MOE_ERR_HIP;
    // the sticky word holds the bits of every cycle since the last status
    // call; the cycle word is left alone (the next route plan overwrites it)
    int32_t word = 0;
    if (hipMemcpy(&word, g->plan.err_sticky, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_ERR_HIP;
    if (word != 0 && hipMemset(g->plan.err_sticky, 0, sizeof(int32_t)) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipDeviceSynchronize() != hipSuccess)
        return MOE_ERR_HIP;
    if (word & moe::ERR_BIT_ROUTING)
        return MOE_ERR_ROUTING;
    if (word & moe::ERR_BIT_CAPACITY)
        return MOE_ERR_CAPACITY;
    if (word & moe::ERR_BIT_INTERNAL)
        return MOE_ERR_INTERNAL;
    return MOE_OK;
}

int moe_hbm_probe(int kind, void* dst, const void* src, size_t bytes, hipStream_t stream)
{
    if (kind < MOE_PROBE_COPY || kind > MOE_PROBE_WRITE || bytes == 0 || bytes % 16 != 0)
        return MOE_ERR_INVALID;
    if (bytes / 16 >= ((size_t)1 << 40))
        return MOE_ERR_INVALID;
    const bool reads = kind != MOE_PROBE_WRITE;
    if (!dst || !aligned16(dst) || (reads && (!src || !aligned16(src))))
        return MOE_ERR_INVALID;
    return from_hip(moe::launch_hbm_probe(kind, dst, src, (int64_t)(bytes / 16), stream));
}

int moe_group_timing_enable(moe_group_t g, int kernel_mask)
{
    if (!g || (kernel_mask & ~MOE_KERNEL_ALL) != 0)
        return MOE_ERR_INVALID;
    g->timing_mask = kernel_mask;
    g->events_used = 0;
    return MOE_OK;
}

int moe_group_timing_read(moe_group_t g, double* total_ms, int64_t* launches)
{
    if (!g || !total_ms || !launches)
        return MOE_ERR_INVALID;
    for (int k = 0; k < MOE_KERNEL_COUNT; ++k) {
        total_ms[k] = 0.0;
        launches[k] = 0;
    }
    for (size_t i = 0; i < g->events_used; ++i) {
        const EventPair& e = g->events[i];
        if (hipEventSynchronize(e.stop) != hipSuccess)
            return MOE_ERR_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess)
            return MOE_ERR_HIP;
        total_ms[e.kernel] += ms;
        launches[e.kernel] += 1;
    }
    g->events_used = 0;
    return MOE_OK;
}

}  // extern "C"
