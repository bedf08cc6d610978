// HIP kernels of the MoE dispatch/combine path for CDNA4 (gfx950, wave64).
//
// Pages cited:
//   [EPMC] "Efficient and portable Mixture-of-Experts communication"
//   [EFA]  "Enabling trillion-parameter models on AWS EFA"
//
// Every step is a permutation copy, a small scan, a codec or a weighted sum:
// nothing is a dense contraction, so there is no MFMA here and the kernels are
// bound by HBM bandwidth.  Rows move as 16-byte vectors; a row is shared by
// up to eight waves with about 2 vectors per lane (a 14 KiB DeepSeek-shaped
// row: eight waves of 1.75 KiB), and every lane issues all its loads before
// its first store.  Row order is driven by small int32 maps that the pack kernel writes
// from the offsets, so the transfer, shuffle and combine kernels are pure
// gathers in destination order.
//
// Every kernel after the route plan checks the cycle's error word first and
// writes nothing once an invalid expert id (or a capacity overflow) has been
// seen in that cycle; the next cycle's route plan overwrites the word, and a
// sticky copy keeps every cycle's bits for the status call.
#include "moe_kernels.h"

#include <hip/hip_ext.h>

namespace moe {
namespace {

// Native clang vectors (not HIP's struct wrappers) so that a value can be an
// inline-asm register operand.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int ROWS_PER_BLOCK = 4;          // waves per 256-thread block
constexpr int COPY_THREADS = WAVE * ROWS_PER_BLOCK;

__device__ inline int lane_id() { return threadIdx.x & (WAVE - 1); }

// Every launch goes through here: with events set, they are attached to the
// dispatch packet (hipExtLaunchKernelGGL) and time exactly this kernel.
template <typename F, typename... Args>
inline void go(F kernel, dim3 grid, dim3 block, size_t lds, const Launch& L, Args... args)
{
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, L.stream, L.start, L.stop, 0u,
                          args...);
}

// Pins loaded values in registers: an empty asm that reads and rewrites each
// vector.  Without it the compiler sinks every load into the predicated store
// that uses it, and the row is copied one vector at a time with a full memory
// wait in between; with it, all U loads of a lane are in flight together.
template <int U>
__device__ inline void hold(v4u (&v)[U])
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        asm volatile("" : "+v"(v[u]));
}

// Streaming access: every row is read once and written once per stage, so row
// loads and stores carry the nontemporal hint and do not displace the small
// tables (maps, offsets) from the caches.
__device__ inline v4u ld_nt(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ inline void st_nt(const v4u& v, v4u* p) { __builtin_nontemporal_store(v, p); }

__device__ inline int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ inline float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// A failed device-side check after the route plan: the cycle's word stops
// the kernels that follow, the sticky word keeps it for moe_group_status.
__device__ inline void raise_err(const Plan& p, int32_t bit)
{
    atomicOr(p.err, bit);
    atomicOr(p.err_sticky, bit);
}

// Exclusive scan of one int per thread over a block of NT threads.  Returns
// the thread's exclusive prefix; *total gets the block sum.  Contains
// barriers: every thread of the block must call it.
template <int NT>
__device__ int block_exclusive_scan(int v, int* wave_sums, int* total)
{
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    int inc = v;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const int t = __shfl_up(inc, d, WAVE);
        if (lane >= d)
            inc += t;
    }
    if (lane == WAVE - 1)
        wave_sums[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < NT / WAVE; ++w) {
            const int c = wave_sums[w];
            wave_sums[w] = run;
            run += c;
        }
        wave_sums[NT / WAVE] = run;
    }
    __syncthreads();
    const int excl = wave_sums[wave] + inc - v;
    *total = wave_sums[NT / WAVE];
    __syncthreads();
    return excl;
}

// ---------------------------------------------------------------------------
// Route plan: one workgroup per logical rank; the last workgroup to finish
// also computes the offsets of the whole group.
//
// Counts ([EFA] "Dispatch and combine": the token counts per expert are formed
// by atomic adds in shared memory of a single block, then summed cumulatively
// to get the offsets inside the contiguous send buffer).  LDS atomics give the
// counts; the order inside an expert is made stable ((t,k) ascending) with a
// per-chunk counting sort: each lane sets its bit in a 64-bit lane mask per
// (wave, key) in LDS, and its position is a running per-key cursor plus the
// set bits of lower waves' masks and of its own wave's mask below its lane.
// With the partial combine every item carries a second key (its destination
// rank, when it is the first item of its token there), ranked in the same
// pass.  With the fixed-slot layout a (sender, expert) count above the slot
// count raises the capacity bit.
//
// Offsets ([EFA] "Send and receive buffers": once the per-expert counts are
// exchanged, each rank derives where to write and the offsets it receives
// from; [EFA] "Dispatch and combine": they are computed once for dispatch and
// combine, off the critical path).  Each workgroup publishes its counts, then
// draws a ticket from a device-wide counter (agent-scope release fence before,
// acquire fence after); the one that draws the last ticket has every rank's
// counts in view and computes the receive offsets per (receiver, sender), the
// pooled receive bases, the expert offsets and the first expert-order row of
// every (sender, expert) run, then resets the counter for the next launch.
// A receive count above N*T*max(K, L) (the page's bound) raises the capacity
// bit.  The loops over ranks run on one workgroup, so they issue BATCH
// independent loads before the first use instead of one latency per rank.
// ---------------------------------------------------------------------------
constexpr int RP_NT = 512;
constexpr int RP_WAVES = RP_NT / WAVE;
constexpr int BATCH = 32;
constexpr int HELD_CHUNKS = 32;     // most idx chunks kept in registers between the two passes

struct RouteArgs {
    const int32_t* idx;
    int N, T, K, E, L;
    int chunk_waves;        // RP_WAVES, or fewer for large E (LDS budget)
    int partial;            // also plan the expert-side partial rows
    int slot_cap;           // fixed-slot layout: most rows per (sender, expert); -1: none
    int table_lds;          // the tail forms the group offsets from a copy of soff in LDS
    int32_t* send_meta;     // when set: each send row's item t*K+k, written with the positions
                            // (the send meta words, or the direct transport's send_item)
    int64_t cap;
};

// One column of an [N][stride] offset table, walked down the senders with
// BATCH loads in flight: .x = sum_s lo[s], and run_out[s] (when given) =
// sum_{s'<s} (hi - lo)[s'], run_out[N] = .y = the column's total span;
// hi_run_out[s] (when given) = sum_{s'<s} hi[s'], hi_run_out[N] = sum of hi.
__device__ int2 walk_column(const int32_t* __restrict__ lo, const int32_t* __restrict__ hi,
                            size_t stride, int N, int32_t* __restrict__ run_out,
                            int32_t* __restrict__ hi_run_out)
{
    int base = 0, run = 0, hrun = 0;
    for (int s0 = 0; s0 < N; s0 += BATCH) {
        int a[BATCH], b[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const size_t row = (size_t)min(s0 + j, N - 1) * stride;
            a[j] = lo[row];
            b[j] = hi[row];
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
            if (s0 + j < N) {
                if (run_out)
                    run_out[s0 + j] = run;
                if (hi_run_out)
                    hi_run_out[s0 + j] = hrun;
                run += b[j] - a[j];
                hrun += b[j];
                base += a[j];
            }
    }
    if (run_out)
        run_out[N] = run;
    if (hi_run_out)
        hi_run_out[N] = hrun;
    return make_int2(base, run);
}

// Every group-wide table is a pass down one column of the send-offset matrix
// soff[s][*] over the senders s, because soff[s][e] already sums sender s's
// counts of the experts before e:
//   eoff[e]      = sum_s soff[s][e]                 (rows of all experts < e)
//   sbase[s][e]  = eoff[e] + sum_{s'<s} cnt[s'][e]   (partial combine only)
//   rbase[d]     = sum_s soff[s][d*L]               (rows received by ranks < d)
//   roff[d][s]   = sum_{s'<s} (soff[s'][(d+1)L] - soff[s'][dL])
// and the partial-row tables are the same walks over psoff[s][*] (one bucket
// per rank instead of per expert):
//   qbase[d]     = sum_s psoff[s][d]                (partial rows of ranks < d)
//   qoff[d][s]   = sum_{s'<s} (psoff[s'][d+1] - psoff[s'][d])
//   pbase[s]     = sum_{s'<s} psoff[s'][N]          (partial rows of senders < s)
// so one thread takes one column (E expert columns, N receiver columns, then
// N partial columns) and walks the senders; no scan across threads.  The
// total rows eoff[E] = rbase[N] are the walk of soff[*][E] (or, when the
// second walk runs, the last expert column's running sum), and the last
// partial column's upper bounds psoff[s][N] are the per-sender totals whose
// running sum is pbase.
// Column `col` of every sender's base row (partial combine): sbase[s][col] =
// base + off[d][s], the first row from sender s on rank d (off, written by
// this thread's walk, is read back).
__device__ inline void sender_rows(const Plan& p, int d, int N, int SB, int col, int base,
                                   const int32_t* off)
{
    for (int s = 0; s < N; ++s)
        p.sbase[(size_t)s * SB + col] = base + off[(size_t)d * (N + 1) + s];
}

__device__ void group_offsets(const RouteArgs& ra, const Plan& p, int32_t* wg_err)
{
    const int N = ra.N, E = ra.E, L = ra.L;
    const int32_t* __restrict__ soff = p.soff;
    const int32_t* __restrict__ cnt = p.cnt;
    const int cols = E + N + (ra.partial ? N : 0);
    const int SB = E + 2 * N + 2;
    for (int col = threadIdx.x; col < cols; col += RP_NT) {
        if (col < E && !ra.partial) {
            // expert column e: its offset alone (the receiver's map kernel
            // forms each sender's first expert row itself)
            const int e = col;
            const int2 br = walk_column(soff + e, soff + e, E + 1, N, nullptr, nullptr);
            p.eoff[e] = br.x;
            if (e == E - 1) {
                // every row of the cycle: the senders' totals, soff[s][E]
                const int tot = walk_column(soff + E, soff + E, E + 1, N, nullptr, nullptr).x;
                p.eoff[E] = tot;
                p.rbase[N] = tot;
            }
        } else if (col < E) {
            // expert column e with the partial combine: its counts are loaded
            // with its offsets and, for N <= BATCH, kept in registers for the
            // second walk, which forms each sender's first expert row (the
            // pack's partial-row records name expert rows)
            const int e = col;
            int base = 0;
            int c[BATCH];
            for (int s0 = 0; s0 < N; s0 += BATCH) {
                int o[BATCH];
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const int sb = min(s0 + b, N - 1);
                    o[b] = soff[(size_t)sb * (E + 1) + e];
                    c[b] = cnt[(size_t)sb * E + e];
                }
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    if (s0 + b < N)
                        base += o[b];
            }
            p.eoff[e] = base;
            int run = base;
            for (int s0 = 0; s0 < N; s0 += BATCH) {
                if (N > BATCH) {
#pragma unroll
                    for (int b = 0; b < BATCH; ++b)
                        c[b] = cnt[(size_t)min(s0 + b, N - 1) * E + e];
                }
#pragma unroll
                for (int b = 0; b < BATCH; ++b)
                    if (s0 + b < N) {
                        p.sbase[(size_t)(s0 + b) * SB + e] = run;
                        run += c[b];
                    }
            }
            if (e == E - 1) {
                p.eoff[E] = run;
                p.rbase[N] = run;
            }
        } else if (col < E + N) {
            const int d = col - E;
            const int2 br = walk_column(soff + d * L, soff + (d + 1) * L, E + 1, N,
                                        p.roff + (size_t)d * (N + 1), nullptr);
            p.rbase[d] = br.x;
            if ((int64_t)br.y > ra.cap)
                atomicOr(wg_err, ERR_BIT_CAPACITY);
            if (ra.partial)
                sender_rows(p, d, N, SB, E + d, br.x, p.roff);
        } else {
            const int d = col - E - N;
            const bool last = d == N - 1;
            const int2 br = walk_column(p.psoff + d, p.psoff + d + 1, N + 1, N,
                                        p.qoff + (size_t)d * (N + 1), last ? p.pbase : nullptr);
            p.qbase[d] = br.x;
            sender_rows(p, d, N, SB, E + N + d, br.x, p.qoff);
            if (last) {
                p.qbase[N] = br.x + br.y;
                for (int s = 0; s < N; ++s) {
                    p.sbase[(size_t)s * SB + E + 2 * N] = p.pbase[s];
                    p.sbase[(size_t)s * SB + E + 2 * N + 1] = br.x + br.y;
                }
            }
        }
    }
}

// The same tables from a copy of soff[N][E+1] (with the partial combine also
// cnt[N][E] and psoff[N][N+1]) in LDS, for small tables: each copy is one
// round of 16-byte loads (up to TAB_VECS per thread), and the column walks
// then read LDS only, where each walk above issues its BATCH loads per column
// (64 for a receiver column, past the 63 a wave can have in flight).
// Mixtral decode (72 ints): the last workgroup's part 4.1 -> 2.0 us;
// DeepSeek-R1 decode (8224 ints) measured 3.8 us either way, the copy's round
// trip taking what the walks saved.
constexpr int TAB_VECS = 2;
constexpr int TAB_MAX_INTS = TAB_VECS * 4 * RP_NT;    // 16 KiB

// One round of 16-byte loads copying n ints (a 16-byte aligned table) into
// LDS at dst (16-byte aligned); n <= TAB_MAX_INTS.
__device__ inline void copy_table(const int32_t* __restrict__ src, int n, int32_t* dst)
{
    const int tid = threadIdx.x, nv = n / 4;
    const int4* __restrict__ src4 = reinterpret_cast<const int4*>(src);
    if (nv > 0) {
        int4 v[TAB_VECS];
#pragma unroll
        for (int j = 0; j < TAB_VECS; ++j)
            v[j] = src4[min(tid + j * RP_NT, nv - 1)];
#pragma unroll
        for (int j = 0; j < TAB_VECS; ++j)
            if (tid + j * RP_NT < nv)
                reinterpret_cast<int4*>(dst)[tid + j * RP_NT] = v[j];
    }
    for (int i = nv * 4 + tid; i < n; i += RP_NT)
        dst[i] = src[i];
}

__host__ __device__ inline int round4(int n)
{
    return (n + 3) & ~3;
}

__device__ void group_offsets_lds(const RouteArgs& ra, const Plan& p, int32_t* wg_err,
                                  int32_t* tab)
{
    const int N = ra.N, E = ra.E, L = ra.L, W = E + 1, SB = E + 2 * N + 2;
    const int tid = threadIdx.x;
    // the send offsets; with the partial combine also the counts and the
    // partial rows' send offsets
    int32_t* tab_cnt = tab + round4(N * W);
    int32_t* tab_ps = tab_cnt + round4(N * E);
    copy_table(p.soff, N * W, tab);
    if (ra.partial) {
        copy_table(p.cnt, N * E, tab_cnt);
        copy_table(p.psoff, N * (N + 1), tab_ps);
    }
    __syncthreads();
    // expert columns and the totals column soff[*][E], a thread each, with 8
    // LDS reads in flight; with the partial combine each expert column also
    // runs down its counts for each sender's first expert row (sbase), and
    // the totals are the last column's running sum
    for (int col = tid; col <= E - (ra.partial ? 1 : 0); col += RP_NT) {
        int sum = 0, s = 0;
        for (; s + 8 <= N; s += 8) {
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = tab[(s + j) * W + col];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sum += v[j];
        }
        for (; s < N; ++s)
            sum += tab[s * W + col];
        p.eoff[col] = sum;
        if (col == E)
            p.rbase[N] = sum;
        if (ra.partial) {
            int run = sum;
            for (int s2 = 0; s2 < N; ++s2) {
                p.sbase[(size_t)s2 * SB + col] = run;
                run += tab_cnt[s2 * E + col];
            }
            if (col == E - 1) {
                p.eoff[E] = run;
                p.rbase[N] = run;
            }
        }
    }
    // the partial rows' columns, a thread each: qoff and qbase down the rank
    // columns of psoff, and down the last one also pbase (the senders' totals)
    if (ra.partial) {
        for (int d = (tid + RP_NT - E % RP_NT) % RP_NT; d < N; d += RP_NT) {
            int32_t* qo = p.qoff + (size_t)d * (N + 1);
            const bool last = d == N - 1;
            int base = 0, run = 0, hrun = 0;
            for (int s2 = 0; s2 < N; ++s2) {
                const int lo = tab_ps[s2 * (N + 1) + d], hi = tab_ps[s2 * (N + 1) + d + 1];
                qo[s2] = run;
                if (last)
                    p.pbase[s2] = hrun;
                run += hi - lo;
                hrun += hi;
                base += lo;
            }
            qo[N] = run;
            if (last)
                p.pbase[N] = hrun;
            p.qbase[d] = base;
            sender_rows(p, d, N, SB, E + N + d, base, p.qoff);
            if (last) {
                p.qbase[N] = base + run;
                for (int s2 = 0; s2 < N; ++s2) {
                    p.sbase[(size_t)s2 * SB + E + 2 * N] = p.pbase[s2];
                    p.sbase[(size_t)s2 * SB + E + 2 * N + 1] = base + run;
                }
            }
        }
    }
    // receiver columns, a thread each, numbered from the top of the block so
    // that their waves are not the expert columns' when both fit
    for (int d = RP_NT - 1 - tid; d < N; d += RP_NT) {
        int32_t* ro = p.roff + (size_t)d * (N + 1);
        const int32_t* lo_col = tab + d * L;
        const int32_t* hi_col = tab + (d + 1) * L;
        int run = 0, base = 0, s = 0;
        for (; s + 8 <= N; s += 8) {
            int lo[8], hi[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lo[j] = lo_col[(s + j) * W];
                hi[j] = hi_col[(s + j) * W];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ro[s + j] = run;
                run += hi[j] - lo[j];
                base += lo[j];
            }
        }
        for (; s < N; ++s) {
            const int lo = lo_col[s * W], hi = hi_col[s * W];
            ro[s] = run;
            run += hi - lo;
            base += lo;
        }
        ro[N] = run;
        p.rbase[d] = base;
        if ((int64_t)run > ra.cap)
            atomicOr(wg_err, ERR_BIT_CAPACITY);
        if (ra.partial)
            sender_rows(p, d, N, SB, E + d, base, p.roff);
    }
}

// The end of the plan, once every sender's counts are in view: the group
// offsets, then their checks' bits ORed into the cycle's word (every
// workgroup has already ORed its sender's bits there) and the sticky word.
// Every thread of the workgroup calls it; wg_err (LDS) holds the workgroup's
// bits; tab, when given, is LDS room for the soff table.
__device__ void close_plan(const RouteArgs& ra, const Plan& p, int32_t* wg_err, int32_t* tab)
{
    if (tab)
        group_offsets_lds(ra, p, wg_err, tab);
    else
        group_offsets(ra, p, wg_err);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int32_t bits = *wg_err;
        if (bits) {
            atomicOr(p.err, bits);
            atomicOr(p.err_sticky, bits);
        }
    }
}

// The counts of one rank's keys sit in cur[0, nkeys): write them out
// (cnt_out may be null), scan them into off_out[0, nkeys] and leave the
// exclusive offsets in cur as the cursors of the ranking pass.  A count above
// cap (when cap >= 0) raises the capacity bit.
__device__ __forceinline__ void publish_counts(int32_t* cur, int nkeys, int32_t* __restrict__ cnt_out,
                                               int32_t* __restrict__ off_out, int* wave_sums,
                                               int cap, int32_t* err,
                                               int32_t* __restrict__ off_col = nullptr,
                                               int col_stride = 0)
{
    const int tid = threadIdx.x;
    const int per = (nkeys + RP_NT - 1) / RP_NT;
    const int k0 = tid * per;
    int local = 0;
    for (int j = 0; j < per; ++j) {
        const int k = k0 + j;
        if (k < nkeys) {
            const int c = cur[k];
            if (cnt_out)
                cnt_out[k] = c;
            if (cap >= 0 && c > cap)
                atomicOr(err, ERR_BIT_CAPACITY);
            local += c;
        }
    }
    int total;
    int run = block_exclusive_scan<RP_NT>(local, wave_sums, &total);
    for (int j = 0; j < per; ++j) {
        const int k = k0 + j;
        if (k < nkeys) {
            const int c = cur[k];
            off_out[k] = run;
            if (off_col)
                off_col[(size_t)k * col_stride] = run;
            cur[k] = run;
            run += c;
        }
    }
    if (tid == 0) {
        off_out[nkeys] = total;
        if (off_col)
            off_col[(size_t)nkeys * col_stride] = total;
    }
    __syncthreads();
}

// Two keys can be packed into one int: the low 16 bits the first, the high 16
// bits the second, NO_KEY for none (keys stay below 2048 here).
constexpr int NO_KEY = 0xFFFF;

__device__ inline int pack_keys(int k1, int k2)
{
    return (k1 < 0 ? NO_KEY : k1) | ((k2 < 0 ? NO_KEY : k2) << 16);
}

// Stable positions, one chunk of CW*64 items at a time (thread tid takes item
// c*CW*64 + tid of chunk c), two barriers per chunk (masks and cursors
// double-buffered by chunk parity).  Each lane sets its bit in
// mask[wave][key] with an LDS 64-bit OR; its rank among equal keys of the
// chunk is then the set bits of lower waves' masks plus the bits of its own
// wave's mask below its lane; the per-key cursor advances by the chunk's
// total into the other buffer.  With TWO, every item carries two keys (packed,
// see pack_keys) from disjoint key ranges, ranked in the same pass.  Keys of
// the first HC chunks come from registers, later ones from
// key_at(i, mine), which every thread calls.  out1[i] (out2[i]) = the item's
// position for its first (second) key, -1 for an item without one; inv1
// (when given) the inverse of out1: inv1[position] = i.
template <bool TWO, int HC, typename KeyAt>
__device__ __forceinline__ void stable_ranks(int items, int nkeys, int CW, uint64_t* mask,
                                             int32_t* cur, const int (&held)[HC],
                                             KeyAt key_at, int32_t* __restrict__ out1,
                                             int32_t* __restrict__ out2,
                                             int32_t* __restrict__ inv1)
{
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int chunk = CW * WAVE;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
    for (int c0 = 0, c = 0; c0 < items; c0 += chunk, ++c) {
        const int A = c & 1;
        uint64_t* mA = mask + (size_t)A * CW * nkeys;
        uint64_t* mB = mask + (size_t)(A ^ 1) * CW * nkeys;
        int32_t* cA = cur + A * nkeys;
        int32_t* cB = cur + (A ^ 1) * nkeys;
        const int i = c0 + tid;
        const bool mine = tid < chunk && i < items;
        int key = TWO ? pack_keys(-1, -1) : -1;
#pragma unroll
        for (int h = 0; h < HC; ++h)
            if (c == h)
                key = held[h];
        if (c >= HC)
            key = key_at(i, mine);
        const int k1 = TWO ? key & 0xFFFF : key;
        const int k2 = TWO ? (key >> 16) & 0xFFFF : NO_KEY;
        const bool v1 = mine && (unsigned)k1 < (unsigned)nkeys;
        const bool v2 = TWO && mine && (unsigned)k2 < (unsigned)nkeys;
        if (v1)
            atomicOr(reinterpret_cast<unsigned long long*>(&mA[(size_t)wave * nkeys + k1]),
                     1ull << lane);
        if (v2)
            atomicOr(reinterpret_cast<unsigned long long*>(&mA[(size_t)wave * nkeys + k2]),
                     1ull << lane);
        for (int j = tid; j < CW * nkeys; j += RP_NT)
            mB[j] = 0ull;
        __syncthreads();
        if (v1) {
            int before = cA[k1] + __popcll(mA[(size_t)wave * nkeys + k1] & lanes_below);
            for (int w = 0; w < wave; ++w)
                before += __popcll(mA[(size_t)w * nkeys + k1]);
            out1[i] = before;
            if (inv1)
                inv1[before] = i;
        } else if (mine) {
            out1[i] = -1;
        }
        if (TWO) {
            if (v2) {
                int before = cA[k2] + __popcll(mA[(size_t)wave * nkeys + k2] & lanes_below);
                for (int w = 0; w < wave; ++w)
                    before += __popcll(mA[(size_t)w * nkeys + k2]);
                out2[i] = before;
            } else if (mine) {
                out2[i] = -1;
            }
        }
        for (int kk = tid; kk < nkeys; kk += RP_NT) {
            int add = 0;
            for (int w = 0; w < CW; ++w)
                add += __popcll(mA[(size_t)w * nkeys + kk]);
            cB[kk] = cA[kk] + add;
        }
        __syncthreads();
    }
}

// Destination rank d = e / L of item i (expert id e; -1 when invalid or not
// this thread's) and whether it is the first item of its token with that
// rank.  A token's K items are consecutive and so are a wave's, so its
// earlier items come from lower lanes by shuffle, or from memory for those
// before the wave.  Every lane of the wave must call it.
__device__ __forceinline__ int rank_of_item(const RouteArgs& ra, const int32_t* __restrict__ my_idx,
                                            int e, int i, bool mine, bool* first)
{
    const int lane = lane_id();
    const int d = (mine && (unsigned)e < (unsigned)ra.E) ? e / ra.L : -1;
    const int k = i % ra.K;
    bool f = d >= 0;
    for (int j = 1; j < ra.K; ++j) {
        int dj = __shfl(d, max(lane - j, 0), WAVE);
        if (mine && j <= k) {
            if (lane < j) {
                const int ej = my_idx[i - j];
                dj = (unsigned)ej < (unsigned)ra.E ? ej / ra.L : -1;
            }
            if (dj == d)
                f = false;
        }
    }
    *first = f;
    return d;
}

// HC: idx chunks held in registers, the fewest of 1, 2, 4, 8, 32 that cover
// a rank's items when possible (a decode batch needs 1 or 2; fewer held
// chunks means fewer loads and shorter unrolled loops).
// Instances: PARTIAL, the partial combine's second key; TAIL, the group
// offsets' tail.  Without the tail the kernel keeps 72 scalar and 36 vector
// registers (94 and 46 with the partial key) and spills none; the tail takes
// it to 106 (149-163 spilled) and 133.
template <int HC, bool PARTIAL, bool TAIL>
__global__ __launch_bounds__(RP_NT) void route_plan_kernel(RouteArgs ra, Plan p)
{
    const bool partial = PARTIAL;
    extern __shared__ __align__(16) uint64_t lds64[];
    const int E = ra.E, N = ra.N;
    // keys: experts [0, E) and, for the partial combine, destination ranks
    // [E, E + N) for the first item of each (token, rank)
    const int NK = partial ? E + N : E;
    const int CW = ra.chunk_waves;              // waves that take items in one chunk
    uint64_t* mask = lds64;                     // [2][CW][NK]: lanes of a wave holding a key
    int32_t* cur = reinterpret_cast<int32_t*>(mask + 2 * (size_t)CW * NK);  // [2][NK] cursors
    __shared__ int32_t wave_sums[RP_WAVES + 1];
    __shared__ int32_t ticket;
    __shared__ int32_t wg_err;             // this workgroup's error bits

    const int s = blockIdx.x;
    const int items = ra.T * ra.K;
    const int32_t* my_idx = ra.idx + (size_t)s * items;
    int32_t* my_pdst = partial ? p.pdst + (size_t)s * items : nullptr;
    const int tid = threadIdx.x;
    const int chunk = CW * WAVE;
    const int held_items = min(items, HC * chunk);

    for (int k = tid; k < NK; k += RP_NT)
        cur[k] = 0;
    for (int j = tid; j < CW * NK; j += RP_NT)
        mask[j] = 0ull;
    if (tid == 0)
        wg_err = 0;
    if (s == 0 && tid == 0)
        *p.err_next = 0;             // the next cycle starts with a clean word
    // expert ids of the first HC chunks stay in registers for both
    // the counting and the ranking (thread tid takes item c*chunk + tid of
    // chunk c); all loads are issued before the first use
    int held_e[HC];
    if (items > 0) {
        // clamped addresses, so the loads are unconditional and issue together
#pragma unroll
        for (int c = 0; c < HC; ++c)
            held_e[c] = my_idx[min(c * chunk + tid, items - 1)];
#pragma unroll
        for (int c = 0; c < HC; ++c)
            if (!(tid < chunk && c * chunk + tid < items))
                held_e[c] = -1;
    } else {
#pragma unroll
        for (int c = 0; c < HC; ++c)
            held_e[c] = -1;
    }
    __syncthreads();
    int bad = 0;
    if (!partial) {
#pragma unroll
        for (int c = 0; c < HC; ++c) {
            const int e = held_e[c];
            if ((unsigned)e < (unsigned)E)
                atomicAdd(&cur[e], 1);
            else if (tid < chunk && c * chunk + tid < items)
                bad = 1;
        }
        for (int i = held_items + tid; i < items; i += RP_NT) {
            const int e = my_idx[i];
            if ((unsigned)e < (unsigned)E)
                atomicAdd(&cur[e], 1);
            else
                bad = 1;
        }
    } else {
        // Each item also gets its rank key when it is the first of its token
        // on that rank (one partial row per (token, rank)); the held ids are
        // replaced by the packed key pair.
#pragma unroll
        for (int c = 0; c < HC; ++c) {
            if (c * chunk >= items)
                break;
            const int i = c * chunk + tid;
            const bool mine = tid < chunk && i < items;
            const int e = held_e[c];
            const bool ok = (unsigned)e < (unsigned)E;
            if (ok)
                atomicAdd(&cur[e], 1);
            else if (mine)
                bad = 1;
            bool first;
            const int d = rank_of_item(ra, my_idx, e, i, mine, &first);
            if (mine)
                my_pdst[i] = d;
            if (first)
                atomicAdd(&cur[E + d], 1);
            held_e[c] = pack_keys(ok ? e : -1, first ? E + d : -1);
        }
        for (int i0 = held_items; i0 < items; i0 += RP_NT) {
            const int i = i0 + tid;
            const bool mine = i < items;
            const int e = mine ? my_idx[i] : -1;
            if ((unsigned)e < (unsigned)E)
                atomicAdd(&cur[e], 1);
            else if (mine)
                bad = 1;
            bool first;
            const int d = rank_of_item(ra, my_idx, e, i, mine, &first);
            if (mine)
                my_pdst[i] = d;
            if (first)
                atomicAdd(&cur[E + d], 1);
        }
    }
    if (bad)
        atomicOr(&wg_err, ERR_BIT_ROUTING);
    __syncthreads();

    // counts out, exclusive scans -> send offsets (and the partial rows'
    // offsets per rank) and the cursors, then the stable position of every
    // item inside its expert's rows (and of every first item of a rank among
    // the sender's partial rows, ordered by rank, then token)
    publish_counts(cur, E, p.cnt + (size_t)s * E, p.soff + (size_t)s * (E + 1), wave_sums,
                   ra.slot_cap, &wg_err,
                   p.soff_col + s, N);
    if (!partial) {
        stable_ranks<false, HC>(items, NK, CW, mask, cur, held_e,
                            [&](int i, bool mine) { return mine ? my_idx[i] : -1; },
                            p.pos + (size_t)s * items, nullptr,
                            ra.send_meta ? ra.send_meta + (size_t)s * items : nullptr);
    } else {
        publish_counts(cur + E, N, nullptr, p.psoff + (size_t)s * (N + 1), wave_sums, -1, &wg_err,
                       p.psoff_col + s, N);
        stable_ranks<true, HC>(items, NK, CW, mask, cur, held_e,
                           [&](int i, bool mine) {
                               const int e = mine ? my_idx[i] : -1;
                               bool first;
                               const int d = rank_of_item(ra, my_idx, e, i, mine, &first);
                               return pack_keys((unsigned)e < (unsigned)E ? e : -1,
                                                first ? E + d : -1);
                           },
                           p.pos + (size_t)s * items, p.ppos + (size_t)s * items,
                           ra.send_meta ? ra.send_meta + (size_t)s * items : nullptr);
    }

    // Publish this rank's error bits (into the cycle's word too).  Where the
    // group offsets are formed here, draw a ticket: every wave waits for its
    // own stores, then one agent-scope release (an L2 write-back) covers the
    // whole workgroup before the ticket is taken, and the last workgroup
    // forms them.
    __syncthreads();
    if (tid == 0) {
        p.err_rank[s] = wg_err;
        if (wg_err) {
            atomicOr(p.err, wg_err);
            atomicOr(p.err_sticky, wg_err);
        }
    }
    if (!TAIL)
        return;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        ticket = atomicAdd(p.ticket, 1);
    }
    __syncthreads();
    if (ticket != ra.N - 1)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // the masks are dead: their LDS takes the soff table
    close_plan(ra, p, &wg_err, ra.table_lds ? reinterpret_cast<int32_t*>(lds64) : nullptr);
    if (tid == 0)
        atomicExch(p.ticket, 0);
}


// ---------------------------------------------------------------------------
// Work split of the row kernels.  SPLIT waves share one row, each moving a
// contiguous part (ALIGN-vector aligned); waves are numbered across blocks,
// so with SPLIT 8 a row spans two 256-thread blocks.  Long rows are split
// until each lane moves about 2 vectors: many short waves keep more rows in
// flight per CU than a few long ones (measured on 7-14 KiB rows).
// ---------------------------------------------------------------------------
struct RowSlot {
    int64_t row;
    int b0, len;      // vectors [b0, b0 + len) of the row
    bool lead;        // part 0 also moves the row's scales and metadata
};

template <int SPLIT, int ALIGN = 1>
__device__ inline RowSlot row_slot(int n, int64_t block = blockIdx.x)
{
    RowSlot rs;
    const int64_t w = block * ROWS_PER_BLOCK + threadIdx.x / WAVE;
    rs.row = w / SPLIT;
    const int part = (int)(w % SPLIT);
    const int plen = ((n + SPLIT - 1) / SPLIT + ALIGN - 1) / ALIGN * ALIGN;
    rs.b0 = min(n, part * plen);
    rs.len = min(n, rs.b0 + plen) - rs.b0;
    rs.lead = part == 0;
    return rs;
}

// The hardware places blocks round-robin over the chip's 8 XCDs (block b on
// XCD b mod 8), so consecutive rows run on different XCDs.  The movers remap
// the block index so that each XCD takes runs of `run` consecutive blocks: an
// XCD's CUs (its L2 and its address translation) then stay in fewer source
// pages at a time.  The transfers, whose rows come in (sender -> receiver)
// segments of contiguous source rows, take one average segment per run:
// DeepSeek-R1 decode (64 blocks a segment) 155 -> 148-150 us; fp8 prefill (256
// and 512) 2610 -> 2460 and 5284 -> 4760 us, where round-robin placement took
// one UTCL1 translation miss per row; the transfer back, against runs of 1,
// 32, 128, 256 and 2048 blocks, was fastest or equal with its segment runs
// (DeepSeek-R1 decode 149.7 us against 151.3-156.5).  The shuffle, the combine pack, the
// combine push and the combine reduce take fixed runs (host side,
// RUN_ROWS_BLOCKS and RUN_TOKEN_BLOCKS).  A ragged last tile keeps its order; run = 1 is plain
// order.
constexpr int XCDS = 8;

// Block b of a part of the grid that starts at a multiple of 8 blocks and
// has nblocks blocks (the whole grid by default).
__device__ inline int64_t xcd_run_block(uint32_t run, uint32_t b = blockIdx.x,
                                        uint32_t nblocks = gridDim.x)
{
    if (run <= 1)
        return b;
    const uint32_t tile = XCDS * run;            // the host keeps run below 2^28
    const uint32_t t0 = b / tile * tile;
    if (t0 + tile > nblocks)
        return b;
    const uint32_t r = b - t0;
    return (int64_t)t0 + (r % XCDS) * run + r / XCDS;
}

// ---------------------------------------------------------------------------
// Pack: one token per wave (or per SPLIT waves).
//
// [EPMC] "Dispatch": activations, block scales and the token's index on the
// sending rank are packed contiguously; [EFA] "Dispatch and combine": with the
// offsets known, rows are packed into contiguous per-peer send buffers.  The
// token row is read once and written K times (one per routed expert).  For
// row (s, t, k) lanes k < K work out where it goes:
//   send row       srow = s*T*K + pos
//   receive row    q    = rbase[d] + roff[d][s] + pos - soff[s][d*L]   (d = e / L)
//   expert row     r    = sbase[s][e] + pos - soff[s][e]   (partial combine)
// and the lead wave records the row maps the movers follow.  With the staged
// transport the rows go to the send buffer (row srow) and the transfer kernel
// moves them; with the direct transport they are pushed straight into the
// receive buffer (row q), as the pages push intra-node tokens into peers'
// buffers ([EFA] "Dispatch and combine").
// ---------------------------------------------------------------------------
struct RowDest {
    int32_t srow, q, qd, r;   // send row, packed receive row, receive-plane row, expert row
    bool ok;
};

// With the fixed-slot layout ([EPMC] "Portable kernels") the receive-plane
// row needs only the sender's own offsets: slot i = pk - soff[s][e] of the
// pair (s, e) is row (e*T_max + i)*N + s (each expert's area slot-major, so
// the filled slots of all senders sit together at its start).
// With Shape::sender_only the group offsets are not formed yet: only the
// send row and the slot are computed (q and r stay 0, unused).
__device__ inline RowDest row_dest(const Shape& sh, const Plan& p, int s, int e, int pk)
{
    const int64_t TK = (int64_t)sh.T * sh.K;
    RowDest rd;
    rd.srow = (int32_t)(s * TK + pk);
    const int32_t* so = p.soff + (size_t)s * (sh.E + 1);
    const int i = pk - so[e];
    bool ok = (uint64_t)pk < (uint64_t)TK;
    rd.q = 0;
    rd.r = 0;
    if (!sh.sender_only) {
        const int d = e / sh.L;
        rd.q = p.rbase[d] + p.roff[(size_t)d * (sh.N + 1) + s] + pk - so[d * sh.L];
        ok = ok && (uint64_t)rd.q < (uint64_t)sh.rows;
    }
    if (sh.partial) {
        // the expert row, named by the partial combine's records
        rd.r = p.sbase[(size_t)s * (sh.E + 2 * sh.N + 2) + e] + i;
        ok = ok && (uint64_t)rd.r < (uint64_t)sh.rows;
    }
    const int64_t slot = ((int64_t)e * sh.slots + i) * sh.N + s;
    rd.qd = sh.fixed ? (int32_t)slot : rd.q;
    if (sh.fixed)
        ok = ok && (uint32_t)i < (uint32_t)sh.slots && (uint64_t)slot < (uint64_t)sh.recv_rows;
    rd.ok = ok;
    return rd;
}

// The map the sender's own transfer follows (the receiver's maps are made by
// recv_map_kernel): for the packed layout the send row of each receive row,
// for the fixed-slot layout the slot of each send row.  The direct transport
// has no transfer.
__device__ inline void record_maps(const Shape& sh, const Plan& p, const RowDest& rd)
{
    if (sh.direct)
        return;
    if (sh.fixed)
        p.send_slot[rd.srow] = rd.qd;
    else
        p.xfer_src[rd.q] = rd.srow;
}

// Whether sender s's rows are to be dropped this cycle: the cycle's error
// word, or with Shape::sender_only (whose senders use nothing from the
// exchange) the sender's own bits from this cycle's route plan.
__device__ inline bool sender_failed(const Shape& sh, const Plan& p, int s)
{
    return sh.sender_only ? p.err_rank[s] != 0 : *p.err != 0;
}

// Records of the expert-side partial combine, made by waves holding the
// items of whole tokens, K lanes a token (all lanes call it; a lane holding
// an item has its index i = tok*K + k, else -1, the first lane of its token
// `seg`, its expert rank d, or -1 if its indices failed, and its
// receive-plane and expert rows).  Each item gets its (expert row,
// receive-plane row); each head item (the first of its rank in the token)
// writes the record of the partial row it heads, in the layout the expert
// side writes (owner layout when staged, token layout when direct): the
// (expert row, receive-plane row) of its first two items, the token, the
// item count and the mask of the token's items on that rank (by k); and,
// staged, the owner row of its token-layout row for the transfer back.  The
// bases: P partial rows in all, pb the sender's first token-layout partial
// row, and per lane ob, the owner-layout row of the sender's first partial
// row on rank d less psoff[s][d], so that a head at ppos pp owns token-layout
// row pb + pp and owner-layout row ob + pp.
__device__ inline void write_partial_records(const Shape& sh, const Plan& p, int64_t i, int seg,
                                             int d, const RowDest& rd, int P, int pb, int ob)
{
    const int lane = lane_id();
    int pp = -1;
    if (i >= 0 && d >= 0) {
        p.pitem[i] = make_int2(rd.r, rd.qd);
        pp = p.ppos[i];
    }
    // every head lane finds its partial rows at once
    int tr = 0, orow = 0;
    bool ok = false;
    if (pp >= 0) {
        tr = pb + pp;
        orow = ob + pp;
        ok = (unsigned)tr < (unsigned)P && (unsigned)orow < (unsigned)P;
        if (!ok)
            raise_err(p, ERR_BIT_INTERNAL);
    }
    // then each lane's mask of its token's items on its rank (bit k: item
    // k), and the rows of the second of them, by shuffles within the token's
    // lanes (no memory access)
    uint64_t my_mask = 0;
    for (int j = 0; j < sh.K; ++j) {
        const int dj = __shfl(d, min(seg + j, WAVE - 1), WAVE);
        if (d >= 0 && dj == d)
            my_mask |= 1ull << j;
    }
    const uint64_t rest = my_mask & (my_mask - 1);
    const int f1 = seg + (rest ? __builtin_ctzll(rest) : lane - seg);
    const int my_r1 = __shfl(rd.r, min(f1, WAVE - 1), WAVE);
    const int my_q1 = __shfl(rd.qd, min(f1, WAVE - 1), WAVE);
    if (ok) {
        int4* rec = p.phead + 2 * (int64_t)(sh.direct ? tr : orow);
        rec[0] = make_int4(rd.r, rd.qd, my_r1, my_q1);
        rec[1] = make_int4((int)(i / sh.K), __popcll(my_mask), (int)(uint32_t)my_mask,
                           (int)(uint32_t)(my_mask >> 32));
        if (!sh.direct)
            p.pmap[tr] = orow;
    }
}

// One token per wave (lanes k < K), the bases read from the sender's base
// row that the route plan formed: pb = sbase[s][E+2N], P = sbase[s][E+2N+1],
// ob = sbase[s][E+N+d] - psoff[s][d].
__device__ inline void record_partial(const Shape& sh, const Plan& p, int64_t tok, int s, int d,
                                      const RowDest& rd)
{
    const int N = sh.N, E = sh.E;
    int P = 0, pb = 0, ob = 0;
    const bool mine = lane_id() < sh.K;
    if (mine && d >= 0) {
        const int32_t* sb = p.sbase + (size_t)s * (E + 2 * N + 2);
        P = sb[E + 2 * N + 1];
        pb = sb[E + 2 * N];
        ob = sb[E + N + d] - p.psoff[(size_t)s * (N + 1) + d];
    }
    write_partial_records(sh, p, mine ? tok * sh.K + lane_id() : -1, 0, d, rd, P, pb, ob);
}

// Lanes k < K: the destination row of (token, k) in the buffer pack writes
// (send row, or receive row when direct), -1 if an index check failed; the
// lead wave also writes the maps, the meta word t*K+k and, for the
// expert-side partial combine, the router weight (dst_w non-null) and the
// partial-row records.
__device__ inline int pack_dest(const Shape& sh, const Plan& p, const int32_t* __restrict__ idx,
                                const float* __restrict__ w, int32_t* __restrict__ dst_meta,
                                float* __restrict__ dst_w, int64_t tok, int s, int t, bool lead)
{
    const int lane = lane_id();
    int row = -1, d = -1;
    RowDest rd{};
    if (lane < sh.K) {
        const int64_t i = tok * sh.K + lane;
        const int e = idx[i];
        rd = row_dest(sh, p, s, e, p.pos[i]);
        if (rd.ok) {
            row = sh.direct ? rd.qd : rd.srow;
            d = e / sh.L;
            if (lead) {
                record_maps(sh, p, rd);
                dst_meta[row] = t * sh.K + lane;
                if (dst_w)
                    dst_w[row] = w[i];
            }
        } else if (lead) {
            raise_err(p, ERR_BIT_INTERNAL);
        }
    }
    if (sh.partial && lead)
        record_partial(sh, p, tok, s, d, rd);
    return row;
}

template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_bf16_kernel(Shape sh, Plan p,
                                                                 const v4u* __restrict__ x,
                                                                 const int32_t* __restrict__ idx,
                                                                 const float* __restrict__ w,
                                                                 v4u* __restrict__ dst_x,
                                                                 int32_t* __restrict__ dst_meta,
                                                                 float* __restrict__ dst_w)
{
    const int lane = lane_id();
    const int n = sh.payload_vecs;
    const RowSlot rs = row_slot<SPLIT>(n);
    const int64_t tok = rs.row;
    if (tok >= (int64_t)sh.N * sh.T)
        return;
    const int s = (int)(tok / sh.T), t = (int)(tok % sh.T);
    if (sender_failed(sh, p, s))
        return;
    const int my_row = pack_dest(sh, p, idx, w, dst_meta, dst_w, tok, s, t, rs.lead);
    const v4u* src = x + tok * n + rs.b0;
    for (int base = 0; base < rs.len; base += WAVE * U) {
        // the caller's tokens are read with ordinary loads (measured faster
        // here than the streaming hint); the K copies are streamed out
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = src[min(base + u * WAVE + lane, rs.len - 1)];
        hold(v);
        for (int k = 0; k < sh.K; ++k) {
            const int row = readlane(my_row, k);
            if ((uint64_t)row >= (uint64_t)(sh.direct ? sh.recv_rows : sh.rows))
                continue;
            v4u* dst = dst_x + (int64_t)row * n + rs.b0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * WAVE + lane;
                if (j < rs.len)
                    st_nt(v[u], dst + j);
            }
        }
    }
}

// OCP e4m3 encode, round to nearest even, saturating at +-448; NaN -> S.1111.111.
// Normal results round the fp32 mantissa at bit 20 (ties to even) and rebias
// the exponent from 127 to 7; below 2^-6 the result is |v|*2^9 rounded to an
// integer (exact scaling, then round-half-even), which also covers rounding
// up into the smallest normal.
__device__ inline uint32_t e4m3_encode(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;
    if (a >= 0x43E00000u)                      // |v| >= 448
        return sign | 0x7Eu;
    if (a < 0x3C800000u) {                     // |v| < 2^-6
        const float m = __uint_as_float(a) * 512.0f;
        return sign | (uint32_t)__builtin_rintf(m);
    }
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    uint32_t c = (r >> 20) - (120u << 3);
    if (c > 0x7Eu)
        c = 0x7Eu;
    return sign | c;
}

// Block-scaled e4m3 of a lane's U 16-element groups (two input vectors of
// bf16 each, va[u] the first 8 elements and vb[u] the next 8): the 16 codes
// of each group as one vector, and its block's scale.  A 128-element block is
// 8 consecutive lanes (the same u), which share amax through xor shuffles, so
// every lane of the wave must call it.
template <int U>
__device__ inline void quant_groups(const v4u (&va)[U], const v4u (&vb)[U], v4u (&q)[U],
                                    float (&sc)[U])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float f[16];
        const uint32_t bits[8] = {va[u].x, va[u].y, va[u].z, va[u].w,
                                  vb[u].x, vb[u].y, vb[u].z, vb[u].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f[2 * i] = __uint_as_float(bits[i] << 16);
            f[2 * i + 1] = __uint_as_float(bits[i] & 0xFFFF0000u);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 4, WAVE));
        amax = fmaxf(amax, __shfl_xor(amax, 2, WAVE));
        amax = fmaxf(amax, __shfl_xor(amax, 1, WAVE));
        float inv = 0.0f, scale = 1.0f;
        if (amax >= 0x1.cp-118f) {             // 448 * 2^-126
            inv = 448.0f / amax;
            scale = amax / 448.0f;
        } else if (amax > 0.0f) {
            inv = 0x1p126f;
            scale = 0x1p-126f;
        }
        uint32_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            c[i] = e4m3_encode(f[i] * inv);
        q[u].x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        q[u].y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        q[u].z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
        q[u].w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
        sc[u] = scale;
    }
}

// [EFA] "Dispatch/combine latency": block-scaled fp8 dispatch; the blocks are
// 128 elements with one fp32 scale each.  Per block: amax = max|x| (exact from
// bf16); for amax >= 448 * 2^-126, inv = 448/amax and scale = amax/448 as
// correctly rounded fp32 divisions; for a smaller nonzero amax the scale is
// held at the smallest normal fp32 value, scale = 2^-126 and inv = 2^126 (so
// the scale never loses bits to an fp32 subnormal and inv never overflows);
// inv = 0, scale = 1 for an all-zero block; code = e4m3(x * inv).
// Each lane encodes 16 consecutive elements (two 16-byte input vectors) into
// one 16-byte store of codes; a 128-element block is 8 lanes, and amax is
// reduced over the 8-lane group with xor shuffles.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_fp8_kernel(Shape sh, Plan p,
                                                                const v4u* __restrict__ x,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ w,
                                                                v4u* __restrict__ dst_q,
                                                                float* __restrict__ dst_scale,
                                                                int32_t* __restrict__ dst_meta,
                                                                float* __restrict__ dst_w,
                                                                uint32_t xrun)
{
    const int lane = lane_id();
    const int n2 = sh.H / 16;                  // 16-element groups per row (= 16-byte code vectors)
    // parts hold whole 128-element blocks
    const RowSlot rs = row_slot<SPLIT, 8>(n2, xcd_run_block(xrun));
    const int64_t tok = rs.row;
    if (tok >= (int64_t)sh.N * sh.T)
        return;
    const int s = (int)(tok / sh.T), t = (int)(tok % sh.T);
    if (sender_failed(sh, p, s))
        return;
    const int my_row = pack_dest(sh, p, idx, w, dst_meta, dst_w, tok, s, t, rs.lead);
    const int nb = sh.scale_blocks;
    const v4u* src = x + tok * (2 * n2);
    const int end = rs.b0 + rs.len;
    for (int base = rs.b0; base < end; base += WAVE * U) {
        // clamped loads (see copy_row); an 8-lane group lies wholly inside or
        // wholly past the part's end because the part bounds and base are
        // multiples of 8.  Ordinary loads, as in the bf16 pack: the
        // nontemporal hint cost 2.5% on the fp8 prefill (each lane's two
        // vectors are interleaved with its neighbours', so each 16-byte load
        // touches lines that its partner load reads again)
        v4u va[U], vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(base + u * WAVE + lane, end - 1);
            va[u] = src[2 * j];
            vb[u] = src[2 * j + 1];
        }
        hold(va);
        hold(vb);
        v4u q[U];
        float sc[U];
        quant_groups<U>(va, vb, q, sc);
        for (int k = 0; k < sh.K; ++k) {
            const int row32 = readlane(my_row, k);
            if ((uint64_t)row32 >= (uint64_t)(sh.direct ? sh.recv_rows : sh.rows))
                continue;
            const int64_t row = row32;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * WAVE + lane;
                if (j < end) {
                    st_nt(q[u], dst_q + row * n2 + j);
                    if ((lane & 7) == 0)
                        dst_scale[row * nb + j / 8] = sc[u];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Pack in send-row order: the same rows as the token-order kernels above,
// written as a gather.  The route plan has already
// written the item t*K+k each send row holds (into the send meta words when
// staged, into send_item when direct), so send row (s, pk) reads its token's
// row x[s][t] and writes it (quantised, for e4m3): staged, in place, so the
// writes stream through the send buffer in address order as the movers' do;
// direct, to its receive-plane row, so they stream through one (s -> d)
// segment after another.  Each token is read K times, mostly from cache (a
// sender's tokens are a few MiB, and one XCD takes a run of its send rows).
// The staged lead wave also records the transfer's map, which needs the
// item's expert (idx) and the offsets: one more dependent load that no other
// wave waits for; the direct lead wave writes the row's meta word.  With the
// expert-side partial combine the lead wave also moves the row's router
// weight, and waves past the rows' write the per-token records.
// ---------------------------------------------------------------------------
// The sum of one int per lane over the wave (every lane active), as a
// wave-uniform value: DPP moves within each row of 16 lanes (swap neighbours,
// swap pairs, mirror within 8, mirror within 16), so every lane holds its
// row's sum, then the four rows' sums are read out.  Register moves only,
// where shuffles would go through the LDS crossbar.
__device__ inline int wave_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);   // row_mirror
    return readlane(v, 0) + readlane(v, 16) + readlane(v, 32) + readlane(v, 48);
}

// The first packed receive row of the (s -> d) rows, rbase[d] + roff[d][s],
// from the senders' offsets alone: what the senders before s send to ranks up
// to d and what s and the senders after it send to ranks before d, i.e. the
// sum of soff[j][(d+1)*L] over j < s and of soff[j][d*L] over j >= s.  Lanes
// take the senders, C*64 of them in one round of loads.  Every lane of the
// wave must call it.
template <int C>
__device__ inline int seg_base_c(const Shape& sh, const Plan& p, int s, int d)
{
    const int lane = lane_id();
    // the two columns, senders consecutive (soff_col is soff transposed)
    const int32_t* lo = p.soff_col + (size_t)d * sh.L * sh.N;
    const int32_t* hi = p.soff_col + (size_t)(d + 1) * sh.L * sh.N;
    int v[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = min(c * WAVE + lane, sh.N - 1);
        v[c] = (j < s ? hi : lo)[j];
    }
    int part = 0;
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (c * WAVE + lane < sh.N)
            part += v[c];
    for (int j = C * WAVE + lane; j < sh.N; j += WAVE)
        part += (j < s ? hi : lo)[j];
    return wave_sum(part);
}

__device__ inline int seg_base(const Shape& sh, const Plan& p, int s, int d)
{
    return sh.N <= WAVE ? seg_base_c<1>(sh, p, s, d) : seg_base_c<4>(sh, p, s, d);
}

// The last bucket b in [0, nb) whose start row[b * stride] is <= key, with
// that start, for non-decreasing starts (the expert or rank parts of a
// sender's send rows); -1 if none.  Lanes take 64 buckets at a time, and up
// to C*64 buckets are loaded in one round.  Every lane of the wave must call
// it with the same arguments.
template <int C>
__device__ inline int2 find_bucket(const int32_t* __restrict__ row, int nb, int stride, int key)
{
    const int lane = lane_id();
    int b = -1, start = 0;
    int v[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
        v[c] = row[(size_t)min(c * WAVE + lane, nb - 1) * stride];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint64_t m = __ballot(c * WAVE + lane < nb && v[c] <= key);
        if (m) {
            const int top = 63 - __builtin_clzll(m);
            b = c * WAVE + top;
            start = readlane(v[c], top);
        }
    }
    for (int b0 = C * WAVE; b0 < nb; b0 += WAVE) {
        const int j = b0 + lane;
        const int w = j < nb ? row[(size_t)j * stride] : 0;
        const uint64_t m = __ballot(j < nb && w <= key);
        if (m) {
            const int top = 63 - __builtin_clzll(m);
            b = b0 + top;
            start = readlane(w, top);
        }
    }
    return make_int2(b, start);
}

// The receive-plane row that the direct transport gives send row (s, pk): the
// rank d whose part of the sender's rows holds pk, then q = rbase[d] +
// roff[d][s] + pk - soff[s][d*L] (from the route plan's tables when it formed
// them, else seg_base); with fixed slots, from the sender's own offsets alone,
// the expert e whose part holds it, then slot i = pk - soff[s][e], row
// (e*T_max + i)*N + s.  -1 if a check fails.  Every lane of the wave must
// call it.
__device__ inline int64_t direct_row(const Shape& sh, const Plan& p, int s, int pk)
{
    const int32_t* so = p.soff + (size_t)s * (sh.E + 1);
    if (sh.fixed) {
        const int2 b = sh.E <= WAVE ? find_bucket<1>(so, sh.E, 1, pk)
                                    : find_bucket<4>(so, sh.E, 1, pk);
        const int i = pk - b.y;
        if (b.x < 0 || (unsigned)i >= (unsigned)sh.slots)
            return -1;
        const int64_t slot = ((int64_t)b.x * sh.slots + i) * sh.N + s;
        return slot < sh.recv_rows ? slot : -1;
    }
    const int2 b = sh.N <= WAVE ? find_bucket<1>(so, sh.N, sh.L, pk)
                                : find_bucket<4>(so, sh.N, sh.L, pk);
    if (b.x < 0)
        return -1;
    const int64_t base = sh.plan_offsets ? (int64_t)p.rbase[b.x] + p.roff[(size_t)b.x * (sh.N + 1) + s]
                                         : (int64_t)seg_base(sh, p, s, b.x);
    const int64_t q = base + pk - b.y;
    return (uint64_t)q < (uint64_t)sh.rows ? q : -1;
}

// The map the staged transfer follows for send row (s, pk) holding item m,
// from the senders' offsets alone: the row's packed receive row q (xfer_src[q]
// = the send row), or with fixed slots its slot (send_slot).  Every lane of
// the lead wave calls it.
__device__ inline void record_send_row(const Shape& sh, const Plan& p,
                                       const int32_t* __restrict__ idx, int s, int pk, int m)
{
    const int lane = lane_id();
    const int64_t TK = (int64_t)sh.T * sh.K;
    const int64_t srow = s * TK + pk;
    const int e = idx[s * TK + m];
    if ((unsigned)e >= (unsigned)sh.E) {
        if (lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    const int32_t* so = p.soff + (size_t)s * (sh.E + 1);
    if (sh.fixed) {
        const int i = pk - so[e];
        const int64_t slot = ((int64_t)e * sh.slots + i) * sh.N + s;
        if (lane == 0) {
            if ((unsigned)i < (unsigned)sh.slots && slot < sh.recv_rows)
                p.send_slot[srow] = (int32_t)slot;
            else
                raise_err(p, ERR_BIT_INTERNAL);
        }
        return;
    }
    const int d = e / sh.L;
    const int64_t q = (int64_t)seg_base(sh, p, s, d) + pk - so[d * sh.L];
    if (lane == 0) {
        if ((uint64_t)q < (uint64_t)sh.rows)
            p.xfer_src[q] = (int32_t)srow;
        else
            raise_err(p, ERR_BIT_INTERNAL);
    }
}

// The partial combine's records in the send-row-order pack, whose row waves
// see one item each: blocks of one sender s each, ahead of the row blocks, a
// wave taking 64/K tokens at a time (K lanes a token) and up to REC_PASSES
// such passes.  A block first puts its sender's bases in LDS (ints:
// so[E+1], ps[N+1], eb[E], qb[N], ob[N], pb, P):
//   so[e] = soff[s][e],  ps[d] = psoff[s][d]
//   eb[e] = first expert row of (s, e) = sum_{j<s} soff[j][e+1] + sum_{j>=s} soff[j][e]
//   qb[d] = first receive row from s on rank d
//         = sum_{j<s} soff[j][(d+1)L] + sum_{j>=s} soff[j][dL]
//   ob[d] = first owner-layout partial row from s on rank d
//         = sum_{j<s} psoff[j][d+1] + sum_{j>=s} psoff[j][d]
//   pb    = first token-layout partial row of s = sum_{j<s} psoff[j][N]
//   P     = partial rows in all = sum_j psoff[j][N]
// (a thread per sum, walking the senders' rows, so that the threads of a
// wave read neighbouring entries; with Shape::plan_offsets they are read
// from the route plan's group tables instead), then each item's lane places
// it from them:
//   expert row        r  = eb[e] + pos - so[e]
//   receive-plane row qd = qb[d] + pos - so[dL], or the slot (e*T_max + pos - so[e])*N + s
// and the head items write the records (write_partial_records).  Measured on
// the decode shapes against records one token per wave (many blocks, each
// summing its sender's bases): those sums cost the pack 4-27 us, and its
// scalar registers (106, occupancy 7 waves per SIMD for every row block)
// another 4-10; one block per sender, a wave's tokens' masks by shuffles
// and 32-bit table indices (94 registers, occupancy 8) brought the staged
// pack back to its time with the route plan's tables.  One, two or four
// passes per wave measured the same.
constexpr int REC_PASSES = 4;

__host__ __device__ inline int rec_lds_ints(const Shape& sh)
{
    return 2 * sh.E + 3 * sh.N + 4;
}

__host__ __device__ inline int rec_tokens_per_block(const Shape& sh)
{
    return ROWS_PER_BLOCK * (WAVE / sh.K) * REC_PASSES;
}

// sum_{j<s} row_j[hi] + sum_{j>=s} row_j[lo] over the rows j < n of a table
// with row stride W: 8 loads issued together per round (clamped rows, the
// ones past n not added).  32-bit indices (the tables hold fewer than 2^21
// entries).
__device__ inline int split_sum(const int32_t* __restrict__ t, int W, int lo, int hi, int n, int s)
{
    int sum = 0;
    for (int j = 0; j < n; j += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = min(j + u, n - 1);
            v[u] = t[r * W + (r < s ? hi : lo)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j + u < n)
                sum += v[u];
    }
    return sum;
}

__device__ inline void sender_bases(const Shape& sh, const Plan& p, int s, int32_t* tab)
{
    const int E = sh.E, N = sh.N, L = sh.L, tid = threadIdx.x;
    int32_t* so = tab;
    int32_t* ps = so + E + 1;
    int32_t* eb = ps + N + 1;
    for (int j = tid; j <= E; j += COPY_THREADS)
        so[j] = p.soff[(size_t)s * (E + 1) + j];
    for (int j = tid; j <= N; j += COPY_THREADS)
        ps[j] = p.psoff[(size_t)s * (N + 1) + j];
    const int nv = E + 2 * N + 2;
    for (int v = tid; v < nv; v += COPY_THREADS) {
        int val;
        if (sh.plan_offsets) {
            val = p.sbase[(size_t)s * nv + v];
        } else if (v < E) {
            val = split_sum(p.soff, E + 1, v, v + 1, N, s);
        } else if (v < E + N) {
            const int d = v - E;
            val = sh.fixed ? 0 : split_sum(p.soff, E + 1, d * L, (d + 1) * L, N, s);
        } else if (v < E + 2 * N) {
            const int d = v - E - N;
            val = split_sum(p.psoff, N + 1, d, d + 1, N, s);
        } else if (v == E + 2 * N) {
            val = split_sum(p.psoff, N + 1, N, N, s, s);
        } else {
            val = split_sum(p.psoff, N + 1, N, N, N, 0);
        }
        eb[v] = val;
    }
    __syncthreads();
}

// One pass of a wave over up to 64/K tokens [t0, t_end) of sender s, K lanes
// a token, from the sender's bases (every lane of the wave calls it).
__device__ inline void token_records(const Shape& sh, const Plan& p,
                                     const int32_t* __restrict__ idx, int s, int t0, int t_end,
                                     const int32_t* tab)
{
    const int lane = lane_id();
    const int E = sh.E, N = sh.N, K = sh.K;
    const int32_t* so = tab;
    const int32_t* ps = so + E + 1;
    const int32_t* eb = ps + N + 1;
    const int32_t* qb = eb + E;
    const int32_t* ob = qb + N;
    const int tl = lane / K, t = t0 + tl;
    const bool mine = tl < WAVE / K && t < t_end;
    const int64_t i = mine ? ((int64_t)s * sh.T + t) * K + lane % K : -1;
    int d = -1, obase = 0;
    RowDest rd{};
    if (mine) {
        const int e = idx[i];
        const int pk = p.pos[i];
        if ((unsigned)e < (unsigned)E && (int64_t)(unsigned)pk < (int64_t)sh.T * K) {
            const int dd = e / sh.L;
            const int ii = pk - so[e];
            const int64_t r = (int64_t)eb[e] + ii;
            int64_t qd;
            bool ok = (uint64_t)r < (uint64_t)sh.rows;
            if (sh.fixed) {
                qd = ((int64_t)e * sh.slots + ii) * N + s;
                ok = ok && (unsigned)ii < (unsigned)sh.slots && (uint64_t)qd < (uint64_t)sh.recv_rows;
            } else {
                qd = (int64_t)qb[dd] + pk - so[dd * sh.L];
                ok = ok && (uint64_t)qd < (uint64_t)sh.rows;
            }
            if (ok) {
                d = dd;
                rd.r = (int32_t)r;
                rd.qd = (int32_t)qd;
                obase = ob[dd] - ps[dd];
            }
        }
        if (d < 0)
            raise_err(p, ERR_BIT_INTERNAL);
    }
    write_partial_records(sh, p, i, tl * K, d, rd, ob[N + 1], ob[N], obase);
}

__device__ inline void pack_record_block(const Shape& sh, const Plan& p,
                                         const int32_t* __restrict__ idx, int32_t* tab)
{
    const int per_block = rec_tokens_per_block(sh);
    const int bps = (sh.T + per_block - 1) / per_block;
    const int s = (int)(blockIdx.x / bps);
    if (s >= sh.N)
        return;
    // one decision for the whole block, before its barrier: another block's
    // error can land while this one's threads read the word, and a block
    // that went on with part of its threads would place records from bases
    // it never formed
    if (__syncthreads_or(sender_failed(sh, p, s)))
        return;
    sender_bases(sh, p, s, tab);
    const int per_pass = WAVE / sh.K;
    const int b0 = (int)(blockIdx.x % bps) * per_block;
    const int t_end = min(sh.T, b0 + per_block);
    for (int t0 = b0 + (int)(threadIdx.x / WAVE) * per_pass; t0 < t_end;
         t0 += ROWS_PER_BLOCK * per_pass)
        token_records(sh, p, idx, s, t0, t_end, tab);
}

// REC: the grid starts with the partial combine's record blocks (a separate
// instance, so that the row blocks of the other modes keep their registers:
// the record path took the kernel's scalar registers from 71 to 94 and the
// receiver-side combine's direct pack from 89 to 93 us on DeepSeek-R1 decode).
template <int U, int SPLIT, bool REC>
__device__ __forceinline__ void pack_rows_bf16(const Shape& sh, const Plan& p,
                                               const v4u* __restrict__ x,
                                               const int32_t* __restrict__ idx,
                                               const int32_t* __restrict__ row_item,
                                               v4u* __restrict__ dst_x,
                                               int32_t* __restrict__ dst_meta,
                                               const float* __restrict__ w,
                                               float* __restrict__ dst_w, uint32_t xrun,
                                               uint32_t rec_blocks)
{
    const int lane = lane_id();
    const int n = sh.payload_vecs;
    if (REC && blockIdx.x < rec_blocks) {
        extern __shared__ __align__(16) int32_t rec_tab[];
        pack_record_block(sh, p, idx, rec_tab);
        return;
    }
    const RowSlot rs = row_slot<SPLIT>(
        n, xcd_run_block(xrun, blockIdx.x - rec_blocks, gridDim.x - rec_blocks));
    const int64_t TK = (int64_t)sh.T * sh.K;
    const int64_t srow = rs.row;
    if (srow >= sh.rows)
        return;
    const int s = (int)(srow / TK), pk = (int)(srow - s * TK);
    if (sender_failed(sh, p, s))
        return;
    const int m = row_item[srow];
    const int64_t drow = sh.direct ? direct_row(sh, p, s, pk) : srow;
    if ((unsigned)m >= (unsigned)TK || drow < 0) {
        if (rs.lead && lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    const v4u* src = x + ((int64_t)s * sh.T + m / sh.K) * n + rs.b0;
    v4u* dst = dst_x + drow * n + rs.b0;
    for (int base = 0; base < rs.len; base += WAVE * U) {
        // ordinary loads: the token's other K-1 rows read it again
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = src[min(base + u * WAVE + lane, rs.len - 1)];
        hold(v);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * WAVE + lane;
            if (j < rs.len)
                st_nt(v[u], dst + j);
        }
    }
    if (rs.lead) {
        if (!sh.direct)
            record_send_row(sh, p, idx, s, pk, m);
        if (lane == 0) {
            if (sh.direct)
                dst_meta[drow] = m;
            if (dst_w)
                dst_w[drow] = w[s * TK + m];
        }
    }
}

template <int U, int SPLIT, bool REC>
__device__ __forceinline__ void pack_rows_fp8(const Shape& sh, const Plan& p,
                                              const v4u* __restrict__ x,
                                              const int32_t* __restrict__ idx,
                                              const int32_t* __restrict__ row_item,
                                              v4u* __restrict__ dst_q,
                                              float* __restrict__ dst_scale,
                                              int32_t* __restrict__ dst_meta,
                                              const float* __restrict__ w,
                                              float* __restrict__ dst_w, uint32_t xrun,
                                              uint32_t rec_blocks)
{
    const int lane = lane_id();
    const int n2 = sh.H / 16;
    if (REC && blockIdx.x < rec_blocks) {
        extern __shared__ __align__(16) int32_t rec_tab[];
        pack_record_block(sh, p, idx, rec_tab);
        return;
    }
    const RowSlot rs = row_slot<SPLIT, 8>(
        n2, xcd_run_block(xrun, blockIdx.x - rec_blocks, gridDim.x - rec_blocks));
    const int64_t TK = (int64_t)sh.T * sh.K;
    const int64_t srow = rs.row;
    if (srow >= sh.rows)
        return;
    const int s = (int)(srow / TK), pk = (int)(srow - s * TK);
    if (sender_failed(sh, p, s))
        return;
    const int m = row_item[srow];
    const int64_t drow = sh.direct ? direct_row(sh, p, s, pk) : srow;
    if ((unsigned)m >= (unsigned)TK || drow < 0) {
        if (rs.lead && lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    const int nb = sh.scale_blocks;
    const v4u* src = x + ((int64_t)s * sh.T + m / sh.K) * (2 * n2);
    const int end = rs.b0 + rs.len;
    for (int base = rs.b0; base < end; base += WAVE * U) {
        // clamped loads; 8-lane groups lie wholly inside or past the part
        v4u va[U], vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(base + u * WAVE + lane, end - 1);
            va[u] = src[2 * j];
            vb[u] = src[2 * j + 1];
        }
        hold(va);
        hold(vb);
        v4u q[U];
        float sc[U];
        quant_groups<U>(va, vb, q, sc);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * WAVE + lane;
            if (j < end) {
                st_nt(q[u], dst_q + drow * n2 + j);
                if ((lane & 7) == 0)
                    dst_scale[drow * nb + j / 8] = sc[u];
            }
        }
    }
    if (rs.lead) {
        if (!sh.direct)
            record_send_row(sh, p, idx, s, pk, m);
        if (lane == 0) {
            if (sh.direct)
                dst_meta[drow] = m;
            if (dst_w)
                dst_w[drow] = w[s * TK + m];
        }
    }
}

template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_rows_bf16_kernel(
    Shape sh, Plan p, const v4u* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_item, v4u* __restrict__ dst_x, int32_t* __restrict__ dst_meta,
    const float* __restrict__ w, float* __restrict__ dst_w, uint32_t xrun, uint32_t rec_blocks)
{
    pack_rows_bf16<U, SPLIT, false>(sh, p, x, idx, row_item, dst_x, dst_meta, w, dst_w, xrun,
                                    rec_blocks);
}

template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_rows_rec_bf16_kernel(
    Shape sh, Plan p, const v4u* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_item, v4u* __restrict__ dst_x, int32_t* __restrict__ dst_meta,
    const float* __restrict__ w, float* __restrict__ dst_w, uint32_t xrun, uint32_t rec_blocks)
{
    pack_rows_bf16<U, SPLIT, true>(sh, p, x, idx, row_item, dst_x, dst_meta, w, dst_w, xrun,
                                   rec_blocks);
}

template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_rows_fp8_kernel(
    Shape sh, Plan p, const v4u* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_item, v4u* __restrict__ dst_q, float* __restrict__ dst_scale,
    int32_t* __restrict__ dst_meta, const float* __restrict__ w, float* __restrict__ dst_w,
    uint32_t xrun, uint32_t rec_blocks)
{
    pack_rows_fp8<U, SPLIT, false>(sh, p, x, idx, row_item, dst_q, dst_scale, dst_meta, w, dst_w,
                                   xrun, rec_blocks);
}

template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void pack_rows_rec_fp8_kernel(
    Shape sh, Plan p, const v4u* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_item, v4u* __restrict__ dst_q, float* __restrict__ dst_scale,
    int32_t* __restrict__ dst_meta, const float* __restrict__ w, float* __restrict__ dst_w,
    uint32_t xrun, uint32_t rec_blocks)
{
    pack_rows_fp8<U, SPLIT, true>(sh, p, x, idx, row_item, dst_q, dst_scale, dst_meta, w, dst_w,
                                  xrun, rec_blocks);
}

// ---------------------------------------------------------------------------
// Row movers: gathers in destination order, a row per one to eight waves.
// ---------------------------------------------------------------------------
// Loads use a clamped index instead of a predicate, so all U loads of a lane
// are issued back to back before the first wait; lanes past the row end
// re-read its last vector (same cache line) and skip the store.
template <int U>
__device__ inline void copy_row(v4u* __restrict__ dst, const v4u* __restrict__ src, int n, int lane)
{
    for (int base = 0; base < n; base += WAVE * U) {
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = ld_nt(src + min(base + u * WAVE + lane, n - 1));
        hold(v);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * WAVE + lane;
            if (j < n)
                st_nt(v[u], dst + j);
        }
    }
}

// Modelled transfer ([EFA] "Dispatch and combine": each peer's rows leave as
// one contiguous write; here rank d's receive row q takes send row
// xfer_src[q], so every (s -> d) segment is copied contiguously).  With the
// fixed-slot layout the copy runs in send order instead: send row srow goes
// to slot send_slot[srow], an address its sender formed from its own counts
// ([EPMC] "Portable kernels").  Moves the payload, the block scales (e4m3),
// the meta word and, for the expert-side partial combine, the router
// weight.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void transfer_kernel(Shape sh, Plan p,
                                                                const v4u* __restrict__ send_x,
                                                                v4u* __restrict__ recv_x,
                                                                const float* __restrict__ send_scale,
                                                                float* __restrict__ recv_scale,
                                                                const int32_t* __restrict__ send_meta,
                                                                int32_t* __restrict__ recv_meta,
                                                                const float* __restrict__ send_w,
                                                                float* __restrict__ recv_w,
                                                                uint32_t xrun)
{
    const int lane = lane_id();
    const int n = sh.payload_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    int64_t srow, q;
    if (sh.fixed) {
        srow = rs.row;
        if (srow >= sh.rows || sender_failed(sh, p, (int)(srow / ((int64_t)sh.T * sh.K))))
            return;
        q = p.send_slot[srow];
    } else {
        q = rs.row;
        if (q >= sh.rows || *p.err)
            return;
        srow = p.xfer_src[q];
    }
    if ((uint64_t)srow >= (uint64_t)sh.rows || (uint64_t)q >= (uint64_t)sh.recv_rows)
        return;
    copy_row<U>(recv_x + q * n + rs.b0, send_x + srow * n + rs.b0, rs.len, lane);
    if (!rs.lead)
        return;
    if (sh.fp8)
        for (int j = lane; j < sh.scale_blocks; j += WAVE)
            recv_scale[q * sh.scale_blocks + j] = send_scale[srow * sh.scale_blocks + j];
    if (lane == 0) {
        recv_meta[q] = send_meta[srow];
        if (send_w)
            recv_w[q] = send_w[srow];
    }
}

// The receiver's row maps, formed at dispatch_recv from the exchanged counts
// and offsets alone ([EFA] "Send and receive buffers": once the counts are
// exchanged, each rank knows where its rows come from), and -- when the route
// plan left them out (Shape::plan_offsets unset) -- the group offsets too.
// One wave per (expert e, sender s) pair, pairs in expert order so
// consecutive waves write consecutive expert rows.  The sums over senders
// (lanes take the senders j, 64 at a time, all loaded in one round):
//   eoff[e]               = sum_j soff[j][e]
//   rbase[d]              = sum_j soff[j][d*L]                      (d = e / L)
//   rbase[d] + roff[d][s] = sum_{j<s} soff[j][(d+1)L] + sum_{j>=s} soff[j][d*L]
//   first expert row r0   = eoff[e] + sum_{j<s} cnt[j][e]
// The pairs publish the tables they own (eoff by s = 0; roff and rbase by
// the rank's first expert; the totals by the first pair; with the partial
// combine qbase[d] = sum_j psoff[j][d] by (dL, 0), pbase[s] = sum_{j<s}
// psoff[j][N] by (0, s) and P by the first pair); then lane i <
// cnt[s][e] takes the pair's i-th row:
//   expert row        r    = r0 + i
//   packed receive row q    = rbase[d] + roff[d][s] + soff[s][e] - soff[s][d*L] + i
//   receive-plane row qd   = q, or the slot (e*T_max + i)*N + s
//   send row          srow = s*T*K + soff[s][e] + i   (its place on the way back)
// and writes shuf_map[r] (the shuffle's gather), shuf_inv[q] and slot_of[q]
// (the combine pack's) and xfer_dst[srow] (the return transfer's and the
// direct combine push's).
__global__ __launch_bounds__(COPY_THREADS) void recv_map_kernel(Shape sh, Plan p)
{
    if (*p.err)
        return;
    const int64_t w = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
    if (w >= (int64_t)sh.E * sh.N)
        return;
    const int lane = lane_id();
    const int N = sh.N, L = sh.L;
    const int e = (int)(w / N), s = (int)(w % N);
    const int d = e / L;
    const size_t W = (size_t)sh.E + 1;
    const int32_t* so = p.soff + (size_t)s * W;
    const int c = p.cnt[(size_t)s * sh.E + e];
    const bool tables = !sh.plan_offsets;
    const bool first_pair = tables && e == 0 && s == 0;
    if (c <= 0 && !(tables && (s == 0 || e == d * L)))
        return;
    const int so_e = so[e], so_d = so[d * L];
    int eo = 0, qb = 0, before = 0;
    // columns of soff transposed (senders consecutive): coalesced loads; a
    // sender's count of e is the difference of its columns e+1 and e
    const int32_t* col_e = p.soff_col + (size_t)e * N;
    const int32_t* col_e1 = col_e + N;
    if (!tables) {
        eo = p.eoff[e];
        qb = p.rbase[d] + p.roff[(size_t)d * (N + 1) + s];
        for (int j = lane; j < s; j += WAVE)
            before += col_e1[j] - col_e[j];
        before = wave_sum(before);
    } else {
        const int32_t* col_lo = p.soff_col + (size_t)d * L * N;
        const int32_t* col_hi = p.soff_col + (size_t)(d + 1) * L * N;
        const int32_t* col_tot = p.soff_col + (size_t)sh.E * N;
        // the partial combine's bases too: qbase[d] = sum_j psoff[j][d] (by
        // the pair (dL, 0)), pbase[s] = sum_{j<s} psoff[j][N] (by (0, s)),
        // and the total P
        const bool part = sh.partial != 0;
        const int32_t* pcol_d = part ? p.psoff_col + (size_t)d * N : nullptr;
        const int32_t* pcol_tot = part ? p.psoff_col + (size_t)N * N : nullptr;
        const bool own_qbase = part && s == 0 && e == d * L, own_pbase = part && e == 0;
        int rb = 0, tot = 0, pq = 0, pbs = 0, ptot = 0;
        for (int j0 = 0; j0 < N; j0 += WAVE) {
            const int j = j0 + lane;
            if (j < N) {
                const int lo = col_lo[j], ce = col_e[j];
                eo += ce;
                rb += lo;
                if (j < s) {
                    qb += col_hi[j];
                    before += col_e1[j] - ce;
                } else {
                    qb += lo;
                }
                if (first_pair)
                    tot += col_tot[j];
                if (own_qbase)
                    pq += pcol_d[j];
                if (own_pbase && (j < s || first_pair)) {
                    const int pt = pcol_tot[j];
                    if (j < s)
                        pbs += pt;
                    if (first_pair)
                        ptot += pt;
                }
            }
        }
        eo = wave_sum(eo);
        rb = wave_sum(rb);
        qb = wave_sum(qb);
        before = wave_sum(before);
        if (first_pair)
            tot = wave_sum(tot);
        if (own_qbase)
            pq = wave_sum(pq);
        if (own_pbase) {
            pbs = wave_sum(pbs);
            if (first_pair)
                ptot = wave_sum(ptot);
        }
        if (lane == 0) {
            if (own_qbase)
                p.qbase[d] = pq;
            if (own_pbase)
                p.pbase[s] = pbs;
            if (part && first_pair) {
                p.qbase[N] = ptot;
                p.pbase[N] = ptot;
            }
            if (s == 0)
                p.eoff[e] = eo;
            if (e == d * L) {
                int32_t* ro = p.roff + (size_t)d * (N + 1);
                ro[s] = qb - rb;
                if (s == N - 1)
                    ro[N] = qb - rb + so[(d + 1) * L] - so_d;
                if (s == 0)
                    p.rbase[d] = rb;
            }
            if (first_pair) {
                p.eoff[sh.E] = tot;
                p.rbase[N] = tot;
            }
        }
    }
    if (c <= 0)
        return;
    const int64_t srow0 = (int64_t)s * sh.T * sh.K + so_e;
    const int64_t q0 = (int64_t)qb + so_e - so_d;
    const int64_t r0 = (int64_t)eo + before;
    for (int i = lane; i < c; i += WAVE) {
        const int64_t q = q0 + i, r = r0 + i, srow = srow0 + i;
        const int64_t qd = sh.fixed ? ((int64_t)e * sh.slots + i) * sh.N + s : q;
        if ((uint64_t)q >= (uint64_t)sh.rows || (uint64_t)r >= (uint64_t)sh.rows ||
            (uint64_t)srow >= (uint64_t)sh.rows || (uint64_t)qd >= (uint64_t)sh.recv_rows ||
            (sh.fixed && i >= sh.slots)) {
            raise_err(p, ERR_BIT_INTERNAL);
            continue;
        }
        p.shuf_map[r] = make_int2((int)qd, s);
        p.shuf_inv[q] = (int32_t)r;
        p.xfer_dst[srow] = make_int2((int)qd, (int)r);
        if (sh.fixed)
            p.slot_of[q] = (int32_t)qd;
    }
}

// Receive shuffle ([EPMC] "Dispatch": received rows are copied into the
// contiguous grouped-GEMM input and the source rank and token index are stored
// for combine; [EFA] "Dispatch and combine": shuffle from the receive buffer
// into the tensor handed to the grouped GEMM).  Expert row r takes receive row
// shuf_map[r].x; block 0 also publishes the expert offsets.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void shuffle_kernel(Shape sh, Plan p,
                                                               const v4u* __restrict__ recv_x,
                                                               const float* __restrict__ recv_scale,
                                                               const int32_t* __restrict__ recv_meta,
                                                               v4u* __restrict__ expert_x,
                                                               float* __restrict__ expert_scale,
                                                               int32_t* __restrict__ src_rank,
                                                               int32_t* __restrict__ src_slot,
                                                               int32_t* __restrict__ expert_offsets,
                                                               uint32_t xrun)
{
    if (*p.err)
        return;
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e <= sh.E; e += COPY_THREADS)
            expert_offsets[e] = p.eoff[e];
    const int lane = lane_id();
    const int n = sh.payload_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    const int64_t r = rs.row;
    if (r >= sh.rows)
        return;
    const int2 m = p.shuf_map[r];
    const int64_t q = m.x;
    if ((uint64_t)q >= (uint64_t)sh.recv_rows)
        return;
    copy_row<U>(expert_x + r * n + rs.b0, recv_x + q * n + rs.b0, rs.len, lane);
    if (!rs.lead)
        return;
    if (sh.fp8)
        for (int j = lane; j < sh.scale_blocks; j += WAVE)
            expert_scale[r * sh.scale_blocks + j] = recv_scale[q * sh.scale_blocks + j];
    if (lane == 0) {
        src_rank[r] = m.y;
        src_slot[r] = recv_meta[q];
    }
}

// Combine send ([EPMC] "Combine": the 16-bit expert outputs go back to the
// slot each row came from; the inverse of the receive shuffle).  Written as a
// gather in destination order (measured faster than scattering the source
// rows): receive-layout row q takes expert row shuf_inv[q].
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void combine_pack_kernel(Shape sh, Plan p,
                                                                    const v4u* __restrict__ y,
                                                                    v4u* __restrict__ comb_send,
                                                                    uint32_t xrun)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const int n = sh.comb_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    const int64_t qp = rs.row;
    if (qp >= sh.rows)
        return;
    const int64_t r = p.shuf_inv[qp];
    const int64_t q = sh.fixed ? (int64_t)p.slot_of[qp] : qp;
    if ((uint64_t)r >= (uint64_t)sh.rows || (uint64_t)q >= (uint64_t)sh.recv_rows)
        return;
    copy_row<U>(comb_send + q * n + rs.b0, y + r * n + rs.b0, rs.len, lane);
}

// Combine transfer ([EFA] "Dispatch and combine": one write per peer back to
// the token's rank), the reverse of the dispatch transfer, as a gather in
// destination order: send row srow takes receive-layout row xfer_dst[srow].x.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void transfer_back_kernel(Shape sh, Plan p,
                                                                     const v4u* __restrict__ comb_send,
                                                                     v4u* __restrict__ comb_recv,
                                                                     uint32_t xrun)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const int n = sh.comb_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    const int64_t srow = rs.row;
    if (srow >= sh.rows)
        return;
    const int64_t q = p.xfer_dst[srow].x;
    if ((uint64_t)q >= (uint64_t)sh.recv_rows)
        return;
    copy_row<U>(comb_recv + srow * n + rs.b0, comb_send + q * n + rs.b0, rs.len, lane);
}

// Combine with the direct transport: the expert output goes straight back
// into the token owner's return rows (send layout), the inverse of the direct
// pack.  Gather in destination order: send row srow takes expert row
// xfer_dst[srow].y.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void combine_push_kernel(Shape sh, Plan p,
                                                                    const v4u* __restrict__ y,
                                                                    v4u* __restrict__ comb_recv,
                                                                    uint32_t xrun)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const int n = sh.comb_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    const int64_t srow = rs.row;
    if (srow >= sh.rows)
        return;
    const int64_t r = p.xfer_dst[srow].y;
    if ((uint64_t)r >= (uint64_t)sh.rows)
        return;
    copy_row<U>(comb_recv + srow * n + rs.b0, y + r * n + rs.b0, rs.len, lane);
}

// bf16 pattern of an fp32 value, round to nearest even (NaN -> 0x7FC0).
__device__ inline uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline void fma_row8(float (&acc)[8], float w, const v4u& v)
{
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w, __uint_as_float(x[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w, __uint_as_float(x[i] & 0xFFFF0000u), acc[2 * i + 1]);
    }
}

__device__ inline v4u pack_bf16x8(const float (&acc)[8])
{
    v4u o;
    o.x = bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16);
    o.y = bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16);
    o.z = bf16_bits(acc[4]) | (bf16_bits(acc[5]) << 16);
    o.w = bf16_bits(acc[6]) | (bf16_bits(acc[7]) << 16);
    return o;
}

// Combine receive: one wave per token ([EPMC] "Introduction": the weighted
// sum of the K expert outputs; [EPMC] "Combine": computed by the receiver
// into the caller's tensor; accumulation only here, on the receive side --
// [EFA] "Dispatch/combine latency").  fp32, k ascending, one fma chain from +0,
// then bf16 round-to-nearest-even.  With K known at compile time (KT > 0) the
// K*U row loads of a chunk are all issued before the first fma.
template <int KT, int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void combine_reduce_kernel(Shape sh, Plan p,
                                                                      const v4u* __restrict__ comb_recv,
                                                                      const float* __restrict__ w,
                                                                      v4u* __restrict__ out,
                                                                      uint32_t xrun)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const RowSlot rs = row_slot<SPLIT>(sh.comb_vecs, xcd_run_block(xrun));
    const int64_t tok = rs.row;
    if (tok >= (int64_t)sh.N * sh.T)
        return;
    const int K = KT > 0 ? KT : sh.K;
    const int64_t s = tok / sh.T;
    const int64_t TK = (int64_t)sh.T * sh.K;
    int my_p = 0;
    float my_w = 0.0f;
    if (lane < K) {
        my_p = p.pos[tok * K + lane];
        my_w = w[tok * K + lane];
    }
    if (__ballot((unsigned)my_p >= (unsigned)TK) != 0) {
        if (lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    const int n = rs.len;                      // this wave's part of the row
    const int stride = sh.comb_vecs;
    const v4u* rows = comb_recv + s * TK * stride + rs.b0;
    v4u* dst = out + tok * stride + rs.b0;
    for (int base = 0; base < n; base += WAVE * U) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[u][i] = 0.0f;
        if constexpr (KT > 0) {
            v4u v[KT][U];
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                const v4u* row = rows + (int64_t)readlane(my_p, k) * stride;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    v[k][u] = ld_nt(row + min(base + u * WAVE + lane, n - 1));
            }
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                const float wk = readlane_f(my_w, k);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    fma_row8(acc[u], wk, v[k][u]);
            }
        } else {
            for (int k = 0; k < K; ++k) {
                const v4u* row = rows + (int64_t)readlane(my_p, k) * stride;
                const float wk = readlane_f(my_w, k);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    fma_row8(acc[u], wk, ld_nt(row + min(base + u * WAVE + lane, n - 1)));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * WAVE + lane;
            if (j < n)
                st_nt(pack_bf16x8(acc[u]), dst + j);
        }
    }
}

// ---------------------------------------------------------------------------
// Combine with expert-side partial sums ([EFA] "Dispatch/combine latency":
// summing on the send side of combine cuts the bytes moved, at some cost in
// precision).  Reading taken here: the expert owner d sums, for each token
// routed to it, the weighted outputs of that token's experts held by d (fp32
// fma chain, k ascending, from +0), rounds the partial once to bf16 and
// returns one row per (token, rank); the token's owner adds its partials in
// fp32, rank ascending, from +0, and rounds to bf16.  The router weights
// travel with the dispatched rows (pack and transfer carry them).
//
// Row layouts of the P partial rows (P = pbase[N]):
//   owner layout  (rank d, sender s, token t): row qbase[d] + qoff[d][s] + rank
//   token layout  (sender s, rank d, token t): row pbase[s] + ppos
// where ppos is the route plan's position of the token's first item on d.
// ---------------------------------------------------------------------------

// Adds the terms of up to M set bits of `bits` (lowest first) into acc as an
// fp32 fma chain in bit order, and clears them from `bits`.  Lane k of
// my_row / my_w holds the expert row and router weight of item k.  The rows
// are loaded together; the weights are read only after the row loads are
// issued.  `bits` is the same on every lane.
template <int M, int U>
__device__ inline void fma_terms(uint64_t& bits, float (&acc)[U][8], const v4u* src, int my_row,
                                 float my_w, int stride, int base, int n, int lane)
{
    if constexpr (M > 1) {
        if (__popcll(bits) < M) {
            fma_terms<M - 1, U>(bits, acc, src, my_row, my_w, stride, base, n, lane);
            return;
        }
    }
    int f[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        f[j] = __builtin_ctzll(bits);
        bits &= bits - 1;
    }
    v4u v[M][U];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const v4u* row = src + (int64_t)readlane(my_row, f[j]) * stride;
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[j][u] = ld_nt(row + min(base + u * WAVE + lane, n - 1));
    }
#pragma unroll
    for (int j = 0; j < M; ++j)
        hold(v[j]);
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const float wj = readlane_f(my_w, f[j]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            fma_row8(acc[u], wj, v[j][u]);
    }
}

// Terms loaded together per round: 2 rows of 2 vectors per lane keep the
// kernel within 64 VGPRs, 8 waves per SIMD like the movers (most partials
// have one term: a token seldom sends two of its K items to one rank).
constexpr int PARTIAL_TERMS = 2;

// One wave group per partial row, in the order of the layout the expert side
// writes (owner layout (rank, sender, token) when staged, token layout
// (sender, rank, token) when direct): a gather like the movers, so each wave
// stores one row part and reads only the expert rows of its own terms.  The
// partial is the fp32 fma chain over the token's items held by this rank, in
// k order from +0, rounded once to bf16.  The row's record (written by pack)
// holds the expert and receive-plane rows of its first two items, so a
// partial of one or two items (most of them: a token seldom sends more than
// two of its K items to one rank) needs no index load beyond the record; a
// larger one reads its items' rows from the item table (lane k of the mask
// holds item k's).  Iterating the owner layout in direct mode too (so
// consecutive rows read one rank's expert rows) and scattering the stores to
// the token layout was slower: DeepSeek-R1 decode 167 -> 167 us, Kimi-K2 Zipf
// 269 -> 293, all-to-rank-0 221 -> 258.  The grid covers the largest possible
// P; rows past the cycle's P exit.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void partial_send_kernel(Shape sh, Plan p,
                                                                    const v4u* __restrict__ y,
                                                                    const float* __restrict__ recv_w,
                                                                    v4u* __restrict__ dst)
{
    const int lane = lane_id();
    const RowSlot rs = row_slot<SPLIT>(sh.comb_vecs);
    const int64_t j = rs.row;
    // at most one partial row per (token, rank): below the rows phead holds,
    // so the record is read together with the error word and the cycle's P
    // (pinned before the branch, or the compiler sinks its load after it)
    if (j >= (int64_t)sh.N * sh.T * min(sh.K, sh.N))
        return;
    const int err = *p.err;
    const int P = p.pbase[sh.N];
    int4 a = p.phead[2 * j];
    int4 h = p.phead[2 * j + 1];
    asm volatile("" : "+v"(a.x), "+v"(a.y), "+v"(a.z), "+v"(a.w));
    asm volatile("" : "+v"(h.x), "+v"(h.y), "+v"(h.z), "+v"(h.w));
    if (err != 0 || j >= P)
        return;
    const int K = sh.K;
    const uint64_t mask = (uint64_t)(uint32_t)h.z | ((uint64_t)(uint32_t)h.w << 32);
    const uint64_t kmask = K >= 64 ? ~0ull : (1ull << K) - 1;
    const int m = h.y;
    bool bad = (uint64_t)h.x >= (uint64_t)sh.N * sh.T || mask == 0 || (mask & ~kmask) != 0 ||
               m != __popcll(mask) ||
               (uint64_t)a.x >= (uint64_t)sh.rows || (uint64_t)a.y >= (uint64_t)sh.recv_rows ||
               (uint64_t)a.z >= (uint64_t)sh.rows || (uint64_t)a.w >= (uint64_t)sh.recv_rows;
    int my_row = 0, my_q = 0;
    if (m > 2 && !bad && lane < K && ((mask >> lane) & 1)) {
        const int2 it = p.pitem[(int64_t)h.x * K + lane];
        bad = (uint64_t)it.x >= (uint64_t)sh.rows || (uint64_t)it.y >= (uint64_t)sh.recv_rows;
        my_row = it.x;
        my_q = it.y;
    }
    if (__ballot(bad) != 0) {
        if (lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    const int n = rs.len;
    const int stride = sh.comb_vecs;
    const v4u* src = y + rs.b0;
    v4u* o = dst + j * stride + rs.b0;
    if (m <= 2) {
        // the record's values are the same on every lane
        const int r0 = __builtin_amdgcn_readfirstlane(a.x);
        const int r1 = __builtin_amdgcn_readfirstlane(a.z);
        const int q0 = __builtin_amdgcn_readfirstlane(a.y);
        const int q1 = __builtin_amdgcn_readfirstlane(a.w);
        const v4u* row0 = src + (int64_t)r0 * stride;
        const v4u* row1 = src + (int64_t)r1 * stride;
        for (int base = 0; base < n; base += WAVE * U) {
            v4u v0[U], v1[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int jj = min(base + u * WAVE + lane, n - 1);
                v0[u] = ld_nt(row0 + jj);
                if (m == 2)
                    v1[u] = ld_nt(row1 + jj);
            }
            // the weights are loaded once the row loads are issued, before
            // the rows are waited for
            const float w0 = recv_w[q0];
            const float w1 = m == 2 ? recv_w[q1] : 0.0f;
            hold(v0);
            if (m == 2)
                hold(v1);
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[u][e] = 0.0f;
                fma_row8(acc[u], w0, v0[u]);
            }
            if (m == 2) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    fma_row8(acc[u], w1, v1[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int jj = base + u * WAVE + lane;
                if (jj < n)
                    st_nt(pack_bf16x8(acc[u]), o + jj);
            }
        }
        return;
    }
    const float my_w = recv_w[my_q];
    for (int base = 0; base < n; base += WAVE * U) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[u][e] = 0.0f;
        for (uint64_t bits = mask; bits != 0;)
            fma_terms<PARTIAL_TERMS, U>(bits, acc, src, my_row, my_w, stride, base, n, lane);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int jj = base + u * WAVE + lane;
            if (jj < n)
                st_nt(pack_bf16x8(acc[u]), o + jj);
        }
    }
}

// Staged transport: the partial rows go back to the token owners, one
// contiguous segment per (rank -> token owner) pair, as a gather in
// destination order: token-layout row j takes owner-layout row pmap[j].  The
// grid covers the largest possible P; rows past the cycle's P exit.
template <int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void partial_transfer_kernel(Shape sh, Plan p,
                                                                        const v4u* __restrict__ psend,
                                                                        v4u* __restrict__ precv,
                                                                        uint32_t xrun)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const int n = sh.comb_vecs;
    const RowSlot rs = row_slot<SPLIT>(n, xcd_run_block(xrun));
    const int64_t j = rs.row;
    const int P = p.pbase[sh.N];
    if (j >= P)
        return;
    const int64_t o = p.pmap[j];
    if ((uint64_t)o >= (uint64_t)P)
        return;
    copy_row<U>(precv + j * n + rs.b0, psend + o * n + rs.b0, rs.len, lane);
}

__device__ inline void add_row8(float (&acc)[8], const v4u& v)
{
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + __uint_as_float(x[i] << 16);
        acc[2 * i + 1] = acc[2 * i + 1] + __uint_as_float(x[i] & 0xFFFF0000u);
    }
}

// Adds the m partial rows of a token (lane j of term_row holds the row of the
// j-th one) into acc in order j = 0..m-1.  m is the same on every lane of the
// wave; the rows are loaded together, exactly m of them (a token visits
// between 1 and min(K, N) ranks, often far fewer than K).
template <int M, int U>
__device__ inline void sum_partials(int m, float (&acc)[U][8], const v4u* src, int term_row,
                                    int stride, int base, int n, int lane)
{
    if constexpr (M > 1) {
        if (m < M) {
            sum_partials<M - 1, U>(m, acc, src, term_row, stride, base, n, lane);
            return;
        }
    }
    v4u v[M][U];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const v4u* row = src + (int64_t)readlane(term_row, j) * stride;
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[j][u] = ld_nt(row + min(base + u * WAVE + lane, n - 1));
    }
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u)
            add_row8(acc[u], v[j][u]);
}

// The token owner's sum: one wave group per token.  The head lanes (one per
// rank the token visited) are put in rank order, lane j then holds the row of
// the j-th partial; the m <= K rows are added in fp32 from +0, then rounded
// to bf16.
template <int KT, int U, int SPLIT>
__global__ __launch_bounds__(COPY_THREADS) void partial_reduce_kernel(Shape sh, Plan p,
                                                                      const v4u* __restrict__ precv,
                                                                      v4u* __restrict__ out)
{
    if (*p.err)
        return;
    const int lane = lane_id();
    const RowSlot rs = row_slot<SPLIT>(sh.comb_vecs);
    const int64_t tok = rs.row;
    if (tok >= (int64_t)sh.N * sh.T)
        return;
    const int K = KT > 0 ? KT : sh.K;
    const int N = sh.N;
    const int64_t s = tok / sh.T;
    int my_d = 0, my_row = 0;
    bool head = false, bad = false;
    if (lane < K) {
        const int64_t i = tok * K + lane;
        const int pp = p.ppos[i];
        if (pp >= 0) {
            head = true;
            my_d = p.pdst[i];
            my_row = p.pbase[s] + pp;
            bad = (unsigned)my_d >= (unsigned)N || (unsigned)my_row >= (unsigned)p.pbase[N];
        }
    }
    const uint64_t heads = __ballot(head);
    if (__ballot(bad) != 0 || heads == 0) {
        if (lane == 0)
            raise_err(p, ERR_BIT_INTERNAL);
        return;
    }
    // a token's heads have distinct ranks: order = number of heads below
    int order = 0;
    for (uint64_t hm = heads; hm != 0; hm &= hm - 1)
        if (readlane(my_d, __builtin_ctzll(hm)) < my_d)
            ++order;
    int term_row = 0;
    for (uint64_t hm = heads; hm != 0; hm &= hm - 1) {
        const int f = __builtin_ctzll(hm);
        if (lane == readlane(order, f))
            term_row = readlane(my_row, f);
    }
    const int m = __popcll(heads);
    const int n = rs.len;
    const int stride = sh.comb_vecs;
    const v4u* src = precv + rs.b0;
    v4u* dst = out + tok * stride + rs.b0;
    for (int base = 0; base < n; base += WAVE * U) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[u][e] = 0.0f;
        if constexpr (KT > 0) {
            sum_partials<KT, U>(m, acc, src, term_row, stride, base, n, lane);
        } else {
            for (int j = 0; j < m; ++j) {
                const v4u* row = src + (int64_t)readlane(term_row, j) * stride;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    add_row8(acc[u], ld_nt(row + min(base + u * WAVE + lane, n - 1)));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * WAVE + lane;
            if (j < n)
                st_nt(pack_bf16x8(acc[u]), dst + j);
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming probes: what HBM delivers to 16-byte nontemporal streams (a
// measurement aid beside the kernels above, not a step of the method).  Each
// 256-thread block moves one vector per lane, the fastest of 1, 2, 4 and 8
// measured (copy 6.6 TB/s against 6.35 with 4; write 6.8 against 5.95); the
// read probe folds its loads into one word that is stored only for a value
// the data never holds, so the loads cannot be dropped.
// ---------------------------------------------------------------------------
constexpr int PROBE_U = 1;
constexpr int PROBE_NT = 256;

__global__ __launch_bounds__(PROBE_NT) void probe_copy_kernel(const v4u* __restrict__ src,
                                                              v4u* __restrict__ dst, int64_t nv)
{
    const int64_t base = (int64_t)blockIdx.x * PROBE_U * PROBE_NT + threadIdx.x;
    v4u v[PROBE_U];
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u) {
        const int64_t j = base + (int64_t)u * PROBE_NT;
        v[u] = ld_nt(src + (j < nv ? j : nv - 1));
    }
    hold(v);
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u) {
        const int64_t j = base + (int64_t)u * PROBE_NT;
        if (j < nv)
            st_nt(v[u], dst + j);
    }
}

__global__ __launch_bounds__(PROBE_NT) void probe_read_kernel(const v4u* __restrict__ src,
                                                              uint32_t* __restrict__ word, int64_t nv)
{
    const int64_t base = (int64_t)blockIdx.x * PROBE_U * PROBE_NT + threadIdx.x;
    v4u v[PROBE_U];
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u) {
        const int64_t j = base + (int64_t)u * PROBE_NT;
        v[u] = ld_nt(src + (j < nv ? j : nv - 1));
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u)
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (acc == 0x9E3779B9u)
        word[0] = acc;
}

__global__ __launch_bounds__(PROBE_NT) void probe_write_kernel(v4u* __restrict__ dst, int64_t nv)
{
    const int64_t base = (int64_t)blockIdx.x * PROBE_U * PROBE_NT + threadIdx.x;
    const v4u v = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, (uint32_t)blockIdx.x};
#pragma unroll
    for (int u = 0; u < PROBE_U; ++u) {
        const int64_t j = base + (int64_t)u * PROBE_NT;
        if (j < nv)
            st_nt(v, dst + j);
    }
}

// Debug poisoning: 16-byte stores over the vector part, then the 4-byte tail.
constexpr int FILL_NT = 256;

__global__ __launch_bounds__(FILL_NT) void fill_kernel(v4u* __restrict__ p, int64_t nvec,
                                                      uint32_t* __restrict__ tail, int ntail,
                                                      uint32_t pattern)
{
    const v4u v = {pattern, pattern, pattern, pattern};
    const int64_t stride = (int64_t)gridDim.x * FILL_NT;
    for (int64_t i = (int64_t)blockIdx.x * FILL_NT + threadIdx.x; i < nvec; i += stride)
        p[i] = v;
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail)
        tail[threadIdx.x] = pattern;
}

// Launch shape of a row kernel: waves per row (SPLIT) and 16-byte vectors
// per lane per round (U), from the number of vectors in a row.
struct RowShape {
    int u, split;
};

inline RowShape row_shape(int n)
{
    // measured against 4 vectors per lane over up to 4 waves: DeepSeek-R1
    // decode step 820 -> 802 us (14 KiB rows, 8 waves of 2), fp8 prefill
    // 21.4 -> 20.6 ms (7 KiB payload rows, 4 waves of 2); 16 waves of 1 lost
    // 8%
    const int per_lane = (n + WAVE - 1) / WAVE;
    if (per_lane <= 1) return {1, 1};
    if (per_lane <= 2) return {2, 1};
    if (per_lane <= 4) return {2, 2};
    if (per_lane <= 8) return {2, 4};
    if (per_lane <= 16) return {2, 8};
    if (per_lane <= 32) return {4, 8};
    return {16, 4};
}

inline unsigned row_blocks(int64_t rows, int split)
{
    const int64_t b = (rows * split + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    return (unsigned)(b > 0 ? b : 1);
}

#define MOE_DISPATCH_ROW(rsh, KERNEL, GRID_ROWS, ...)                                              \
    MOE_DISPATCH_ROW_BLOCKS(rsh, KERNEL, row_blocks((GRID_ROWS), (rsh).split), __VA_ARGS__)

#define MOE_DISPATCH_ROW_BLOCKS(rsh, KERNEL, GRID_BLOCKS, ...)                                     \
    MOE_DISPATCH_ROW_BLOCKS_LDS(rsh, KERNEL, GRID_BLOCKS, 0, __VA_ARGS__)

#define MOE_DISPATCH_ROW_BLOCKS_LDS(rsh, KERNEL, GRID_BLOCKS, LDS, ...)                            \
    do {                                                                                           \
        const dim3 grid_(GRID_BLOCKS), block_(COPY_THREADS);                                       \
        const size_t lds_ = (LDS);                                                                 \
        if ((rsh).split == 1 && (rsh).u == 1)                                                      \
            go((KERNEL<1, 1>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else if ((rsh).split == 1)                                                                 \
            go((KERNEL<2, 1>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else if ((rsh).split == 2)                                                                 \
            go((KERNEL<2, 2>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else if ((rsh).split == 4 && (rsh).u == 2)                                                 \
            go((KERNEL<2, 4>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else if ((rsh).split == 4 && (rsh).u == 4)                                                 \
            go((KERNEL<4, 4>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else if ((rsh).split == 4)                                                                 \
            go((KERNEL<16, 4>), grid_, block_, lds_, __VA_ARGS__);                                 \
        else if ((rsh).u == 2)                                                                     \
            go((KERNEL<2, 8>), grid_, block_, lds_, __VA_ARGS__);                                  \
        else                                                                                       \
            go((KERNEL<4, 8>), grid_, block_, lds_, __VA_ARGS__);                                  \
    } while (0)

// The group offsets are formed from an LDS copy of the send offsets
// soff[N][E+1] when it fits (receiver-side combine; the partial combine's
// walks also need the counts and the partial offsets).
inline size_t table_lds_bytes(const Shape& sh)
{
    int64_t n = round4(sh.N * (sh.E + 1));
    if (sh.partial)
        n += round4(sh.N * sh.E) + (int64_t)sh.N * (sh.N + 1);
    return (size_t)n * sizeof(int32_t);
}

inline int table_in_lds(const Shape& sh)
{
    const int64_t per = std::max<int64_t>((int64_t)sh.N * (sh.E + 1),
                                          sh.partial ? std::max<int64_t>((int64_t)sh.N * sh.E,
                                                                         (int64_t)sh.N * (sh.N + 1))
                                                     : 0);
    return per <= TAB_MAX_INTS && table_lds_bytes(sh) <= 48 * 1024;
}


}  // namespace

hipError_t launch_route_plan(const Shape& sh, const int32_t* idx, const Plan& p, const Rows& r,
                             const Launch& L)
{
    RouteArgs ra;
    ra.idx = idx;
    ra.send_meta = !pack_in_row_order(sh) ? nullptr : sh.direct ? p.send_item : r.send_meta;
    ra.N = sh.N;
    ra.T = sh.T;
    ra.K = sh.K;
    ra.E = sh.E;
    ra.L = sh.L;
    ra.partial = sh.partial;
    ra.slot_cap = sh.fixed ? sh.slots : -1;
    ra.cap = (int64_t)sh.N * sh.T * (sh.K > sh.L ? sh.K : sh.L);
    // keys: E experts, plus N ranks for the partial combine.  Two buffers of
    // lane masks take 16 bytes per (wave, key) and the cursors 8 bytes per
    // key: (16*CW + 8)*NK bytes, kept within 64 KiB: 8 waves up to 481 keys,
    // 4 up to 910, 2 up to 1638, 1 above
    const int nk = sh.E + (sh.partial ? sh.N : 0);
    ra.chunk_waves = nk <= 481 ? RP_WAVES : nk <= 910 ? RP_WAVES / 2 : nk <= 1638 ? RP_WAVES / 4
                                                                                   : RP_WAVES / 8;
    size_t lds = 2 * (size_t)ra.chunk_waves * nk * sizeof(uint64_t) +
                 (size_t)2 * nk * sizeof(int32_t);
    ra.table_lds = table_in_lds(sh);
    if (ra.table_lds)
        lds = std::max(lds, table_lds_bytes(sh));
    const int chunks = (sh.T * sh.K + ra.chunk_waves * WAVE - 1) / (ra.chunk_waves * WAVE);
    const dim3 grid(sh.N), block(RP_NT);
#define MOE_ROUTE_PLAN(HC)                                                                         \
    (sh.partial ? (sh.plan_offsets ? go(route_plan_kernel<HC, true, true>, grid, block, lds, L, ra, p)  \
                                   : go(route_plan_kernel<HC, true, false>, grid, block, lds, L, ra, p)) \
                : (sh.plan_offsets ? go(route_plan_kernel<HC, false, true>, grid, block, lds, L, ra, p) \
                                   : go(route_plan_kernel<HC, false, false>, grid, block, lds, L, ra, p)))
    if (chunks <= 1)
        MOE_ROUTE_PLAN(1);
    else if (chunks <= 2)
        MOE_ROUTE_PLAN(2);
    else if (chunks <= 4)
        MOE_ROUTE_PLAN(4);
    else if (chunks <= 8)
        MOE_ROUTE_PLAN(8);
    else
        MOE_ROUTE_PLAN(HELD_CHUNKS);
#undef MOE_ROUTE_PLAN
    return hipGetLastError();
}


hipError_t launch_recv_map(const Shape& sh, const Plan& p, const Launch& L)
{
    const int64_t pairs = (int64_t)sh.E * sh.N;
    go(recv_map_kernel, dim3(row_blocks(pairs, 1)), dim3(COPY_THREADS), 0, L, sh, p);
    return hipGetLastError();
}

// Grids below this many blocks keep round-robin placement: they are resident
// at once, so there is no later block to keep in the same pages (Mixtral
// decode, 2048 blocks: 61.2 -> 63.0 us with runs in the transfers).
constexpr int64_t XCD_RUN_MIN_BLOCKS = 8192;

// Fixed XCD runs for the shuffle, the combine pack and the direct combine
// push (RUN_ROWS_BLOCKS: 128 blocks move about 1 MiB of destination rows) and
// for the combine reduce (RUN_TOKEN_BLOCKS), measured per kernel on
// DeepSeek-R1 decode, Kimi-K2 Zipf decode and the fp8 prefill against runs of
// 1 to 512 blocks: shuffle 149 -> 144, 310 -> 292, 2578 -> 2430 us; combine
// pack 147 -> 146, 302 -> 297, 4993 -> 4769 us; combine push 156 -> 150,
// 308 -> 304, 5036 -> 4750 us; combine reduce flat on the decode shapes,
// 2923 -> 2836 us on the prefill; runs of 256 and more lost up to 10% on the
// decode shapes.  The bf16 pack and partial send gained nothing from runs
// (partial send lost 3-6%); the partial reduce gained on the prefill and lost
// on the all-to-rank-0 decode, and keeps plain order; the partial transfer
// takes segment runs where segments are long (launch_partial_transfer).
constexpr uint32_t RUN_ROWS_BLOCKS = 128;
constexpr uint32_t RUN_TOKEN_BLOCKS = 32;
// The fp8 pack: runs of 256 blocks (256 tokens of one sender per run) on the
// prefill 1859-1868 -> 1821-1823 us; 64 and 1024 gained less.
constexpr uint32_t RUN_FP8_PACK_BLOCKS = 256;
constexpr int64_t PARTIAL_RUN_MIN_BLOCKS = 64;

inline uint32_t fixed_run(int64_t blocks, uint32_t run)
{
    return blocks < XCD_RUN_MIN_BLOCKS ? 1u : run;
}

// The send-row-order pack takes runs of one sender's rows (T*K rows), so an
// XCD reads one sender's tokens at a time: 86.9 -> 74.5 us on DeepSeek-R1
// decode, where runs of 128 blocks (107 us) and plain order (92.5 us) were
// slower.
inline uint32_t sender_run(const Shape& sh, const RowShape& rsh)
{
    if ((int64_t)row_blocks(sh.rows, rsh.split) < XCD_RUN_MIN_BLOCKS)
        return 1;
    const int64_t run = row_blocks((int64_t)sh.T * sh.K, rsh.split);
    return (uint32_t)std::min<int64_t>(run, (int64_t)1 << 24);
}

hipError_t launch_pack(const Shape& sh, const void* x, const int32_t* idx, const float* w,
                       const Plan& p, const Rows& r, const Launch& L)
{
    float* dst_w = sh.partial ? (sh.direct ? r.recv_w : r.send_w) : nullptr;
    const int64_t tokens = (int64_t)sh.N * sh.T;
    if (tokens == 0)
        return hipSuccess;
    if (pack_in_row_order(sh)) {
        const int32_t* item = sh.direct ? p.send_item : r.send_meta;
        v4u* dx = (v4u*)(sh.direct ? r.recv_x : r.send_x);
        int32_t* dmeta = sh.direct ? r.recv_meta : nullptr;
        // the partial combine's token records: blocks of one sender each,
        // ahead of the row blocks (so that their latency overlaps the rows),
        // padded to a multiple of 8 blocks (the row blocks keep their XCDs)
        unsigned tblocks = 0;
        size_t lds = 0;
        if (sh.partial) {
            const int per_block = rec_tokens_per_block(sh);
            const int64_t nb = (int64_t)sh.N * ((sh.T + per_block - 1) / per_block);
            tblocks = (unsigned)((nb + XCDS - 1) / XCDS * XCDS);
            lds = (size_t)rec_lds_ints(sh) * sizeof(int32_t);
        }
        if (sh.fp8) {
            RowShape rsh = row_shape(sh.H / 16);
            if (rsh.u > 4)
                rsh.u = 4;
            const unsigned rb = row_blocks(sh.rows, rsh.split);
            float* dscale = sh.direct ? r.recv_scale : r.send_scale;
            if (sh.partial)
                MOE_DISPATCH_ROW_BLOCKS_LDS(rsh, pack_rows_rec_fp8_kernel, rb + tblocks, lds, L, sh,
                                            p, (const v4u*)x, idx, item, dx, dscale, dmeta, w,
                                            dst_w, sender_run(sh, rsh), tblocks);
            else
                MOE_DISPATCH_ROW_BLOCKS(rsh, pack_rows_fp8_kernel, rb, L, sh, p, (const v4u*)x,
                                        idx, item, dx, dscale, dmeta, w, dst_w,
                                        sender_run(sh, rsh), 0u);
        } else if (sh.payload_vecs == 7 * 2 * WAVE) {
            // hidden 7168: seven waves of exactly 2 vectors per lane instead of
            // eight with an eighth of the lanes idle in the second round.
            // DeepSeek-R1 decode pack, warm / MALL-flushed: direct 84-92 ->
            // 79-86 / 111 -> 106 us, staged 75-78 -> 74-75 / 99 -> 99 us;
            // the other movers lost 1-3 us with the same split, the combine
            // and partial reduces 1-2 us
            const RowShape rsh{2, 7};
            const unsigned rb = row_blocks(sh.rows, rsh.split);
            if (sh.partial)
                go((pack_rows_rec_bf16_kernel<2, 7>), dim3(rb + tblocks), dim3(COPY_THREADS), lds,
                   L, sh, p, (const v4u*)x, idx, item, dx, dmeta, w, dst_w, sender_run(sh, rsh),
                   tblocks);
            else
                go((pack_rows_bf16_kernel<2, 7>), dim3(rb), dim3(COPY_THREADS), 0, L, sh, p,
                   (const v4u*)x, idx, item, dx, dmeta, w, dst_w, sender_run(sh, rsh), 0u);
        } else {
            const RowShape rsh = row_shape(sh.payload_vecs);
            const unsigned rb = row_blocks(sh.rows, rsh.split);
            if (sh.partial)
                MOE_DISPATCH_ROW_BLOCKS_LDS(rsh, pack_rows_rec_bf16_kernel, rb + tblocks, lds, L,
                                            sh, p, (const v4u*)x, idx, item, dx, dmeta, w, dst_w,
                                            sender_run(sh, rsh), tblocks);
            else
                MOE_DISPATCH_ROW_BLOCKS(rsh, pack_rows_bf16_kernel, rb, L, sh, p, (const v4u*)x,
                                        idx, item, dx, dmeta, w, dst_w, sender_run(sh, rsh), 0u);
        }
        return hipGetLastError();
    }
    if (sh.fp8) {
        // a row is H/16 groups of 16 elements (16 codes out per lane); each
        // lane holds two input vectors per group, so at most 4 groups per
        // lane per round.  A DeepSeek-shaped row takes 4 waves of 112 groups;
        // 2 or 8 waves, or 4 groups per lane, were equal or up to 6% slower
        // on the fp8 prefill
        RowShape rsh = row_shape(sh.H / 16);
        if (rsh.u > 4)
            rsh.u = 4;
        MOE_DISPATCH_ROW(rsh, pack_fp8_kernel, tokens, L, sh, p, (const v4u*)x, idx, w,
                         (v4u*)(sh.direct ? r.recv_x : r.send_x),
                         sh.direct ? r.recv_scale : r.send_scale,
                         sh.direct ? r.recv_meta : r.send_meta, dst_w,
                         fixed_run(row_blocks(tokens, rsh.split), RUN_FP8_PACK_BLOCKS));
    } else {
        MOE_DISPATCH_ROW(row_shape(sh.payload_vecs), pack_bf16_kernel, tokens, L, sh, p,
                         (const v4u*)x, idx, w, (v4u*)(sh.direct ? r.recv_x : r.send_x),
                         sh.direct ? r.recv_meta : r.send_meta, dst_w);
    }
    return hipGetLastError();
}

// Blocks of an average (sender -> receiver) segment, R / N^2 rows: the
// transfers' XCD runs.
inline uint32_t segment_blocks(const Shape& sh, const RowShape& rsh)
{
    if ((int64_t)row_blocks(sh.rows, rsh.split) < XCD_RUN_MIN_BLOCKS)
        return 1;
    const int64_t seg_rows = std::max<int64_t>(1, sh.rows / ((int64_t)sh.N * sh.N));
    const int64_t run = (seg_rows * rsh.split + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    return (uint32_t)std::min<int64_t>(std::max<int64_t>(run, 1), (int64_t)1 << 24);
}

hipError_t launch_transfer(const Shape& sh, const Plan& p, const Rows& r, const Launch& L)
{
    if (sh.rows == 0)
        return hipSuccess;
    const RowShape rsh = row_shape(sh.payload_vecs);
    MOE_DISPATCH_ROW(rsh, transfer_kernel, sh.rows, L, sh, p, (const v4u*)r.send_x,
                     (v4u*)r.recv_x, r.send_scale, r.recv_scale, r.send_meta, r.recv_meta,
                     sh.partial ? r.send_w : nullptr, r.recv_w, segment_blocks(sh, rsh));
    return hipGetLastError();
}

hipError_t launch_shuffle(const Shape& sh, const Plan& p, const Rows& r, void* expert_x,
                          float* expert_scale, int32_t* expert_offsets, const Launch& L)
{
    // launched even with no rows: block 0 publishes the expert offsets
    const RowShape rsh = row_shape(sh.payload_vecs);
    MOE_DISPATCH_ROW(rsh, shuffle_kernel, sh.rows, L, sh, p, (const v4u*)r.recv_x, r.recv_scale,
                     r.recv_meta, (v4u*)expert_x, expert_scale, r.src_rank, r.src_slot,
                     expert_offsets, fixed_run(row_blocks(sh.rows, rsh.split), RUN_ROWS_BLOCKS));
    return hipGetLastError();
}

hipError_t launch_combine_pack(const Shape& sh, const Plan& p, const Rows& r, const void* y,
                               const Launch& L)
{
    if (sh.rows == 0)
        return hipSuccess;
    const RowShape rsh = row_shape(sh.comb_vecs);
    MOE_DISPATCH_ROW(rsh, combine_pack_kernel, sh.rows, L, sh, p, (const v4u*)y,
                     (v4u*)r.comb_send,
                     fixed_run(row_blocks(sh.rows, rsh.split), RUN_ROWS_BLOCKS));
    return hipGetLastError();
}

hipError_t launch_transfer_back(const Shape& sh, const Plan& p, const Rows& r, const Launch& L)
{
    if (sh.rows == 0)
        return hipSuccess;
    const RowShape rsh = row_shape(sh.comb_vecs);
    MOE_DISPATCH_ROW(rsh, transfer_back_kernel, sh.rows, L, sh, p, (const v4u*)r.comb_send,
                     (v4u*)r.comb_recv, segment_blocks(sh, rsh));
    return hipGetLastError();
}

hipError_t launch_combine_push(const Shape& sh, const Plan& p, const Rows& r, const void* y,
                               const Launch& L)
{
    if (sh.rows == 0)
        return hipSuccess;
    const RowShape rsh = row_shape(sh.comb_vecs);
    MOE_DISPATCH_ROW(rsh, combine_push_kernel, sh.rows, L, sh, p, (const v4u*)y,
                     (v4u*)r.comb_recv,
                     fixed_run(row_blocks(sh.rows, rsh.split), RUN_ROWS_BLOCKS));
    return hipGetLastError();
}

// Token kernels (one wave group per token, all K rows in flight) are
// compiled for the common K (1, 2, 4, 6, 8) and for any other K, with UK
// vectors per lane per row; rows are split across waves as for the movers.
#define MOE_TOKEN_SPLIT(KERNEL, KT, U, split, grid, block, L, ...)                                  \
    do {                                                                                           \
        if ((split) == 1)                                                                          \
            go((KERNEL<KT, U, 1>), grid, block, 0, L, __VA_ARGS__);                                \
        else if ((split) == 2)                                                                     \
            go((KERNEL<KT, U, 2>), grid, block, 0, L, __VA_ARGS__);                                \
        else if ((split) == 4)                                                                     \
            go((KERNEL<KT, U, 4>), grid, block, 0, L, __VA_ARGS__);                                \
        else                                                                                       \
            go((KERNEL<KT, U, 8>), grid, block, 0, L, __VA_ARGS__);                                \
    } while (0)

// The token kernels (combine reduce, partial reduce) hold all K rows' vectors
// of a token at once: with the movers' split and 2 vectors per lane per row,
// K = 8 rows take 64 VGPRs of data (94 in all, 5 waves per SIMD); at 4
// vectors per lane over 4 waves such kernels took 160-180 VGPRs and ran at 2
// (an earlier per-token partial send: 172 -> 165 us on DeepSeek-R1 decode);
// at 1 vector per lane (56 VGPRs, 8 waves per SIMD, two rounds a wave) the
// combine reduce took 91.8 us against 87.0 (Kimi-K2 decode 183.6 against 172.4).
#define MOE_DISPATCH_TOKEN(sh, KERNEL, UK, tokens, L, ...)                                         \
    do {                                                                                           \
        const int split_ = row_shape((sh).comb_vecs).split;                                        \
        const dim3 grid_(row_blocks((tokens), split_)), block_(COPY_THREADS);                      \
        switch ((sh).K) {                                                                          \
        case 1: MOE_TOKEN_SPLIT(KERNEL, 1, UK, split_, grid_, block_, L, __VA_ARGS__); break;      \
        case 2: MOE_TOKEN_SPLIT(KERNEL, 2, UK, split_, grid_, block_, L, __VA_ARGS__); break;      \
        case 4: MOE_TOKEN_SPLIT(KERNEL, 4, UK, split_, grid_, block_, L, __VA_ARGS__); break;      \
        case 6: MOE_TOKEN_SPLIT(KERNEL, 6, UK, split_, grid_, block_, L, __VA_ARGS__); break;      \
        case 8: MOE_TOKEN_SPLIT(KERNEL, 8, UK, split_, grid_, block_, L, __VA_ARGS__); break;      \
        default: MOE_TOKEN_SPLIT(KERNEL, 0, UK, split_, grid_, block_, L, __VA_ARGS__); break;     \
        }                                                                                          \
    } while (0)

hipError_t launch_combine_reduce(const Shape& sh, const Plan& p, const Rows& r, const float* w,
                                 void* out, const Launch& L)
{
    const int64_t tokens = (int64_t)sh.N * sh.T;
    if (tokens == 0)
        return hipSuccess;
    const uint32_t run =
        fixed_run(row_blocks(tokens, row_shape(sh.comb_vecs).split), RUN_TOKEN_BLOCKS);
    MOE_DISPATCH_TOKEN(sh, combine_reduce_kernel, 2, tokens, L, sh, p, (const v4u*)r.comb_recv, w,
                       (v4u*)out, run);
    return hipGetLastError();
}

hipError_t launch_partial_send(const Shape& sh, const Plan& p, const Rows& r, const void* y,
                               const Launch& L)
{
    // at most one partial row per (token, rank), and at most K ranks per token
    const int64_t p_max = (int64_t)sh.N * sh.T * (sh.K < sh.N ? sh.K : sh.N);
    if (p_max == 0)
        return hipSuccess;
    // 2 vectors per lane per row and round whatever the row length (a round
    // holds up to PARTIAL_TERMS rows and an fp32 accumulator); the movers' split
    const int split = row_shape(sh.comb_vecs).split;
    const dim3 grid(row_blocks(p_max, split)), block(COPY_THREADS);
    const v4u* ysrc = (const v4u*)y;
    v4u* dst = (v4u*)(sh.direct ? r.comb_recv : r.comb_send);
    if (split == 1)
        go(partial_send_kernel<2, 1>, grid, block, 0, L, sh, p, ysrc, r.recv_w, dst);
    else if (split == 2)
        go(partial_send_kernel<2, 2>, grid, block, 0, L, sh, p, ysrc, r.recv_w, dst);
    else if (split == 4)
        go(partial_send_kernel<2, 4>, grid, block, 0, L, sh, p, ysrc, r.recv_w, dst);
    else
        go(partial_send_kernel<2, 8>, grid, block, 0, L, sh, p, ysrc, r.recv_w, dst);
    return hipGetLastError();
}

hipError_t launch_partial_transfer(const Shape& sh, const Plan& p, const Rows& r, const Launch& L)
{
    // at most one partial row per (token, rank), and at most K ranks per token
    const int64_t p_max = (int64_t)sh.N * sh.T * (sh.K < sh.N ? sh.K : sh.N);
    if (p_max == 0)
        return hipSuccess;
    // XCD runs of one (rank -> token owner) segment of the largest P, only
    // where a segment spans PARTIAL_RUN_MIN_BLOCKS blocks: runs of 64 blocks
    // on DeepSeek-R1 decode 139 -> 134 us, of 512 on the fp8 prefill
    // 5033 -> 4642 us; on the Kimi-K2 decode shapes (32-block segments, the
    // partial rows piled on few ranks) runs of 32 lost 2-6%
    const RowShape rsh = row_shape(sh.comb_vecs);
    const int64_t seg_rows = std::max<int64_t>(1, p_max / ((int64_t)sh.N * sh.N));
    const int64_t seg = (seg_rows * rsh.split + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    const uint32_t run = seg >= PARTIAL_RUN_MIN_BLOCKS
                             ? fixed_run(row_blocks(p_max, rsh.split),
                                         (uint32_t)std::min<int64_t>(seg, (int64_t)1 << 24))
                             : 1u;
    MOE_DISPATCH_ROW(rsh, partial_transfer_kernel, p_max, L, sh, p, (const v4u*)r.comb_send,
                     (v4u*)r.comb_recv, run);
    return hipGetLastError();
}

hipError_t launch_partial_reduce(const Shape& sh, const Plan& p, const Rows& r, void* out,
                                 const Launch& L)
{
    const int64_t tokens = (int64_t)sh.N * sh.T;
    if (tokens == 0)
        return hipSuccess;
    MOE_DISPATCH_TOKEN(sh, partial_reduce_kernel, 2, tokens, L, sh, p, (const v4u*)r.comb_recv,
                       (v4u*)out);
    return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream)
{
    if (bytes < 4)
        return hipSuccess;
    const int64_t nvec = (int64_t)(bytes / 16);
    const int ntail = (int)((bytes % 16) / 4);
    const int64_t blocks = std::min<int64_t>(std::max<int64_t>((nvec + FILL_NT - 1) / FILL_NT, 1),
                                             (int64_t)1 << 16);
    const Launch L{stream, nullptr, nullptr};
    go(fill_kernel, dim3((unsigned)blocks), dim3(FILL_NT), 0, L, (v4u*)p, nvec,
       (uint32_t*)((uint8_t*)p + nvec * 16), ntail, pattern);
    return hipGetLastError();
}

hipError_t launch_hbm_probe(int kind, void* dst, const void* src, int64_t vecs, hipStream_t stream)
{
    const int64_t per_block = (int64_t)PROBE_U * PROBE_NT;
    const dim3 grid((unsigned)((vecs + per_block - 1) / per_block)), block(PROBE_NT);
    const Launch L{stream, nullptr, nullptr};
    if (kind == 0)
        go(probe_copy_kernel, grid, block, 0, L, (const v4u*)src, (v4u*)dst, vecs);
    else if (kind == 1)
        go(probe_read_kernel, grid, block, 0, L, (const v4u*)src, (uint32_t*)dst, vecs);
    else
        go(probe_write_kernel, grid, block, 0, L, (v4u*)dst, vecs);
    return hipGetLastError();
}

}  // namespace moe
