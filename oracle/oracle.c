/*
 * CPU oracle for the MoE dispatch/combine path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library) never calls it, includes it or shares code with it.
 *
 * It is the plain definition of each step, written as scalar loops in the
 * order the pages describe, with its own bf16 and fp8-e4m3 codecs.  It is
 * built with gcc -O2 -ffp-contract=off, so no multiply-add is fused unless
 * fmaf() is written out.
 *
 * Pages cited:
 *   [EPMC] "Efficient and portable Mixture-of-Experts communication"
 *   [EFA]  "Enabling trillion-parameter models on AWS EFA"
 *
 * Notation: N logical ranks, T tokens per rank, K experts per token, E experts,
 * L = E/N experts per rank (expert e lives on rank e / L), H hidden elements.
 * idx[s][t][k] is the k-th expert of token t on rank s.  Row arrays are flat:
 * the send rows of sender s are rows [s*T*K, (s+1)*T*K); the receive rows of
 * receiver d are rows [G[d], G[d+1]) of one pooled array.
 *
 * Error behaviour: functions that validate their input return 0 on success and
 * a negative value if an expert id is outside [0, E); they never abort.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* bf16 -> fp32: a bf16 value is the top 16 bits of the fp32 value. */
float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Value of a bf16 pattern as a double, with the all-ones exponent read as
 * 2^128 (the value it would have with an unbounded exponent), so that rounding
 * up past the largest finite bf16 picks infinity exactly when IEEE does. */
static double bf16_mag_value(uint32_t mag16)
{
    if (mag16 == 0x7F80u)
        return ldexp(1.0, 128);
    return (double)orc_bf16_to_f32((uint16_t)mag16);
}

/* fp32 -> bf16, round to nearest, ties to even: pick the nearer of the two
 * bf16 neighbours of |f| (the truncation and the next pattern up); on a tie
 * take the one whose last mantissa bit is 0. */
uint16_t orc_f32_to_bf16(float f)
{
    if (isnan(f))
        return 0x7FC0u;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag >= 0x7F800000u)                /* infinity stays infinity */
        return (uint16_t)((sign | mag) >> 16);
    uint32_t lo = mag >> 16, hi = lo + 1;
    double a = fabs((double)f);
    double dlo = a - bf16_mag_value(lo);
    double dhi = bf16_mag_value(hi) - a;
    uint32_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1u) ? hi : lo;
    return (uint16_t)((sign >> 16) | pick);
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits (bias
 * 7), 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the pattern
 * S.1111.111 is NaN; there is no infinity; largest finite value 448. */
double orc_e4m3_value(uint8_t code)
{
    int sign = code >> 7, ex = (code >> 3) & 15, m = code & 7;
    double v;
    if (ex == 15 && m == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, ex - 7);
    return sign ? -v : v;
}

/* fp32 -> e4m3, round to nearest with ties to even, saturating: |v| >= 448
 * (infinity included) gives +-448; NaN gives the NaN pattern.  The nearest
 * finite code is found by bisection over the increasing positive code values;
 * a tie between two adjacent codes goes to the even code (mantissa bit 0).
 * The sign bit is copied, so values that round to zero keep their sign. */
uint8_t orc_f32_to_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* largest code c in [0, 0x7E] with value(c) <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (orc_e4m3_value((uint8_t)c) != a) {
        double dlo = a - orc_e4m3_value((uint8_t)c);
        double dhi = orc_e4m3_value((uint8_t)(c + 1)) - a;
        if (dhi < dlo || (dhi == dlo && ((c + 1) & 1) == 0))
            c = c + 1;
    }
    return (uint8_t)(sign | c);
}

/* ------------------------------------------------ dispatch: count and offsets */

/* Per-expert token counts of every sender ([EFA] "Dispatch and combine": the
 * dispatch-send kernel first aggregates the routing information into token
 * counts per expert).  cnt[s][e] = #{(t,k) : idx[s][t][k] == e}. */
int orc_route_count(int N, int T, int K, int E, const int32_t* idx, int32_t* cnt)
{
    int bad = 0;
    memset(cnt, 0, sizeof(int32_t) * (size_t)N * E);
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                int e = idx[((size_t)s * T + t) * K + k];
                if (e < 0 || e >= E) {
                    bad = 1;
                    continue;
                }
                cnt[(size_t)s * E + e] += 1;
            }
    return bad ? -1 : 0;
}

/* Offsets inside each sender's contiguous send buffer ([EFA] "Dispatch and
 * combine": the cumulative sum of the token counts gives the offsets at which
 * tokens are packed into contiguous per-peer send buffers).
 * soff[s][e] = sum_{e' < e} cnt[s][e'], soff[s][E] = T*K. */
void orc_send_offsets(int N, int E, const int32_t* cnt, int32_t* soff)
{
    for (int s = 0; s < N; ++s) {
        int32_t run = 0;
        for (int e = 0; e < E; ++e) {
            soff[(size_t)s * (E + 1) + e] = run;
            run += cnt[(size_t)s * E + e];
        }
        soff[(size_t)s * (E + 1) + E] = run;
    }
}

/* Position of each (t,k) in its sender's buffer: rows grouped by expert, and
 * within one expert in (t,k) order -- a stable counting sort.  The pages leave
 * the order inside an expert free (the receive order is not deterministic,
 * [EPMC] "Dispatch"); a fixed order makes every byte checkable. */
void orc_positions(int N, int T, int K, int E, const int32_t* idx,
                   const int32_t* soff, int32_t* pos)
{
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int s = 0; s < N; ++s) {
        for (int e = 0; e < E; ++e)
            cursor[e] = soff[(size_t)s * (E + 1) + e];
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                size_t i = ((size_t)s * T + t) * K + k;
                pos[i] = cursor[idx[i]]++;
            }
    }
    free(cursor);
}

/* Receive-side offsets ([EFA] "Send and receive buffers": after the per-expert
 * counts are exchanged, every rank knows where to write and from which offsets
 * it receives).  scnt(s,d) = rows sender s sends to rank d = soff[s][(d+1)L] -
 * soff[s][dL].  roff[d][s] = sum_{s' < s} scnt(s',d), roff[d][N] = rows d
 * receives; G[d] = sum_{d' < d} roff[d'][N] is rank d's base in the pooled
 * receive array, G[N] = N*T*K. */
void orc_recv_offsets(int N, int E, const int32_t* soff, int32_t* roff, int32_t* G)
{
    int L = E / N;
    for (int d = 0; d < N; ++d) {
        int32_t run = 0;
        for (int s = 0; s < N; ++s) {
            roff[(size_t)d * (N + 1) + s] = run;
            run += soff[(size_t)s * (E + 1) + (d + 1) * L] - soff[(size_t)s * (E + 1) + d * L];
        }
        roff[(size_t)d * (N + 1) + N] = run;
    }
    int32_t run = 0;
    for (int d = 0; d < N; ++d) {
        G[d] = run;
        run += roff[(size_t)d * (N + 1) + N];
    }
    G[N] = run;
}

/* First row of every expert in the expert-contiguous grouped-GEMM input
 * ([EPMC] "Dispatch": received tokens are laid out contiguously for the
 * grouped GEMM).  eoff[e] = sum_{e' < e} sum_s cnt[s][e'], eoff[E] = N*T*K. */
void orc_expert_offsets(int N, int E, const int32_t* cnt, int32_t* eoff)
{
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
        eoff[e] = run;
        for (int s = 0; s < N; ++s)
            run += cnt[(size_t)s * E + e];
    }
    eoff[E] = run;
}

/* --------------------------------------------------------------- dispatch: pack */

/* Pack, bf16 payload ([EPMC] "Dispatch": activations and the token's index on
 * the sending rank are packed into one contiguous chunk; [EFA] "Dispatch and
 * combine": packed into contiguous per-peer send buffers).  Row pos[s][t][k] of
 * sender s receives token t unchanged; its meta word is t*K+k. */
void orc_pack_bf16(int N, int T, int K, int H, const uint16_t* x, const int32_t* pos,
                   uint16_t* send_x, int32_t* send_meta)
{
    size_t TK = (size_t)T * K;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                size_t row = (size_t)s * TK + pos[((size_t)s * T + t) * K + k];
                memcpy(send_x + row * H, x + ((size_t)s * T + t) * H, sizeof(uint16_t) * H);
                send_meta[row] = t * K + k;
            }
}

/* Block-scaled fp8 quantisation of one token row ([EFA] "Dispatch/combine
 * latency": block-scaled fp8 dispatch; [EPMC] "Dispatch": block scaling
 * factors travel with the tokens).  For each block b of 128 elements, with
 * amax = max |x| and m = the smallest normal fp32 number, 2^-126:
 *   amax >= 448*m:    inv = 448 / amax and scale = amax / 448 (each one fp32
 *                     division; scale >= m, a normal number);
 *   0 < amax < 448*m: scale = m and inv = 1/m = 2^126 (the scale is kept
 *                     normal: amax / 448 would be an fp32 subnormal with few
 *                     significant bits, and 448 / amax can overflow to
 *                     infinity);
 *   amax == 0:        inv = 0 and scale = 1.
 * code = e4m3(x * inv) with one fp32 multiply.  Dequantised value = e4m3
 * value * scale.  Every finite input gives a finite code and a finite,
 * normal scale. */
void orc_quant_row_fp8(int H, const uint16_t* xrow, uint8_t* q, float* scale)
{
    const float m = ldexpf(1.0f, -126);
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float v = fabsf(orc_bf16_to_f32(xrow[b * 128 + i]));
            if (v > amax)
                amax = v;
        }
        float inv, sc;
        if (amax >= 448.0f * m) {
            inv = 448.0f / amax;
            sc = amax / 448.0f;
        } else if (amax > 0.0f) {
            inv = 1.0f / m;
            sc = m;
        } else {
            inv = 0.0f;
            sc = 1.0f;
        }
        for (int i = 0; i < 128; ++i) {
            float prod = orc_bf16_to_f32(xrow[b * 128 + i]) * inv;
            q[b * 128 + i] = orc_f32_to_e4m3(prod);
        }
        scale[b] = sc;
    }
}

/* orc_quant_row_fp8 of n consecutive rows of H elements. */
void orc_quant_rows_fp8(int64_t n, int H, const uint16_t* x, uint8_t* q, float* scale)
{
    for (int64_t i = 0; i < n; ++i)
        orc_quant_row_fp8(H, x + (size_t)i * H, q + (size_t)i * H, scale + (size_t)i * (H / 128));
}

/* Pack, fp8 payload: as orc_pack_bf16 but each token is quantised once and the
 * K copies carry its codes and its H/128 block scales. */
void orc_pack_fp8(int N, int T, int K, int H, const uint16_t* x, const int32_t* pos,
                  uint8_t* send_q, float* send_scale, int32_t* send_meta)
{
    size_t TK = (size_t)T * K;
    int nb = H / 128;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sc = (float*)malloc(sizeof(float) * (size_t)nb);
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t) {
            orc_quant_row_fp8(H, x + ((size_t)s * T + t) * H, q, sc);
            for (int k = 0; k < K; ++k) {
                size_t row = (size_t)s * TK + pos[((size_t)s * T + t) * K + k];
                memcpy(send_q + row * H, q, (size_t)H);
                memcpy(send_scale + row * nb, sc, sizeof(float) * nb);
                send_meta[row] = t * K + k;
            }
        }
    free(q);
    free(sc);
}

/* ------------------------------------------------------ dispatch: transfer */

/* The modelled network transfer ([EFA] "Dispatch and combine": the rows for
 * one peer leave in a single write; [EFA] "Send and receive buffers"): for each
 * sender s and receiver d, the scnt(s,d) rows starting at send row
 * soff[s][dL] of sender s land at receive row G[d] + roff[d][s].  Rows are
 * opaque byte strings of row_bytes bytes; the call is made once per plane
 * (payload, scales, meta). */
void orc_transfer_range(int N, int E, int T, int K, size_t row_bytes, const int32_t* soff,
                        const int32_t* roff, const int32_t* G, const uint8_t* send,
                        uint8_t* recv, int s0, int s1)
{
    int L = E / N;
    size_t TK = (size_t)T * K;
    for (int s = s0; s < s1; ++s)
        for (int d = 0; d < N; ++d) {
            int32_t first = soff[(size_t)s * (E + 1) + d * L];
            int32_t n = soff[(size_t)s * (E + 1) + (d + 1) * L] - first;
            size_t src = (size_t)s * TK + first;
            size_t dst = (size_t)G[d] + roff[(size_t)d * (N + 1) + s];
            memcpy(recv + dst * row_bytes, send + src * row_bytes, row_bytes * (size_t)n);
        }
}

void orc_transfer(int N, int E, int T, int K, size_t row_bytes, const int32_t* soff,
                  const int32_t* roff, const int32_t* G, const uint8_t* send, uint8_t* recv)
{
    orc_transfer_range(N, E, T, K, row_bytes, soff, roff, G, send, recv, 0, N);
}

/* ------------------------------------------------------ dispatch: shuffle */

/* Receive shuffle into grouped-GEMM order ([EPMC] "Dispatch": the receiver
 * copies tokens into contiguous buffers for the expert kernels and stores
 * source rank, expert and token index separately; [EFA] "Dispatch and combine":
 * rows are shuffled from the receive buffer into the tensor handed to the
 * grouped GEMM).  For expert e on rank d = e/L, for s ascending, the cnt[s][e]
 * rows of e from sender s (at receive row G[d] + roff[d][s] + soff[s][e] -
 * soff[s][dL] onward) go to expert rows eoff[e] + sum_{s'<s} cnt[s'][e] onward.
 * Metadata: src_rank[r] = s, src_slot[r] = the row's meta word (t*K+k).
 * The payload plane has row_bytes bytes per row; scales (scale_bytes per row,
 * 0 when there are none) move with it. */
void orc_shuffle_range(int N, int E, int T, int K, size_t row_bytes, size_t scale_bytes,
                       const int32_t* cnt, const int32_t* soff, const int32_t* roff,
                       const int32_t* G, const int32_t* eoff,
                       const uint8_t* recv_x, const uint8_t* recv_scale, const int32_t* recv_meta,
                       uint8_t* expert_x, uint8_t* expert_scale,
                       int32_t* src_rank, int32_t* src_slot, int e0, int e1)
{
    int L = E / N;
    (void)T;
    (void)K;
    for (int e = e0; e < e1; ++e) {
        int d = e / L;
        int32_t r = eoff[e];
        for (int s = 0; s < N; ++s) {
            int32_t n = cnt[(size_t)s * E + e];
            int32_t q0 = G[d] + roff[(size_t)d * (N + 1) + s] +
                         soff[(size_t)s * (E + 1) + e] - soff[(size_t)s * (E + 1) + d * L];
            for (int32_t i = 0; i < n; ++i, ++r) {
                size_t q = (size_t)q0 + i;
                memcpy(expert_x + (size_t)r * row_bytes, recv_x + q * row_bytes, row_bytes);
                if (scale_bytes)
                    memcpy(expert_scale + (size_t)r * scale_bytes, recv_scale + q * scale_bytes,
                           scale_bytes);
                src_rank[r] = s;
                src_slot[r] = recv_meta[q];
            }
        }
    }
}

void orc_shuffle(int N, int E, int T, int K, size_t row_bytes, size_t scale_bytes,
                 const int32_t* cnt, const int32_t* soff, const int32_t* roff,
                 const int32_t* G, const int32_t* eoff,
                 const uint8_t* recv_x, const uint8_t* recv_scale, const int32_t* recv_meta,
                 uint8_t* expert_x, uint8_t* expert_scale,
                 int32_t* src_rank, int32_t* src_slot)
{
    orc_shuffle_range(N, E, T, K, row_bytes, scale_bytes, cnt, soff, roff, G, eoff, recv_x,
                      recv_scale, recv_meta, expert_x, expert_scale, src_rank, src_slot, 0, E);
}

/* ------------------------------------------------- the expert (not the path) */

/* Stand-in for the grouped GEMM, outside the path: y[r] = bf16(v * (e+1)) where
 * e is row r's expert and v the row's value (bf16, or e4m3 value * block scale
 * when scales are given), one fp32 multiply per factor. */
void orc_expert_standin(int E, int H, const int32_t* eoff, const uint8_t* expert_x,
                        const float* expert_scale, int fp8, uint16_t* y)
{
    int nb = H / 128;
    for (int e = 0; e < E; ++e)
        for (int32_t r = eoff[e]; r < eoff[e + 1]; ++r)
            for (int h = 0; h < H; ++h) {
                float v;
                if (fp8) {
                    v = (float)orc_e4m3_value(expert_x[(size_t)r * H + h]) *
                        expert_scale[(size_t)r * nb + h / 128];
                } else {
                    uint16_t b;
                    memcpy(&b, expert_x + ((size_t)r * H + h) * 2, 2);
                    v = orc_bf16_to_f32(b);
                }
                y[(size_t)r * H + h] = orc_f32_to_bf16(v * (float)(e + 1));
            }
}

/* --------------------------------------------------------------- combine */

/* Combine send ([EPMC] "Combine": senders copy the unquantised 16-bit expert
 * outputs back toward the token's rank; [EFA] "Dispatch and combine": combine
 * is the reverse route, one write per peer).  The inverse of orc_shuffle: the
 * expert-order row r of expert e from sender s, i-th of its run, goes back to
 * receive-layout row G[d] + roff[d][s] + soff[s][e] - soff[s][dL] + i. */
void orc_combine_send_range(int N, int E, size_t row_bytes, const int32_t* cnt,
                            const int32_t* soff, const int32_t* roff, const int32_t* G,
                            const int32_t* eoff, const uint8_t* y, uint8_t* comb_send,
                            int e0, int e1)
{
    int L = E / N;
    for (int e = e0; e < e1; ++e) {
        int d = e / L;
        int32_t r = eoff[e];
        for (int s = 0; s < N; ++s) {
            int32_t n = cnt[(size_t)s * E + e];
            int32_t q0 = G[d] + roff[(size_t)d * (N + 1) + s] +
                         soff[(size_t)s * (E + 1) + e] - soff[(size_t)s * (E + 1) + d * L];
            for (int32_t i = 0; i < n; ++i, ++r)
                memcpy(comb_send + ((size_t)q0 + i) * row_bytes, y + (size_t)r * row_bytes,
                       row_bytes);
        }
    }
}

void orc_combine_send(int N, int E, size_t row_bytes, const int32_t* cnt,
                      const int32_t* soff, const int32_t* roff, const int32_t* G,
                      const int32_t* eoff, const uint8_t* y, uint8_t* comb_send)
{
    orc_combine_send_range(N, E, row_bytes, cnt, soff, roff, G, eoff, y, comb_send, 0, E);
}

/* Combine transfer: the reverse of orc_transfer.  The rows rank d holds for
 * sender s (receive rows G[d] + roff[d][s] ...) return to sender s's buffer at
 * rows s*T*K + soff[s][dL] ..., i.e. where s packed them. */
void orc_combine_transfer_range(int N, int E, int T, int K, size_t row_bytes,
                                const int32_t* soff, const int32_t* roff, const int32_t* G,
                                const uint8_t* comb_send, uint8_t* comb_recv, int d0, int d1)
{
    int L = E / N;
    size_t TK = (size_t)T * K;
    for (int d = d0; d < d1; ++d)
        for (int s = 0; s < N; ++s) {
            int32_t first = soff[(size_t)s * (E + 1) + d * L];
            int32_t n = soff[(size_t)s * (E + 1) + (d + 1) * L] - first;
            size_t src = (size_t)G[d] + roff[(size_t)d * (N + 1) + s];
            size_t dst = (size_t)s * TK + first;
            memcpy(comb_recv + dst * row_bytes, comb_send + src * row_bytes, row_bytes * (size_t)n);
        }
}

void orc_combine_transfer(int N, int E, int T, int K, size_t row_bytes, const int32_t* soff,
                          const int32_t* roff, const int32_t* G, const uint8_t* comb_send,
                          uint8_t* comb_recv)
{
    orc_combine_transfer_range(N, E, T, K, row_bytes, soff, roff, G, comb_send, comb_recv, 0, N);
}

/* Combine receive: the router-weighted sum of the K expert outputs of every
 * token ([EPMC] "Introduction": the output is the sum of the expert outputs
 * multiplied by weights from the router distribution; [EPMC] "Combine": the
 * receiver computes the weighted average locally into an externally allocated
 * tensor).  Precision: fp32, k ascending, as one fused multiply-add chain
 * from +0, rounded once to bf16 (nearest even):
 *   acc = +0; for k: acc = fmaf(w[s][t][k], y_k[h], acc); out = bf16(acc)
 * where y_k is the returned row at sender row pos[s][t][k]. */
void orc_combine_recv(int N, int T, int K, int H, const int32_t* pos, const float* w,
                      const uint16_t* comb_recv, uint16_t* out)
{
    size_t TK = (size_t)T * K;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                float acc = +0.0f;
                for (int k = 0; k < K; ++k) {
                    size_t i = ((size_t)s * T + t) * K + k;
                    size_t row = (size_t)s * TK + pos[i];
                    acc = fmaf(w[i], orc_bf16_to_f32(comb_recv[row * H + h]), acc);
                }
                out[((size_t)s * T + t) * H + h] = orc_f32_to_bf16(acc);
            }
}

/* The same weighted sum in double precision, unrounded (each product of a
 * float weight and a bf16 value is exact in double; the sum of K <= 16 such
 * terms is exact to within 2^-50 relative).  Used only to bound the fp32
 * chain above. */
void orc_combine_recv_f64(int N, int T, int K, int H, const int32_t* pos, const float* w,
                          const uint16_t* comb_recv, double* out, double* abs_sum)
{
    size_t TK = (size_t)T * K;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                double acc = 0.0, mag = 0.0;
                for (int k = 0; k < K; ++k) {
                    size_t i = ((size_t)s * T + t) * K + k;
                    size_t row = (size_t)s * TK + pos[i];
                    double term = (double)w[i] * (double)orc_bf16_to_f32(comb_recv[row * H + h]);
                    acc += term;
                    mag += fabs(term);
                }
                out[((size_t)s * T + t) * H + h] = acc;
                abs_sum[((size_t)s * T + t) * H + h] = mag;
            }
}

/* Combine receive of a single token (sampled checks at sizes where the whole
 * output is too large for the CPU): same chain as orc_combine_recv.  rows[k]
 * points at the k-th returned row, w at the token's K weights. */
void orc_combine_token(int K, int H, const uint16_t* const* rows, const float* w, uint16_t* out)
{
    for (int h = 0; h < H; ++h) {
        float acc = +0.0f;
        for (int k = 0; k < K; ++k)
            acc = fmaf(w[k], orc_bf16_to_f32(rows[k][h]), acc);
        out[h] = orc_f32_to_bf16(acc);
    }
}

/* Many tokens of the same combine, for whole-workload checks where the
 * returned rows sit in one array: token i's k-th returned row is row
 * rows[i*K + k] of y ([*][H]), its weights w[i*K ...]; out[i] is
 * orc_combine_token of those rows. */
void orc_combine_tokens(int64_t n, int K, int H, const int64_t* rows, const float* w,
                        const uint16_t* y, uint16_t* out)
{
    const uint16_t** r = (const uint16_t**)malloc(sizeof(*r) * (size_t)K);
    for (int64_t i = 0; i < n; ++i) {
        for (int k = 0; k < K; ++k)
            r[k] = y + (size_t)rows[i * K + k] * H;
        orc_combine_token(K, H, r, w + i * K, out + (size_t)i * H);
    }
    free(r);
}

/* ------------------------------------------------ array forms of the codecs */

void orc_f32_to_bf16_n(size_t n, const float* in, uint16_t* out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(in[i]);
}

void orc_f32_to_e4m3_n(size_t n, const float* in, uint8_t* out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_e4m3(in[i]);
}

/* ---------------------------------------- per-row definitions for sampling */

/* The meta word of every send row (the index part of the pack step, without
 * the payload): send_meta[s*T*K + pos[s][t][k]] = t*K+k. */
void orc_send_meta(int N, int T, int K, const int32_t* pos, int32_t* send_meta)
{
    size_t TK = (size_t)T * K;
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k)
                send_meta[(size_t)s * TK + pos[((size_t)s * T + t) * K + k]] = t * K + k;
}

/* The expert-order row that (s,t,k) lands in (the shuffle's destination):
 * expert e = idx[s][t][k] starts at eoff[e]; the rows of e from senders
 * s' < s come first; then s's own rows of e in its send order. */
void orc_expert_rows_range(int N, int T, int K, int E, const int32_t* idx, const int32_t* cnt,
                           const int32_t* soff, const int32_t* pos, const int32_t* eoff,
                           int32_t* rows, int s0, int s1)
{
    (void)N;
    for (int s = s0; s < s1; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                size_t i = ((size_t)s * T + t) * K + k;
                int e = idx[i];
                int32_t before = 0;
                for (int s2 = 0; s2 < s; ++s2)
                    before += cnt[(size_t)s2 * E + e];
                rows[i] = eoff[e] + before + pos[i] - soff[(size_t)s * (E + 1) + e];
            }
}

void orc_expert_rows(int N, int T, int K, int E, const int32_t* idx, const int32_t* cnt,
                     const int32_t* soff, const int32_t* pos, const int32_t* eoff, int32_t* rows)
{
    orc_expert_rows_range(N, T, K, E, idx, cnt, soff, pos, eoff, rows, 0, N);
}

/* ------------------------------------------------ fixed-slot receive layout */
/*
 * [EPMC] "Portable kernels": the most tokens a DP rank may dispatch is fixed
 * for the group, and that also bounds what a rank can receive from each
 * source rank for each of its local experts, so a sender can work out a
 * unique address on the receiver without synchronising with other ranks.
 * Reading taken here: receiver d holds the areas of its experts e = d*L + j,
 * each T_max*N rows of the pooled receive array (N*E*T_max rows in all), slot
 * index major and source rank minor: sender s's i-th row for expert e (i = its
 * rank among s's rows for e, (t,k) order) goes to row (e*T_max + i)*N + s.
 * Each (source, expert) pair so owns T_max slots (every N-th row of the
 * expert's area), and the filled slots, i < count, gather at the start of
 * each expert's area.  A (sender, expert) count above T_max -- possible only
 * when a token names an expert more than once -- does not fit.
 */

/* 1 when every (sender, expert) count fits its T_max slots, else 0. */
int orc_slot_capacity_ok(int N, int E, int T_max, const int32_t* cnt)
{
    for (size_t i = 0; i < (size_t)N * E; ++i)
        if (cnt[i] > T_max)
            return 0;
    return 1;
}

/* Slot row of every (s,t,k): (e*T_max + i)*N + s, with i the item's rank
 * among sender s's rows for its expert (pos - soff[s][e]). */
void orc_slot_rows(int N, int T, int K, int E, int T_max, const int32_t* idx, const int32_t* soff,
                   const int32_t* pos, int64_t* slot)
{
    for (int s = 0; s < N; ++s)
        for (int t = 0; t < T; ++t)
            for (int k = 0; k < K; ++k) {
                size_t it = ((size_t)s * T + t) * K + k;
                int e = idx[it];
                int64_t i = pos[it] - soff[(size_t)s * (E + 1) + e];
                slot[it] = ((int64_t)e * T_max + i) * N + s;
            }
}

/* The transfer into the slots: every send row (sender s, position pos) goes
 * to its slot; slots no row names are left as they were. */
void orc_transfer_slots(int N, int T, int K, size_t row_bytes, const int32_t* pos,
                        const int64_t* slot, const uint8_t* send, uint8_t* recv)
{
    size_t TK = (size_t)T * K;
    for (int s = 0; s < N; ++s)
        for (size_t tk = 0; tk < TK; ++tk) {
            size_t i = (size_t)s * TK + tk;
            memcpy(recv + (size_t)slot[i] * row_bytes, send + ((size_t)s * TK + pos[i]) * row_bytes,
                   row_bytes);
        }
}

/* The receive shuffle out of the slots, from the layout alone: expert e
 * takes, for s ascending, source s's first cnt[s][e] slots, in slot order
 * (rows (e*T_max + i)*N + s, i = 0, 1, ...), into expert rows eoff[e]
 * onward; metadata as in orc_shuffle. */
void orc_shuffle_slots(int N, int E, int T_max, size_t row_bytes, size_t scale_bytes,
                       const int32_t* cnt, const int32_t* eoff, const uint8_t* recv_x,
                       const uint8_t* recv_scale, const int32_t* recv_meta, uint8_t* expert_x,
                       uint8_t* expert_scale, int32_t* src_rank, int32_t* src_slot)
{
    for (int e = 0; e < E; ++e) {
        int32_t r = eoff[e];
        for (int s = 0; s < N; ++s) {
            for (int32_t i = 0; i < cnt[(size_t)s * E + e]; ++i, ++r) {
                size_t q = ((size_t)e * T_max + (size_t)i) * N + s;
                memcpy(expert_x + (size_t)r * row_bytes, recv_x + q * row_bytes, row_bytes);
                if (scale_bytes)
                    memcpy(expert_scale + (size_t)r * scale_bytes, recv_scale + q * scale_bytes,
                           scale_bytes);
                src_rank[r] = s;
                src_slot[r] = recv_meta[q];
            }
        }
    }
}

/* ------------------------------------- combine with sender-side partial sums */
/*
 * [EFA] "Dispatch/combine latency": accumulating on the send side of combine
 * cuts the bytes moved, at some cost in precision.  Reading taken here: the
 * rank d owning some of token (s,t)'s experts sums their weighted outputs
 * (fp32, k ascending, fma chain from +0), rounds the partial once to bf16 and
 * returns ONE row per (token, destination rank); the token's owner adds the
 * partials in fp32, destination rank ascending, from +0, and rounds to bf16.
 *
 * visits(s,t,d) = some k has idx[s][t][k] / L == d.
 * pc[s][d]      = #{t : visits(s,t,d)}          (partial rows from d back to s)
 * prank(s,t,d)  = #{t' < t : visits(s,t',d)}
 * Owner-side rows ("partial send", like the receive layout): owner d's rows
 * start at sum_{d'<d} sum_s pc[s][d']; inside, sender s ascending, then t.
 * Token-owner rows ("partial receive", like the send layout): sender s's rows
 * start at sum_{s'<s} sum_d pc[s'][d]; inside, d ascending, then t.
 */
void orc_partial_counts_range(int N, int T, int K, int E, const int32_t* idx, int32_t* pc,
                              int s0, int s1)
{
    int L = E / N;
    memset(pc + (size_t)s0 * N, 0, sizeof(int32_t) * (size_t)(s1 - s0) * N);
    for (int s = s0; s < s1; ++s)
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < N; ++d) {
                int v = 0;
                for (int k = 0; k < K; ++k)
                    if (idx[((size_t)s * T + t) * K + k] / L == d)
                        v = 1;
                pc[(size_t)s * N + d] += v;
            }
}

void orc_partial_counts(int N, int T, int K, int E, const int32_t* idx, int32_t* pc)
{
    orc_partial_counts_range(N, T, K, E, idx, pc, 0, N);
}

/* Row of partial (s,t,d) in the owner-side and token-owner-side layouts, for
 * every (s,t,d) visited (-1 elsewhere); arrays [N][T][N].  The owner-side
 * rows are ordered by (d, s, t): the rows before (d, s) are a running count of
 * pc taken in (d, s) order.  The token-side rows are ordered by (s, d, t):
 * a running count of pc in (s, d) order.  Inside a (d, s) pair, tokens in
 * order (the running rank of the pair). */
void orc_partial_rows_range(int N, int T, int K, int E, const int32_t* idx, const int32_t* pc,
                            int32_t* owner_row, int32_t* token_row, int s0, int s1)
{
    int L = E / N;
    int32_t* obase = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * N);  /* [d][s] */
    int32_t* tbase = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * N);  /* [s][d] */
    int32_t* rank = (int32_t*)calloc((size_t)N * N, sizeof(int32_t));    /* [s][d] running prank */
    int32_t run = 0;
    for (int d = 0; d < N; ++d)
        for (int s = 0; s < N; ++s) {
            obase[(size_t)d * N + s] = run;
            run += pc[(size_t)s * N + d];
        }
    run = 0;
    for (int s = 0; s < N; ++s)
        for (int d = 0; d < N; ++d) {
            tbase[(size_t)s * N + d] = run;
            run += pc[(size_t)s * N + d];
        }
    for (int s = s0; s < s1; ++s)
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < N; ++d) {
                size_t o = ((size_t)s * T + t) * N + d;
                int v = 0;
                for (int k = 0; k < K; ++k)
                    if (idx[((size_t)s * T + t) * K + k] / L == d)
                        v = 1;
                if (!v) {
                    owner_row[o] = -1;
                    token_row[o] = -1;
                    continue;
                }
                int32_t pr = rank[(size_t)s * N + d]++;
                owner_row[o] = obase[(size_t)d * N + s] + pr;
                token_row[o] = tbase[(size_t)s * N + d] + pr;
            }
    free(obase);
    free(tbase);
    free(rank);
}

void orc_partial_rows(int N, int T, int K, int E, const int32_t* idx, const int32_t* pc,
                      int32_t* owner_row, int32_t* token_row)
{
    orc_partial_rows_range(N, T, K, E, idx, pc, owner_row, token_row, 0, N);
}

/* The owner's partial sums: for every visited (s,t,d), the fp32 fma chain over
 * the token's k (ascending) whose expert lives on d, of w[s][t][k] times the
 * expert output row y[expert_rows[s][t][k]], rounded to bf16, written to the
 * owner-side row. */
void orc_partial_send_range(int N, int T, int K, int E, int H, const int32_t* idx,
                            const float* w, const int32_t* expert_rows, const uint16_t* y,
                            const int32_t* owner_row, uint16_t* psend, int s0, int s1)
{
    int L = E / N;
    float* acc = (float*)malloc(sizeof(float) * (size_t)H);
    for (int s = s0; s < s1; ++s)
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < N; ++d) {
                int32_t row = owner_row[((size_t)s * T + t) * N + d];
                if (row < 0)
                    continue;
                for (int h = 0; h < H; ++h)
                    acc[h] = +0.0f;
                for (int k = 0; k < K; ++k) {
                    size_t i = ((size_t)s * T + t) * K + k;
                    if (idx[i] / L != d)
                        continue;
                    const uint16_t* yr = y + (size_t)expert_rows[i] * H;
                    for (int h = 0; h < H; ++h)
                        acc[h] = fmaf(w[i], orc_bf16_to_f32(yr[h]), acc[h]);
                }
                for (int h = 0; h < H; ++h)
                    psend[(size_t)row * H + h] = orc_f32_to_bf16(acc[h]);
            }
    free(acc);
}

void orc_partial_send(int N, int T, int K, int E, int H, const int32_t* idx, const float* w,
                      const int32_t* expert_rows, const uint16_t* y, const int32_t* owner_row,
                      uint16_t* psend)
{
    orc_partial_send_range(N, T, K, E, H, idx, w, expert_rows, y, owner_row, psend, 0, N);
}

/* The transfer of the partial rows back to each token's owner. */
void orc_partial_transfer_range(int N, int T, int H, const int32_t* owner_row,
                                const int32_t* token_row, const uint16_t* psend,
                                uint16_t* precv, int s0, int s1)
{
    for (size_t o = (size_t)s0 * T * N; o < (size_t)s1 * T * N; ++o)
        if (owner_row[o] >= 0)
            memcpy(precv + (size_t)token_row[o] * H, psend + (size_t)owner_row[o] * H,
                   sizeof(uint16_t) * H);
}

void orc_partial_transfer(int N, int T, int H, const int32_t* owner_row, const int32_t* token_row,
                          const uint16_t* psend, uint16_t* precv)
{
    orc_partial_transfer_range(N, T, H, owner_row, token_row, psend, precv, 0, N);
}

/* The token owner's sum of its partial rows: fp32, destination rank
 * ascending, from +0, rounded once to bf16. */
void orc_partial_recv_range(int N, int T, int H, const int32_t* token_row,
                            const uint16_t* precv, uint16_t* out, int s0, int s1)
{
    for (int s = s0; s < s1; ++s)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                float acc = +0.0f;
                for (int d = 0; d < N; ++d) {
                    int32_t row = token_row[((size_t)s * T + t) * N + d];
                    if (row >= 0)
                        acc = acc + orc_bf16_to_f32(precv[(size_t)row * H + h]);
                }
                out[((size_t)s * T + t) * H + h] = orc_f32_to_bf16(acc);
            }
}

void orc_partial_recv(int N, int T, int H, const int32_t* token_row, const uint16_t* precv,
                      uint16_t* out)
{
    orc_partial_recv_range(N, T, H, token_row, precv, out, 0, N);
}

/* One token of the same combine, for checking single tokens of workloads too
 * large for the whole-batch functions: rows[k] is the expert output of item
 * k, rank[k] its destination rank.  Ranks ascending: the partial of rank d is
 * the fp32 fma chain from +0 over the k with rank[k] == d, k ascending,
 * rounded to bf16; the partials are added in fp32 from +0 and the sum is
 * rounded to bf16. */
void orc_partial_token(int K, int H, const uint16_t* const* rows, const float* w,
                       const int32_t* rank, uint16_t* out)
{
    for (int h = 0; h < H; ++h) {
        float acc = +0.0f;
        int32_t prev = -1;
        for (;;) {
            /* the smallest rank above the previous one */
            int32_t d = -1;
            for (int k = 0; k < K; ++k)
                if (rank[k] > prev && (d < 0 || rank[k] < d))
                    d = rank[k];
            if (d < 0)
                break;
            float part = +0.0f;
            for (int k = 0; k < K; ++k)
                if (rank[k] == d)
                    part = fmaf(w[k], orc_bf16_to_f32(rows[k][h]), part);
            acc = acc + orc_bf16_to_f32(orc_f32_to_bf16(part));
            prev = d;
        }
        out[h] = orc_f32_to_bf16(acc);
    }
}

/* orc_partial_token of many tokens: token i's k-th returned row is row
 * rows[i*K + k] of y ([*][H]), its weight w[i*K + k] and destination rank
 * rank[i*K + k]. */
void orc_partial_tokens(int64_t n, int K, int H, const int64_t* rows, const float* w,
                        const int32_t* rank, const uint16_t* y, uint16_t* out)
{
    const uint16_t** r = (const uint16_t**)malloc(sizeof(*r) * (size_t)K);
    for (int64_t i = 0; i < n; ++i) {
        for (int k = 0; k < K; ++k)
            r[k] = y + (size_t)rows[i * K + k] * H;
        orc_partial_token(K, H, r, w + i * K, rank + i * K, out + (size_t)i * H);
    }
    free(r);
}
