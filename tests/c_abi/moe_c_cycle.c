/* A dispatch + combine cycle driven from plain C through include/moe_ep.h,
 * with no Python: identity experts (expert_y = expert_x) and router weights
 * summing to one, so every output token must equal its input token (an input
 * -0 comes back as +0, the fma chain starting from +0).  Prints one line and
 * exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_ep.h"

#define CHECK_HIP(x)                                                        \
    do {                                                                    \
        hipError_t e_ = (x);                                                \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s failed: %d\n", #x, (int)e_);                \
            return 2;                                                       \
        }                                                                   \
    } while (0)
#define CHECK_MOE(x)                                                        \
    do {                                                                    \
        int s_ = (x);                                                       \
        if (s_ != MOE_OK) {                                                 \
            fprintf(stderr, "%s: %s\n", #x, moe_strerror(s_));              \
            return 3;                                                       \
        }                                                                   \
    } while (0)

static uint32_t lcg(uint32_t* s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

int main(void)
{
    const int N = 4, T = 24, H = 256, E = 16, K = 3;
    const int L = E / N;
    const size_t R = (size_t)N * T * K;
    uint16_t* x = malloc(sizeof(uint16_t) * N * T * H);
    int32_t* idx = malloc(sizeof(int32_t) * N * T * K);
    float* w = malloc(sizeof(float) * N * T * K);
    uint16_t* out = malloc(sizeof(uint16_t) * N * T * H);
    uint32_t seed = 12345u;
    for (size_t i = 0; i < (size_t)N * T * H; ++i) {
        /* bf16 values 1..2 with a random sign: sign | exponent 127 | 7 mantissa bits */
        x[i] = (uint16_t)(((lcg(&seed) & 1u) << 15) | 0x3F80u | (lcg(&seed) & 0x7Fu));
    }
    for (int t = 0; t < N * T; ++t) {
        /* K distinct experts; weights 1/2, 1/4, 1/4 sum to one exactly */
        int first = (int)(lcg(&seed) % (uint32_t)E);
        for (int k = 0; k < K; ++k) {
            idx[t * K + k] = (first + k * (L + 1)) % E;
            w[t * K + k] = k == 0 ? 0.5f : 0.25f;
        }
    }
    void *d_x, *d_idx, *d_w, *d_ex, *d_out;
    int32_t* d_offs;
    CHECK_HIP(hipMalloc(&d_x, sizeof(uint16_t) * N * T * H));
    CHECK_HIP(hipMalloc(&d_idx, sizeof(int32_t) * N * T * K));
    CHECK_HIP(hipMalloc(&d_w, sizeof(float) * N * T * K));
    CHECK_HIP(hipMalloc(&d_ex, sizeof(uint16_t) * R * H));
    CHECK_HIP(hipMalloc((void**)&d_offs, sizeof(int32_t) * (E + 1)));
    CHECK_HIP(hipMalloc(&d_out, sizeof(uint16_t) * N * T * H));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * N * T * H, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_idx, idx, sizeof(int32_t) * N * T * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w, w, sizeof(float) * N * T * K, hipMemcpyHostToDevice));

    moe_group_desc desc;
    memset(&desc, 0, sizeof(desc));
    desc.num_ranks = N;
    desc.num_experts = E;
    desc.top_k = K;
    desc.hidden = H;
    desc.max_tokens = T;
    desc.dispatch_dtype = MOE_BF16;
    desc.transport = MOE_TRANSPORT_STAGED;
    desc.combine_mode = MOE_COMBINE_RECEIVER;
    desc.layout = MOE_LAYOUT_PACKED;
    moe_group_t g = NULL;
    CHECK_MOE(moe_group_create(&desc, &g));
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    for (int cycle = 0; cycle < 2; ++cycle) {
        CHECK_MOE(moe_dispatch_send(g, T, d_x, (const int32_t*)d_idx, NULL, st));
        CHECK_MOE(moe_dispatch_recv(g, d_ex, NULL, d_offs, st));
        CHECK_MOE(moe_combine_send(g, d_ex, st));         /* identity experts */
        CHECK_MOE(moe_combine_recv(g, (const float*)d_w, d_out, st));
        CHECK_MOE(moe_group_status(g, st));
    }
    CHECK_HIP(hipMemcpy(out, d_out, sizeof(uint16_t) * N * T * H, hipMemcpyDeviceToHost));
    int32_t offs[17];
    CHECK_HIP(hipMemcpy(offs, d_offs, sizeof(offs), hipMemcpyDeviceToHost));
    size_t bad = 0;
    for (size_t i = 0; i < (size_t)N * T * H; ++i)
        if (out[i] != (x[i] == 0x8000u ? 0u : x[i]))
            ++bad;
    const int rows_ok = offs[0] == 0 && offs[E] == (int32_t)R;
    CHECK_MOE(moe_group_destroy(g));
    CHECK_HIP(hipStreamDestroy(st));
    hipFree(d_x);
    hipFree(d_idx);
    hipFree(d_w);
    hipFree(d_ex);
    hipFree(d_offs);
    hipFree(d_out);
    printf("c-abi cycle: N=%d T=%d H=%d E=%d K=%d mismatches=%zu expert_offsets=%s\n", N, T, H, E, K,
           bad, rows_ok ? "ok" : "bad");
    free(x);
    free(idx);
    free(w);
    free(out);
    return bad == 0 && rows_ok ? 0 : 1;
}
