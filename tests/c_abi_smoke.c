/*
 * c_abi_smoke.c - the library used from plain C, without Python or torch:
 * device buffers from hipMalloc, one routing + dispatch + combine pass, and
 * checks that need no reference implementation.
 *
 *   - route count: cnt sums to the number of valid ids, off is its scan;
 *   - dispatch (bf16, compact): every valid entry got a row of its expert's
 *     segment, packed_src names the entry's token, the row holds x[t] bit for
 *     bit, and no two entries share a row;
 *   - combine with one entry per token and weight 1: out == x bit for bit
 *     (bf16 -> f32 -> times 1 -> plus 0 -> bf16 is exact), out_weights == 1;
 *   - the error path: a short workspace returns MOE_ERR_WORKSPACE and a message.
 *
 * Prints "c abi smoke: ok" and exits 0 on success; exits 1 with a message on
 * the first failed check, 2 when no GPU is usable.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_route.h"

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

#define EXPECT(cond, ...)                                                         \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "c abi smoke: check failed: " __VA_ARGS__);           \
            fprintf(stderr, "\n");                                                \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static void* dmalloc(size_t n) {
    void* p = NULL;
    CHECK_HIP(hipMalloc(&p, n ? n : 1));
    return p;
}

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {  /* xorshift32 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        fprintf(stderr, "c abi smoke: no GPU\n");
        return 2;
    }
    const int64_t T = 777, H = 256;
    const int K = 4, E = 12;
    const int64_t N = T * K, rows = N;

    /* inputs: random ids with some -1 and some out of range, random bf16 rows */
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * N);
    uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * T * H);
    int64_t valid = 0;
    for (int64_t f = 0; f < N; ++f) {
        uint32_t r = rnd() % 100;
        idx[f] = r < 5 ? -1 : (r < 8 ? E + (int32_t)(r % 3) : (int32_t)(rnd() % E));
        valid += idx[f] >= 0 && idx[f] < E;
    }
    for (int64_t i = 0; i < T * H; ++i)  /* normal bf16 of either sign, no zeros */
        x[i] = (uint16_t)(((rnd() & 1u) << 15) | ((0x30u + rnd() % 32u) << 8) | (rnd() & 0xFFu));

    int32_t* d_idx = (int32_t*)dmalloc(sizeof(int32_t) * N);
    uint16_t* d_x = (uint16_t*)dmalloc(sizeof(uint16_t) * T * H);
    CHECK_HIP(hipMemcpy(d_idx, idx, sizeof(int32_t) * N, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

    const size_t ws_bytes = moe_workspace_size(T, K, E, 0);
    EXPECT(ws_bytes > 0, "workspace size %zu", ws_bytes);
    void* ws = dmalloc(ws_bytes);
    int32_t* d_cnt = (int32_t*)dmalloc(sizeof(int32_t) * E);
    int32_t* d_off = (int32_t*)dmalloc(sizeof(int32_t) * (E + 1));
    int32_t* d_stats = (int32_t*)dmalloc(sizeof(int32_t) * 3);

    /* the error path: nothing is launched, a message is left */
    EXPECT(moe_route_count(d_idx, T, K, E, d_cnt, d_off, d_stats, ws, ws_bytes - 1, NULL) ==
               MOE_ERR_WORKSPACE,
           "short workspace accepted");
    EXPECT(strlen(moe_last_error()) > 0, "no error message");

    /* route count */
    EXPECT(moe_route_count(d_idx, T, K, E, d_cnt, d_off, d_stats, ws, ws_bytes, NULL) == MOE_OK,
           "moe_route_count: %s", moe_last_error());
    int32_t cnt[64], off[65], stats[3];
    CHECK_HIP(hipMemcpy(cnt, d_cnt, sizeof(int32_t) * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(off, d_off, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(stats, d_stats, sizeof(int32_t) * 3, hipMemcpyDeviceToHost));
    int64_t sum = 0;
    for (int e = 0; e < E; ++e) {
        EXPECT(off[e] == sum, "off[%d] = %d, expected %lld", e, off[e], (long long)sum);
        sum += cnt[e];
    }
    EXPECT(sum == valid && off[E] == sum, "counts sum to %lld, valid ids %lld", (long long)sum,
           (long long)valid);

    /* dispatch, compact bf16 */
    uint16_t* d_packed = (uint16_t*)dmalloc(sizeof(uint16_t) * rows * H);
    int32_t* d_pcnt = (int32_t*)dmalloc(sizeof(int32_t) * E);
    int32_t* d_poff = (int32_t*)dmalloc(sizeof(int32_t) * (E + 1));
    int32_t* d_psrc = (int32_t*)dmalloc(sizeof(int32_t) * rows);
    int64_t* d_tm = (int64_t*)dmalloc(sizeof(int64_t) * N);
    EXPECT(moe_dispatch(d_x, MOE_BF16, T, H, d_idx, K, E, 0, rows, d_packed, MOE_BF16, NULL,
                        d_pcnt, d_poff, d_psrc, d_tm, d_stats, ws, ws_bytes, NULL) == MOE_OK,
           "moe_dispatch: %s", moe_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    int64_t* tm = (int64_t*)malloc(sizeof(int64_t) * N);
    int32_t* psrc = (int32_t*)malloc(sizeof(int32_t) * rows);
    uint16_t* packed = (uint16_t*)malloc(sizeof(uint16_t) * rows * H);
    unsigned char* seen = (unsigned char*)calloc((size_t)rows, 1);
    CHECK_HIP(hipMemcpy(tm, d_tm, sizeof(int64_t) * N, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(psrc, d_psrc, sizeof(int32_t) * rows, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(packed, d_packed, sizeof(uint16_t) * rows * H, hipMemcpyDeviceToHost));
    for (int64_t f = 0; f < N; ++f) {
        const int64_t t = f / K;
        const int32_t e = idx[f];
        if (!(e >= 0 && e < E)) {
            EXPECT(tm[f] == -1, "entry %lld with id %d has row %lld", (long long)f, e,
                   (long long)tm[f]);
            continue;
        }
        const int64_t r = tm[f];
        EXPECT(r >= off[e] && r < off[e + 1], "entry %lld: row %lld outside expert %d", (long long)f,
               (long long)r, e);
        EXPECT(!seen[r], "row %lld given twice", (long long)r);
        seen[r] = 1;
        EXPECT(psrc[r] == t, "packed_src[%lld] = %d, expected %lld", (long long)r, psrc[r],
               (long long)t);
        EXPECT(memcmp(packed + r * H, x + t * H, sizeof(uint16_t) * H) == 0,
               "row %lld differs from token %lld", (long long)r, (long long)t);
    }

    /* combine: one entry per token (the first), weight 1, identity expert */
    int64_t* tm1 = (int64_t*)malloc(sizeof(int64_t) * T);
    float* w1 = (float*)malloc(sizeof(float) * T);
    for (int64_t t = 0; t < T; ++t) {
        tm1[t] = tm[t * K];
        w1[t] = 1.0f;
    }
    int64_t* d_tm1 = (int64_t*)dmalloc(sizeof(int64_t) * T);
    float* d_w1 = (float*)dmalloc(sizeof(float) * T);
    uint16_t* d_out = (uint16_t*)dmalloc(sizeof(uint16_t) * T * H);
    float* d_ow = (float*)dmalloc(sizeof(float) * T);
    CHECK_HIP(hipMemcpy(d_tm1, tm1, sizeof(int64_t) * T, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_w1, w1, sizeof(float) * T, hipMemcpyHostToDevice));
    EXPECT(moe_combine(d_packed, MOE_BF16, rows, H, d_tm1, d_w1, T, 1, E, NULL, d_out, MOE_BF16,
                       d_ow, NULL) == MOE_OK,
           "moe_combine: %s", moe_last_error());
    CHECK_HIP(hipDeviceSynchronize());
    uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * T * H);
    float* ow = (float*)malloc(sizeof(float) * T);
    CHECK_HIP(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(ow, d_ow, sizeof(float) * T, hipMemcpyDeviceToHost));
    for (int64_t t = 0; t < T; ++t) {
        if (tm1[t] < 0) {
            EXPECT(ow[t] == 0.0f, "token %lld without entry has weight %g", (long long)t, ow[t]);
            for (int64_t h = 0; h < H; ++h)
                EXPECT(out[t * H + h] == 0, "token %lld without entry is not zero", (long long)t);
            continue;
        }
        EXPECT(ow[t] == 1.0f, "out_weights[%lld] = %g", (long long)t, ow[t]);
        EXPECT(memcmp(out + t * H, x + t * H, sizeof(uint16_t) * H) == 0,
               "combine of token %lld differs from x", (long long)t);
    }
    printf("c abi smoke: ok (library version %d.%d, %lld valid entries)\n", moe_version() >> 16,
           moe_version() & 0xFFFF, (long long)valid);
    return 0;
}
