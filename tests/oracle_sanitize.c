/*
 * oracle_sanitize.c -- drives every function of oracle/moe_oracle.c over small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles the
 * two files together with gcc -fsanitize=address,undefined -fno-sanitize-recover=all and runs the
 * program). Values are not checked here (the pin tests do that); a read or write outside a buffer,
 * a use of freed memory, a leak or undefined arithmetic makes the program abort, and a function
 * that rejects valid arguments makes it return 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { F32 = 0, BF16 = 1, FP8 = 2 };

void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
void oracle_f64_to_bf16(const double* in, uint16_t* out, int64_t n);
void oracle_f32_to_e4m3(const float* in, uint8_t* out, int64_t n);
void oracle_e4m3_to_f32(const uint8_t* in, float* out, int64_t n);
int oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                 float* topk_w);
int oracle_dispatch(const void* x, int32_t x_dtype, int32_t T, int32_t H, const int32_t* topk_idx,
                    int32_t k, int32_t E, int32_t N, int32_t payload_dtype, void* recv,
                    float* recv_scales, int32_t* expert_counts, int32_t* expert_offsets,
                    int32_t* rank_counts, int32_t* rank_offsets, int32_t* token_row,
                    int32_t* row_token);
int oracle_experts(const void* recv, int32_t payload_dtype, const float* recv_scales, int32_t R,
                   int32_t H, const int32_t* expert_offsets, int32_t E, int32_t rule, void* y,
                   int32_t y_dtype);
int oracle_combine(const void* y, int32_t y_dtype, int32_t T, int32_t H, int32_t k,
                   const int32_t* token_row, const float* topk_w, void* out, int32_t out_dtype);
int oracle_ep_send(const void* x, int32_t x_dtype, int32_t T, int32_t H, const int32_t* topk_idx,
                   int32_t k, int32_t E, int32_t N, int32_t source, int32_t S, int32_t cap,
                   void* regions, int32_t* region_counts, int32_t* send_row);
int oracle_ep_recv(const void* regions, int32_t dtype, int32_t H, int32_t E, int32_t N, int32_t rank,
                   int32_t S, int32_t cap, const int32_t* region_counts, void* grouped,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* grouped_src);
int oracle_ep_return(const void* y_grouped, int32_t dtype, int32_t H, int64_t n_rows,
                     const int32_t* grouped_src, void* returns);
int oracle_ep_partial_rows(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t N,
                           int32_t source, int32_t S, int32_t pcap, int32_t* part_row,
                           int32_t* part_counts);
int oracle_ep_reduce(const void* y_grouped, int32_t dtype, int32_t H, int32_t E, int32_t N,
                     int32_t rank, int32_t S, int32_t cap, const int32_t* grouped_src, int32_t T,
                     int32_t k, const int32_t* topk_idx, const float* topk_w,
                     const int32_t* send_row, const int32_t* part_row, void* partials);
int oracle_ep_combine_reduced(const void* partials, int32_t dtype, int32_t T, int32_t H, int32_t N,
                              const int32_t* part_row, void* out, int32_t out_dtype);
int oracle_check_topk(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int64_t* counts);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform(void)      /* xorshift64*, in [0, 1) */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}

static size_t esize(int dt) { return dt == F32 ? 4 : dt == BF16 ? 2 : 1; }

static void* xalloc(size_t n)
{
    void* p = calloc(n ? n : 1, 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

#define REQUIRE(call)                                                                             \
    do {                                                                                          \
        if ((call) != 0) {                                                                        \
            fprintf(stderr, "rejected: %s (line %d)\n", #call, __LINE__);                         \
            return 1;                                                                             \
        }                                                                                         \
    } while (0)

/* route -> dispatch -> experts -> combine on one batch, then the id check */
static int chain(int T, int H, int E, int k, int N, int x_dt, int payload, int y_dt)
{
    const int R = T * k;
    float* logits = xalloc((size_t)T * E * sizeof(float));
    float* xf = xalloc((size_t)T * H * sizeof(float));
    void* x = xalloc((size_t)T * H * esize(x_dt));
    for (int64_t i = 0; i < (int64_t)T * E; i++)
        logits[i] = (float)(uniform() * 6.0 - 3.0);
    for (int64_t i = 0; i < (int64_t)T * H; i++)
        xf[i] = (float)(uniform() * 4.0 - 2.0);
    if (x_dt == F32)
        memcpy(x, xf, (size_t)T * H * sizeof(float));
    else
        oracle_f32_to_bf16(xf, (uint16_t*)x, (int64_t)T * H);
    int32_t* idx = xalloc((size_t)R * sizeof(int32_t));
    float* w = xalloc((size_t)R * sizeof(float));
    REQUIRE(oracle_route(logits, T, E, k, idx, w));
    void* recv = xalloc((size_t)R * H * esize(payload));
    float* scales = payload == FP8 ? xalloc((size_t)R * (H / 128) * sizeof(float)) : NULL;
    int32_t* ec = xalloc((size_t)E * sizeof(int32_t));
    int32_t* eo = xalloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* rc = xalloc((size_t)N * sizeof(int32_t));
    int32_t* ro = xalloc((size_t)(N + 1) * sizeof(int32_t));
    int32_t* tr = xalloc((size_t)R * sizeof(int32_t));
    int32_t* rt = xalloc((size_t)R * sizeof(int32_t));
    REQUIRE(oracle_dispatch(x, x_dt, T, H, idx, k, E, N, payload, recv, scales, ec, eo, rc, ro, tr,
                            rt));
    void* y = xalloc((size_t)R * H * esize(y_dt));
    REQUIRE(oracle_experts(recv, payload, scales, R, H, eo, E, 1, y, y_dt));
    void* out = xalloc((size_t)T * H * 4);
    REQUIRE(oracle_combine(y, y_dt, T, H, k, tr, w, out, F32));
    REQUIRE(oracle_combine(y, y_dt, T, H, k, tr, w, out, BF16));
    int64_t counts[2];
    REQUIRE(oracle_check_topk(idx, T, k, E, counts));
    if (T > 0)
        idx[0] = E;                                      /* out of range: dispatch must reject */
    if (T > 0 && oracle_dispatch(x, x_dt, T, H, idx, k, E, N, payload, recv, scales, ec, eo, rc,
                                 ro, tr, rt) == 0) {
        fprintf(stderr, "an out-of-range id was accepted\n");
        return 1;
    }
    REQUIRE(oracle_check_topk(idx, T, k, E, counts));
    free(logits); free(xf); free(x); free(idx); free(w); free(recv); free(scales);
    free(ec); free(eo); free(rc); free(ro); free(tr); free(rt); free(y); free(out);
    return 0;
}

/* expert parallelism over S sources and N ranks, with and without pre-reduction */
static int ep_chain(int S, int T, int H, int E, int k, int N, int dt)
{
    const int L = E / N, cap = T * (k < L ? k : L), TT = S * T, R = TT * k;
    float* logits = xalloc((size_t)TT * E * sizeof(float));
    float* xf = xalloc((size_t)TT * H * sizeof(float));
    void* x = xalloc((size_t)TT * H * esize(dt));
    for (int64_t i = 0; i < (int64_t)TT * E; i++)
        logits[i] = (float)(uniform() * 6.0 - 3.0);
    for (int64_t i = 0; i < (int64_t)TT * H; i++)
        xf[i] = (float)(uniform() * 4.0 - 2.0);
    if (dt == F32)
        memcpy(x, xf, (size_t)TT * H * sizeof(float));
    else
        oracle_f32_to_bf16(xf, (uint16_t*)x, (int64_t)TT * H);
    int32_t* idx = xalloc((size_t)R * sizeof(int32_t));
    float* w = xalloc((size_t)R * sizeof(float));
    REQUIRE(oracle_route(logits, TT, E, k, idx, w));
    const size_t rb = (size_t)H * esize(dt);
    char* regions = xalloc((size_t)N * S * cap * rb);
    int32_t* counts = xalloc((size_t)N * S * L * sizeof(int32_t));
    int32_t* send = xalloc((size_t)R * sizeof(int32_t));
    for (int s = 0; s < S; s++)
        REQUIRE(oracle_ep_send((const char*)x + (size_t)s * T * rb, dt, T, H, idx + (size_t)s * T * k,
                               k, E, N, s, S, cap, regions, counts, send + (size_t)s * T * k));
    char* returns = xalloc((size_t)N * S * cap * rb);
    int32_t* pcounts = xalloc((size_t)N * S * sizeof(int32_t));
    int32_t* prow = xalloc((size_t)TT * N * sizeof(int32_t));
    for (int s = 0; s < S; s++)
        REQUIRE(oracle_ep_partial_rows(idx + (size_t)s * T * k, T, k, E, N, s, S, T,
                                       prow + (size_t)s * T * N, pcounts));
    char* partials = xalloc((size_t)N * S * T * rb);
    for (int r = 0; r < N; r++) {
        char* grouped = xalloc((size_t)S * cap * rb);
        int32_t* gc = xalloc((size_t)L * sizeof(int32_t));
        int32_t* go = xalloc((size_t)(L + 1) * sizeof(int32_t));
        int32_t* gs = xalloc((size_t)S * cap * sizeof(int32_t));
        REQUIRE(oracle_ep_recv(regions, dt, H, E, N, r, S, cap, counts, grouped, gc, go, gs));
        char* y = xalloc((size_t)S * cap * rb);
        REQUIRE(oracle_experts(grouped, dt, NULL, go[L], H, go, L, 1, y, dt));
        REQUIRE(oracle_ep_return(y, dt, H, (int64_t)S * cap, gs, returns));
        REQUIRE(oracle_ep_reduce(y, dt, H, E, N, r, S, cap, gs, T, k, idx, w, send, prow,
                                 partials));
        free(grouped); free(gc); free(go); free(gs); free(y);
    }
    void* out = xalloc((size_t)T * H * 4);
    for (int s = 0; s < S; s++) {
        REQUIRE(oracle_combine(returns, dt, T, H, k, send + (size_t)s * T * k, w + (size_t)s * T * k,
                               out, dt));
        REQUIRE(oracle_ep_combine_reduced(partials, dt, T, H, N, prow + (size_t)s * T * N, out,
                                          F32));
    }
    free(logits); free(xf); free(x); free(idx); free(w); free(regions); free(counts); free(send);
    free(returns); free(pcounts); free(prow); free(partials); free(out);
    return 0;
}

static int conversions(void)
{
    enum { n = 4096 };
    float* f = xalloc(n * sizeof(float));
    double* d = xalloc(n * sizeof(double));
    uint16_t* b = xalloc(n * sizeof(uint16_t));
    uint8_t* q = xalloc(n);
    float* back = xalloc(n * sizeof(float));
    const float special[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 448.0f, -448.0f, 449.0f,
                             1e-30f, -1e-45f, 3.4e38f, 1.0f / 512.0f, 0.0009765625f};
    for (int i = 0; i < n; i++) {
        f[i] = i < (int)(sizeof special / sizeof special[0]) ? special[i]
                                                               : (float)((uniform() - 0.5) * 1000.0);
        d[i] = (double)f[i] * (1.0 + 1e-12);
        q[i] = (uint8_t)i;
    }
    oracle_f32_to_bf16(f, b, n);
    oracle_f64_to_bf16(d, b, n);
    oracle_f32_to_e4m3(f, q, n);
    for (int i = 0; i < 256; i++)
        q[i] = (uint8_t)i;
    oracle_e4m3_to_f32(q, back, n);
    free(f); free(d); free(b); free(q); free(back);
    return 0;
}

int main(void)
{
    if (conversions())
        return 1;
    /* T, H, E, k, N, x, payload, y */
    if (chain(16, 256, 8, 2, 2, F32, F32, F32) || chain(37, 256, 12, 3, 4, BF16, BF16, BF16) ||
        chain(9, 384, 16, 4, 8, BF16, FP8, BF16) || chain(5, 128, 8, 8, 1, F32, FP8, F32) ||
        chain(0, 128, 8, 2, 2, BF16, BF16, BF16) || chain(3, 128, 64, 64, 64, F32, F32, F32))
        return 1;
    /* S, T, H, E, k, N, dtype */
    if (ep_chain(3, 10, 256, 8, 2, 4, F32) || ep_chain(4, 7, 128, 32, 8, 8, BF16) ||
        ep_chain(2, 6, 128, 8, 2, 4, F32))
        return 1;
    /* arguments the oracle must reject */
    int32_t idx[4] = {0, 1, 2, 3};
    float w[4];
    if (oracle_route(NULL, 1, 4, 5, idx, w) == 0 || oracle_check_topk(idx, 1, 0, 4, NULL) == 0)
        return 1;
    printf("oracle sanitizer run: ok\n");
    return 0;
}
