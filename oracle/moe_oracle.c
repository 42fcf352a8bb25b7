/*
 * moe_oracle.c -- plain, slow, single-threaded CPU oracle for MoE top-k routing, token dispatch and
 * weighted combine.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU-baseline leg are
 * the only callers. The HIP library neither links nor calls this code, and the two share no
 * source, header, table or helper.
 *
 * What is computed follows Perplexity, "Enabling trillion-parameter models on AWS EFA":
 *   - "Introductie": a small linear router picks the experts of each token; dispatch sends every
 *     token to the ranks hosting its experts, combine takes back the processed copies and forms
 *     their weighted average.
 *   - "MoE all-to-all over EFA": dispatch receives the tokens and the per-token experts; combine
 *     returns the tokens to their source and averages them before handing them to the model.
 *   - "Verzend- en ontvangstbuffers": per-expert token counts are known before any row is written,
 *     so writes to each destination are laid out contiguously.
 *   - "Dispatch en Combine": per-expert counts, then a cumulative sum gives the offsets at which
 *     tokens are packed into contiguous per-destination buffers; combine accumulates the received
 *     rows into the output tensor.
 *   - "Evaluatie / Dispatch/Combine-latentie": block-scaled fp8 dispatch and bf16 combine.
 * Readings where the page is silent (softmax scoring with renormalisation over the top-k, ties to
 * the lower expert id, rows ordered by (rank, expert, token, slot), 1x128 fp8 blocks with an fp32
 * absmax/448 scale, contiguous expert-to-rank blocks) are stated at each function.
 *
 * Precision: real-valued results (routing weights, combine sums) are computed in double and rounded
 * once to the output format. Where floating point decides an integer code (fp8 quantisation), the
 * decision is taken in fp32, the precision of the GPU kernel. Build with
 * gcc -O2 -ffp-contract=off (no fast-math), so every C operator is one IEEE-754 operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2 };
enum { ORC_EXPERTS_IDENTITY = 0, ORC_EXPERTS_SCALE = 1 };

/* ------------------------------------------------------------------------------------------------
 * Number formats, from their definitions.
 * bf16: IEEE-754 binary32 with the significand cut to 8 bits (same exponent range).
 * e4m3fn (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; smallest
 * normal 2^-6; subnormals m/8 * 2^-6.
 * ---------------------------------------------------------------------------------------------- */

/* Nearest value to a >= 0 (finite) that has `p` significand bits and an exponent of at least
 * `emin`; below 2^emin every value shares the quantum 2^(emin-p+1). Ties go to the even
 * neighbour: the default rounding mode of nearbyint is round-to-nearest-even. Every step is exact
 * in double for the formats used here, so this is one correctly rounded operation. */
static double round_to_format(double a, int p, int emin)
{
    if (a == 0.0)
        return 0.0;
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2 with f in [0.5, 1): floor(log2 a) = e2 - 1 */
    int ex = e2 - 1;
    if (ex < emin)
        ex = emin;
    double quantum = ldexp(1.0, ex - (p - 1));
    return nearbyint(a / quantum) * quantum;
}

static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bf16 nearest to a double (ties to even); overflow gives infinity, NaN gives the quiet NaN. */
static uint16_t bf16_bits_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    double r = round_to_format(a, 8, -126);
    if (r >= 0x1p128)
        return sign | 0x7F80;
    float rf = (float)r;    /* exact: r has at most 8 significand bits and lies in float range */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return sign | (uint16_t)(u >> 16);
}

/* Value of an e4m3fn code. */
static double e4m3_value(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    if (ex == 15 && m == 7)
        return NAN;
    double mag = (ex == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), ex - 10);
    return s ? -mag : mag;
}

/* e4m3fn code nearest to a float, ties to even, saturating: magnitudes beyond the largest finite
 * value 448 (infinity included) give +-448. NaN gives the NaN code with the input's sign. */
static uint8_t e4m3_from_float(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v))
        return sign | 0x7F;
    double a = fabs((double)v);
    if (a > 448.0)
        a = 448.0;
    double r = round_to_format(a, 4, -6);
    if (r == 0.0)
        return sign;
    int e2;
    frexp(r, &e2);
    int ex = e2 - 1;
    if (ex < -6)                                   /* subnormal: r = m * 2^-9, m in 1..7 */
        return sign | (uint8_t)(r * 512.0);
    int m = (int)ldexp(r, 3 - ex) - 8;             /* r = (8 + m) * 2^(ex-3), m in 0..7 */
    return sign | (uint8_t)(((ex + 7) << 3) | m);
}

/* Element i of a row-major buffer in format `dt`, as a double (fp8 elements exclude the scale). */
static double load_elem(const void* p, int dt, int64_t i)
{
    switch (dt) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return (double)bf16_bits_to_float(((const uint16_t*)p)[i]);
    default: return e4m3_value(((const uint8_t*)p)[i]);
    }
}

static size_t elem_size(int dt) { return dt == ORC_F32 ? 4 : dt == ORC_BF16 ? 2 : 1; }

/* ------------------------------------------------------------------------------------------------
 * Conversions exported for the tests that pin the formats above.
 * ---------------------------------------------------------------------------------------------- */
void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_bits_from_double((double)in[i]);
}

void oracle_f64_to_bf16(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_bits_from_double(in[i]);
}

void oracle_f32_to_e4m3(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = e4m3_from_float(in[i]);
}

void oracle_e4m3_to_f32(const uint8_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (float)e4m3_value(in[i]);
}

/* ------------------------------------------------------------------------------------------------
 * Routing ("Introductie": a small linear routing layer decides which experts multiply a token).
 * Reading: softmax over all E logits, the k experts of largest logit are kept, and their
 * probabilities are renormalised to sum to one. Slots are ordered by logit, largest first; equal
 * logits go to the lower expert id (so -0.0 and +0.0 tie). Logits must be finite.
 * ---------------------------------------------------------------------------------------------- */

/* Expert a comes before expert b in the selection order of logit row l. */
static int selected_before(const float* l, int a, int b)
{
    return l[a] > l[b] || (l[a] == l[b] && a < b);
}

int oracle_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                 float* topk_w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return 1;
    char* taken = (char*)malloc((size_t)E);
    double* p = (double*)malloc((size_t)E * sizeof(double));
    if (!taken || !p) {
        free(taken);
        free(p);
        return 2;
    }
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * (int64_t)E;
        int32_t* idx = topk_idx + t * (int64_t)k;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {           /* j-th best of the experts not yet taken */
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || selected_before(l, e, best)))
                    best = e;
            taken[best] = 1;
            idx[j] = best;
        }
        /* softmax over all experts, shifted by the largest logit (that of slot 0) */
        double mx = (double)l[idx[0]];
        double z = 0.0;
        for (int e = 0; e < E; e++) {
            p[e] = exp((double)l[e] - mx);
            z += p[e];
        }
        for (int e = 0; e < E; e++)
            p[e] /= z;
        double kept = 0.0;                      /* renormalise over the k kept experts */
        for (int j = 0; j < k; j++)
            kept += p[idx[j]];
        for (int j = 0; j < k; j++)
            topk_w[t * (int64_t)k + j] = (float)(p[idx[j]] / kept);
    }
    free(taken);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Dispatch ("Verzend- en ontvangstbuffers", "Dispatch en Combine").
 *   counts: expert_counts[e] = number of (token, slot) pairs routed to expert e;
 *   rank r hosts the contiguous expert block [r*E/N, (r+1)*E/N) (reading; the page names no
 *   mapping), rank_counts[r] = sum of its experts' counts;
 *   offsets: exclusive cumulative sums, expert_offsets[E] = rank_offsets[N] = T*k;
 *   layout: every (token, slot) pair gets one row; rows are ordered by the key
 *   (rank, expert, token, slot), so each rank's rows are contiguous and, inside, grouped per expert
 *   in token order (the grouped-GEMM input the receiver fills in "Dispatch en Combine");
 *   payload: row token_row[t*k+j] holds token t, as the same bytes for f32/bf16, or as block-scaled
 *   fp8 (reading of "block-scaled fp8-dispatch": per token and per block of 128 consecutive
 *   elements, amax = max |x| over the elements that are not NaN, scale s = amax/448 in fp32, or 1
 *   if amax = 0, code = e4m3(x/s) rounded to nearest even and saturated at 448; all fp32
 *   operations, as on the GPU. s is positive, so every quotient has the sign of x; IEEE 754 leaves
 *   the sign of a NaN result open (an infinite x over an infinite s), and it is taken as x's too).
 * Expert ids must lie in [0, E); a repeated id in one token is two separate items.
 * ---------------------------------------------------------------------------------------------- */
typedef struct {
    int32_t rank, expert, token, slot;
} orc_item_t;

static int item_cmp(const void* pa, const void* pb)
{
    const orc_item_t* a = (const orc_item_t*)pa;
    const orc_item_t* b = (const orc_item_t*)pb;
    if (a->rank != b->rank) return a->rank < b->rank ? -1 : 1;
    if (a->expert != b->expert) return a->expert < b->expert ? -1 : 1;
    if (a->token != b->token) return a->token < b->token ? -1 : 1;
    if (a->slot != b->slot) return a->slot < b->slot ? -1 : 1;
    return 0;
}

int oracle_dispatch(const void* x, int32_t x_dtype, int32_t T, int32_t H, const int32_t* topk_idx,
                    int32_t k, int32_t E, int32_t N, int32_t payload_dtype, void* recv,
                    float* recv_scales, int32_t* expert_counts, int32_t* expert_offsets,
                    int32_t* rank_counts, int32_t* rank_offsets, int32_t* token_row,
                    int32_t* row_token)
{
    if (T < 0 || H < 1 || k < 1 || E < 1 || N < 1 || E % N != 0)
        return 1;
    if (x_dtype == ORC_FP8_E4M3 || (payload_dtype != x_dtype && payload_dtype != ORC_FP8_E4M3))
        return 1;
    if (payload_dtype == ORC_FP8_E4M3 && H % 128 != 0)
        return 1;
    const int64_t R = (int64_t)T * k;
    const int32_t epr = E / N;
    for (int64_t i = 0; i < R; i++)
        if (topk_idx[i] < 0 || topk_idx[i] >= E)
            return 1;

    /* counts and offsets */
    for (int e = 0; e < E; e++)
        expert_counts[e] = 0;
    for (int64_t i = 0; i < R; i++)
        expert_counts[topk_idx[i]]++;
    expert_offsets[0] = 0;
    for (int e = 0; e < E; e++)
        expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];
    for (int r = 0; r < N; r++) {
        rank_counts[r] = 0;
        for (int e = r * epr; e < (r + 1) * epr; e++)
            rank_counts[r] += expert_counts[e];
    }
    rank_offsets[0] = 0;
    for (int r = 0; r < N; r++)
        rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];

    /* layout: sort every (token, slot) item by (rank, expert, token, slot); its position is its row */
    orc_item_t* items = (orc_item_t*)malloc((size_t)(R > 0 ? R : 1) * sizeof(orc_item_t));
    if (!items)
        return 2;
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            orc_item_t* it = &items[t * k + j];
            it->expert = topk_idx[t * k + j];
            it->rank = it->expert / epr;
            it->token = (int32_t)t;
            it->slot = j;
        }
    qsort(items, (size_t)R, sizeof(orc_item_t), item_cmp);
    for (int64_t row = 0; row < R; row++) {
        token_row[(int64_t)items[row].token * k + items[row].slot] = (int32_t)row;
        row_token[row] = items[row].token;
    }
    free(items);

    /* payload */
    if (payload_dtype != ORC_FP8_E4M3) {
        const size_t rb = (size_t)H * elem_size(x_dtype);
        for (int64_t i = 0; i < R; i++)
            memcpy((char*)recv + (size_t)token_row[i] * rb, (const char*)x + (size_t)(i / k) * rb,
                   rb);
        return 0;
    }
    const int nb = H / 128;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* s = (float*)malloc((size_t)nb * sizeof(float));
    if (!q || !s) {
        free(q);
        free(s);
        return 2;
    }
    for (int64_t t = 0; t < T; t++) {
        for (int b = 0; b < nb; b++) {
            float amax = 0.0f;
            for (int h = b * 128; h < (b + 1) * 128; h++) {
                float a = fabsf((float)load_elem(x, x_dtype, t * (int64_t)H + h));
                if (a > amax)
                    amax = a;
            }
            s[b] = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            for (int h = b * 128; h < (b + 1) * 128; h++) {
                float xv = (float)load_elem(x, x_dtype, t * (int64_t)H + h);
                float scaled = copysignf(xv / s[b], xv);   /* s > 0: changes only a NaN's sign */
                q[h] = e4m3_from_float(scaled);
            }
        }
        for (int j = 0; j < k; j++) {
            int64_t row = token_row[t * k + j];
            memcpy((uint8_t*)recv + row * H, q, (size_t)H);
            memcpy(recv_scales + row * nb, s, (size_t)nb * sizeof(float));
        }
    }
    free(q);
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Emulated experts (stand-in for the grouped GEMM of "MoE all-to-all over EFA"; harness only).
 * Row r belongs to the expert e whose segment [expert_offsets[e], expert_offsets[e+1]) holds it.
 * identity: y = value of the row; scale: y = value * (e+1)/256. The value of an fp8 element is
 * code value * block scale. Each result is rounded once to y's format.
 * ---------------------------------------------------------------------------------------------- */
int oracle_experts(const void* recv, int32_t payload_dtype, const float* recv_scales, int32_t R,
                   int32_t H, const int32_t* expert_offsets, int32_t E, int32_t rule, void* y,
                   int32_t y_dtype)
{
    if (y_dtype == ORC_FP8_E4M3 || (payload_dtype == ORC_FP8_E4M3 && H % 128 != 0))
        return 1;
    int e = 0;
    for (int64_t r = 0; r < R; r++) {
        while (e < E && expert_offsets[e + 1] <= r)
            e++;
        double f = (rule == ORC_EXPERTS_SCALE) ? (double)(e + 1) / 256.0 : 1.0;
        for (int64_t h = 0; h < H; h++) {
            double v = load_elem(recv, payload_dtype, r * H + h);
            if (payload_dtype == ORC_FP8_E4M3)
                v *= (double)recv_scales[r * (H / 128) + h / 128];
            v *= f;
            if (y_dtype == ORC_F32)
                ((float*)y)[r * H + h] = (float)v;
            else
                ((uint16_t*)y)[r * H + h] = bf16_bits_from_double(v);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Combine ("Dispatch en Combine": the receiver accumulates the returned rows of every token into
 * the output tensor, as the weighted average of "Introductie"; the weights are renormalised, so
 * the weighted sum is that average).
 *   out[t, h] = sum_j w[t, j] * y[token_row[t*k+j], h], in double, rounded once to out's format.
 * ---------------------------------------------------------------------------------------------- */
int oracle_combine(const void* y, int32_t y_dtype, int32_t T, int32_t H, int32_t k,
                   const int32_t* token_row, const float* topk_w, void* out, int32_t out_dtype)
{
    if (y_dtype == ORC_FP8_E4M3 || out_dtype == ORC_FP8_E4M3)
        return 1;
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) {
                int64_t row = token_row[t * k + j];
                acc += (double)topk_w[t * k + j] * load_elem(y, y_dtype, row * H + h);
            }
            if (out_dtype == ORC_F32)
                ((float*)out)[t * H + h] = (float)acc;
            else
                ((uint16_t*)out)[t * H + h] = bf16_bits_from_double(acc);
        }
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Expert parallelism over several devices, emulated on one: S sources (the devices that own the
 * tokens) and N destination ranks (the devices that host the experts; rank r hosts the L = E/N
 * experts [r*L, (r+1)*L)). The pages split dispatch and combine into a sender half and a receiver
 * half ("MoE all-to-all over EFA"), size every receive buffer for the worst case before any row is
 * written, and let each sender write its rows into the receiver's buffer, after which the receiver
 * copies them into the input of its grouped GEMM ("Verzend- en ontvangstbuffers", "Dispatch en
 * Combine"). Readings:
 *   - the receive buffer of rank r holds one region of `cap` rows per source s, at rows
 *     [(r*S + s)*cap, (r*S + s + 1)*cap) of one [N*S*cap, H] array; cap >= T*min(k, L), the most
 *     rows one source can send to one rank when a token's experts are distinct (ids repeated
 *     within a token that overflow a region are rejected);
 *   - inside its region a source's rows are ordered by (local expert, token, slot), and the
 *     source publishes region_counts[(r*S + s)*L + l], its rows for expert r*L + l;
 *   - the receiver's grouped layout is ordered by (local expert, source, token, slot);
 *   - combine sends every grouped row back to the region row it came from, and the source then
 *     forms the weighted sum over its token's rows there (the combine above, with the region rows
 *     as token_row).
 * ---------------------------------------------------------------------------------------------- */

/* Sender half of dispatch for source `source`: region rows, region counts, and for every (token,
 * slot) item its row in the region array (send_row[t*k + j]). Payload is x's format. */
int oracle_ep_send(const void* x, int32_t x_dtype, int32_t T, int32_t H, const int32_t* topk_idx,
                   int32_t k, int32_t E, int32_t N, int32_t source, int32_t S, int32_t cap,
                   void* regions, int32_t* region_counts, int32_t* send_row)
{
    if (T < 0 || H < 1 || k < 1 || E < 1 || N < 1 || E % N != 0 || S < 1 || source < 0 ||
        source >= S || x_dtype == ORC_FP8_E4M3)
        return 1;
    const int32_t L = E / N;
    if ((int64_t)cap < (int64_t)T * (k < L ? k : L))
        return 1;
    const int64_t R = (int64_t)T * k;
    for (int64_t i = 0; i < R; i++)
        if (topk_idx[i] < 0 || topk_idx[i] >= E)
            return 1;
    for (int r = 0; r < N; r++)
        for (int l = 0; l < L; l++)
            region_counts[((int64_t)r * S + source) * L + l] = 0;
    for (int64_t i = 0; i < R; i++) {
        const int e = topk_idx[i];
        region_counts[((int64_t)(e / L) * S + source) * L + e % L]++;
    }
    for (int r = 0; r < N; r++) {                      /* ids repeated in a token can overflow */
        int64_t n = 0;
        for (int l = 0; l < L; l++)
            n += region_counts[((int64_t)r * S + source) * L + l];
        if (n > cap)
            return 1;
    }
    orc_item_t* items = (orc_item_t*)malloc((size_t)(R > 0 ? R : 1) * sizeof(orc_item_t));
    if (!items)
        return 2;
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            orc_item_t* it = &items[t * k + j];
            it->expert = topk_idx[t * k + j];
            it->rank = it->expert / L;
            it->token = (int32_t)t;
            it->slot = j;
        }
    qsort(items, (size_t)R, sizeof(orc_item_t), item_cmp);
    const size_t rb = (size_t)H * elem_size(x_dtype);
    int64_t pos = 0;
    for (int64_t n = 0; n < R; n++) {
        if (n > 0 && items[n].rank != items[n - 1].rank)
            pos = 0;                                   /* a new destination rank: its region */
        const int64_t row = ((int64_t)items[n].rank * S + source) * cap + pos;
        pos++;
        send_row[(int64_t)items[n].token * k + items[n].slot] = (int32_t)row;
        memcpy((char*)regions + (size_t)row * rb, (const char*)x + (size_t)items[n].token * rb, rb);
    }
    free(items);
    return 0;
}

/* Receiver half of dispatch for rank `rank`: the grouped layout [S*cap, H] ordered by (local
 * expert, source, token, slot), its per-expert counts and offsets, and for every grouped row the
 * region row it was copied from (grouped_src; -1 past the last row). */
int oracle_ep_recv(const void* regions, int32_t dtype, int32_t H, int32_t E, int32_t N, int32_t rank,
                   int32_t S, int32_t cap, const int32_t* region_counts, void* grouped,
                   int32_t* expert_counts, int32_t* expert_offsets, int32_t* grouped_src)
{
    if (H < 1 || E < 1 || N < 1 || E % N != 0 || S < 1 || rank < 0 || rank >= N ||
        dtype == ORC_FP8_E4M3 || cap < 0)
        return 1;
    const int32_t L = E / N;
    const size_t rb = (size_t)H * elem_size(dtype);
    int64_t g = 0;
    for (int l = 0; l < L; l++) {
        expert_offsets[l] = (int32_t)g;
        for (int s = 0; s < S; s++) {
            const int32_t* c = region_counts + ((int64_t)rank * S + s) * L;
            int64_t start = 0;
            for (int q = 0; q < l; q++)
                start += c[q];
            if (start + c[l] > cap)
                return 1;
            for (int64_t i = 0; i < c[l]; i++) {
                const int64_t src = ((int64_t)rank * S + s) * cap + start + i;
                grouped_src[g] = (int32_t)src;
                memcpy((char*)grouped + (size_t)g * rb, (const char*)regions + (size_t)src * rb,
                       rb);
                g++;
            }
        }
        expert_counts[l] = (int32_t)g - expert_offsets[l];
    }
    expert_offsets[L] = (int32_t)g;
    for (int64_t q = g; q < (int64_t)S * cap; q++)
        grouped_src[q] = -1;
    return 0;
}

/* Receiver half of combine: every grouped row of expert output goes back to the region row it
 * came from (returns has the layout of the region array). */
int oracle_ep_return(const void* y_grouped, int32_t dtype, int32_t H, int64_t n_rows,
                     const int32_t* grouped_src, void* returns)
{
    if (H < 1 || dtype == ORC_FP8_E4M3 || n_rows < 0)
        return 1;
    const size_t rb = (size_t)H * elem_size(dtype);
    for (int64_t g = 0; g < n_rows; g++)
        if (grouped_src[g] >= 0)
            memcpy((char*)returns + (size_t)grouped_src[g] * rb, (const char*)y_grouped + g * rb,
                   rb);
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * Combine with pre-reduction on the expert side ("Evaluatie / Dispatch/Combine-latentie": the pages
 * accumulate only on the receiver, which is why they lag at prefill). Reading: before the return
 * trip, rank r sums, for every token t of source s that has experts on r, the weighted outputs of
 * those experts into one partial row, P[r, s, t] = sum over slots j with rank(idx[t, j]) = r of
 * w[t, j] * y(t, j), rounded once to the wire format; only partial rows travel back, and the
 * source finishes out[t] = sum over ranks of P[r, s, t], rounded once.
 *   - the partial rows of (rank r, source s) sit in a region of pcap >= T rows at rows
 *     [(r*S + s)*pcap, ...) of the partial array, one row per token of s with experts on r, in
 *     token order; part_row[t*N + r] is that row, or -1 when t has no expert on r;
 *   - sums are exact (double) and rounded once, at the partial and at the output.
 * ---------------------------------------------------------------------------------------------- */

/* Where the partial rows of source `source` go: part_row [T, N] and part_counts[r*S + source]. */
int oracle_ep_partial_rows(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int32_t N,
                           int32_t source, int32_t S, int32_t pcap, int32_t* part_row,
                           int32_t* part_counts)
{
    if (T < 0 || k < 1 || E < 1 || N < 1 || E % N != 0 || S < 1 || source < 0 || source >= S ||
        pcap < T)
        return 1;
    const int32_t L = E / N;
    for (int r = 0; r < N; r++) {
        int32_t p = 0;
        for (int64_t t = 0; t < T; t++) {
            int on_rank = 0;
            for (int j = 0; j < k; j++)
                if (topk_idx[t * k + j] / L == r)
                    on_rank = 1;
            part_row[t * N + r] = on_rank ? (int32_t)(((int64_t)r * S + source) * pcap + p) : -1;
            p += on_rank;
        }
        part_counts[(int64_t)r * S + source] = p;
    }
    return 0;
}

/* Expert side: the partial rows of rank `rank` for every source. y_grouped holds the rank's
 * expert outputs in its grouped layout and grouped_src (from receive) names each grouped row's
 * region row; topk_idx / topk_w / send_row / part_row are the sources' tables, source s at
 * [s*T, (s+1)*T) tokens. */
int oracle_ep_reduce(const void* y_grouped, int32_t dtype, int32_t H, int32_t E, int32_t N,
                     int32_t rank, int32_t S, int32_t cap, const int32_t* grouped_src, int32_t T,
                     int32_t k, const int32_t* topk_idx, const float* topk_w,
                     const int32_t* send_row, const int32_t* part_row, void* partials)
{
    if (H < 1 || E < 1 || N < 1 || E % N != 0 || S < 1 || rank < 0 || rank >= N || T < 0 ||
        k < 1 || dtype == ORC_FP8_E4M3)
        return 1;
    const int32_t L = E / N;
    /* grouped row of every region row of this rank */
    const int64_t base = (int64_t)rank * S * cap, nreg = (int64_t)S * cap;
    int64_t* grouped_of = (int64_t*)malloc((size_t)(nreg > 0 ? nreg : 1) * sizeof(int64_t));
    if (!grouped_of)
        return 2;
    for (int64_t q = 0; q < nreg; q++)
        grouped_of[q] = -1;
    for (int64_t g = 0; g < nreg; g++)
        if (grouped_src[g] >= 0)
            grouped_of[grouped_src[g] - base] = g;
    for (int s = 0; s < S; s++)
        for (int64_t t = 0; t < T; t++) {
            const int64_t tt = (int64_t)s * T + t;
            const int32_t pr = part_row[tt * N + rank];
            if (pr < 0)
                continue;
            for (int64_t h = 0; h < H; h++) {
                double acc = 0.0;
                for (int j = 0; j < k; j++) {
                    if (topk_idx[tt * k + j] / L != rank)
                        continue;
                    const int64_t q = send_row[tt * k + j] - base;
                    const int64_t g = (q >= 0 && q < nreg) ? grouped_of[q] : -1;
                    if (g < 0) {
                        free(grouped_of);
                        return 1;
                    }
                    acc += (double)topk_w[tt * k + j] * load_elem(y_grouped, dtype, g * H + h);
                }
                if (dtype == ORC_F32)
                    ((float*)partials)[(int64_t)pr * H + h] = (float)acc;
                else
                    ((uint16_t*)partials)[(int64_t)pr * H + h] = bf16_bits_from_double(acc);
            }
        }
    free(grouped_of);
    return 0;
}

/* Source side: out[t] = sum over ranks of the partial rows of token t, rounded once. */
int oracle_ep_combine_reduced(const void* partials, int32_t dtype, int32_t T, int32_t H, int32_t N,
                              const int32_t* part_row, void* out, int32_t out_dtype)
{
    if (T < 0 || H < 1 || N < 1 || dtype == ORC_FP8_E4M3 || out_dtype == ORC_FP8_E4M3)
        return 1;
    for (int64_t t = 0; t < T; t++)
        for (int64_t h = 0; h < H; h++) {
            double acc = 0.0;
            for (int r = 0; r < N; r++) {
                const int32_t pr = part_row[t * N + r];
                if (pr >= 0)
                    acc += load_elem(partials, dtype, (int64_t)pr * H + h);
            }
            if (out_dtype == ORC_F32)
                ((float*)out)[t * H + h] = (float)acc;
            else
                ((uint16_t*)out)[t * H + h] = bf16_bits_from_double(acc);
        }
    return 0;
}

/* ------------------------------------------------------------------------------------------------
 * The routing precondition of dispatch. Dispatch is handed, for every token, the experts it goes
 * to ("MoE all-to-all over EFA"); the router picks k of the E experts for each token
 * ("Introductie"), so every id names an expert and no token names one expert twice.
 * counts[0] = number of slots (t, j) whose id lies outside [0, E);
 * counts[1] = number of slots (t, j) whose id lies in [0, E) and equals the id of an earlier slot
 *             j' < j of the same token (a token naming one expert three times counts 2).
 * ---------------------------------------------------------------------------------------------- */
int oracle_check_topk(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, int64_t* counts)
{
    if (T < 0 || k < 1 || E < 1)
        return 1;
    counts[0] = 0;
    counts[1] = 0;
    for (int64_t t = 0; t < T; t++)
        for (int32_t j = 0; j < k; j++) {
            const int32_t id = topk_idx[t * k + j];
            if (id < 0 || id >= E) {
                counts[0]++;
                continue;
            }
            for (int32_t jj = 0; jj < j; jj++)
                if (topk_idx[t * k + jj] == id) {
                    counts[1]++;
                    break;
                }
        }
    return 0;
}
