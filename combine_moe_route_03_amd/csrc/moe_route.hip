// moe_route.hip -- HIP kernels for CDNA4 (gfx950) and the C ABI declared in include/moe_route.h.
//
// MoE token routing on one GPU, after Perplexity, "Enabling trillion-parameter models on AWS EFA":
// top-k routing ("Introductie"), per-expert counts and their cumulative sum ("Verzend- en
// ontvangstbuffers", "Dispatch en Combine"), packing of token rows into contiguous per-destination
// buffers, optionally block-scaled fp8 ("Evaluatie / Dispatch/Combine-latentie"), and the
// receiver-side weighted accumulation of combine ("Dispatch en Combine").
//
// The path moves bytes; it has no dense contraction, so it uses no MFMA. Every kernel is bound by
// HBM bandwidth or by latency:
//   k_route_topk     one wavefront per token, k rounds of a wave-wide 64-bit max built from DPP
//                    row operations and four readlanes;
//   k_layout_hist    per block of items: stable in-block ranks from LDS bit masks, and the
//                    block's expert histogram, stored expert-major;
//   k_layout_scan    one workgroup: per expert, a DPP wave scan over the blocks' counts gives
//                    the rows of that expert in earlier blocks; a block scan over the expert
//                    totals gives the expert offsets;
//   k_layout_rows    token_row / row_token from the scan, the in-block ranks and the ids;
//   k_pack_rows      one wavefront per (token, slot, part of the row): reads the x row (from the
//                    XCD's L2 after the first of the token's wavefronts) and writes one whole
//                    contiguous row with 16-byte non-temporal stores;
//   k_pack_rows_fp8  same, quantising 1x128 blocks to e4m3 with an fp32 absmax/448 scale;
//   k_combine        one wavefront per (token, 512-element segment): all k row loads in flight,
//                    fp32 fused multiply-adds, one 16-byte store per 8 outputs.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe_route.h"

namespace {

constexpr int kThreads = 256;            // route / layout workgroups: 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kScanThreads = 1024;       // the single scan workgroup: 16 wavefronts
constexpr int kMaxLayoutBlocks = 64;     // histogram blocks: one per lane of a scan wavefront
constexpr int kPackWaves = 2;            // wavefronts per pack workgroup
constexpr int kCombineWaves = 2;         // wavefronts per combine workgroup
constexpr int kXcds = 8;                 // workgroup b runs on XCD b % 8 (round-robin dispatch)
constexpr int64_t kTargetWaves = 16384;  // wavefronts the row kernels aim for (64 per CU)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------- number formats --
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// bf16 nearest to f, ties to even (add half an ulp minus one, plus the kept lsb, then truncate).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) | 0x40u) & 0xFFFFu;           // NaN stays a quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP e4m3fn code nearest to v, ties to even, saturating to +-448 (the largest finite value).
// Normal codes: keep 3 of the 23 fp32 mantissa bits with round-to-nearest-even on the 20 dropped
// bits, then rebias the exponent from 127 to 7. Below 2^-6 the quantum is 2^-9 for every value.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;                            // NaN
    if (a >= 0x43E00000u)                               // |v| >= 448 (infinity included)
        return sign | 0x7Eu;
    if (a < 0x3C800000u) {                              // |v| < 2^-6: multiples of 2^-9
        const float m = rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE to 0..8
        return sign | (uint32_t)m;
    }
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // exponent(8) | mantissa(3)
    return sign | (r - (120u << 3));                    // 120 = 127 - 7
}

// ------------------------------------------------------------------------------- wave helpers --
// DPP controls (CDNA row = 16 lanes): quad_perm [1,0,3,2] and [2,3,0,1] exchange within quads,
// row_half_mirror pairs lane i with 7-i, row_mirror pairs lane i with 15-i. Applied in that order
// with an associative operator they leave the row's reduction in every lane of the row.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ double dpp_add_f64(double x)
{
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    return x + __longlong_as_double((long long)dpp_u64<CTRL>(b));
}

// Sum over all 64 lanes (all active), the same value in every lane; fixed summation order.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v = dpp_add_f64<kDppQuadXor1>(v);
    v = dpp_add_f64<kDppQuadXor2>(v);
    v = dpp_add_f64<kDppRowHalfMirror>(v);
    v = dpp_add_f64<kDppRowMirror>(v);
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const double r0 = __longlong_as_double((long long)readlane_u64(b, 0));
    const double r1 = __longlong_as_double((long long)readlane_u64(b, 16));
    const double r2 = __longlong_as_double((long long)readlane_u64(b, 32));
    const double r3 = __longlong_as_double((long long)readlane_u64(b, 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float max_row16_f32(float v)
{
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadXor1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuadXor2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(v))));
    return v;
}

// ---------------------------------------------------------------------------------- routing --
// Selection key: larger logit first, equal logits to the lower id. The float is mapped to an
// unsigned integer with the same order (sign-magnitude to offset binary; -0 folded onto +0) and
// the id is stored inverted in the low word. Key 0 never wins: every finite logit maps above it.
__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u)
        u = 0u;
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float route_key_logit(uint64_t key)
{
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Maximum over all 64 lanes (all active), the same value in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// One wavefront per token. Lane l holds experts l, l+64, ... (coalesced loads) and sorts its
// keys once, largest first, so its best remaining candidate is always key[0]. Each of the k
// rounds takes the wave-wide maximum of the candidates' logit words; when a single lane holds it
// (the usual case, found with one ballot) that lane wins, otherwise the lowest expert id among
// the tied lanes wins. The winner drops its head. The weights use double-precision exp and
// division, rounded once to fp32.
template <int PL>
__global__ __launch_bounds__(kThreads) void k_route_topk(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= T)
        return;                                          // uniform: whole wavefronts leave
    const float* l = logits + t * E;
    uint64_t key[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        const int e = lane + 64 * p;
        key[p] = (e < E) ? route_key(l[e], e) : 0ull;
    }
#pragma unroll
    for (int r = 0; r < PL; ++r)                        // odd-even transposition sort, descending
#pragma unroll
        for (int p = r & 1; p + 1 < PL; p += 2)
            if (key[p] < key[p + 1]) {
                const uint64_t tmp = key[p];
                key[p] = key[p + 1];
                key[p + 1] = tmp;
            }
    int my_id = 0;
    float my_logit = 0.0f, top_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        const uint32_t hi = (uint32_t)(key[0] >> 32);
        const uint32_t best_hi = wave_max_u32(hi);
        const uint64_t holders = __builtin_amdgcn_ballot_w64(hi == best_hi);
        uint32_t id;
        if (__popcll(holders) == 1) {
            id = ~(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0],
                                                      (int)__builtin_ctzll(holders));
        } else {                                        // equal logits: lowest id wins
            const uint32_t lo = (hi == best_hi) ? (uint32_t)key[0] : 0u;   // low word = ~id
            id = ~wave_max_u32(lo);
        }
        if ((uint32_t)lane == (id & 63u)) {             // the owner drops its head
#pragma unroll
            for (int p = 0; p + 1 < PL; ++p)
                key[p] = key[p + 1];
            key[PL - 1] = 0ull;
        }
        const float lg = route_key_logit((uint64_t)best_hi << 32);
        if (j == 0)
            top_logit = lg;
        if (lane == j) {
            my_id = (int)id;
            my_logit = lg;
        }
    }
    const double ex = (lane < k) ? exp((double)my_logit - (double)top_logit) : 0.0;
    const double sum = wave_sum_f64(ex);
    if (lane < k) {
        topk_idx[t * k + lane] = my_id;
        topk_w[t * k + lane] = (float)(ex / sum);
    }
}

// --------------------------------------------------------------------------------- layout --
// Items are the (token, slot) pairs in index order i = t*k + j. Block b owns the contiguous items
// [b*rows_per_block, (b+1)*rows_per_block) and walks them 64*W at a time (W wavefronts). For
// each group, every item sets its lane bit in the LDS mask of (its wavefront, its expert); its
// rank among the block's items of the same expert is then
//   run[e] + (bits of e in lower wavefronts) + (bits of e in lower lanes of its own wavefront),
// which keeps index order without any atomic deciding a position. The first item of each expert
// in the group then advances run[e] and clears the masks. The block's counts go to
// hist_t[e * nblk + b] (expert-major). LDS: masks [W][E] u64, run [E] u32.
template <int W>
__device__ __forceinline__ void block_histogram(const int32_t* __restrict__ topk_idx, int32_t R,
                                                int32_t E, int32_t rows_per_block, int32_t nblk,
                                                uint32_t* __restrict__ hist_t,
                                                uint32_t* __restrict__ local_rank,
                                                uint64_t* lds)
{
    constexpr int NT = 64 * W;
    uint64_t* mask = lds;
    uint32_t* run = reinterpret_cast<uint32_t*>(mask + W * E);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < W * E; i += NT)
        mask[i] = 0ull;
    for (int i = tid; i < E; i += NT)
        run[i] = 0u;
    const uint64_t lower_lanes = (1ull << lane) - 1ull;
    const int64_t first = (int64_t)blockIdx.x * rows_per_block;
    const int64_t last = first + rows_per_block < R ? first + rows_per_block : R;
    int e_next = (first + tid < last) ? topk_idx[first + tid] : -1;
    __syncthreads();
    for (int64_t i = first + tid; i - tid < last; i += NT) {
        int e = e_next;
        if (i + NT < last)
            e_next = topk_idx[i + NT];                  // prefetch the next group's id
        if (i >= last || (uint32_t)e >= (uint32_t)E)
            e = -1;                                      // past the range, or an id outside [0, E)
        if (e >= 0)
            atomicOr(&mask[wave * E + e], 1ull << lane);
        __syncthreads();
        uint32_t rank = 0u;
        bool leader = false;
        if (e >= 0) {
            uint32_t before = 0u;
            for (int w = 0; w < wave; ++w)
                before += (uint32_t)__popcll(mask[w * E + e]);
            before += (uint32_t)__popcll(mask[wave * E + e] & lower_lanes);
            rank = run[e] + before;
            leader = (before == 0u);
        }
        __syncthreads();
        if (leader) {
            uint32_t n = 0u;
            for (int w = 0; w < W; ++w) {
                n += (uint32_t)__popcll(mask[w * E + e]);
                mask[w * E + e] = 0ull;
            }
            run[e] += n;
        }
        __syncthreads();
        if (i < last)
            local_rank[i] = rank;
    }
    for (int e = tid; e < E; e += NT)
        hist_t[(int64_t)e * nblk + blockIdx.x] = run[e];
}

// Exclusive scan of one value per thread over the NT threads of the block; returns the prefix
// and writes the block total to *total. `scratch` holds NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, d, 64);
        if (lane >= d)
            x += y;
    }
    if (lane == 63)
        scratch[wave] = x;
    __syncthreads();
    uint32_t base = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t s = scratch[w];
        base += (w < wave) ? s : 0u;
        all += s;
    }
    *total = all;
    return base + x - v;
}

// Inclusive prefix sum over the 64 lanes (all active): row_shr 1, 2, 4, 8 within 16-lane rows
// (lanes that would read before their row get 0), then row_bcast:15 and row_bcast:31 carry row
// totals into the following rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // bcast:31
    return v;
}

// Offsets from the expert-major histograms, by one workgroup of 16 wavefronts. Wavefront w
// takes experts w, w+16, ...; for expert e, lane b holds hist_t[e * nblk + b] (nblk <= 64) and a
// wave scan gives prefix[e * nblk + b] = rows of e in blocks before b (stored at once, so the
// stores drain during the rest); the last lane gives e's total. A block scan over the E totals
// gives the expert offsets; the row of item i of block b with expert e is then
// expert_offsets[e] + prefix[e * nblk + b] + local_rank[i]. Also writes the rank counts and
// offsets. EPW >= ceil(E / 16).
template <int EPW>
__device__ __forceinline__ void scan_histograms(const uint32_t* __restrict__ hist_t, int32_t E,
                                                int32_t N, int32_t nblk,
                                                uint32_t* __restrict__ prefix,
                                                int32_t* __restrict__ expert_counts,
                                                int32_t* __restrict__ expert_offsets,
                                                int32_t* __restrict__ rank_counts,
                                                int32_t* __restrict__ rank_offsets,
                                                uint32_t* scratch, uint32_t* eoff)
{
    constexpr int kWavesS = kScanThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t cnt[EPW];
#pragma unroll
    for (int u = 0; u < EPW; ++u) {
        const int e = wave + kWavesS * u;
        cnt[u] = (e < E && lane < nblk) ? hist_t[(int64_t)e * nblk + lane] : 0u;
    }
#pragma unroll
    for (int u = 0; u < EPW; ++u) {
        const int e = wave + kWavesS * u;
        if (e < E) {                                    // uniform per wavefront
            const uint32_t incl = wave_inclusive_scan_u32(cnt[u]);
            if (lane < nblk)
                prefix[(int64_t)e * nblk + lane] = incl - cnt[u];
            if (lane == 63)
                eoff[e] = incl;                         // expert total, for now
        }
    }
    __syncthreads();
    const uint32_t mine = tid < E ? eoff[tid] : 0u;     // E <= 1024: one expert per thread
    uint32_t total = 0u;
    const uint32_t ex = block_exclusive_scan<kScanThreads>(mine, scratch, &total);
    __syncthreads();                                    // every total read before overwriting
    if (tid < E)
        eoff[tid] = ex;
    if (tid == 0)
        eoff[E] = total;
    __syncthreads();
    const int epr = E / N;
    for (int i = tid; i < E; i += kScanThreads) {
        expert_offsets[i] = (int32_t)eoff[i];
        expert_counts[i] = (int32_t)(eoff[i + 1] - eoff[i]);
    }
    for (int r = tid; r < N; r += kScanThreads) {
        rank_offsets[r] = (int32_t)eoff[r * epr];
        rank_counts[r] = (int32_t)(eoff[(r + 1) * epr] - eoff[r * epr]);
    }
    if (tid == 0) {
        expert_offsets[E] = (int32_t)total;
        rank_offsets[N] = (int32_t)total;
    }
}

// Histogram blocks of 4 wavefronts (256 items per pass).
__global__ __launch_bounds__(kThreads) void k_layout_hist(const int32_t* __restrict__ topk_idx,
                                                          int32_t R, int32_t E,
                                                          int32_t rows_per_block, int32_t nblk,
                                                          uint32_t* __restrict__ hist_t,
                                                          uint32_t* __restrict__ local_rank)
{
    extern __shared__ uint64_t lds_u64[];
    block_histogram<kWaves>(topk_idx, R, E, rows_per_block, nblk, hist_t, local_rank, lds_u64);
}

// The scan as its own launch of one workgroup; with T = 0 it alone runs and writes zero counts.
template <int EPW>
__global__ __launch_bounds__(kScanThreads) void k_layout_scan(
    const uint32_t* __restrict__ hist_t, int32_t E, int32_t N, int32_t nblk,
    uint32_t* __restrict__ prefix, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets)
{
    __shared__ uint32_t scratch[kScanThreads / 64];
    __shared__ uint32_t eoff[MOE_MAX_EXPERTS + 1];
    scan_histograms<EPW>(hist_t, E, N, nblk, prefix, expert_counts, expert_offsets, rank_counts,
                         rank_offsets, scratch, eoff);
}

// Everything a kernel needs to place item i = t*k + j: either the finished token_row, or the
// layout results from which the row is computed (and token_row / row_token written).
struct RowPlan {
    const int32_t* topk_idx;
    const uint32_t* local_rank;
    const uint32_t* prefix;
    const int32_t* expert_offsets;
    int32_t* token_row;
    int32_t* row_token;
    int32_t E, nblk, rows_per_block;
};

// Row of item i from the layout results, or -1 for an expert id outside [0, E).
__device__ __forceinline__ int32_t planned_row(const RowPlan& rp, int64_t i)
{
    const int e = rp.topk_idx[i];
    if ((uint32_t)e >= (uint32_t)rp.E)
        return -1;
    const int64_t b = i / rp.rows_per_block;
    return (int32_t)((uint32_t)rp.expert_offsets[e] + rp.prefix[(int64_t)e * rp.nblk + b] +
                     rp.local_rank[i]);
}

__global__ __launch_bounds__(kThreads) void k_layout_rows(RowPlan rp, int32_t R, int32_t k)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < R;
         i += (int64_t)gridDim.x * kThreads) {
        const int32_t row = planned_row(rp, i);
        rp.token_row[i] = row;
        if ((uint32_t)row < (uint32_t)R)
            rp.row_token[row] = (int32_t)(i / k);
    }
}

// ----------------------------------------------------------------------------------- packing --
// Wavefront placement of the row kernels. Wavefront w of workgroup blk handles item
// m = (blk / 8) * waves_per_group + w of XCD blk % 8. Items of XCD x belong to tokens
// x, x+8, x+16, ... (items_per_token consecutive items each), so every wavefront that reads the
// row of token t runs on the same XCD and finds it in that XCD's L2 after the first read.
struct XcdItem {
    int64_t token;
    int sub;           // item index inside the token: slot * parts + part
};

__device__ __forceinline__ XcdItem xcd_item(int waves_per_group, int items_per_token)
{
    const int64_t m = (int64_t)(blockIdx.x / kXcds) * waves_per_group + (threadIdx.x >> 6);
    const int64_t q = m / items_per_token;
    XcdItem it;
    it.token = q * kXcds + (blockIdx.x % kXcds);
    it.sub = (int)(m - q * items_per_token);
    return it;
}

// Row of (token t, slot j): from token_row, or planned (the part-0 wavefront then records it).
template <bool PLANNED>
__device__ __forceinline__ int32_t pack_row(const RowPlan& rp, int64_t t, int j, int k, int part,
                                            int32_t R)
{
    const int64_t i = t * k + j;
    int32_t row;
    if constexpr (PLANNED) {
        row = planned_row(rp, i);
        if (part == 0 && (threadIdx.x & 63) == 0) {
            rp.token_row[i] = row;
            if ((uint32_t)row < (uint32_t)R)
                rp.row_token[row] = (int32_t)t;
        }
    } else {
        row = rp.token_row[i];
    }
    return row;
}

// One wavefront per (token, slot, part): chunks [part*cpp, (part+1)*cpp) (16 bytes each) of x's
// row t are loaded (plain loads: the k wavefronts of the token share them through L2) and
// stored to row token_row[t*k+j] with non-temporal stores, U chunks per lane at a time. The
// first loads are issued before the row is known.
template <int U, bool PLANNED>
__global__ __launch_bounds__(64 * kPackWaves) void k_pack_rows(const u32x4* __restrict__ x,
                                                               int32_t T, int32_t k, int32_t R,
                                                               int32_t chunks_per_row,
                                                               int32_t parts,
                                                               int32_t chunks_per_part,
                                                               RowPlan rp,
                                                               u32x4* __restrict__ recv)
{
    const XcdItem it = xcd_item(kPackWaves, k * parts);
    if (it.token >= T)
        return;
    const int j = it.sub / parts, part = it.sub - j * parts;
    const int lane = threadIdx.x & 63;
    const int c0 = part * chunks_per_part;
    const int c1 = min(chunks_per_row, c0 + chunks_per_part);
    const u32x4* src = x + it.token * chunks_per_row;
    u32x4 v[U];
    int cb = c0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = cb + u * 64 + lane;
        if (c < c1)
            v[u] = src[c];
    }
    const int32_t row = pack_row<PLANNED>(rp, it.token, j, k, part, R);
    if ((uint32_t)row >= (uint32_t)R)
        return;
    u32x4* dst = recv + (int64_t)row * chunks_per_row;
    while (true) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + u * 64 + lane;
            if (c < c1)
                __builtin_nontemporal_store(v[u], dst + c);
        }
        cb += 64 * U;
        if (cb >= c1)
            break;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + u * 64 + lane;
            if (c < c1)
                v[u] = src[c];
        }
    }
}

// Eight consecutive elements of x as fp32.
template <typename XT>
struct Load8;

template <>
struct Load8<float> {
    static __device__ __forceinline__ void run(const float* p, float (&v)[8])
    {
        const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
        const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
};

template <>
struct Load8<uint16_t> {
    static __device__ __forceinline__ void run(const uint16_t* p, float (&v)[8])
    {
        const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
};

// fp8 packing, one wavefront per (token, slot, part). A chunk is 8 elements; the 16 lanes of a
// DPP row hold the 128 elements of one scale block (parts are multiples of 16 chunks, so rows
// never straddle two blocks). Every lane stays active through the reduction; only stores are
// masked. The row is resolved after the first chunk group has been loaded and quantised.
template <typename XT, bool PLANNED>
__global__ __launch_bounds__(64 * kPackWaves) void k_pack_rows_fp8(
    const XT* __restrict__ x, int32_t T, int32_t H, int32_t k, int32_t R, int32_t parts,
    int32_t chunks_per_part, RowPlan rp, uint8_t* __restrict__ recv,
    float* __restrict__ recv_scales)
{
    const XcdItem it = xcd_item(kPackWaves, k * parts);
    if (it.token >= T)
        return;
    const int j = it.sub / parts, part = it.sub - j * parts;
    const int lane = threadIdx.x & 63;
    const int chunks_per_row = H / 8;
    const int nb = H / 128;
    const int c0 = part * chunks_per_part;
    const int c1 = min(chunks_per_row, c0 + chunks_per_part);
    const XT* src = x + it.token * H;
    int32_t row = -1;
    uint8_t* dst = nullptr;
    for (int cb = c0; cb < c1; cb += 64) {
        const int c = cb + lane;
        const bool active = c < c1;
        float v[8];
        if (active) {
            Load8<XT>::run(src + (int64_t)c * 8, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = 0.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
        amax = max_row16_f32(amax);
        const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;   // correctly rounded division
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = f32_to_e4m3(v[i] / s);
        u32x2 packed;
        packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        if (cb == c0) {
            row = pack_row<PLANNED>(rp, it.token, j, k, part, R);
            if ((uint32_t)row >= (uint32_t)R)
                return;
            dst = recv + (int64_t)row * H;
        }
        if (active) {
            __builtin_nontemporal_store(packed, reinterpret_cast<u32x2*>(dst) + c);
            if ((lane & 15) == 0)
                recv_scales[(int64_t)row * nb + c / 16] = s;
        }
    }
}

// ----------------------------------------------------------------------------------- combine --
template <typename YT>
struct Y8;

template <>
struct Y8<uint16_t> {       // bf16: one 16-byte load per 8 elements
    u32x4 a;
    __device__ __forceinline__ void load(const uint16_t* p)
    {
        a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ void fma_into(float w, float (&acc)[8]) const
    {
        const uint32_t v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, bf16_to_f32(v[i] & 0xFFFFu), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, bf16_to_f32(v[i] >> 16), acc[2 * i + 1]);
        }
    }
};

template <>
struct Y8<float> {          // fp32: two 16-byte loads per 8 elements
    u32x4 a, b;
    __device__ __forceinline__ void load(const float* p)
    {
        a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
    }
    __device__ __forceinline__ void fma_into(float w, float (&acc)[8]) const
    {
        const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = fmaf(w, __uint_as_float(v[i]), acc[i]);
    }
};

template <typename OT>
struct Store8;

template <>
struct Store8<uint16_t> {
    static __device__ __forceinline__ void run(uint16_t* p, const float (&acc)[8])
    {
        u32x4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p));
    }
};

template <>
struct Store8<float> {
    static __device__ __forceinline__ void run(float* p, const float (&acc)[8])
    {
        u32x4 a, b;
        a.x = __float_as_uint(acc[0]); a.y = __float_as_uint(acc[1]);
        a.z = __float_as_uint(acc[2]); a.w = __float_as_uint(acc[3]);
        b.x = __float_as_uint(acc[4]); b.y = __float_as_uint(acc[5]);
        b.z = __float_as_uint(acc[6]); b.w = __float_as_uint(acc[7]);
        __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(p) + 1);
    }
};

// One wavefront per (token, segment of 64 chunks = 512 elements); lane l owns chunk
// segment*64 + l. KC is k when it is a compile-time constant (all k loads issued before the
// first multiply-add), else 0.
template <typename YT, typename OT, int KC>
__global__ __launch_bounds__(64 * kCombineWaves) void k_combine(
    const YT* __restrict__ y, int32_t T, int32_t H, int32_t k_rt, int32_t R, int32_t nseg,
    const int32_t* __restrict__ token_row, const float* __restrict__ topk_w,
    OT* __restrict__ out)
{
    const int k = KC > 0 ? KC : k_rt;
    const int64_t item = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
    const int64_t t = item / nseg;
    if (t >= T)
        return;
    const int seg = (int)(item - t * nseg);
    const int c = seg * 64 + (threadIdx.x & 63);
    if (c >= H / 8)
        return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.0f;
    const int64_t off = (int64_t)c * 8;
    if constexpr (KC > 0) {
        Y8<YT> v[KC];
        float w[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int row = token_row[t * KC + j];
            w[j] = topk_w[t * KC + j];
            if ((uint32_t)row < (uint32_t)R) {
                v[j].load(y + (int64_t)row * H + off);
            } else {
                w[j] = 0.0f;
                v[j] = Y8<YT>{};
            }
        }
#pragma unroll
        for (int j = 0; j < KC; ++j)
            v[j].fma_into(w[j], acc);
    } else {
        for (int j = 0; j < k; ++j) {
            const int row = token_row[t * k + j];
            if ((uint32_t)row >= (uint32_t)R)
                continue;
            Y8<YT> v;
            v.load(y + (int64_t)row * H + off);
            v.fma_into(topk_w[t * k + j], acc);
        }
    }
    Store8<OT>::run(out + t * H + off, acc);
}

// ------------------------------------------------------------------------------ host helpers --
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t dtype_size(moe_dtype_t d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

inline bool is_wide(moe_dtype_t d) { return d == MOE_F32 || d == MOE_BF16; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Layout launch plan: histogram blocks of 4 wavefronts walk their items 256 at a time; at most
// 64 blocks (one lane each in the scan).
struct LayoutPlan {
    int32_t rows_per_block;
    int32_t nblk;
};

inline size_t hist_lds_bytes(int32_t E)
{
    return (size_t)kWaves * E * sizeof(uint64_t) + (size_t)E * sizeof(uint32_t);
}

inline LayoutPlan layout_plan(int64_t R)
{
    LayoutPlan p;
    const int64_t groups = R > 0 ? ceil_div(R, (int64_t)kThreads * kMaxLayoutBlocks) : 1;
    p.rows_per_block = (int32_t)(groups * kThreads);
    p.nblk = (int32_t)ceil_div(R, p.rows_per_block);
    return p;
}

// Workspace: expert-major histograms [E * nblk], in-expert prefixes [E * nblk], in-block ranks
// [R]; each piece 256-byte aligned.
struct Workspace {
    uint32_t* hist_t;
    uint32_t* prefix;
    uint32_t* local_rank;
};

inline size_t ws_hist_bytes(int64_t R, int32_t E)
{
    return align_up(((size_t)layout_plan(R).nblk * E + 1) * sizeof(uint32_t), 256);
}

inline size_t ws_bytes(int64_t R, int32_t E)
{
    return 2 * ws_hist_bytes(R, E) + align_up((size_t)(R > 0 ? R : 1) * 4, 256);
}

inline Workspace carve_workspace(void* base, int64_t R, int32_t E)
{
    char* p = static_cast<char*>(base);
    const size_t hb = ws_hist_bytes(R, E);
    Workspace w;
    w.hist_t = reinterpret_cast<uint32_t*>(p);
    w.prefix = reinterpret_cast<uint32_t*>(p + hb);
    w.local_rank = reinterpret_cast<uint32_t*>(p + 2 * hb);
    return w;
}

// Parts per row for the row kernels: enough wavefronts to fill the GPU, each part at least
// `min_chunks` long and a multiple of `align` chunks.
struct PartPlan {
    int32_t parts;
    int32_t chunks_per_part;
};

inline PartPlan part_plan(int64_t R, int32_t chunks_per_row, int32_t align, int32_t min_chunks)
{
    int64_t parts = R > 0 ? ceil_div(kTargetWaves, R) : 1;
    const int64_t max_parts = ceil_div(chunks_per_row, min_chunks);
    if (parts > max_parts)
        parts = max_parts;
    if (parts < 1)
        parts = 1;
    int64_t cpp = ceil_div(chunks_per_row, parts);
    cpp = ceil_div(cpp, align) * align;
    PartPlan p;
    p.chunks_per_part = (int32_t)cpp;
    p.parts = (int32_t)ceil_div(chunks_per_row, cpp);
    return p;
}

inline dim3 xcd_grid(int32_t T, int64_t items_per_token, int waves_per_group)
{
    const int64_t per_xcd = ceil_div(ceil_div(T, kXcds) * items_per_token, waves_per_group);
    return dim3((unsigned)(per_xcd * kXcds));
}

inline moe_status_t launch_status()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t check_layout_args(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                               int32_t n_ranks, const moe_dispatch_out_t* out)
{
    if (T < 0 || k < 1 || E < 1 || n_ranks < 1 || E % n_ranks != 0 || out == nullptr)
        return MOE_ERR_INVALID;
    if ((int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS)
        return MOE_ERR_UNSUPPORTED;
    if (!out->expert_counts || !out->expert_offsets || !out->rank_counts || !out->rank_offsets)
        return MOE_ERR_INVALID;
    if (T > 0 && (!topk_idx || !out->token_row || !out->row_token))
        return MOE_ERR_INVALID;
    return MOE_OK;
}

moe_status_t check_pack_args(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H, int32_t k,
                             const int32_t* token_row, moe_dtype_t payload_dtype,
                             const void* recv, const float* recv_scales)
{
    if (T < 0 || H < 1 || k < 1 || (int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    if (!is_wide(x_dtype) || (payload_dtype != x_dtype && payload_dtype != MOE_FP8_E4M3))
        return MOE_ERR_UNSUPPORTED;
    if (T > 0 && (!x || !token_row || !recv))
        return MOE_ERR_INVALID;
    if (payload_dtype == MOE_FP8_E4M3) {
        if (H % 128 != 0)
            return MOE_ERR_UNSUPPORTED;
        if (T > 0 && !recv_scales)
            return MOE_ERR_INVALID;
        if (!aligned(recv_scales, 4))
            return MOE_ERR_UNSUPPORTED;
    }
    if (((int64_t)H * (int64_t)dtype_size(x_dtype)) % 16 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(recv, 16))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

template <int EPW>
void launch_counts_epw(const int32_t* topk_idx, int64_t R, int32_t E, int32_t n_ranks,
                       const moe_dispatch_out_t* out, const Workspace& ws, const LayoutPlan& plan,
                       hipStream_t stream)
{
    if (plan.nblk > 0)
        k_layout_hist<<<plan.nblk, kThreads, hist_lds_bytes(E), stream>>>(
            topk_idx, (int32_t)R, E, plan.rows_per_block, plan.nblk, ws.hist_t, ws.local_rank);
    k_layout_scan<EPW><<<1, kScanThreads, 0, stream>>>(ws.hist_t, E, n_ranks, plan.nblk,
                                                       ws.prefix, out->expert_counts,
                                                       out->expert_offsets, out->rank_counts,
                                                       out->rank_offsets);
}

// The counting half of dispatch: histograms, scan, counts and offsets. With T = 0 only the scan
// runs, which writes zero counts.
void launch_layout_counts(const int32_t* topk_idx, int64_t R, int32_t E, int32_t n_ranks,
                          const moe_dispatch_out_t* out, const Workspace& ws,
                          const LayoutPlan& plan, hipStream_t stream)
{
    const int64_t epw = ceil_div(E, kScanThreads / 64);
    if (epw <= 8)
        launch_counts_epw<8>(topk_idx, R, E, n_ranks, out, ws, plan, stream);
    else if (epw <= 16)
        launch_counts_epw<16>(topk_idx, R, E, n_ranks, out, ws, plan, stream);
    else if (epw <= 32)
        launch_counts_epw<32>(topk_idx, R, E, n_ranks, out, ws, plan, stream);
    else
        launch_counts_epw<64>(topk_idx, R, E, n_ranks, out, ws, plan, stream);
}

RowPlan make_row_plan(const int32_t* topk_idx, const Workspace& ws, const LayoutPlan& plan,
                      int32_t E, const moe_dispatch_out_t* out)
{
    RowPlan rp;
    rp.topk_idx = topk_idx;
    rp.local_rank = ws.local_rank;
    rp.prefix = ws.prefix;
    rp.expert_offsets = out->expert_offsets;
    rp.token_row = out->token_row;
    rp.row_token = out->row_token;
    rp.E = E;
    rp.nblk = plan.nblk;
    rp.rows_per_block = plan.rows_per_block;
    return rp;
}

template <bool PLANNED>
void launch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H, int32_t k,
                 const RowPlan& rp, moe_dtype_t payload_dtype, void* recv, float* recv_scales,
                 hipStream_t stream)
{
    const int32_t R = T * k;
    if (payload_dtype != MOE_FP8_E4M3) {
        const int32_t cpr = (int32_t)((int64_t)H * (int64_t)dtype_size(x_dtype) / 16);
        const PartPlan pp = part_plan(R, cpr, 1, 64);
        const dim3 grid = xcd_grid(T, (int64_t)k * pp.parts, kPackWaves);
        const u32x4* xs = static_cast<const u32x4*>(x);
        u32x4* rv = static_cast<u32x4*>(recv);
        const int64_t u = ceil_div(pp.chunks_per_part, 64);
#define MOE_PACK(UU)                                                                              \
    k_pack_rows<UU, PLANNED><<<grid, 64 * kPackWaves, 0, stream>>>(xs, T, k, R, cpr, pp.parts,   \
                                                                   pp.chunks_per_part, rp, rv)
        if (u <= 1)
            MOE_PACK(1);
        else if (u <= 2)
            MOE_PACK(2);
        else if (u <= 4)
            MOE_PACK(4);
        else if (u <= 8)
            MOE_PACK(8);
        else
            MOE_PACK(16);
#undef MOE_PACK
    } else {
        const PartPlan pp = part_plan(R, H / 8, 16, 64);
        const dim3 grid = xcd_grid(T, (int64_t)k * pp.parts, kPackWaves);
        if (x_dtype == MOE_F32)
            k_pack_rows_fp8<float, PLANNED><<<grid, 64 * kPackWaves, 0, stream>>>(
                static_cast<const float*>(x), T, H, k, R, pp.parts, pp.chunks_per_part, rp,
                static_cast<uint8_t*>(recv), recv_scales);
        else
            k_pack_rows_fp8<uint16_t, PLANNED><<<grid, 64 * kPackWaves, 0, stream>>>(
                static_cast<const uint16_t*>(x), T, H, k, R, pp.parts, pp.chunks_per_part, rp,
                static_cast<uint8_t*>(recv), recv_scales);
    }
}

template <typename YT, typename OT>
void launch_combine_typed(const void* y, int32_t T, int32_t H, int32_t k,
                          const int32_t* token_row, const float* topk_w, void* out,
                          hipStream_t stream)
{
    const int32_t R = T * k;
    const int32_t nseg = (int32_t)ceil_div(H / 8, 64);
    const dim3 grid((unsigned)ceil_div((int64_t)T * nseg, kCombineWaves));
    const YT* yp = static_cast<const YT*>(y);
    OT* op = static_cast<OT*>(out);
#define MOE_COMBINE(KK)                                                                           \
    k_combine<YT, OT, KK><<<grid, 64 * kCombineWaves, 0, stream>>>(yp, T, H, k, R, nseg,         \
                                                                   token_row, topk_w, op)
    switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 6: MOE_COMBINE(6); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
    }
#undef MOE_COMBINE
}

}  // namespace

// ------------------------------------------------------------------------------------ C ABI --
extern "C" {

const char* moe_status_str(moe_status_t status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported dtype, size or alignment";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    }
    return "unknown moe_status_t";
}

moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T > 0 && (!logits || !topk_idx || !topk_w))
        return MOE_ERR_INVALID;
    if ((int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    if (T == 0)
        return MOE_OK;
    const int pl = (E + 63) / 64;
    const dim3 grid((unsigned)ceil_div(T, kWaves));
#define MOE_ROUTE(PP)                                                                             \
    k_route_topk<PP><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w)
    if (pl <= 1)
        MOE_ROUTE(1);
    else if (pl <= 2)
        MOE_ROUTE(2);
    else if (pl <= 4)
        MOE_ROUTE(4);
    else if (pl <= 6)
        MOE_ROUTE(6);
    else if (pl <= 8)
        MOE_ROUTE(8);
    else
        MOE_ROUTE(16);
#undef MOE_ROUTE
    return launch_status();
}

size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k)
{
    if (T < 0 || E < 1 || k < 1 || (int64_t)T * k > INT32_MAX)
        return 0;
    const int64_t R = (int64_t)T * k;
    return ws_bytes(R, E);
}

moe_status_t moe_dispatch_layout(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                 int32_t n_ranks, const moe_dispatch_out_t* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    moe_status_t st = check_layout_args(topk_idx, T, k, E, n_ranks, out);
    if (st != MOE_OK)
        return st;
    if (!workspace || workspace_bytes < moe_dispatch_workspace_bytes(T, E, k))
        return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return MOE_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = layout_plan(R);
    const Workspace ws = carve_workspace(workspace, R, E);
    launch_layout_counts(topk_idx, R, E, n_ranks, out, ws, plan, stream);
    if (R > 0) {
        const RowPlan rp = make_row_plan(topk_idx, ws, plan, E, out);
        const int64_t want = ceil_div(R, kThreads);
        const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
        k_layout_rows<<<blocks, kThreads, 0, stream>>>(rp, (int32_t)R, k);
    }
    return launch_status();
}

moe_status_t moe_dispatch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                               int32_t k, const int32_t* token_row, moe_dtype_t payload_dtype,
                               void* recv, float* recv_scales, hipStream_t stream)
{
    moe_status_t st =
        check_pack_args(x, x_dtype, T, H, k, token_row, payload_dtype, recv, recv_scales);
    if (st != MOE_OK)
        return st;
    if (T == 0)
        return MOE_OK;
    RowPlan rp = {};
    rp.token_row = const_cast<int32_t*>(token_row);   // read only on this path
    launch_pack<false>(x, x_dtype, T, H, k, rp, payload_dtype, recv, recv_scales, stream);
    return launch_status();
}

moe_status_t moe_dispatch(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                          const int32_t* topk_idx, int32_t k, int32_t E, int32_t n_ranks,
                          moe_dtype_t payload_dtype, const moe_dispatch_out_t* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    moe_status_t st = check_layout_args(topk_idx, T, k, E, n_ranks, out);
    if (st != MOE_OK)
        return st;
    st = check_pack_args(x, x_dtype, T, H, k, out->token_row, payload_dtype, out->recv,
                         out->recv_scales);
    if (st != MOE_OK)
        return st;
    if (!workspace || workspace_bytes < moe_dispatch_workspace_bytes(T, E, k))
        return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return MOE_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = layout_plan(R);
    const Workspace ws = carve_workspace(workspace, R, E);
    launch_layout_counts(topk_idx, R, E, n_ranks, out, ws, plan, stream);
    if (R > 0) {
        const RowPlan rp = make_row_plan(topk_idx, ws, plan, E, out);
        launch_pack<true>(x, x_dtype, T, H, k, rp, payload_dtype, out->recv, out->recv_scales,
                          stream);
    }
    return launch_status();
}

moe_status_t moe_combine(const void* y, moe_dtype_t y_dtype, int32_t T, int32_t H, int32_t k,
                         const int32_t* token_row, const float* topk_w, void* out,
                         moe_dtype_t out_dtype, hipStream_t stream)
{
    if (T < 0 || H < 1 || k < 1 || (int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    if (!is_wide(y_dtype) || !is_wide(out_dtype))
        return MOE_ERR_UNSUPPORTED;
    if (H % 8 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (T > 0 && (!y || !token_row || !topk_w || !out))
        return MOE_ERR_INVALID;
    if (!aligned(y, 16) || !aligned(out, 16))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16)
        launch_combine_typed<uint16_t, uint16_t>(y, T, H, k, token_row, topk_w, out, stream);
    else if (y_dtype == MOE_BF16)
        launch_combine_typed<uint16_t, float>(y, T, H, k, token_row, topk_w, out, stream);
    else if (out_dtype == MOE_BF16)
        launch_combine_typed<float, uint16_t>(y, T, H, k, token_row, topk_w, out, stream);
    else
        launch_combine_typed<float, float>(y, T, H, k, token_row, topk_w, out, stream);
    return launch_status();
}

}  // extern "C"
