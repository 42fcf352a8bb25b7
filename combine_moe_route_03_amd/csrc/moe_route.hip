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
//   k_route_topk     top-k routing, 16 lanes a token (k <= 16, large batches: k rounds of a row
//                    maximum and a row minimum by DPP) or, as k_route_topk_wide, a wavefront a
//                    token (lane-sorted candidates give up their heads over k wave-wide maxima);
//   k_route_layout   the same routing, 16 tokens per workgroup, and in the same launch the
//                    workgroup's expert histogram and the stable in-workgroup rank of every
//                    (token, slot) from one LDS bit mask per expert;
//   k_layout_hist    for caller-given expert ids: per block of items, stable in-block ranks from
//                    per-wavefront LDS bit masks, and the block's expert histogram;
//   k_expert_scan    four experts per workgroup: coalesced gathers of the blocks' counts, then a
//                    wavefront per expert scans them into per-block prefixes and the total;
//   k_layout_rows    every workgroup scans the expert totals into offsets in LDS, then writes
//                    token_row / row_token; workgroup 0 writes the counts and offsets;
//   k_pack_rows      window order: one wavefront per (destination row, 1 KB piece), a 16-byte
//                    load of x (from the XCD's L2 after the window's first touch) and a 16-byte
//                    non-temporal store per lane; token order: one wavefront per (token, 1 KB
//                    piece), one load stored to all k rows; the pieces of a row run side by side;
//   k_pack_rows_fp8  same, quantising 1x128 blocks to e4m3 with an fp32 absmax/448 scale;
//   k_layout_pack    batches of up to 512 tokens (896 routed ones for row copies): every
//                    workgroup rebuilds the whole layout in LDS from the ids (LDS counts, one
//                    block scan, token bit masks for the ranks) and packs its pieces, so layout
//                    and packing take one launch; up to 32 routed tokens every workgroup also
//                    routes the batch itself, so dispatch is one launch;
//   k_combine        one wavefront per (token, 512-element segment): all k row loads in flight,
//                    fp32 fused multiply-adds, one 16-byte non-temporal store per 8 outputs;
//   k_ep_recv_plan   expert-parallel receive: every workgroup scans a rank's per-(source, expert)
//                    region counts into the grouped layout and finds the region row of its share
//                    of the grouped rows;
//   k_copy_rows      grid-stride row gather / scatter by a row map (expert-parallel receive and
//                    the return half of combine);
//   k_ep_partial_rows, k_ep_invert, k_ep_reduce, k_ep_finish  combine with pre-reduction on the
//                    expert side: one partial row per (token, rank), summed by the source.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "moe_route.h"

namespace {

constexpr int kThreads = 256;            // route / histogram workgroups: 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kGroupThreads = 1024;      // 16-wavefront workgroups (route-layout, totals, scan)
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kRouteTokens = kGroupWaves;   // route-layout workgroup, k > 16: a token a wave
constexpr int kRouteTokens16 = kThreads / 16;   // route-layout workgroup, k <= 16: 16 lanes each
constexpr int kMaxScanBlocks = 64 * 16;  // histogram blocks one scan takes (64 threads of 16 each)
constexpr int kScanExperts = kThreads / 64;   // experts per scan workgroup (a wavefront each)
constexpr int kPackWaves = 16;           // wavefronts per pack / copy workgroup
constexpr int kPackWavesWindows = 8;     //   (8 for the window-ordered pack)
constexpr int kPackSplitPieces = 12;     // window order: rows of fewer 1 KB pieces take 2 a wave
constexpr int kMaxEpSegments = 4096;     // expert-parallel receive: sources x local experts
constexpr int kCombineWaves = 1;         // wavefronts per combine workgroup
constexpr int kXcds = 8;                 // workgroup b runs on XCD b % 8 (round-robin dispatch)
constexpr int kLpTokens = 512;           // layout folded into packing: at most this many tokens
constexpr int kLpThreads = 512;          //   (8 wavefronts a workgroup, two experts a thread)
constexpr int kLpWaves = kLpThreads / 64;
constexpr int kLpMaxGroups = 1024;       //   (grid-stride beyond this many workgroups)
constexpr int kLpWideThreads = 1024;     //   above kLpWideTokens tokens, 16 wavefronts a
constexpr int kLpWideTokens = 256;       //   workgroup (row copies without routing),
constexpr int kLpCopyTokens = 896;       //   up to this many routed tokens for row copies,
constexpr int kLpWideMaxGroups = 512;    //   at most one round of them (two on each of 256 CUs)
constexpr int kLpRouteTokens = kLpThreads / 16;   // routing in the same launch: at most 32 tokens

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------- number formats --
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// bf16 nearest to f, ties to even (add half an ulp minus one, plus the kept lsb, then truncate);
// every NaN becomes the one quiet NaN 0x7FC0 (its sign and payload are not kept).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
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

// Exclusive scan of one value per thread over the NT threads of the block (every lane active);
// returns the prefix and writes the block total to *total. `wave_tot` holds NT/64 words of LDS.
// The wavefront scan is the DPP one: at 128 decode tokens it makes the step 0.25 us faster than a
// scan by __shfl_up (14.97 -> 14.72 us).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot,
                                                         uint32_t* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan_u32(v);
    if (lane == 63)
        wave_tot[wave] = x;
    __syncthreads();
    uint32_t base = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t s = wave_tot[w];
        base += (w < wave) ? s : 0u;
        all += s;
    }
    *total = all;
    return base + x - v;
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

// Maximum over all 64 lanes (all active), the same value in every lane: the maximum within each
// 16-lane row (every lane of the row ends with it), then row_bcast:15 and row_bcast:31 carry row
// maxima forward so lane 63 holds the wave's, and one readlane broadcasts it.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(v));
    v = max(v, dpp_u32<kDppRowMirror>(v));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The logits of one token, lane l holding experts l, l+64, ... (entries past E are not read).
template <int PL>
__device__ __forceinline__ void load_logits(const float* __restrict__ l, int32_t E, float (&v)[PL])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        const int e = lane + 64 * p;
        v[p] = (e < E) ? l[e] : 0.0f;
    }
}

// Top-k of one token by one whole wavefront (all lanes active). Lane l holds experts l, l+64, ...
// (coalesced loads) and sorts its keys once, largest first, so its best remaining candidate is
// always key[0]. Each of the k rounds takes the wave-wide maximum of the candidates' logit words;
// when a single lane holds it (the usual case, found with one ballot) that lane wins, otherwise the
// lowest expert id among the tied lanes wins. The winner drops its head. The weights use
// double-precision exp and division, rounded once to fp32. Lane j < k writes slot j and returns
// its expert id (other lanes return -1). The logits come from load_logits.
template <int PL>
__device__ __forceinline__ int route_token_from(const float (&v)[PL], int32_t E, int32_t k,
                                                int32_t* __restrict__ idx_out,
                                                float* __restrict__ w_out)
{
    const int lane = threadIdx.x & 63;
    uint64_t key[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        const int e = lane + 64 * p;
        key[p] = (e < E) ? route_key(v[p], e) : 0ull;
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
    int my_id = -1;
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
        idx_out[lane] = my_id;
        w_out[lane] = (float)(ex / sum);
    }
    return my_id;
}

template <int PL>
__device__ __forceinline__ int route_token(const float* __restrict__ l, int32_t E, int32_t k,
                                           int32_t* __restrict__ idx_out,
                                           float* __restrict__ w_out)
{
    float v[PL];
    load_logits<PL>(l, E, v);
    return route_token_from<PL>(v, E, k, idx_out, w_out);
}

// Routing with one whole wavefront per token (any k up to 64), one wavefront a workgroup: the
// tokens' logit loads go out from as many CUs as there are tokens (128 decode tokens: the step
// 13.95 -> 13.46 us against four wavefronts a workgroup).
template <int PL>
__global__ __launch_bounds__(64) void k_route_topk_wide(const float* __restrict__ logits,
                                                   int32_t T, int32_t E, int32_t k,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w)
{
    const int64_t t = blockIdx.x;
    if (t >= T)
        return;
    route_token<PL>(logits + t * E, E, k, topk_idx + t * k, topk_w + t * k);
}

// The counts of routing block b, popcount(mask[e]), stored block-major: as u32 at hist[b*E + e],
// or, with hist8 non-null, as one byte each at hist8[b*E16 + e], the row padded with zeros to E16
// (E rounded up to 16). A block holds 16 tokens and a routed token names an expert at most once,
// so a count is at most 16 and fits a byte; the whole table (96 KB for 4096 tokens and 384
// experts) is then small enough for every rows workgroup to sum it itself (k_layout_rows8).
__device__ __forceinline__ void store_block_counts(const uint32_t* mask, int32_t E, int64_t b,
                                                   uint32_t* __restrict__ hist,
                                                   uint8_t* __restrict__ hist8, int32_t E16)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    if (hist8 != nullptr) {
        uint32_t* row = reinterpret_cast<uint32_t*>(hist8 + b * E16);
        for (int q = tid; q < E16 / 4; q += nt) {
            uint32_t packed = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 4 * q + j;
                packed |= (e < E ? (uint32_t)__popc(mask[e]) : 0u) << (8 * j);
            }
            row[q] = packed;
        }
    } else {
        for (int e = tid; e < E; e += nt)
            hist[b * E + e] = (uint32_t)__popc(mask[e]);
    }
}

// Routing plus the counting half of dispatch in one launch, one wavefront per token (used for
// k > 16). Workgroup b routes tokens
// 16b .. 16b+15 (wavefront w takes token 16b + w); each selected (token, slot) sets bit w of
// the LDS mask of its expert. A token's k experts are distinct, so the rank of (token, slot)
// among the workgroup's items of the same expert, in (token, slot) order, is the number of bits
// below w, and the workgroup's count of expert e is popcount(mask[e]), stored block-major at
// hist[b * E + e] (one coalesced row per workgroup). LDS: mask [E] u32.
template <int PL>
__global__ __launch_bounds__(kGroupThreads) void k_route_layout_wide(
    const float* __restrict__ logits, int32_t T, int32_t E, int32_t k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ local_rank, uint8_t* __restrict__ hist8, int32_t E16)
{
    extern __shared__ uint32_t lds_mask[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E; e += kGroupThreads)
        lds_mask[e] = 0u;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kRouteTokens + wave;
    const bool active = t < T;                          // uniform per wavefront
    int my_id = -1;
    if (active)
        my_id = route_token<PL>(logits + t * E, E, k, topk_idx + t * k, topk_w + t * k);
    if (my_id >= 0)
        atomicOr(&lds_mask[my_id], 1u << wave);
    __syncthreads();
    if (my_id >= 0)
        local_rank[t * k + lane] = (uint32_t)__popc(lds_mask[my_id] & ((1u << wave) - 1u));
    store_block_counts(lds_mask, E, blockIdx.x, hist, hist8, E16);
}

// ------------------------------------------------------------------------ x prefetch --
// The packing launch reads x with plain loads and then writes k rows per token. When x comes from
// HBM, those reads arrive in the middle of the row writes and the mixed traffic runs far below
// either stream alone (prefill: about 110 us for the pack instead of 85). The three layout
// launches before it (counting, scan, rows) are bound by latency and leave HBM idle, so extra
// workgroups of each read a third of x ahead: the lines stay in the 256 MB memory-side Infinity
// Cache, and the pack finds them there.
struct Prefetch {
    const u32x4* x;       // first chunk to read (null: no prefetch)
    int64_t chunks;       // 16-byte chunks to read
    int32_t groups;       // workgroups that share them
    int32_t sleeps;       // s_sleep(16) (1024 shader clocks) before the first load, this many
    uint32_t* sink;       // a workspace word that nothing reads
};

constexpr int kPrefetchChunksPerThread = 16;
// At most 7/8 of the 256 MB Infinity Cache is read ahead. Measured, µs per step (hidden 7168,
// 8 buffer sets): 16384 tokens, E 256 (235 MB of x) 778.9 with a 128 MiB cap, 766-767 (160 MiB),
// 752-753 (192), 741 (224), 742 (256); 12288 tokens, E 384 (176 MB) 602 (128), 597 (160), 585-587
// from 192 MiB on.
constexpr int64_t kPrefetchMaxBytes = 224ll << 20;

// Workgroup g of pf.groups reads its contiguous span of the chunks, four loads in flight per
// thread, after pf.sleeps sleeps of about half a microsecond. The loaded words feed one
// data-dependent store to pf.sink, which keeps the loads.
__device__ __forceinline__ void prefetch_span(const Prefetch& pf, int g)
{
    for (int z = 0; z < pf.sleeps; ++z)
        __builtin_amdgcn_s_sleep(16);
    const int64_t per = (pf.chunks + pf.groups - 1) / pf.groups;
    const int64_t b = (int64_t)g * per;
    const int64_t e = b + per < pf.chunks ? b + per : pf.chunks;
    uint32_t acc = 0u;
    for (int64_t i = b + threadIdx.x; i < e; i += 4 * (int64_t)blockDim.x) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t c = i + (int64_t)u * blockDim.x;
            v[u] = c < e ? pf.x[c] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u)
        *pf.sink = acc;
}

// ------------------------------------------------------------------ routing, 16 lanes a token --
// For k <= 16 a wavefront routes 4 tokens at once, one per 16-lane DPP row, which takes about a
// third of the instructions per token of the wavefront-per-token selection (routing is bound by
// issue: 4096 tokens give every SIMD only a few wavefronts).
__device__ __forceinline__ uint32_t logit_key(float v)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u)
        u = 0u;                                          // -0 equals +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // every finite logit maps above 0
}

__device__ __forceinline__ float key_logit(uint32_t ord)
{
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppRowHalfMirror>(v));
    return max(v, dpp_u32<kDppRowMirror>(v));
}

__device__ __forceinline__ uint32_t row16_min_u32(uint32_t v)
{
    v = min(v, dpp_u32<kDppQuadXor1>(v));
    v = min(v, dpp_u32<kDppQuadXor2>(v));
    v = min(v, dpp_u32<kDppRowHalfMirror>(v));
    return min(v, dpp_u32<kDppRowMirror>(v));
}

// The logits of a row's token: lane l of the row holds experts l, l+16, ... (entries past `E`
// are not read; a row with E = 0 routes nothing).
template <int P>
__device__ __forceinline__ void load_logits16(const float* __restrict__ l, int32_t E,
                                              float (&v)[P])
{
    const int l16 = threadIdx.x & 15;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int e = l16 + 16 * p;
        v[p] = (e < E) ? l[e] : 0.0f;
    }
}

// Top-k of the token of each 16-lane row (all lanes active, k <= 16). Each lane keeps its keys
// (0 marks an expert taken or absent) and its best remaining one: the largest key, the lowest
// expert among equal keys of the lane. Round j takes the row's largest key and, among the lanes
// holding it, the lowest expert id (two DPP reductions inside the row), so the winner is the
// largest logit with ties to the lower id; its owner clears the key and rescans. Lane j < k of the
// row keeps slot j; `valid` = false (a row past the last token) routes nothing and writes
// nothing. The weights use double-precision exp and division, rounded once to fp32. Returns the
// lane's expert id for lanes j < k of a valid row, else -1.
template <int P>
__device__ __forceinline__ int route_row16(const float (&v)[P], int32_t E, int32_t k, bool valid,
                                           int32_t* __restrict__ idx_out,
                                           float* __restrict__ w_out)
{
    const int l16 = threadIdx.x & 15;
    uint32_t key[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        key[p] = (valid && l16 + 16 * p < E) ? logit_key(v[p]) : 0u;
    uint32_t bk = 0u;
    int bp = 0;
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (key[p] > bk) {
            bk = key[p];
            bp = p;
        }
    int my_id = -1;
    uint32_t my_key = 0u, top_key = 0u;
    for (int j = 0; j < k; ++j) {
        const uint32_t m = row16_max_u32(bk);
        const uint32_t mine = (uint32_t)(l16 + 16 * bp);
        const uint32_t cand = row16_min_u32((m != 0u && bk == m) ? mine : 0xFFFFFFFFu);
        if (j == 0)
            top_key = m;
        if (l16 == j && m != 0u) {
            my_id = (int)cand;
            my_key = m;
        }
        if (m != 0u && bk == m && mine == cand) {      // the owner clears its key and rescans
#pragma unroll
            for (int p = 0; p < P; ++p)
                key[p] = (p == bp) ? 0u : key[p];
            bk = 0u;
            bp = 0;
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (key[p] > bk) {
                    bk = key[p];
                    bp = p;
                }
        }
    }
    const bool slot = valid && l16 < k;
    double ex = slot ? exp((double)key_logit(my_key) - (double)key_logit(top_key)) : 0.0;
    double sum = ex;
    sum = dpp_add_f64<kDppQuadXor1>(sum);
    sum = dpp_add_f64<kDppQuadXor2>(sum);
    sum = dpp_add_f64<kDppRowHalfMirror>(sum);
    sum = dpp_add_f64<kDppRowMirror>(sum);
    if (slot && idx_out != nullptr) {                   // null outputs: the ids only
        idx_out[l16] = my_id;
        w_out[l16] = (float)(ex / sum);
    }
    return slot ? my_id : -1;
}

// Routing only, 16 lanes a token: 4 tokens per wavefront, 16 per workgroup.
template <int P>
__global__ __launch_bounds__(kThreads) void k_route_topk(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w)
{
    const int64_t t = (int64_t)blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
    const bool valid = t < T;
    float v[P];
    load_logits16<P>(logits + (valid ? t : 0) * E, valid ? E : 0, v);
    route_row16<P>(v, E, k, valid, topk_idx + t * k, topk_w + t * k);
}

// Routing plus the counting half of dispatch, 16 lanes a token (k <= 16). Workgroup b (4
// wavefronts) routes tokens 16b .. 16b+15 (token q of the block in row q % 4 of wavefront q / 4);
// each selected (token, slot) sets bit q of the LDS mask of its expert. A token's k experts are
// distinct, so the rank of (token, slot) among the block's items of the same expert, in (token,
// slot) order, is the number of mask bits below q, and the block's count of expert e is
// popcount(mask[e]), stored block-major at hist[b * E + e]. LDS: mask [E] u32.
// Workgroups past the routing blocks (blockIdx.x >= nblk) read x ahead for packing instead.
template <int P>
__global__ __launch_bounds__(kThreads) void k_route_layout(
    const float* __restrict__ logits, int32_t T, int32_t E, int32_t k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ local_rank, int32_t nblk, Prefetch pf, uint8_t* __restrict__ hist8,
    int32_t E16)
{
    if ((int32_t)blockIdx.x >= nblk) {                   // uniform per workgroup, before barriers
        prefetch_span(pf, (int)blockIdx.x - nblk);
        return;
    }
    extern __shared__ uint32_t lds_mask32[];
    const int tid = threadIdx.x, l16 = tid & 15;
    const int q = tid >> 4;                              // token of the block, 0..15
    for (int e = tid; e < E; e += kThreads)
        lds_mask32[e] = 0u;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * kRouteTokens16 + q;
    const bool valid = t < T;
    float v[P];
    load_logits16<P>(logits + (valid ? t : 0) * E, valid ? E : 0, v);
    const int my_id = route_row16<P>(v, E, k, valid, topk_idx + t * k, topk_w + t * k);
    if (my_id >= 0)
        atomicOr(&lds_mask32[my_id], 1u << q);
    __syncthreads();
    if (my_id >= 0)
        local_rank[t * k + l16] = (uint32_t)__popc(lds_mask32[my_id] & ((1u << q) - 1u));
    store_block_counts(lds_mask32, E, blockIdx.x, hist, hist8, E16);
}

// --------------------------------------------------------------------------------- layout --
// Items are the (token, slot) pairs in index order i = t*k + j.
//
// Caller-given ids (which may repeat within a token): block b owns the contiguous items
// [b*rows_per_block, (b+1)*rows_per_block) and walks them 256 at a time. For each group, every
// item sets its lane bit in the LDS mask of (its wavefront, its expert); its rank among the
// block's items of the same expert is then
//   run[e] + (bits of e in lower wavefronts) + (bits of e in lower lanes of its own wavefront),
// which keeps index order without any atomic deciding a position. The first item of each expert
// in the group then advances run[e] and clears the masks. The block's counts go to
// hist[b * E + e] (block-major, one coalesced row). LDS: masks [4][E] u64, run [E] u32.
// Workgroups past the blocks (blockIdx.x >= nblk) read x ahead for packing instead.
__global__ __launch_bounds__(kThreads) void k_layout_hist(const int32_t* __restrict__ topk_idx,
                                                          int32_t R, int32_t E,
                                                          int32_t rows_per_block,
                                                          uint32_t* __restrict__ hist,
                                                          uint32_t* __restrict__ local_rank,
                                                          int32_t nblk, Prefetch pf)
{
    if ((int32_t)blockIdx.x >= nblk) {                   // uniform per workgroup, before barriers
        prefetch_span(pf, (int)blockIdx.x - nblk);
        return;
    }
    extern __shared__ uint64_t lds_u64[];
    uint64_t* mask = lds_u64;
    uint32_t* run = reinterpret_cast<uint32_t*>(mask + kWaves * E);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < kWaves * E; i += kThreads)
        mask[i] = 0ull;
    for (int i = tid; i < E; i += kThreads)
        run[i] = 0u;
    const uint64_t lower_lanes = (1ull << lane) - 1ull;
    const int64_t first = (int64_t)blockIdx.x * rows_per_block;
    const int64_t last = first + rows_per_block < R ? first + rows_per_block : R;
    int e_next = (first + tid < last) ? topk_idx[first + tid] : -1;
    __syncthreads();
    for (int64_t i = first + tid; i - tid < last; i += kThreads) {
        int e = e_next;
        if (i + kThreads < last)
            e_next = topk_idx[i + kThreads];            // prefetch the next group's id
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
            for (int w = 0; w < kWaves; ++w) {
                n += (uint32_t)__popcll(mask[w * E + e]);
                mask[w * E + e] = 0ull;
            }
            run[e] += n;
        }
        __syncthreads();
        if (i < last)
            local_rank[i] = rank;
    }
    for (int e = tid; e < E; e += kThreads)
        hist[(int64_t)blockIdx.x * E + e] = run[e];
}

// Scan of the block histograms (stored block-major, hist[b * E + e]). A workgroup takes
// kScanExperts neighbouring experts: thread (q, u) = (tid / kScanExperts, tid % kScanExperts)
// gathers the counts of expert e = first + u in blocks q*S .. q*S+S-1, so one load instruction of a
// wavefront reads 16 short runs of kScanExperts words instead of 64 scattered words. Wavefront u
// then scans the 64 per-thread sums of expert u in LDS, and every thread writes its S exclusive
// prefixes: prefix[e * nblk + b] = rows of e in blocks before b; e's total goes to totals[e].
// Requires nblk <= 64 * S (nblk = 0 gives zero totals). Workgroups from `groups` on read x ahead
// for packing instead.
template <int S>
__global__ __launch_bounds__(kThreads) void k_expert_scan(const uint32_t* __restrict__ hist,
                                                          int32_t E, int32_t nblk,
                                                          uint32_t* __restrict__ prefix,
                                                          uint32_t* __restrict__ totals,
                                                          int32_t groups, Prefetch pf)
{
    if ((int32_t)blockIdx.x >= groups) {                 // uniform per workgroup, before barriers
        prefetch_span(pf, (int)blockIdx.x - groups);
        return;
    }
    static_assert(kThreads == 64 * kScanExperts, "one scanning wavefront per expert");
    __shared__ uint32_t part[kScanExperts * 64];
    const int u = threadIdx.x % kScanExperts;
    const int q = threadIdx.x / kScanExperts;
    const int e = blockIdx.x * kScanExperts + u;
    const bool valid = e < E;                            // no early return: barriers follow
    uint32_t c[S];
    uint32_t sum = 0u;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int b = q * S + s;
        c[s] = (valid && b < nblk) ? hist[(int64_t)b * E + e] : 0u;
        sum += c[s];
    }
    part[u * 64 + q] = sum;
    __syncthreads();
    {
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
        const uint32_t v = part[w * 64 + lane];
        const uint32_t incl = wave_inclusive_scan_u32(v);
        part[w * 64 + lane] = incl - v;
        const int ew = blockIdx.x * kScanExperts + w;
        if (lane == 63 && ew < E)
            totals[ew] = incl;
    }
    __syncthreads();
    uint32_t run = part[u * 64 + q];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int b = q * S + s;
        if (valid && b < nblk)
            prefix[(int64_t)e * nblk + b] = run;
        run += c[s];
    }
}

// The count outputs of dispatch: expert and rank counts and offsets (offsets end with the row
// count at [E] / [N]); rank r hosts experts [r*E/N, (r+1)*E/N).
struct CountOutputs {
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* rank_counts;
    int32_t* rank_offsets;
    int32_t N;
};

// Packing windows. A window is `blocks_per_window` consecutive layout blocks, sized so that the
// x rows of its tokens fit in one XCD's L2. For every window the rows kernel lists the window's
// (row, token) pairs in ascending row order: list[w0 + q] is the q-th smallest destination row
// of the window that starts at item w0 (entries past the window's valid rows hold (-1, -1)).
//
// Expert-parallel send (ep_counts != nullptr): the rows go to the source's regions instead. Rank
// r's rows of source s fill region (r, s) = rows [(r*S + s)*cap, ...) in (expert, token, slot)
// order, so row = (r*S + s)*cap + (expert_offset[e] - expert_offset[r*L]) + prefix + rank (-1
// past the region's cap rows, which only ids repeated within a token can reach); the
// per-(rank, source, local expert) counts go to ep_counts, and row_token is not written.
struct RowPlan {
    const int32_t* topk_idx;
    const uint32_t* local_rank;
    const uint32_t* prefix;
    const uint32_t* totals;
    int32_t* token_row;
    int32_t* row_token;
    int2* list;
    int32_t E, nblk, rows_per_block;
    int32_t blocks_per_window, groups_per_window;
    int32_t* ep_counts;
    int32_t ep_source, ep_sources, ep_cap, ep_L;
};

// Rows of the items. Workgroup g of window w takes kThreads items of the window. Every workgroup
// first turns the E expert totals into expert offsets (an exclusive scan in LDS: E <= 1024 is four
// values a thread) and the window's per-expert row counts
// n[e] = prefix[e * nblk + b1] - prefix[e * nblk + b0] into their exclusive scan C[e] (rows of
// lower experts in the window); workgroup 0 also writes the count outputs. Item i of block b with
// expert e then takes row expert_offset[e] + prefix[e * nblk + b] + local_rank[i] (recorded in
// token_row[i] and row_token[row]) and list position C[e] + prefix[e * nblk + b] -
// prefix[e * nblk + b0] + local_rank[i] within its window. An id outside [0, E) gets token_row -1
// and no row. LDS: eoff [E + 1] u32, qbase [E] i32.
// Workgroups from `groups` on read x ahead for packing instead.
__global__ __launch_bounds__(kThreads) void k_layout_rows(RowPlan rp, int32_t R, int32_t k,
                                                          CountOutputs co, int32_t groups,
                                                          Prefetch pf)
{
    if ((int32_t)blockIdx.x >= groups) {                 // uniform per workgroup, before barriers
        prefetch_span(pf, (int)blockIdx.x - groups);
        return;
    }
    constexpr int kPer = (MOE_MAX_EXPERTS + kThreads - 1) / kThreads;
    __shared__ uint32_t eoff[MOE_MAX_EXPERTS + 1];
    __shared__ int32_t qbase[MOE_MAX_EXPERTS];
    __shared__ uint32_t wave_tot[kWaves];
    const int tid = threadIdx.x, E = rp.E;
    const int w = blockIdx.x / rp.groups_per_window;
    const int g = blockIdx.x - w * rp.groups_per_window;
    const int b0 = w * rp.blocks_per_window;
    const int b1 = min(b0 + rp.blocks_per_window, rp.nblk);
    const bool in_window = b0 < rp.nblk;                 // uniform: false only for an empty batch
    uint32_t v[kPer], p0[kPer], n[kPer];
    uint32_t mine = 0u, mine_n = 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = tid * kPer + u;
        const bool ok = e < E;
        v[u] = ok ? rp.totals[e] : 0u;
        p0[u] = (ok && in_window) ? rp.prefix[(int64_t)e * rp.nblk + b0] : 0u;
        const uint32_t p1 = (ok && in_window)
                                ? (b1 < rp.nblk ? rp.prefix[(int64_t)e * rp.nblk + b1] : v[u])
                                : 0u;
        n[u] = p1 - p0[u];
        mine += v[u];
        mine_n += n[u];
    }
    uint32_t total = 0u, window_rows = 0u;
    uint32_t run = block_exclusive_scan<kThreads>(mine, wave_tot, &total);
    __syncthreads();                                     // wave_tot is reused below
    uint32_t run_n = block_exclusive_scan<kThreads>(mine_n, wave_tot, &window_rows);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int e = tid * kPer + u;
        if (e < E) {
            eoff[e] = run;
            qbase[e] = (int32_t)(run_n - p0[u]);
        }
        run += v[u];
        run_n += n[u];
    }
    if (tid == 0)
        eoff[E] = total;
    __syncthreads();
    const bool ep = rp.ep_counts != nullptr;
    if (blockIdx.x == 0 && ep) {
        for (int e = tid; e < E; e += kThreads)
            rp.ep_counts[((int64_t)(e / rp.ep_L) * rp.ep_sources + rp.ep_source) * rp.ep_L +
                         e % rp.ep_L] = (int32_t)(eoff[e + 1] - eoff[e]);
    } else if (blockIdx.x == 0) {
        const int epr = E / co.N;
        for (int e = tid; e < E; e += kThreads) {
            co.expert_offsets[e] = (int32_t)eoff[e];
            co.expert_counts[e] = (int32_t)(eoff[e + 1] - eoff[e]);
        }
        for (int r = tid; r < co.N; r += kThreads) {
            co.rank_offsets[r] = (int32_t)eoff[r * epr];
            co.rank_counts[r] = (int32_t)(eoff[(r + 1) * epr] - eoff[r * epr]);
        }
        if (tid == 0) {
            co.expert_offsets[E] = (int32_t)total;
            co.rank_offsets[co.N] = (int32_t)total;
        }
    }
    if (!in_window)
        return;
    const int64_t w0 = (int64_t)b0 * rp.rows_per_block;
    const int64_t w1 = min((int64_t)b1 * rp.rows_per_block, (int64_t)R);
    const int64_t i = w0 + (int64_t)g * kThreads + tid;
    if (i >= w1)
        return;
    const int e = rp.topk_idx[i];
    const int32_t t = (int32_t)(i / k);
    int32_t row = -1;
    if ((uint32_t)e < (uint32_t)E) {
        const uint32_t pf =
            rp.prefix[(int64_t)e * rp.nblk + i / rp.rows_per_block] + rp.local_rank[i];
        if (ep) {                                        // a row past the region is skipped
            const int r = e / rp.ep_L;
            const uint32_t pos = (eoff[e] - eoff[r * rp.ep_L]) + pf;
            row = pos < (uint32_t)rp.ep_cap
                      ? (int32_t)(((int64_t)r * rp.ep_sources + rp.ep_source) * rp.ep_cap + pos)
                      : -1;
        } else {
            row = (int32_t)(eoff[e] + pf);
        }
        rp.list[w0 + (qbase[e] + (int32_t)pf)] = make_int2(row, t);
    }
    rp.token_row[i] = row;
    if (!ep && (uint32_t)row < (uint32_t)R)
        rp.row_token[row] = t;
    if (i - w0 >= (int64_t)window_rows)                  // past the window's valid rows
        rp.list[i] = make_int2(-1, -1);
}

// Rows of routed items without a separate scan launch. The routing launch stores the blocks'
// counts as bytes, block-major (store_block_counts), and every workgroup of this launch sums the
// whole table itself: e's total, e's rows in the blocks before the workgroup's window, and the
// exclusive prefix of e's counts over the window's blocks. Workgroup g of window w then takes
// kRows8Threads items of the window; item i of block b with expert e takes
//   row = expert_offset[e] + before_window[e] + in_window_prefix[b][e] + local_rank[i]
// and list position qbase[e] + in_window_prefix[b][e] + local_rank[i] of its window, qbase[e]
// being the window's rows of lower experts. Outputs are those of k_layout_rows (without the
// expert-parallel mode).
//
// Summing the table: a 16-lane DPP row takes one 16-byte column c (16 experts) and lane l of it
// the table rows l, l + 16, l + 32, ...: every load instruction of a wavefront reads 16 rows x 64
// contiguous bytes, all loads of a lane are issued at once, and the bytes are added as pairs of
// 16-bit lanes (even and odd bytes of each word; no sum reaches 2^16: a count is at most 16 and a
// total at most the token count). Reductions over the 16 lanes of a row are DPP butterflies, and
// the window's prefixes a DPP row scan with a carry from one group of 16 rows to the next, so no
// value goes through LDS before the per-expert results. LDS (dynamic): wpre [bpw][E16] u16, then
// tot, pre, wcnt, eoff, qbase [E16] u32. Workgroups from `groups` on read x ahead for packing.
constexpr int kRows8Threads = 512;
constexpr int kRows8Waves = kRows8Threads / 64;
constexpr int kRows8Batch = 16;                    // table rows a lane loads at once

struct RowPlan8 {
    const int32_t* topk_idx;
    const uint32_t* local_rank;
    const uint8_t* hist8;     // [nblk][E16] counts
    int32_t* token_row;
    int32_t* row_token;
    int2* list;
    int32_t E, E16, nblk, rows_per_block;
    int32_t blocks_per_window, groups_per_window;
};

// Pairs of bytes of 16 experts in 16-bit lanes: p[j] holds experts 4j and 4j + 2 of the column
// (low, high half), p[4 + j] experts 4j + 1 and 4j + 3.
struct BytePairs {
    uint32_t p[8];
};

__device__ __forceinline__ void add_pairs(BytePairs& a, const u32x4& v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a.p[j] += w[j] & 0x00FF00FFu;
        a.p[4 + j] += (w[j] >> 8) & 0x00FF00FFu;
    }
}

// Sum over the 16 lanes of each DPP row, in every lane of the row.
__device__ __forceinline__ void row16_sum(BytePairs& a)
{
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t v = a.p[q];
        v += dpp_u32<kDppQuadXor1>(v);
        v += dpp_u32<kDppQuadXor2>(v);
        v += dpp_u32<kDppRowHalfMirror>(v);
        v += dpp_u32<kDppRowMirror>(v);
        a.p[q] = v;
    }
}

// Inclusive prefix over the lanes of each DPP row (lanes before the row's start add 0).
__device__ __forceinline__ void row16_inclusive(BytePairs& a)
{
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t v = a.p[q];
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // shr:1
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // shr:2
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);   // shr:4
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);   // shr:8
        a.p[q] = v;
    }
}

// The 16-bit value of expert x (0..15) of the column.
__device__ __forceinline__ uint32_t pair_value(const BytePairs& a, int x)
{
    const int j = x >> 2, q = x & 3;
    uint32_t w = 0u;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
        w = (jj == j) ? ((q & 1) ? a.p[4 + jj] : a.p[jj]) : w;
    return (q & 2) ? (w >> 16) : (w & 0xFFFFu);
}

// The 16 values in expert order as 16-bit words (two 16-byte stores).
__device__ __forceinline__ void store_pairs_u16(uint16_t* dst, const BytePairs& a)
{
    u32x4 lo, hi;
    lo.x = (a.p[0] & 0xFFFFu) | (a.p[4] << 16);
    lo.y = (a.p[0] >> 16) | (a.p[4] & 0xFFFF0000u);
    lo.z = (a.p[1] & 0xFFFFu) | (a.p[5] << 16);
    lo.w = (a.p[1] >> 16) | (a.p[5] & 0xFFFF0000u);
    hi.x = (a.p[2] & 0xFFFFu) | (a.p[6] << 16);
    hi.y = (a.p[2] >> 16) | (a.p[6] & 0xFFFF0000u);
    hi.z = (a.p[3] & 0xFFFFu) | (a.p[7] << 16);
    hi.w = (a.p[3] >> 16) | (a.p[7] & 0xFFFF0000u);
    reinterpret_cast<u32x4*>(dst)[0] = lo;
    reinterpret_cast<u32x4*>(dst)[1] = hi;
}

// Two exclusive scans over the block at once (one value of each per thread), one barrier.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* wave_tot,
                                                      uint32_t& ea, uint32_t& eb, uint32_t& ta,
                                                      uint32_t& tb)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t ia = wave_inclusive_scan_u32(a), ib = wave_inclusive_scan_u32(b);
    if (lane == 63) {
        wave_tot[2 * wave] = ia;
        wave_tot[2 * wave + 1] = ib;
    }
    __syncthreads();
    uint32_t ba = 0u, bb = 0u;
    ta = 0u;
    tb = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t sa = wave_tot[2 * w], sb = wave_tot[2 * w + 1];
        ba += (w < wave) ? sa : 0u;
        bb += (w < wave) ? sb : 0u;
        ta += sa;
        tb += sb;
    }
    ea = ba + ia - a;
    eb = bb + ib - b;
}

__global__ __launch_bounds__(kRows8Threads) void k_layout_rows8(RowPlan8 rp, int32_t R, int32_t k,
                                                                CountOutputs co, int32_t groups,
                                                                Prefetch pf)
{
    if ((int32_t)blockIdx.x >= groups) {                 // uniform per workgroup, before barriers
        prefetch_span(pf, (int)blockIdx.x - groups);
        return;
    }
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_r8[];
    __shared__ uint32_t wave_tot[2 * kRows8Waves];
    const int tid = threadIdx.x, E = rp.E, E16 = rp.E16, bpw = rp.blocks_per_window;
    uint16_t* wpre = reinterpret_cast<uint16_t*>(lds_r8);                        // [bpw][E16]
    uint32_t* tot = reinterpret_cast<uint32_t*>(lds_r8 + (int64_t)2 * bpw * E16);
    uint32_t* pre = tot + E16;                                                    // [E16]
    uint32_t* wcnt = pre + E16;                                                   // [E16]
    uint32_t* eoff = wcnt + E16;                                                  // [E16]
    uint32_t* qbase = eoff + E16;                                                 // [E16]
    const int w = blockIdx.x / rp.groups_per_window;
    const int g = blockIdx.x - w * rp.groups_per_window;
    const int b0 = w * bpw;
    const int b1 = min(b0 + bpw, rp.nblk);
    const int64_t w0 = (int64_t)b0 * rp.rows_per_block;
    const int64_t w1 = min((int64_t)b1 * rp.rows_per_block, (int64_t)R);
    const int64_t i = w0 + (int64_t)g * kRows8Threads + tid;
    const bool item = b0 < rp.nblk && i < w1;
    int e_i = -1;
    uint32_t lr = 0u;
    if (item) {                                          // in flight while the table is summed
        e_i = rp.topk_idx[i];
        lr = rp.local_rank[i];
    }

    // the table: DPP row d of the workgroup takes columns d, d + 32, ...; lane l16 the rows
    // l16, l16 + 16, ... (every lane of a wavefront runs the same iterations)
    const int C = E16 / 16, l16 = tid & 15;
    const int passes = (C + kRows8Threads / 16 - 1) / (kRows8Threads / 16);
    const u32x4* h = reinterpret_cast<const u32x4*>(rp.hist8);
    for (int pass = 0; pass < passes; ++pass) {
        const int c = (tid >> 4) + pass * (kRows8Threads / 16);
        const bool col = c < C;                          // uniform per DPP row
        BytePairs all = {}, bef = {}, carry = {};
        for (int r0 = 0; r0 < rp.nblk; r0 += 16 * kRows8Batch) {   // uniform
            u32x4 v[kRows8Batch];
#pragma unroll
            for (int u = 0; u < kRows8Batch; ++u) {
                const int r = r0 + 16 * u + l16;
                v[u] = (col && r < rp.nblk) ? h[(int64_t)r * C + c] : u32x4{0u, 0u, 0u, 0u};
            }
            // 8 rows at a time as plain bytes (a byte sum of 8 counts <= 16 stays below 256),
            // then widened once into the 16-bit pairs
#pragma unroll
            for (int u0 = 0; u0 < kRows8Batch; u0 += 8) {
                const int rlo = r0 + 16 * u0, rhi = r0 + 16 * (u0 + 8);   // rows [rlo, rhi)
                u32x4 acc = v[u0];
#pragma unroll
                for (int u = u0 + 1; u < u0 + 8; ++u)
                    acc += v[u];
                add_pairs(all, acc);
                if (rhi <= b0) {                         // every row before the window (uniform)
                    add_pairs(bef, acc);
                } else if (rlo < b0) {                   // the chunk holding b0 (uniform)
                    u32x4 part = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int u = u0; u < u0 + 8; ++u)
                        if (r0 + 16 * u + l16 < b0)
                            part += v[u];
                    add_pairs(bef, part);
                }
            }
        }
        // the window's rows again (from cache), 16 at a time: row scan plus the carry so far
        for (int rb = b0 & ~15; rb < b1; rb += 16) {     // uniform
            const int r = rb + l16;
            const bool in = col && r >= b0 && r < b1;
            BytePairs x = {};
            if (in)
                add_pairs(x, h[(int64_t)r * C + c]);
            BytePairs incl = x, grp = x;
            row16_inclusive(incl);
            row16_sum(grp);
            if (in) {
                BytePairs ex;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    ex.p[q] = carry.p[q] + incl.p[q] - x.p[q];
                store_pairs_u16(wpre + (int64_t)(r - b0) * E16 + 16 * c, ex);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                carry.p[q] += grp.p[q];
        }
        row16_sum(all);
        row16_sum(bef);
        if (col) {                                       // lane l16 writes expert 16c + l16
            const int e = 16 * c + l16;
            tot[e] = pair_value(all, l16);
            pre[e] = pair_value(bef, l16);
            wcnt[e] = pair_value(carry, l16);
        }
    }
    __syncthreads();

    // expert offsets and the window's list bases; thread u takes experts 2u and 2u + 1
    // (E16 <= 2 * kRows8Threads)
    uint32_t tc[2] = {0u, 0u}, wc[2] = {0u, 0u};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int e = 2 * tid + u;
        if (e < E16) {
            tc[u] = tot[e];
            wc[u] = wcnt[e];
        }
    }
    uint32_t ex, qx, total, window_rows;
    block_exclusive_scan2<kRows8Threads>(tc[0] + tc[1], wc[0] + wc[1], wave_tot, ex, qx, total,
                                         window_rows);
    if (2 * tid < E16) {
        eoff[2 * tid] = ex;
        qbase[2 * tid] = qx;
    }
    if (2 * tid + 1 < E16) {
        eoff[2 * tid + 1] = ex + tc[0];
        qbase[2 * tid + 1] = qx + wc[0];
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        const int epr = E / co.N;
        for (int e = tid; e < E; e += kRows8Threads) {
            co.expert_offsets[e] = (int32_t)eoff[e];
            co.expert_counts[e] = (int32_t)tot[e];
        }
        for (int r = tid; r < co.N; r += kRows8Threads) {
            co.rank_offsets[r] = (int32_t)eoff[r * epr];
            uint32_t n = 0u;
            for (int e = r * epr; e < (r + 1) * epr; ++e)
                n += tot[e];
            co.rank_counts[r] = (int32_t)n;
        }
        if (tid == 0) {
            co.expert_offsets[E] = (int32_t)total;
            co.rank_offsets[co.N] = (int32_t)total;
        }
    }
    if (!item)
        return;
    const int32_t t = (int32_t)(i / k);
    int32_t row = -1;
    if ((uint32_t)e_i < (uint32_t)E) {
        const int bi = (int)(i / rp.rows_per_block) - b0;
        const uint32_t inw = (uint32_t)wpre[bi * E16 + e_i] + lr;
        row = (int32_t)(eoff[e_i] + pre[e_i] + inw);
        rp.list[w0 + (int64_t)(qbase[e_i] + inw)] = make_int2(row, t);
    }
    rp.token_row[i] = row;
    if ((uint32_t)row < (uint32_t)R)
        rp.row_token[row] = t;
    if (i - w0 >= (int64_t)window_rows)                  // past the window's valid rows
        rp.list[i] = make_int2(-1, -1);
}

// ------------------------------------------------------------ routing precondition check --
// What dispatch takes for granted about ids that do not come from the router: every slot names one
// of the E experts, and no token names one expert twice. counts[0] += slots whose id lies outside
// [0, E); counts[1] += slots whose in-range id equals the id of an earlier slot of the same token.
// Grid-stride over the slots; each wavefront adds its two sums with one atomic each to the counts
// that k_zero_i32 cleared before it.
__global__ __launch_bounds__(64) void k_zero_i32(int32_t* __restrict__ p, int32_t n)
{
    if ((int32_t)threadIdx.x < n)
        p[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kThreads) void k_check_topk(const int32_t* __restrict__ topk_idx,
                                                         int64_t R, int32_t k, int32_t E,
                                                         int32_t* __restrict__ counts)
{
    uint32_t bad = 0u, rep = 0u;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < R; i += stride) {
        const int32_t id = topk_idx[i];
        if ((uint32_t)id >= (uint32_t)E) {
            ++bad;
            continue;
        }
        for (int64_t q = i - i % k; q < i; ++q)
            if (topk_idx[q] == id) {
                ++rep;
                break;
            }
    }
    bad = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan_u32(bad), 63);
    rep = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan_u32(rep), 63);
    if ((threadIdx.x & 63) == 0 && (bad | rep) != 0u) {
        atomicAdd(&counts[0], (int32_t)bad);
        atomicAdd(&counts[1], (int32_t)rep);
    }
}

// ---------------------------------------------------------------------- expert-parallel receive --
// Receiver half of dispatch for one rank, planning step. The S*L segments
// (local expert l, source s) are taken in (l, s) order: segment (l, s) holds the
// region_counts[(rank*S + s)*L + l] rows that source s wrote for expert rank*L + l, which start in
// its region (rank, s) after its rows of lower experts. An exclusive scan of the segment sizes
// gives the grouped layout (expert, source, token, slot); every grouped row g then finds its
// segment by binary search and records its region row in grouped_src[g] (-1 past the last row).
// Every workgroup repeats the (small) scan and takes its share of the grouped rows; workgroup 0
// also writes the rank's per-expert counts and offsets. LDS: 3 * kMaxEpSegments u32.
__global__ __launch_bounds__(kGroupThreads) void k_ep_recv_plan(
    const int32_t* __restrict__ region_counts, int32_t rank, int32_t S, int32_t L, int32_t cap,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ grouped_src)
{
    constexpr int kPer = kMaxEpSegments / kGroupThreads;
    __shared__ uint32_t cnt[kMaxEpSegments];             // source-major: s*L + l
    __shared__ uint32_t srcoff[kMaxEpSegments];          // source-major: start in the region
    __shared__ uint32_t dst[kMaxEpSegments + 1];         // (l, s) order: start in the grouped rows
    __shared__ uint32_t wave_tot[kGroupWaves];
    const int tid = threadIdx.x;
    const int nseg = S * L;
    for (int q = tid; q < nseg; q += kGroupThreads)
        cnt[q] = (uint32_t)region_counts[(int64_t)rank * nseg + q];
    __syncthreads();
    for (int s = tid; s < S; s += kGroupThreads) {       // per-source scan over its experts
        uint32_t run = 0u;
        for (int l = 0; l < L; ++l) {
            srcoff[s * L + l] = run;
            run += cnt[s * L + l];
        }
    }
    uint32_t v[kPer];
    uint32_t mine = 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int q = tid * kPer + u;                    // (l, s) order: q = l*S + s
        v[u] = q < nseg ? cnt[(q % S) * L + q / S] : 0u;
        mine += v[u];
    }
    uint32_t total = 0u;
    uint32_t run = block_exclusive_scan<kGroupThreads>(mine, wave_tot, &total);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int q = tid * kPer + u;
        if (q < nseg)
            dst[q] = run;
        run += v[u];
    }
    if (tid == 0)
        dst[nseg] = total;
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int l = tid; l < L; l += kGroupThreads) {
            expert_offsets[l] = (int32_t)dst[l * S];
            expert_counts[l] = (int32_t)(dst[(l + 1) * S] - dst[l * S]);
        }
        if (tid == 0)
            expert_offsets[L] = (int32_t)total;
    }
    for (int64_t g = (int64_t)blockIdx.x * kGroupThreads + tid; g < (int64_t)S * cap;
         g += (int64_t)gridDim.x * kGroupThreads) {
        int32_t src = -1;
        if (g < (int64_t)total) {
            int lo = 0, hi = nseg - 1;                   // last q with dst[q] <= g
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (dst[mid] <= (uint32_t)g)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int s = lo % S, l = lo / S;
            src = (int32_t)(((int64_t)rank * S + s) * cap + srcoff[s * L + l] + (g - dst[lo]));
        }
        grouped_src[g] = src;
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

// Which rows a packing wavefront writes, and from which token. TOKEN_ORDER: wavefront (token t,
// piece) loads its piece of x once and stores it to all k rows token_row[t*k + j]; the pieces
// wavefronts of a token run on one XCD (tokens x, x+8, ... on XCD x). One load for k stores keeps
// k times more bytes in flight per wavefront than one store per load, which is what hides x
// coming from HBM (prefill, x cold, the pack alone: 105-108 us against 130-138 us). WINDOWS: wavefront (window w, list position q, piece) with (row, token) = list[w*rw + q];
// the windows of XCD x are x, x+8, ..., so the window's x rows stay in one L2 while its rows go
// out in ascending order, which keeps the writes of the whole GPU in a narrow address range.
enum PackOrder { PACK_TOKEN_ORDER = 0, PACK_WINDOWS = 1 };

// Wavefronts per packing workgroup: 16 in token order, 8 in window order (each measured best).
template <int ORDER>
constexpr int pack_waves()
{
    return ORDER == PACK_WINDOWS ? kPackWavesWindows : kPackWaves;
}

struct PackPlan {
    const int32_t* token_row;
    const int2* list;
    int32_t T, k, R, pieces;          // R = T*k items
    int32_t window_pieces;            // window order: work items per row (pieces / pieces a wave)
    int32_t rows_per_window, nwin;
    int64_t row_limit;                // rows of the destination buffer
};

// The (token, row, piece) of a wavefront: for TOKEN_ORDER the k rows are read by the caller
// after the x load has been issued (row = -1 here), for WINDOWS both come from the list.
// token = -1: nothing to copy.
struct PackItem {
    int64_t token;
    int32_t row;
    int piece;
};

template <int ORDER>
__device__ __forceinline__ PackItem pack_item(const PackPlan& pp)
{
    PackItem it;
    it.token = -1;
    it.row = -1;
    it.piece = 0;
    if constexpr (ORDER == PACK_TOKEN_ORDER) {
        const XcdItem xi = xcd_item(pack_waves<ORDER>(), pp.pieces);
        if (xi.token < pp.T) {
            it.piece = xi.sub;
            it.token = xi.token;
        }
    } else {
        const XcdItem xi = xcd_item(pack_waves<ORDER>(), pp.rows_per_window * pp.window_pieces);
        const int q = xi.sub / pp.window_pieces;
        const int64_t pos = xi.token * pp.rows_per_window + q;   // "token" is the window here
        if (xi.token < pp.nwin && pos < pp.R) {
            it.piece = xi.sub - q * pp.window_pieces;
            const int2 rt = pp.list[pos];
            if ((uint64_t)(uint32_t)rt.x < (uint64_t)pp.row_limit && rt.x >= 0) {
                it.row = rt.x;
                it.token = rt.y;
            }
        }
    }
    return it;
}

// One wavefront per (row, PPW consecutive 1 KB pieces of it) in window order, per (token, 1 KB
// piece) in token order: lane l copies chunks (piece*PPW + p)*64 + l (16 bytes each) of x's row
// to the destination row (to each of the token's k rows in token order) with non-temporal stores,
// all loads issued before the stores; x is read with plain loads so the wavefronts of a window
// find it in L2. The pieces of a row run side by side. A row outside [0, row_limit) is skipped.
// PPW > 1 only in window order.
template <int ORDER, int PPW>
__global__ __launch_bounds__(64 * pack_waves<ORDER>()) void k_pack_rows(
    const u32x4* __restrict__ x, int32_t chunks_per_row, PackPlan pp, u32x4* __restrict__ recv)
{
    const PackItem it = pack_item<ORDER>(pp);
    if (it.token < 0)
        return;                                          // uniform per wavefront
    const int c0 = it.piece * (64 * PPW) + (threadIdx.x & 63);
    u32x4 v[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        v[p] = u32x4{0u, 0u, 0u, 0u};
        if (c0 + 64 * p < chunks_per_row)
            v[p] = x[it.token * chunks_per_row + c0 + 64 * p];
    }
    if constexpr (ORDER == PACK_TOKEN_ORDER) {
        // the token's rows, 64 slots at a time: lane j of a group reads slot j0 + j, and the
        // wavefront stores its piece to each of them in slot order
        const int lane = threadIdx.x & 63;
        const int32_t* rows = pp.token_row + it.token * pp.k;
        for (int j0 = 0; j0 < pp.k; j0 += 64) {
            const int32_t mine = j0 + lane < pp.k ? rows[j0 + lane] : -1;
            const int n = pp.k - j0 < 64 ? pp.k - j0 : 64;
            for (int j = 0; j < n; ++j) {
                const int32_t row = __builtin_amdgcn_readlane(mine, j);
                if (row < 0 || (int64_t)row >= pp.row_limit)
                    continue;                            // uniform per wavefront
#pragma unroll
                for (int p = 0; p < PPW; ++p)
                    if (c0 + 64 * p < chunks_per_row)
                        __builtin_nontemporal_store(
                            v[p], recv + (int64_t)row * chunks_per_row + c0 + 64 * p);
            }
        }
    } else {
        const int32_t row = it.row;
        if (row < 0 || (int64_t)row >= pp.row_limit)
            return;
#pragma unroll
        for (int p = 0; p < PPW; ++p)
            if (c0 + 64 * p < chunks_per_row)
                __builtin_nontemporal_store(v[p],
                                            recv + (int64_t)row * chunks_per_row + c0 + 64 * p);
    }
}

// Copies of whole rows by a row map, grid-stride over (row, 1 KB piece) by wavefronts: GATHER
// dst[g] = src[map[g]], SCATTER dst[map[g]] = src[g], for g < min(*n_rows, max_rows); a map
// entry outside [0, row_limit) is skipped. The row count is read on the device (it is the output
// of the previous kernel), so every wavefront's loop ends at the same bound.
enum CopyDir { COPY_GATHER = 0, COPY_SCATTER = 1 };

template <int DIR>
__global__ __launch_bounds__(64 * kPackWaves) void k_copy_rows(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst,
                                                               int32_t chunks_per_row,
                                                               int32_t pieces,
                                                               const int32_t* __restrict__ map,
                                                               const int32_t* __restrict__ n_rows,
                                                               int64_t max_rows,
                                                               int64_t row_limit)
{
    int64_t n = *n_rows;
    n = n < 0 ? 0 : n > max_rows ? max_rows : n;
    const int64_t waves = (int64_t)gridDim.x * kPackWaves;
    const int lane = threadIdx.x & 63;
    for (int64_t m = (int64_t)blockIdx.x * kPackWaves + (threadIdx.x >> 6); m < n * pieces;
         m += waves) {
        const int64_t g = m / pieces;
        const int c = (int)(m - g * pieces) * 64 + lane;
        const int32_t r = map[g];
        if (r < 0 || (int64_t)r >= row_limit || c >= chunks_per_row)
            continue;
        if (DIR == COPY_GATHER)
            __builtin_nontemporal_store(src[(int64_t)r * chunks_per_row + c],
                                        dst + g * chunks_per_row + c);
        else
            __builtin_nontemporal_store(src[g * chunks_per_row + c],
                                        dst + (int64_t)r * chunks_per_row + c);
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

// Four e4m3 codes of quotients d with |d| < 464 or NaN, by the hardware conversion (round to
// nearest even; byte i of the result is the code of d[i]). The magnitude bits are kept and the sign
// is taken from d: for every such fp32 pattern this equals f32_to_e4m3 (checked over all 2^32
// patterns on gfx950; the hardware gives NaN one fixed sign, f32_to_e4m3 keeps the input's).
__device__ __forceinline__ uint32_t e4m3x4_hw(float d0, float d1, float d2, float d3)
{
    uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(d0, d1, 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(d2, d3, c, true);
    const uint32_t sign = ((__float_as_uint(d0) >> 31) << 7) | ((__float_as_uint(d1) >> 31) << 15) |
                          ((__float_as_uint(d2) >> 31) << 23) | (__float_as_uint(d3) & 0x80000000u);
    return (c & 0x7F7F7F7Fu) | sign;
}

// Block-scaled e4m3 of the 8 elements a lane holds, the 16 lanes of each DPP row forming one
// 128-element block (every lane of the wavefront takes part in the row maximum): scale
// s = amax / 448 (1 for an all-zero block, the division correctly rounded), codes e4m3(v / s) with
// v / s the correctly rounded fp32 quotient, packed little-endian into 8 bytes. Returns s.
//   - Usual blocks (amax finite, s normal, amax < 2^127): the quotient comes from the correctly
//     rounded reciprocal r = 1/s, q0 = |v|*r and one fused correction q0 + (|v| - q0*s)*r
//     (Markstein's division theorem: with r correctly rounded and q0 within an ulp, the corrected
//     quotient is the correctly rounded one, as long as the residual |v| - q0*s is exact). The
//     residual is formed on |v| and s scaled by 2^(127 - exponent of amax), exactly, so it cannot
//     underflow where the code is not zero; below 2^-11 the quotient may differ in its last bits but
//     both round to a zero code. The sign is copied from v. The codes then come from the hardware
//     conversion. Checked on gfx950 for every pair of bf16 values (v, amax) with |v| <= amax: the
//     codes equal those of the correctly rounded division and f32_to_e4m3.
//   - An all-zero block: s = 1, the quotient is v itself.
//   - Otherwise (amax infinite, s below the normal range, amax >= 2^127) the correctly rounded
//     division and f32_to_e4m3, which also saturate the infinite quotients these blocks can give.
// The case is the same for the 16 lanes of a row.
__device__ __forceinline__ float quantise8_e4m3(const float (&v)[8], u32x2& packed)
{
    // NaN elements, signalling ones too, take no part in the maximum: a comparison skips them,
    // where fmaxf would return NaN for a signalling NaN operand
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = fabsf(v[i]);
        amax = a > amax ? a : amax;
    }
    amax = max_row16_f32(amax);
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    const uint32_t ea = __float_as_uint(amax) >> 23;    // amax >= +0, never NaN
    float d[8];
    if (amax == 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            d[i] = v[i];
    } else if (ea <= 253u && s >= 0x1p-126f) {
        const float r = 1.0f / s;
        const float up = __uint_as_float((254u - ea) << 23);     // 2^(127 - ea)
        const float down = __uint_as_float(ea << 23);            // 2^(ea - 127)
        const float s_up = s * up, r_down = r * down;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a = fabsf(v[i]);
            const float q0 = a * r;
            d[i] = copysignf(fmaf(fmaf(-q0, s_up, a * up), r_down, q0), v[i]);
        }
    } else {
        // s > 0, so a quotient has the sign of v; that of a NaN quotient (an infinite v over an
        // infinite s) is left open by IEEE 754 and taken from v as well
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = f32_to_e4m3(copysignf(v[i] / s, v[i]));
        packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        return s;
    }
    packed.x = e4m3x4_hw(d[0], d[1], d[2], d[3]);
    packed.y = e4m3x4_hw(d[4], d[5], d[6], d[7]);
    return s;
}

// fp8 packing, one wavefront per (token t, piece of 64 chunks of 8 elements), placed like the
// token-order packing (tokens x, x+8, ... on XCD x). The 16 lanes of a DPP row hold the 128
// elements of one scale block (H % 128 == 0, so a row of lanes is all active or all inactive);
// every lane takes part in the reduction, only the stores are masked. Scale s = amax / 448 (1 for
// an all-zero block), codes e4m3(x / s). Each block is quantised once and its codes and scale are
// stored to all k rows of the token: lanes j < k read the k rows with one load, and store round j
// takes row j by readlane. A row outside [0, R) is skipped.
template <typename XT>
__global__ __launch_bounds__(64 * kPackWaves) void k_pack_rows_fp8(
    const XT* __restrict__ x, int32_t H, PackPlan pp, uint8_t* __restrict__ recv,
    float* __restrict__ recv_scales)
{
    const XcdItem xi = xcd_item(kPackWaves, pp.pieces);
    if (xi.token >= pp.T)
        return;                                          // uniform per wavefront
    const int lane = threadIdx.x & 63;
    const int c = xi.sub * 64 + lane;
    const bool active = c < H / 8;
    float v[8];
    if (active) {
        Load8<XT>::run(x + xi.token * H + (int64_t)c * 8, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = 0.0f;
    }
    const int32_t my_row = lane < pp.k ? pp.token_row[xi.token * pp.k + lane] : -1;
    u32x2 packed;
    const float s = quantise8_e4m3(v, packed);
    for (int j = 0; j < pp.k; ++j) {
        const int32_t row = __builtin_amdgcn_readlane(my_row, j);
        if (row < 0 || (int64_t)row >= pp.row_limit)
            continue;                                    // uniform per wavefront
        if (active) {
            __builtin_nontemporal_store(packed,
                                        reinterpret_cast<u32x2*>(recv + (int64_t)row * H) + c);
            if ((lane & 15) == 0)
                recv_scales[(int64_t)row * (H / 128) + c / 16] = s;
        }
    }
}

// ------------------------------------------------------------- layout and packing in one launch --
// Layout and packing of a batch of at most kLpTokens tokens (kLpCopyTokens for row copies) in one
// launch: at these sizes every launch costs more than its work, so the scan and row kernels are
// folded into the packing. Every workgroup rebuilds the whole layout in LDS from the T*k expert ids
// (read from L2):
//   - counts: one LDS atomic add per slot (order does not matter for a count); one block scan turns
//     them into expert offsets;
//   - ranks: token t sets bit t % 32 of word t / 32 of the mask of each of its experts. When no
//     token names an expert twice (always so for routed ids), item (t, j) with expert e takes row
//       eoff[e] + (bits of e's mask below bit t),
//     the stable (expert, token, slot) order of the layout kernels. A token naming an expert twice
//     finds its bit already set when inserting it; then every workgroup (they all read the same
//     ids) takes the exact rank instead: the wavefront counts the earlier slots with the same
//     expert, 64 slots a step.
// Wavefront m of the grid takes the units (token, piece) m, m + waves, ...: lanes j < k compute the
// token's k rows, the wavefront of piece 0 writes token_row and row_token, and every wavefront
// stores its piece of x to the k rows. LP_COPY copies 16-byte chunks; the fp8 modes quantise 8
// elements a lane (bf16 or fp32 x) once, as the fp8 packing kernel does, and store codes and scales
// to the k rows; LP_LAYOUT writes the row maps only (one unit a token). x and the ids of the
// wavefront's first unit are loaded before the layout is built, so those loads overlap it.
// Out-of-range ids are skipped (token_row -1). Workgroup 0 writes the count outputs.
// LDS: masks [words][E] u32 (word-major), offsets [E + 1] u32.
enum LayoutPackMode { LP_COPY = 0, LP_FP8_BF16 = 1, LP_FP8_F32 = 2, LP_LAYOUT = 3 };

struct LayoutPackPlan {
    const void* x;
    const int32_t* topk_idx;
    int32_t* token_row;
    int32_t* row_token;
    void* recv;
    float* recv_scales;
    int32_t T, k, E, H;
    int32_t words;        // ceil(T / 32) mask words per expert
    int32_t chunks;       // lane chunks per row: 16 bytes (copy) or 8 elements (fp8); 0 for layout
    int32_t pieces;       // ceil(chunks / 64), at least 1
    // expert-parallel send (ep_L > 0): rows go to the regions of this source, as in k_layout_rows
    int32_t* ep_counts;
    int32_t ep_source, ep_sources, ep_cap, ep_L;
    // routing in the same launch (RP > 0): logits in, ids and weights out (workgroup 0 writes them)
    const float* logits;
    int32_t* route_idx;
    float* route_w;
};

// Row of an item of expert e (in range) with rank `rank` among the expert's items: the packed row,
// or for an expert-parallel send the row in region (rank of e, source), -1 past the region.
__device__ __forceinline__ int32_t lp_row(const LayoutPackPlan& lp, const uint32_t* eoff, int32_t e,
                                          uint32_t rank)
{
    if (lp.ep_L == 0)
        return (int32_t)(eoff[e] + rank);
    const int32_t r = e / lp.ep_L;
    const uint32_t pos = eoff[e] - eoff[r * lp.ep_L] + rank;
    return pos < (uint32_t)lp.ep_cap
               ? (int32_t)(((int64_t)r * lp.ep_sources + lp.ep_source) * lp.ep_cap + pos)
               : -1;
}

template <int MODE>
__device__ __forceinline__ void lp_load(const LayoutPackPlan& lp, int64_t t, int c, u32x4& xv,
                                        float (&v)[8])
{
    if constexpr (MODE == LP_COPY)
        xv = static_cast<const u32x4*>(lp.x)[t * lp.chunks + c];
    else if constexpr (MODE == LP_FP8_BF16)
        Load8<uint16_t>::run(static_cast<const uint16_t*>(lp.x) + t * lp.H + c * 8, v);
    else if constexpr (MODE == LP_FP8_F32)
        Load8<float>::run(static_cast<const float*>(lp.x) + t * lp.H + c * 8, v);
}

template <int MODE, int RP, int NT = kLpThreads>
__global__ __launch_bounds__(NT) void k_layout_pack(LayoutPackPlan lp, CountOutputs co)
{
    extern __shared__ uint32_t lds_lp[];
    __shared__ uint32_t wave_tot[NT / 64];
    __shared__ uint32_t repeated;
    const int32_t E = lp.E, W = lp.words, k = lp.k;
    uint32_t* mask = lds_lp;                             // [W][E]
    uint32_t* eoff = lds_lp + (int64_t)W * E;            // [E + 1]: counts, then offsets
    int32_t* ids = reinterpret_cast<int32_t*>(eoff + E + 1);     // [T * k] when routing here
    const int32_t* __restrict__ topk_idx = RP > 0 ? ids : lp.topk_idx;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t waves = (int64_t)gridDim.x * (NT / 64);
    const int64_t units = (int64_t)lp.T * lp.pieces;
    int64_t u = (int64_t)blockIdx.x * (NT / 64) + (tid >> 6);       // uniform per wavefront

    // the first unit's payload and ids, in flight while the layout is built
    u32x4 xv = {0u, 0u, 0u, 0u};
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = 0.0f;
    int32_t id = -1;
    int64_t t = u / lp.pieces;
    int c = (int)(u - t * lp.pieces) * 64 + lane;
    if (u < units) {
        if (c < lp.chunks)
            lp_load<MODE>(lp, t, c, xv, v);
        if (RP == 0 && lane < k)
            id = lp.topk_idx[t * k + lane];
    }

    // routing (RP > 0, k <= 16): every workgroup routes the whole batch into LDS, 16 lanes a
    // token, NT / 16 tokens a pass; workgroup 0 also writes the ids and weights
    if constexpr (RP > 0) {
        for (int q0 = 0; q0 < lp.T; q0 += NT / 16) {     // uniform across the workgroup
            const int q = q0 + (tid >> 4);
            const bool valid = q < lp.T;
            float lg[RP];
            load_logits16<RP>(lp.logits + (int64_t)(valid ? q : 0) * E, valid ? E : 0, lg);
            const bool out = blockIdx.x == 0 && valid;
            const int my = route_row16<RP>(lg, E, k, valid, out ? lp.route_idx + q * k : nullptr,
                                           out ? lp.route_w + q * k : nullptr);
            if (valid && (tid & 15) < k)
                ids[q * k + (tid & 15)] = my;
        }
        __syncthreads();
        if (u < units && lane < k)
            id = ids[t * k + lane];
    }

    // the layout, in every workgroup. The thread's first ids are loaded before LDS is cleared, so
    // their latency overlaps the clearing and its barrier (at 128 decode tokens, two ids a thread:
    // 14.72 -> 14.50 us a step, decode-fp8 14.85 -> 14.56 us)
    const int32_t R = lp.T * k;
    constexpr int kPre = 2;
    int32_t pre_id[kPre];
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
        const int32_t i = tid + q * NT;
        pre_id[q] = (i < R) ? topk_idx[i] : -1;
    }
    for (int i = tid; i < W * E; i += NT)
        mask[i] = 0u;
    for (int i = tid; i <= E; i += NT)
        eoff[i] = 0u;
    if (tid == 0)
        repeated = 0u;
    __syncthreads();
    auto add_item = [&](int32_t i, int32_t e) {
        if ((uint32_t)e < (uint32_t)E) {
            const int32_t tt = i / k;
            const uint32_t bit = 1u << (tt & 31);
            if (atomicOr(&mask[(tt >> 5) * E + e], bit) & bit)
                repeated = 1u;                           // the token names e twice
            atomicAdd(&eoff[e], 1u);
        }
    };
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
        const int32_t i = tid + q * NT;
        if (i < R)
            add_item(i, pre_id[q]);
    }
    for (int32_t i = tid + kPre * NT; i < R; i += NT)
        add_item(i, topk_idx[i]);
    __syncthreads();
    const int e0 = 2 * tid, e1 = 2 * tid + 1;            // E <= 2 * NT
    const uint32_t c0 = e0 < E ? eoff[e0] : 0u;
    const uint32_t c1 = e1 < E ? eoff[e1] : 0u;
    uint32_t total = 0u;
    const uint32_t ex = block_exclusive_scan<NT>(c0 + c1, wave_tot, &total);
    if (e0 < E)
        eoff[e0] = ex;
    if (e1 < E)
        eoff[e1] = ex + c0;
    if (tid == 0)
        eoff[E] = total;
    __syncthreads();
    const bool exact = repeated != 0u;                   // uniform over the grid
    if (blockIdx.x == 0 && lp.ep_L > 0) {
        for (int e = tid; e < E; e += NT)
            lp.ep_counts[((int64_t)(e / lp.ep_L) * lp.ep_sources + lp.ep_source) * lp.ep_L +
                         e % lp.ep_L] = (int32_t)(eoff[e + 1] - eoff[e]);
    } else if (blockIdx.x == 0) {
        const int epr = E / co.N;
        for (int e = tid; e < E; e += NT) {
            co.expert_offsets[e] = (int32_t)eoff[e];
            co.expert_counts[e] = (int32_t)(eoff[e + 1] - eoff[e]);
        }
        for (int r = tid; r < co.N; r += NT) {
            co.rank_offsets[r] = (int32_t)eoff[r * epr];
            co.rank_counts[r] = (int32_t)(eoff[(r + 1) * epr] - eoff[r * epr]);
        }
        if (tid == 0) {
            co.expert_offsets[E] = (int32_t)total;
            co.rank_offsets[co.N] = (int32_t)total;
        }
    }

    // the wavefront's units; no barrier from here on
    for (bool first = true; u < units; u += waves, first = false) {
        if (!first) {
            t = u / lp.pieces;
            c = (int)(u - t * lp.pieces) * 64 + lane;
            if (c < lp.chunks) {
                lp_load<MODE>(lp, t, c, xv, v);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[i] = 0.0f;
            }
            id = lane < k ? topk_idx[t * k + lane] : -1;
        }
        // an item's own slot is among its expert's count, so its rank is below that count and
        // every packed row is below eoff[e + 1] <= R
        int32_t row = -1;
        if (!exact) {
            if ((uint32_t)id < (uint32_t)E) {
                const int tw = (int)(t >> 5);
                uint32_t r = 0u;
                for (int w = 0; w < tw; ++w)
                    r += (uint32_t)__popc(mask[w * E + id]);
                r += (uint32_t)__popc(mask[tw * E + id] & ((1u << (t & 31)) - 1u));
                row = lp_row(lp, eoff, id, r);
            }
        } else {
            for (int j = 0; j < k; ++j) {
                const int32_t ej = __builtin_amdgcn_readlane(id, j);
                if ((uint32_t)ej >= (uint32_t)E)
                    continue;                            // uniform per wavefront
                uint32_t n = 0u;
                for (int64_t q = lane; q < t * k + j; q += 64)
                    n += topk_idx[q] == ej ? 1u : 0u;
                n = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan_u32(n), 63);
                if (lane == j)
                    row = lp_row(lp, eoff, ej, n);
            }
        }
        if (c < 64 && lane < k) {                        // piece 0: the row maps
            lp.token_row[t * k + lane] = row;
            if (row >= 0 && lp.row_token)
                lp.row_token[row] = (int32_t)t;
        }
        const bool active = c < lp.chunks;
        if constexpr (MODE == LP_COPY) {
            u32x4* rv = static_cast<u32x4*>(lp.recv);
            for (int j = 0; j < k; ++j) {
                const int32_t rj = __builtin_amdgcn_readlane(row, j);
                if (rj >= 0 && active)
                    __builtin_nontemporal_store(xv, rv + (int64_t)rj * lp.chunks + c);
            }
        } else if constexpr (MODE == LP_FP8_BF16 || MODE == LP_FP8_F32) {
            u32x2 packed;
            const float s = quantise8_e4m3(v, packed);
            uint8_t* rv = static_cast<uint8_t*>(lp.recv);
            for (int j = 0; j < k; ++j) {
                const int32_t rj = __builtin_amdgcn_readlane(row, j);
                if (rj >= 0 && active) {
                    __builtin_nontemporal_store(
                        packed, reinterpret_cast<u32x2*>(rv + (int64_t)rj * lp.H) + c);
                    if ((lane & 15) == 0)
                        lp.recv_scales[(int64_t)rj * (lp.H / 128) + c / 16] = s;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------------- combine --
template <typename YT>
struct Y8;

// Loads of expert-output rows: non-temporal (NT, the default: rows read once, more of them than
// the Infinity Cache holds), or plain, which lets a small batch's rows come from, and stay in, the
// Infinity Cache (combine picks by the bytes it reads; see launch_combine_typed).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <>
struct Y8<uint16_t> {       // bf16: one 16-byte load per 8 elements
    u32x4 a;
    template <bool NT = true>
    __device__ __forceinline__ void load(const uint16_t* p)
    {
        a = load16<NT>(reinterpret_cast<const u32x4*>(p));
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
    template <bool NT = true>
    __device__ __forceinline__ void load(const float* p)
    {
        a = load16<NT>(reinterpret_cast<const u32x4*>(p));
        b = load16<NT>(reinterpret_cast<const u32x4*>(p) + 1);
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
// first multiply-add), else 0; NT selects non-temporal row loads (Y8::load).
template <typename YT, typename OT, int KC, bool NT>
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
        if constexpr (!NT) {
            // small batches (plain loads): every row id and weight first, then the k row loads.
            // One counter tracks a wavefront's loads in order, so a row load issued before the
            // next id would make that id wait for the row; at 128 decode tokens loading the ids
            // first takes the step from 14.48 to 13.91 us. Large batches keep the interleaved
            // order: there, more rows in flight per wavefront slowed combine (87.6 -> 89.5 us at
            // prefill).
            int rows[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                rows[j] = token_row[t * KC + j];
                w[j] = topk_w[t * KC + j];
            }
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                if ((uint32_t)rows[j] < (uint32_t)R) {
                    v[j].template load<NT>(y + (int64_t)rows[j] * H + off);
                } else {
                    w[j] = 0.0f;
                    v[j] = Y8<YT>{};
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int row = token_row[t * KC + j];
                w[j] = topk_w[t * KC + j];
                if ((uint32_t)row < (uint32_t)R) {
                    v[j].template load<NT>(y + (int64_t)row * H + off);
                } else {
                    w[j] = 0.0f;
                    v[j] = Y8<YT>{};
                }
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
            v.template load<NT>(y + (int64_t)row * H + off);
            v.fma_into(topk_w[t * k + j], acc);
        }
    }
    Store8<OT>::run(out + t * H + off, acc);
}


// ------------------------------------------------------------ combine with pre-reduction (EP) --
// Where the partial rows of one source go: workgroup r scans the source's tokens in order, 1024 at
// a time; token t takes row (r*S + source)*pcap + p when one of its experts sits on rank r (p
// counts such tokens before t), else -1. part_counts[r*S + source] = the number of such tokens.
__global__ __launch_bounds__(kGroupThreads) void k_ep_partial_rows(
    const int32_t* __restrict__ topk_idx, int32_t T, int32_t k, int32_t L, int32_t S,
    int32_t source, int32_t pcap, int32_t N, int32_t* __restrict__ part_row,
    int32_t* __restrict__ part_counts)
{
    __shared__ uint32_t wave_tot[kGroupWaves];
    const int r = blockIdx.x, tid = threadIdx.x;
    uint32_t base = 0u;
    for (int t0 = 0; t0 < T; t0 += kGroupThreads) {     // uniform across the workgroup
        const int t = t0 + tid;
        uint32_t on = 0u;
        if (t < T)
            for (int j = 0; j < k; ++j)
                on |= (topk_idx[(int64_t)t * k + j] / L == r) ? 1u : 0u;
        uint32_t n = 0u;
        const uint32_t before = block_exclusive_scan<kGroupThreads>(on, wave_tot, &n);
        if (t < T)
            part_row[(int64_t)t * N + r] =
                on ? (int32_t)(((int64_t)r * S + source) * pcap + base + before) : -1;
        base += n;
        __syncthreads();                                 // wave_tot is reused next round
    }
    if (tid == 0)
        part_counts[(int64_t)r * S + source] = (int32_t)base;
}

// Grouped row of every region row of one rank: inv[grouped_src[g] - base] = g.
__global__ __launch_bounds__(kThreads) void k_ep_invert(const int32_t* __restrict__ grouped_src,
                                                        int64_t n, int64_t base,
                                                        int32_t* __restrict__ inv)
{
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n;
         g += (int64_t)gridDim.x * kThreads) {
        const int64_t q = (int64_t)grouped_src[g] - base;
        if (grouped_src[g] >= 0 && q >= 0 && q < n)
            inv[q] = (int32_t)g;
    }
}

// Expert side: one wavefront per (token of any source, 512-element segment). Lanes j < k read
// the token's slots; the slots whose expert sits on this rank are added in slot order, fp32
// multiply-adds of w * y[grouped row], and the sum is rounded once into the token's partial row.
template <typename YT>
__global__ __launch_bounds__(64 * kCombineWaves) void k_ep_reduce(
    const YT* __restrict__ y, int32_t H, int32_t nseg, int64_t tokens, int32_t k, int32_t L,
    int32_t N, int32_t rank, int64_t base, int64_t nreg, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const int32_t* __restrict__ send_row,
    const int32_t* __restrict__ part_row, const int32_t* __restrict__ inv, int64_t part_limit,
    YT* __restrict__ partials)
{
    const int64_t item = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
    const int64_t tt = item / nseg;
    if (tt >= tokens)
        return;
    const int32_t pr = part_row[tt * N + rank];
    if (pr < 0 || (int64_t)pr >= part_limit)
        return;                                          // uniform per wavefront
    const int lane = threadIdx.x & 63;
    int32_t g_mine = -1;
    float w_mine = 0.0f;
    if (lane < k && topk_idx[tt * k + lane] / L == rank) {
        const int64_t q = (int64_t)send_row[tt * k + lane] - base;
        g_mine = (q >= 0 && q < nreg) ? inv[q] : -1;
        if (g_mine >= nreg)
            g_mine = -1;                                 // never outside the grouped rows
        w_mine = topk_w[tt * k + lane];
    }
    const int seg = (int)(item - tt * nseg);
    const int c = seg * 64 + lane;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc[i] = 0.0f;
    const bool active = c < H / 8;
    for (int j = 0; j < k; ++j) {
        const int32_t g = __builtin_amdgcn_readlane(g_mine, j);
        if (g < 0)
            continue;                                    // uniform per wavefront
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), j));
        if (active) {
            Y8<YT> v;
            v.load(y + (int64_t)g * H + (int64_t)c * 8);
            v.fma_into(wj, acc);
        }
    }
    if (active)
        Store8<YT>::run(partials + (int64_t)pr * H + (int64_t)c * 8, acc);
}

// Source side: one wavefront per (token, 512-element segment); the token's partial rows are added
// in rank order in fp32 and the sum is rounded once.
template <typename YT, typename OT>
__global__ __launch_bounds__(64 * kCombineWaves) void k_ep_finish(
    const YT* __restrict__ partials, int32_t T, int32_t H, int32_t nseg, int32_t N,
    const int32_t* __restrict__ part_row, int64_t part_limit, OT* __restrict__ out)
{
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
    for (int r = 0; r < N; ++r) {
        const int32_t pr = part_row[t * N + r];
        if (pr < 0 || (int64_t)pr >= part_limit)
            continue;
        Y8<YT> v;
        v.load(partials + (int64_t)pr * H + (int64_t)c * 8);
        v.fma_into(1.0f, acc);
    }
    Store8<OT>::run(out + t * H + (int64_t)c * 8, acc);
}

// ----------------------------------------------------------------- fixed device scratch --
// The workspace of moe_route_dispatch_noalloc: device memory of the library itself, one array per
// device, held until the process ends, so that the call allocates nothing. Host code never passes
// `scratch` itself to a kernel (on the host the name is a stand-in, not a device address); the
// device address comes from hipGetSymbolAddress (device_scratch).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

// ------------------------------------------------------------------------------ host helpers --
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t dtype_size(moe_dtype_t d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

inline bool is_wide(moe_dtype_t d) { return d == MOE_F32 || d == MOE_BF16; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Layout blocks. Caller-given ids: blocks of 4 wavefronts walk their items 256 at a time, at
// most kMaxScanBlocks blocks. Fused routing: one block per 16 tokens (T <= 16 * kMaxScanBlocks).
struct LayoutPlan {
    int32_t rows_per_block;
    int32_t nblk;
};

inline LayoutPlan hist_plan(int64_t R)
{
    LayoutPlan p;
    const int64_t groups = R > 0 ? ceil_div(R, (int64_t)kThreads * kMaxScanBlocks) : 1;
    p.rows_per_block = (int32_t)(groups * kThreads);
    p.nblk = (int32_t)ceil_div(R, p.rows_per_block);
    return p;
}

// Tokens per routing-and-counting workgroup: 16 either way (4 wavefronts of 4 tokens for k <= 16,
// 16 wavefronts of one token otherwise). Below 1024 tokens routing is bound by the latency of one
// selection, not by issue, and the wavefront-per-token kernels finish sooner.
inline bool route_rows16(int32_t T, int32_t k) { return k <= 16 && T >= 1024; }

inline int32_t route_block_tokens(int32_t k) { return k <= 16 ? kRouteTokens16 : kRouteTokens; }

inline bool fused_route_fits(int32_t T, int32_t k)
{
    return ceil_div(T, route_block_tokens(k)) <= kMaxScanBlocks;
}

inline LayoutPlan route_plan(int32_t T, int32_t k)
{
    LayoutPlan p;
    p.rows_per_block = route_block_tokens(k) * k;
    p.nblk = (int32_t)ceil_div(T, route_block_tokens(k));
    return p;
}

inline size_t hist_lds_bytes(int32_t E)
{
    return (size_t)kWaves * E * sizeof(uint64_t) + (size_t)E * sizeof(uint32_t);
}

// Workspace: block-major histograms [nblk * E], expert-major prefixes [E * nblk], expert totals
// [E], in-block ranks [R], the windows' (row, token) lists [R]; each piece 256-byte aligned; nblk
// covers both layout plans.
struct Workspace {
    uint32_t* sink;          // the word after the largest histogram, written by nothing else
    uint32_t* hist;
    uint32_t* prefix;
    uint32_t* totals;
    uint32_t* local_rank;
    int2* list;
    uint8_t* hist8;          // routing blocks' byte counts (k_layout_rows8), in the prefix piece
};

inline int64_t ws_nblk(int32_t T, int32_t k)
{
    int64_t n = hist_plan((int64_t)T * k).nblk;
    if (fused_route_fits(T, k) && route_plan(T, k).nblk > n)
        n = route_plan(T, k).nblk;
    return n;
}

inline int32_t e16(int32_t E) { return (int32_t)align_up((size_t)E, 16); }

// The histograms of the largest layout plan, plus one word (the prefetch's sink); also large
// enough for the byte counts of the routing blocks (nblk rows of E16 bytes, in the prefix piece).
inline size_t ws_hist_bytes(int32_t T, int32_t E, int32_t k)
{
    const size_t words = ((size_t)ws_nblk(T, k) * E + 1) * sizeof(uint32_t);
    const size_t bytes8 = (size_t)ws_nblk(T, k) * e16(E);
    return align_up(words > bytes8 ? words : bytes8, 256);
}

inline size_t ws_bytes(int32_t T, int32_t E, int32_t k)
{
    const int64_t R = (int64_t)T * k;
    const size_t rr = (size_t)(R > 0 ? R : 1);
    return 2 * ws_hist_bytes(T, E, k) + align_up((size_t)E * sizeof(uint32_t), 256) +
           align_up(rr * sizeof(uint32_t), 256) + align_up(rr * sizeof(int2), 256);
}

inline Workspace carve_workspace(void* base, int32_t T, int32_t E, int32_t k)
{
    char* p = static_cast<char*>(base);
    const size_t hb = ws_hist_bytes(T, E, k);
    const size_t tb = align_up((size_t)E * sizeof(uint32_t), 256);
    Workspace w;
    w.hist = reinterpret_cast<uint32_t*>(p);
    w.sink = w.hist + ws_nblk(T, k) * E;
    w.prefix = reinterpret_cast<uint32_t*>(p + hb);
    w.hist8 = reinterpret_cast<uint8_t*>(p + hb);
    w.totals = reinterpret_cast<uint32_t*>(p + 2 * hb);
    w.local_rank = reinterpret_cast<uint32_t*>(p + 2 * hb + tb);
    const int64_t R = (int64_t)T * k;
    w.list = reinterpret_cast<int2*>(p + 2 * hb + tb +
                                     align_up((size_t)(R > 0 ? R : 1) * sizeof(uint32_t), 256));
    return w;
}

// Packing windows: about as many layout blocks as keep the window's x rows within kWindowBytes
// (they stay in the 4 MB L2 of one XCD while the window is packed), with the window count rounded
// up to a multiple of 8 so that every XCD gets the same number of windows where the block count
// allows it. x_row_bytes = 0 (no packing follows) takes 8 windows. With whole_groups (the routed
// layout, k_layout_rows8) a window of more than 16 blocks is cut to whole groups of 16, the rows its
// window pass reads per step: measured on the skewed batch (8192 tokens, hidden 4096, E 128, k 4),
// 16-block windows of 2 MiB take the step from 120.8-120.9 to 118.5 us (16384 tokens: 237.4-237.7 to
// 231.9-232.1), where the byte rule alone gave 22-block windows.
constexpr int64_t kWindowBytes = 3584 * 1024;

struct WindowPlan {
    int32_t blocks_per_window;
    int32_t rows_per_window;
    int32_t nwin;
};

inline WindowPlan window_plan(const LayoutPlan& lp, int64_t x_row_bytes, int32_t k,
                              bool whole_groups = false)
{
    int64_t fit = lp.nblk;
    if (x_row_bytes > 0) {
        const int64_t tokens = kWindowBytes / x_row_bytes > 1 ? kWindowBytes / x_row_bytes : 1;
        fit = tokens * k / lp.rows_per_block;
        if (fit < 1)
            fit = 1;
        if (whole_groups && fit > 16)
            fit &= ~(int64_t)15;
    }
    const int64_t nwin_target = kXcds * (lp.nblk > 0 ? ceil_div(lp.nblk, kXcds * fit) : 1);
    const int64_t bpw = lp.nblk > 0 ? ceil_div(lp.nblk, nwin_target) : 1;
    WindowPlan wp;
    wp.blocks_per_window = (int32_t)bpw;
    wp.rows_per_window = (int32_t)(bpw * lp.rows_per_block);
    wp.nwin = (int32_t)ceil_div(lp.nblk, bpw);
    return wp;
}

inline int64_t xcd_blocks(int32_t T, int64_t items_per_token, int waves_per_group)
{
    return ceil_div(ceil_div(T, kXcds) * items_per_token, waves_per_group) * kXcds;
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
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)         // the one-launch layout keeps a
        return MOE_ERR_UNSUPPORTED;                      // token's slots in one wavefront
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

moe_status_t check_route_args(const float* logits, int32_t T, int32_t E, int32_t k,
                              const int32_t* topk_idx, const float* topk_w)
{
    if (T < 0 || E < 1 || k < 1 || k > E)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T > 0 && (!logits || !topk_idx || !topk_w))
        return MOE_ERR_INVALID;
    if ((int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    return MOE_OK;
}

#define MOE_ROUTE_LAUNCH(KERNEL, GRID, BLOCK, LDS, ...)                                          \
    do {                                                                                          \
        const int pl_ = (int)ceil_div(E, 64);                                                     \
        if (pl_ <= 1)                                                                             \
            KERNEL<1><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (pl_ <= 2)                                                                        \
            KERNEL<2><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (pl_ <= 4)                                                                        \
            KERNEL<4><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (pl_ <= 6)                                                                        \
            KERNEL<6><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (pl_ <= 8)                                                                        \
            KERNEL<8><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else                                                                                      \
            KERNEL<16><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
    } while (0)

// 16 lanes a token: P = ceil(E / 16) keys a lane, rounded up to an instantiated width.
#define MOE_ROUTE16_LAUNCH(KERNEL, GRID, BLOCK, LDS, ...)                                        \
    do {                                                                                          \
        const int p16_ = (int)ceil_div(E, 16);                                                    \
        if (p16_ <= 1)                                                                            \
            KERNEL<1><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (p16_ <= 2)                                                                       \
            KERNEL<2><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (p16_ <= 4)                                                                       \
            KERNEL<4><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (p16_ <= 8)                                                                       \
            KERNEL<8><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                 \
        else if (p16_ <= 16)                                                                      \
            KERNEL<16><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
        else if (p16_ <= 24)                                                                      \
            KERNEL<24><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
        else if (p16_ <= 32)                                                                      \
            KERNEL<32><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
        else if (p16_ <= 48)                                                                      \
            KERNEL<48><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
        else                                                                                      \
            KERNEL<64><<<GRID, BLOCK, LDS, stream>>>(__VA_ARGS__);                                \
    } while (0)

void launch_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                  float* topk_w, hipStream_t stream)
{
    if (route_rows16(T, k)) {
        const dim3 grid((unsigned)ceil_div(T, kThreads / 16));
        MOE_ROUTE16_LAUNCH(k_route_topk, grid, kThreads, 0, logits, T, E, k, topk_idx, topk_w);
    } else {
        MOE_ROUTE_LAUNCH(k_route_topk_wide, dim3((unsigned)T), 64, 0, logits, T, E, k, topk_idx,
                         topk_w);
    }
}

inline Prefetch no_prefetch()
{
    Prefetch pf;
    pf.x = nullptr;
    pf.chunks = 0;
    pf.groups = 0;
    pf.sleeps = 0;
    pf.sink = nullptr;
    return pf;
}

// Parts [part, part + n) of `parts` equal parts of the x prefetch: the first kPrefetchMaxBytes of
// x at most (the first windows pack first), in 16-byte chunks, 16 chunks a thread, after `sleeps`
// sleeps. x null, or a range outside [0, parts): none.
Prefetch make_prefetch(const void* x, int64_t x_bytes, const Workspace& ws, int part, int parts,
                       int n = 1, int sleeps = 0)
{
    if (part < 0 || n < 1 || part + n > parts)
        return no_prefetch();
    Prefetch pf;
    const int64_t bytes = x_bytes < kPrefetchMaxBytes ? x_bytes : kPrefetchMaxBytes;
    const int64_t all = x != nullptr && bytes > 0 ? bytes / 16 : 0;
    const int64_t b = all * part / parts, e = all * (part + n) / parts;
    pf.x = static_cast<const u32x4*>(x) + b;
    pf.chunks = e - b;
    pf.groups = (int32_t)ceil_div(pf.chunks, (int64_t)kThreads * kPrefetchChunksPerThread);
    pf.sleeps = sleeps;
    pf.sink = ws.sink;
    return pf;
}





// Routing and counting; with bytes8 the block counts go out as bytes (ws.hist8) for
// k_layout_rows8, else as u32 (ws.hist) for the scan.
void launch_route_layout(const float* logits, int32_t T, int32_t E, int32_t k,
                         int32_t* topk_idx, float* topk_w, const Workspace& ws,
                         const LayoutPlan& plan, const Prefetch& pf, bool bytes8,
                         hipStream_t stream)
{
    uint8_t* h8 = bytes8 ? ws.hist8 : nullptr;
    if (route_rows16(T, k)) {
        const dim3 grid((unsigned)(plan.nblk + pf.groups));
        MOE_ROUTE16_LAUNCH(k_route_layout, grid, kThreads, (size_t)E * sizeof(uint32_t), logits,
                           T, E, k, topk_idx, topk_w, ws.hist, ws.local_rank, plan.nblk, pf, h8,
                           e16(E));
        return;
    }
    const dim3 grid((unsigned)plan.nblk);               // wavefront a token: no prefetch
    MOE_ROUTE_LAUNCH(k_route_layout_wide, grid, kGroupThreads, (size_t)E * sizeof(uint32_t),
                     logits, T, E, k, topk_idx, topk_w, ws.hist, ws.local_rank, h8, e16(E));
}

void launch_hist(const int32_t* topk_idx, int64_t R, int32_t E, const Workspace& ws,
                 const LayoutPlan& plan, const Prefetch& pf, hipStream_t stream)
{
    if (plan.nblk > 0)
        k_layout_hist<<<plan.nblk + pf.groups, kThreads, hist_lds_bytes(E), stream>>>(
            topk_idx, (int32_t)R, E, plan.rows_per_block, ws.hist, ws.local_rank, plan.nblk, pf);
}

CountOutputs count_outputs(const moe_dispatch_out_t* out, int32_t n_ranks)
{
    CountOutputs co;
    co.expert_counts = out->expert_counts;
    co.expert_offsets = out->expert_offsets;
    co.rank_counts = out->rank_counts;
    co.rank_offsets = out->rank_offsets;
    co.N = n_ranks;
    return co;
}

// Scan of the histograms, then the rows (whose workgroup 0 also writes the count outputs, so it
// runs even for an empty batch).
// Expert-parallel send: where the rows of one source go (its regions) and its region counts.
struct EpSend {
    int32_t* counts;
    int32_t source, sources, cap, L;
};

void launch_scan_rows(const int32_t* topk_idx, int32_t R, int32_t k, int32_t E,
                      int32_t* token_row, int32_t* row_token, const CountOutputs& co,
                      const EpSend* ep, const Workspace& ws, const LayoutPlan& plan,
                      const WindowPlan& wp, const Prefetch& pf_scan, const Prefetch& pf_rows,
                      hipStream_t stream)
{
    const int32_t scan_groups = (int32_t)ceil_div(E, kScanExperts);
    const dim3 grid((unsigned)(scan_groups + pf_scan.groups));
    const int64_t s = ceil_div(plan.nblk, 64);
#define MOE_SCAN(SS)                                                                              \
    k_expert_scan<SS><<<grid, kThreads, 0, stream>>>(ws.hist, E, plan.nblk, ws.prefix, ws.totals, \
                                                     scan_groups, pf_scan)
    if (s <= 1)
        MOE_SCAN(1);
    else if (s <= 2)
        MOE_SCAN(2);
    else if (s <= 4)
        MOE_SCAN(4);
    else if (s <= 8)
        MOE_SCAN(8);
    else
        MOE_SCAN(16);
#undef MOE_SCAN
    RowPlan rp;
    rp.topk_idx = topk_idx;
    rp.local_rank = ws.local_rank;
    rp.prefix = ws.prefix;
    rp.totals = ws.totals;
    rp.token_row = token_row;
    rp.row_token = row_token;
    rp.E = E;
    rp.nblk = plan.nblk;
    rp.rows_per_block = plan.rows_per_block;
    rp.list = ws.list;
    rp.blocks_per_window = wp.blocks_per_window;
    rp.groups_per_window = (int32_t)ceil_div(wp.rows_per_window, kThreads);
    rp.ep_counts = ep ? ep->counts : nullptr;
    rp.ep_source = ep ? ep->source : 0;
    rp.ep_sources = ep ? ep->sources : 1;
    rp.ep_cap = ep ? ep->cap : 0;
    rp.ep_L = ep ? ep->L : 1;
    const int64_t want = (int64_t)wp.nwin * rp.groups_per_window;
    const int32_t rows_groups = (int32_t)(want < 1 ? 1 : want);
    k_layout_rows<<<(unsigned)(rows_groups + pf_rows.groups), kThreads, 0, stream>>>(
        rp, R, k, co, rows_groups, pf_rows);
}

// The rows of routed items in one launch after routing (k_layout_rows8): taken when every
// workgroup can sum the whole byte-count table quickly and the window's part fits LDS.
constexpr int64_t kRows8TableBytes = 256 * 1024;
constexpr int64_t kRows8WindowBytes = 40 * 1024;

inline bool rows8_fits(const LayoutPlan& plan, const WindowPlan& wp, int32_t E)
{
    return (int64_t)plan.nblk * e16(E) <= kRows8TableBytes &&
           (int64_t)2 * wp.blocks_per_window * e16(E) <= kRows8WindowBytes;
}

inline size_t rows8_lds_bytes(const WindowPlan& wp, int32_t E)
{
    return (size_t)2 * wp.blocks_per_window * e16(E) + (size_t)5 * e16(E) * 4;
}

void launch_rows8(const int32_t* topk_idx, int32_t R, int32_t k, int32_t E, int32_t* token_row,
                  int32_t* row_token, const CountOutputs& co, const Workspace& ws,
                  const LayoutPlan& plan, const WindowPlan& wp, const Prefetch& pf,
                  hipStream_t stream)
{
    RowPlan8 rp;
    rp.topk_idx = topk_idx;
    rp.local_rank = ws.local_rank;
    rp.hist8 = ws.hist8;
    rp.token_row = token_row;
    rp.row_token = row_token;
    rp.list = ws.list;
    rp.E = E;
    rp.E16 = e16(E);
    rp.nblk = plan.nblk;
    rp.rows_per_block = plan.rows_per_block;
    rp.blocks_per_window = wp.blocks_per_window;
    rp.groups_per_window = (int32_t)ceil_div(wp.rows_per_window, kRows8Threads);
    const int64_t want = (int64_t)wp.nwin * rp.groups_per_window;
    const int32_t rows_groups = (int32_t)(want < 1 ? 1 : want);
    k_layout_rows8<<<(unsigned)(rows_groups + pf.groups), kRows8Threads,
                     rows8_lds_bytes(wp, E), stream>>>(rp, R, k, co, rows_groups, pf);
}

// Packing in token order (token_row given), or by windows from the list the rows kernel wrote.
void launch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H, int32_t k,
                 const int32_t* token_row, const int2* list, const WindowPlan* wp,
                 moe_dtype_t payload_dtype, void* recv, float* recv_scales, int64_t row_limit,
                 hipStream_t stream)
{
    const int32_t R = T * k;
    if (R == 0)
        return;
    const bool fp8 = payload_dtype == MOE_FP8_E4M3;
    const int32_t cpr = (int32_t)((int64_t)H * (int64_t)dtype_size(x_dtype) / 16);
    PackPlan pp;
    pp.token_row = token_row;
    pp.list = list;
    pp.T = T;
    pp.k = k;
    pp.R = R;
    pp.pieces = (int32_t)ceil_div(fp8 ? H / 8 : cpr, 64);
    // window order: rows of fewer than kPackSplitPieces pieces take two pieces a wavefront
    const bool two = pp.pieces < kPackSplitPieces;
    pp.window_pieces = two ? (pp.pieces + 1) / 2 : pp.pieces;
    pp.rows_per_window = wp ? wp->rows_per_window : 0;
    pp.nwin = wp ? wp->nwin : 0;
    pp.row_limit = row_limit;
    const bool windows = wp && (int64_t)pp.rows_per_window * pp.pieces < (int64_t)INT32_MAX / 2;
    const u32x4* xs = static_cast<const u32x4*>(x);
    if (!fp8) {
        u32x4* rv = static_cast<u32x4*>(recv);
        if (windows) {
            constexpr int wpg = pack_waves<PACK_WINDOWS>();
            const dim3 grid((unsigned)xcd_blocks(
                pp.nwin, (int64_t)pp.rows_per_window * pp.window_pieces, wpg));
            if (two)
                k_pack_rows<PACK_WINDOWS, 2><<<grid, 64 * wpg, 0, stream>>>(xs, cpr, pp, rv);
            else
                k_pack_rows<PACK_WINDOWS, 1><<<grid, 64 * wpg, 0, stream>>>(xs, cpr, pp, rv);
        } else {
            constexpr int wpg = pack_waves<PACK_TOKEN_ORDER>();
            const dim3 grid((unsigned)xcd_blocks(T, pp.pieces, wpg));
            k_pack_rows<PACK_TOKEN_ORDER, 1><<<grid, 64 * wpg, 0, stream>>>(xs, cpr, pp, rv);
        }
        return;
    }
    // fp8: one wavefront per (token, piece), quantised once and stored to the token's k rows
    const dim3 block(64 * kPackWaves);
    const dim3 grid8((unsigned)xcd_blocks(T, pp.pieces, kPackWaves));
    uint8_t* rv = static_cast<uint8_t*>(recv);
    if (x_dtype == MOE_F32)
        k_pack_rows_fp8<float><<<grid8, block, 0, stream>>>(static_cast<const float*>(x), H, pp,
                                                            rv, recv_scales);
    else
        k_pack_rows_fp8<uint16_t><<<grid8, block, 0, stream>>>(static_cast<const uint16_t*>(x), H,
                                                               pp, rv, recv_scales);
}

// Layout (and packing, unless payload is null) of a batch in one launch: up to kLpTokens tokens
// (kLpCopyTokens for row copies), with the masks and offsets in 64 KB of LDS.
inline size_t lp_lds_bytes(int32_t T, int32_t E)
{
    return ((size_t)ceil_div(T, 32) * E + E + 1) * sizeof(uint32_t);
}

// copy: routed ids (never repeated within a token) whose payload is x's own bytes take the
// one-launch layout up to kLpCopyTokens. Caller-given ids keep kLpTokens: a token that names an
// expert twice sends every wavefront through the exact-rank scan of all earlier slots, which grows
// with T squared (896 tokens with repeats: 144 us a dispatch, against 32 us in the multi-launch
// layout).
inline bool lp_fits(int32_t T, int32_t E, bool copy = false)
{
    return T >= 1 && T <= (copy ? kLpCopyTokens : kLpTokens) &&
           lp_lds_bytes(T, E) + 256 <= 64 * 1024;        // + static LDS
}

// Routing in the same launch as layout and packing: small batches of routed tokens.
inline bool lp_route_fits(int32_t T, int32_t E, int32_t k)
{
    return T >= 1 && T <= kLpRouteTokens && k <= 16 && E <= 256 &&
           lp_lds_bytes(T, E) + (size_t)T * k * sizeof(int32_t) + 256 <= 64 * 1024;
}

// Layout and packing in one launch; with `logits` non-null also the routing (lp_route_fits), whose
// ids and weights go to topk_idx / topk_w.
void launch_layout_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H, int32_t E,
                        int32_t k, const int32_t* topk_idx, const moe_dtype_t* payload_dtype,
                        const moe_dispatch_out_t* out, const CountOutputs& co, hipStream_t stream,
                        const EpSend* ep = nullptr, const float* logits = nullptr,
                        float* topk_w = nullptr)
{
    const bool layout_only = payload_dtype == nullptr;
    const bool fp8 = !layout_only && *payload_dtype == MOE_FP8_E4M3;
    LayoutPackPlan lp;
    lp.x = x;
    lp.topk_idx = topk_idx;
    lp.token_row = out->token_row;
    lp.row_token = out->row_token;
    lp.recv = layout_only ? nullptr : out->recv;
    lp.recv_scales = layout_only ? nullptr : out->recv_scales;
    lp.T = T;
    lp.k = k;
    lp.E = E;
    lp.H = H;
    lp.words = (int32_t)ceil_div(T, 32);
    lp.chunks = layout_only ? 0
                : fp8       ? H / 8
                            : (int32_t)((int64_t)H * (int64_t)dtype_size(x_dtype) / 16);
    lp.pieces = layout_only ? 1 : (int32_t)ceil_div(lp.chunks, 64);
    lp.ep_counts = ep ? ep->counts : nullptr;
    lp.ep_source = ep ? ep->source : 0;
    lp.ep_sources = ep ? ep->sources : 1;
    lp.ep_cap = ep ? ep->cap : 0;
    lp.ep_L = ep ? ep->L : 0;
    lp.logits = logits;
    lp.route_idx = const_cast<int32_t*>(topk_idx);
    lp.route_w = topk_w;
    const int64_t groups = ceil_div((int64_t)T * lp.pieces, kLpWaves);
    const dim3 grid((unsigned)(groups < kLpMaxGroups ? groups : kLpMaxGroups));
    if (logits != nullptr) {                             // routing here: payload modes only
        const size_t lds = lp_lds_bytes(T, E) + (size_t)T * k * sizeof(int32_t);
        const int p16 = (int)ceil_div(E, 16);
#define MOE_LP_ROUTE(MODE)                                                                        \
    do {                                                                                          \
        if (p16 <= 1)                                                                             \
            k_layout_pack<MODE, 1><<<grid, kLpThreads, lds, stream>>>(lp, co);                    \
        else if (p16 <= 2)                                                                        \
            k_layout_pack<MODE, 2><<<grid, kLpThreads, lds, stream>>>(lp, co);                    \
        else if (p16 <= 4)                                                                        \
            k_layout_pack<MODE, 4><<<grid, kLpThreads, lds, stream>>>(lp, co);                    \
        else if (p16 <= 8)                                                                        \
            k_layout_pack<MODE, 8><<<grid, kLpThreads, lds, stream>>>(lp, co);                    \
        else                                                                                      \
            k_layout_pack<MODE, 16><<<grid, kLpThreads, lds, stream>>>(lp, co);                   \
    } while (0)
        if (!fp8)
            MOE_LP_ROUTE(LP_COPY);
        else if (x_dtype == MOE_F32)
            MOE_LP_ROUTE(LP_FP8_F32);
        else
            MOE_LP_ROUTE(LP_FP8_BF16);
#undef MOE_LP_ROUTE
        return;
    }
    const size_t lds = lp_lds_bytes(T, E);
    if (T > kLpWideTokens && !layout_only && !fp8) {
        // 16 wavefronts a workgroup: half the workgroups, so half the layouts rebuilt. Measured
        // at hidden 7168 bf16, E 256, k 8 (µs per step): 384 tokens 27.05 -> 26.7, 512 tokens
        // 34.2 -> 32.6, 256 and fewer unchanged or slower. The fp8 modes keep 8 wavefronts: their
        // quantising workgroups ran 24.2 -> 28.0 us at 384 tokens (fewer, longer workgroups than
        // CUs can take in one round). The grid stays within one round of workgroups (wavefronts
        // take further units in turn): a second round rebuilds the layout again, 42.9 -> 40.3 us
        // at 640 tokens; with it, row copies take this launch up to 896 tokens.
        const int64_t groups16 = ceil_div((int64_t)T * lp.pieces, kLpWideThreads / 64);
        const dim3 grid16((unsigned)(groups16 < kLpWideMaxGroups ? groups16 : kLpWideMaxGroups));
        k_layout_pack<LP_COPY, 0, kLpWideThreads><<<grid16, kLpWideThreads, lds, stream>>>(lp, co);
        return;
    }
    if (layout_only)
        k_layout_pack<LP_LAYOUT, 0><<<grid, kLpThreads, lds, stream>>>(lp, co);
    else if (!fp8)
        k_layout_pack<LP_COPY, 0><<<grid, kLpThreads, lds, stream>>>(lp, co);
    else if (x_dtype == MOE_F32)
        k_layout_pack<LP_FP8_F32, 0><<<grid, kLpThreads, lds, stream>>>(lp, co);
    else
        k_layout_pack<LP_FP8_BF16, 0><<<grid, kLpThreads, lds, stream>>>(lp, co);
}

// Rows read by combine up to this many bytes are loaded plainly (they fit the 256 MB Infinity
// Cache many times over, and a small batch's rows were just written): measured at hidden 7168,
// 256 experts, top-8, the decode step takes 15.3 us with plain loads against 17.2 us with
// non-temporal ones, and 256 tokens (29 MB of rows) 21.4 against 22.1 us; from 512 tokens (59 MB)
// on, non-temporal loads win (34.3 against 35.6 us; the 4096-token prefill step 186.9 against
// 192.2 us).
constexpr int64_t kCombinePlainLoadBytes = 32ll << 20;

template <typename YT, typename OT>
void launch_combine_typed(const void* y, int32_t T, int32_t H, int32_t k,
                          const int32_t* token_row, const float* topk_w, void* out, int32_t R,
                          hipStream_t stream)
{
    const int32_t nseg = (int32_t)ceil_div(H / 8, 64);
    const dim3 grid((unsigned)ceil_div((int64_t)T * nseg, kCombineWaves));
    const YT* yp = static_cast<const YT*>(y);
    OT* op = static_cast<OT*>(out);
    const bool nt = (int64_t)T * k * H * (int64_t)sizeof(YT) > kCombinePlainLoadBytes;
#define MOE_COMBINE(KK)                                                                           \
    do {                                                                                          \
        if (nt)                                                                                   \
            k_combine<YT, OT, KK, true><<<grid, 64 * kCombineWaves, 0, stream>>>(                 \
                yp, T, H, k, R, nseg, token_row, topk_w, op);                                     \
        else                                                                                      \
            k_combine<YT, OT, KK, false><<<grid, 64 * kCombineWaves, 0, stream>>>(                \
                yp, T, H, k, R, nseg, token_row, topk_w, op);                                     \
    } while (0)
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
    const moe_status_t st = check_route_args(logits, T, E, k, topk_idx, topk_w);
    if (st != MOE_OK)
        return st;
    if (T == 0)
        return MOE_OK;
    launch_route(logits, T, E, k, topk_idx, topk_w, stream);
    return launch_status();
}

size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k)
{
    if (T < 0 || E < 1 || k < 1 || (int64_t)T * k > INT32_MAX)
        return 0;
    return ws_bytes(T, E, k);
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
    if (lp_fits(T, E)) {
        launch_layout_pack(nullptr, MOE_F32, T, 0, E, k, topk_idx, nullptr, out,
                           count_outputs(out, n_ranks), stream);
        return launch_status();
    }
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = hist_plan(R);
    const Workspace ws = carve_workspace(workspace, T, E, k);
    launch_hist(topk_idx, R, E, ws, plan, no_prefetch(), stream);
    launch_scan_rows(topk_idx, (int32_t)R, k, E, out->token_row, out->row_token,
                     count_outputs(out, n_ranks), nullptr, ws, plan, window_plan(plan, 0, k),
                     no_prefetch(), no_prefetch(), stream);
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
    launch_pack(x, x_dtype, T, H, k, token_row, nullptr, nullptr, payload_dtype, recv,
                recv_scales, (int64_t)T * k, stream);
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
    if (lp_fits(T, E)) {
        launch_layout_pack(x, x_dtype, T, H, E, k, topk_idx, &payload_dtype, out,
                           count_outputs(out, n_ranks), stream);
        return launch_status();
    }
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = hist_plan(R);
    const Workspace ws = carve_workspace(workspace, T, E, k);
    const int64_t x_bytes = (int64_t)T * H * (int64_t)dtype_size(x_dtype);
    launch_hist(topk_idx, R, E, ws, plan, make_prefetch(x, x_bytes, ws, 0, 3), stream);
    const WindowPlan wp = window_plan(plan, (int64_t)H * (int64_t)dtype_size(x_dtype), k);
    launch_scan_rows(topk_idx, (int32_t)R, k, E, out->token_row, out->row_token,
                     count_outputs(out, n_ranks), nullptr, ws, plan, wp,
                     make_prefetch(x, x_bytes, ws, 1, 3),
                     make_prefetch(x, x_bytes, ws, 2, 3), stream);
    launch_pack(x, x_dtype, T, H, k, out->token_row, ws.list, &wp, payload_dtype, out->recv,
                out->recv_scales, R, stream);
    return launch_status();
}

}  // extern "C"

namespace {

moe_status_t check_route_dispatch_args(const float* logits, const void* x, moe_dtype_t x_dtype,
                                       int32_t T, int32_t H, int32_t E, int32_t k,
                                       int32_t n_ranks, moe_dtype_t payload_dtype,
                                       const int32_t* topk_idx, const float* topk_w,
                                       const moe_dispatch_out_t* out)
{
    moe_status_t st = check_route_args(logits, T, E, k, topk_idx, topk_w);
    if (st != MOE_OK)
        return st;
    st = check_layout_args(topk_idx, T, k, E, n_ranks, out);
    if (st != MOE_OK)
        return st;
    return check_pack_args(x, x_dtype, T, H, k, out->token_row, payload_dtype, out->recv,
                           out->recv_scales);
}

// Routing and dispatch once the arguments and the workspace are known to be valid.
moe_status_t route_dispatch(const float* logits, const void* x, moe_dtype_t x_dtype, int32_t T,
                            int32_t H, int32_t E, int32_t k, int32_t n_ranks,
                            moe_dtype_t payload_dtype, int32_t* topk_idx, float* topk_w,
                            const moe_dispatch_out_t* out, void* workspace, hipStream_t stream)
{
    const int64_t R = (int64_t)T * k;
    if (lp_route_fits(T, E, k)) {
        // the smallest batches: routing, layout and packing in one launch
        launch_layout_pack(x, x_dtype, T, H, E, k, topk_idx, &payload_dtype, out,
                           count_outputs(out, n_ranks), stream, nullptr, logits, topk_w);
        return launch_status();
    }
    if (lp_fits(T, E, payload_dtype != MOE_FP8_E4M3)) {
        // small batches: routing, then layout and packing in one launch
        launch_route(logits, T, E, k, topk_idx, topk_w, stream);
        launch_layout_pack(x, x_dtype, T, H, E, k, topk_idx, &payload_dtype, out,
                           count_outputs(out, n_ranks), stream);
        return launch_status();
    }
    const Workspace ws = carve_workspace(workspace, T, E, k);
    const int64_t x_bytes = (int64_t)T * H * (int64_t)dtype_size(x_dtype);
    const int64_t row_bytes = (int64_t)H * (int64_t)dtype_size(x_dtype);
    const bool fused = T > 0 && fused_route_fits(T, k);
    const bool wide = fused && !route_rows16(T, k);
    const LayoutPlan plan = fused ? route_plan(T, k) : hist_plan(R);
    const WindowPlan wp8 = window_plan(plan, row_bytes, k, true);
    const bool rows8 = fused && rows8_fits(plan, wp8, E);
    const WindowPlan wp = rows8 ? wp8 : window_plan(plan, row_bytes, k);
    if (rows8) {
        // two layout launches: routing with counting (byte counts), then the rows, each reading
        // half of x ahead; the wavefront-per-token routing launch carries none, and the rows
        // launch reads all of it. The routing launch's read-ahead starts about 1 us late, so the
        // routing workgroups' logit loads go first: measured at prefill (200 steps, 3 runs, one
        // box) 183.8-183.9 us per step against 184.8-185.5 with no sleep; 1, 3, 4 and 6 sleeps
        // gave 184.8-184.9, 183.7-184.0, 184.3-184.5 and 185.3; a sleep in the rows launch's
        // read-ahead costs (186.8-187.2 with 2).
        const Prefetch pf_route = wide ? no_prefetch() : make_prefetch(x, x_bytes, ws, 0, 2, 1, 2);
        const Prefetch pf_rows = wide ? make_prefetch(x, x_bytes, ws, 0, 1)
                                      : make_prefetch(x, x_bytes, ws, 1, 2);
        launch_route_layout(logits, T, E, k, topk_idx, topk_w, ws, plan, pf_route, true, stream);
        launch_rows8(topk_idx, (int32_t)R, k, E, out->token_row, out->row_token,
                     count_outputs(out, n_ranks), ws, plan, wp, pf_rows, stream);
    } else {
        // x is read ahead by the counting, scan and rows launches, a third each; the
        // wavefront-per-token routing launch (k > 16 or small batches) carries none, and scan and
        // rows take halves.
        const int parts = wide ? 2 : 3;
        const int q_route = wide ? 0 : 1;                        // parts of each launch, in order
        const Prefetch pf_route = make_prefetch(x, x_bytes, ws, 0, parts, q_route);
        const Prefetch pf_scan = make_prefetch(x, x_bytes, ws, q_route, parts, 1);
        const Prefetch pf_rows = make_prefetch(x, x_bytes, ws, q_route + 1, parts, 1);
        if (fused) {
            launch_route_layout(logits, T, E, k, topk_idx, topk_w, ws, plan, pf_route, false,
                                stream);
        } else {
            if (T > 0)
                launch_route(logits, T, E, k, topk_idx, topk_w, stream);
            launch_hist(topk_idx, R, E, ws, plan, pf_route, stream);
        }
        launch_scan_rows(topk_idx, (int32_t)R, k, E, out->token_row, out->row_token,
                         count_outputs(out, n_ranks), nullptr, ws, plan, wp, pf_scan, pf_rows,
                         stream);
    }
    launch_pack(x, x_dtype, T, H, k, out->token_row, ws.list, &wp, payload_dtype, out->recv,
                out->recv_scales, R, stream);
    return launch_status();
}

// Device address of `scratch` on the device of `stream` (the current device for the null
// stream): looked up once per device with that device current, then kept.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxScratchDevices];

moe_status_t device_scratch(hipStream_t stream, void** addr)
{
    int dev = 0;
    const hipError_t ge = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (ge != hipSuccess)
        return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess)
            return MOE_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return MOE_ERR_HIP;
        void* p = nullptr;
        const hipError_t se = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess)
            return MOE_ERR_HIP;
        if (se != hipSuccess || p == nullptr)
            return MOE_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_route_dispatch(const float* logits, const void* x, moe_dtype_t x_dtype,
                                int32_t T, int32_t H, int32_t E, int32_t k, int32_t n_ranks,
                                moe_dtype_t payload_dtype, int32_t* topk_idx, float* topk_w,
                                const moe_dispatch_out_t* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream)
{
    const moe_status_t st = check_route_dispatch_args(logits, x, x_dtype, T, H, E, k, n_ranks,
                                                      payload_dtype, topk_idx, topk_w, out);
    if (st != MOE_OK)
        return st;
    if (!workspace || workspace_bytes < moe_dispatch_workspace_bytes(T, E, k))
        return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return MOE_ERR_UNSUPPORTED;
    return route_dispatch(logits, x, x_dtype, T, H, E, k, n_ranks, payload_dtype, topk_idx,
                          topk_w, out, workspace, stream);
}

moe_status_t moe_route_dispatch_noalloc(const float* logits, const void* x, moe_dtype_t x_dtype,
                                        int32_t T, int32_t H, int32_t E, int32_t k,
                                        int32_t n_ranks, moe_dtype_t payload_dtype,
                                        int32_t* topk_idx, float* topk_w,
                                        const moe_dispatch_out_t* out, hipStream_t stream)
{
    moe_status_t st = check_route_dispatch_args(logits, x, x_dtype, T, H, E, k, n_ranks,
                                                payload_dtype, topk_idx, topk_w, out);
    if (st != MOE_OK)
        return st;
    if (moe_dispatch_workspace_bytes(T, E, k) > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    st = device_scratch(stream, &ws);
    if (st != MOE_OK)
        return st;
    return route_dispatch(logits, x, x_dtype, T, H, E, k, n_ranks, payload_dtype, topk_idx,
                          topk_w, out, ws, stream);
}

moe_status_t moe_check_topk(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                            int32_t* counts, hipStream_t stream)
{
    if (T < 0 || k < 1 || E < 1 || (int64_t)T * k > INT32_MAX || !counts)
        return MOE_ERR_INVALID;
    if (T > 0 && !topk_idx)
        return MOE_ERR_INVALID;
    k_zero_i32<<<1, 64, 0, stream>>>(counts, 2);
    const int64_t R = (int64_t)T * k;
    if (R > 0) {
        const int64_t g = ceil_div(R, (int64_t)kThreads);
        k_check_topk<<<(unsigned)(g < 1024 ? g : 1024), kThreads, 0, stream>>>(topk_idx, R, k, E,
                                                                              counts);
    }
    return launch_status();
}

static moe_status_t combine_checked(const void* y, moe_dtype_t y_dtype, int32_t T, int32_t H,
                                    int32_t k, const int32_t* token_row, const float* topk_w,
                                    void* out, moe_dtype_t out_dtype, int32_t y_rows,
                                    hipStream_t stream)
{
    if (T < 0 || H < 1 || k < 1 || (int64_t)T * k > INT32_MAX || y_rows < 0)
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
        launch_combine_typed<uint16_t, uint16_t>(y, T, H, k, token_row, topk_w, out, y_rows,
                                                 stream);
    else if (y_dtype == MOE_BF16)
        launch_combine_typed<uint16_t, float>(y, T, H, k, token_row, topk_w, out, y_rows, stream);
    else if (out_dtype == MOE_BF16)
        launch_combine_typed<float, uint16_t>(y, T, H, k, token_row, topk_w, out, y_rows, stream);
    else
        launch_combine_typed<float, float>(y, T, H, k, token_row, topk_w, out, y_rows, stream);
    return launch_status();
}

moe_status_t moe_combine(const void* y, moe_dtype_t y_dtype, int32_t T, int32_t H, int32_t k,
                         const int32_t* token_row, const float* topk_w, void* out,
                         moe_dtype_t out_dtype, hipStream_t stream)
{
    if ((int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    return combine_checked(y, y_dtype, T, H, k, token_row, topk_w, out, out_dtype, T * k, stream);
}

// ------------------------------------------------------------------- expert parallelism (one GPU)
int64_t moe_ep_capacity(int32_t T, int32_t E, int32_t k, int32_t n_ranks)
{
    if (T < 0 || E < 1 || k < 1 || n_ranks < 1 || E % n_ranks != 0)
        return 0;
    const int32_t L = E / n_ranks;
    return (int64_t)T * (k < L ? k : L);
}

static moe_status_t ep_region_args(int32_t E, int32_t n_ranks, int32_t n_sources, int32_t cap)
{
    if (E < 1 || n_ranks < 1 || E % n_ranks != 0 || n_sources < 1 || cap < 0)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)n_ranks * n_sources * cap > INT32_MAX)
        return MOE_ERR_INVALID;
    return MOE_OK;
}

moe_status_t moe_ep_send(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                         const int32_t* topk_idx, int32_t k, int32_t E, int32_t n_ranks,
                         int32_t source, int32_t n_sources, int32_t cap, void* regions,
                         int32_t* region_counts, int32_t* send_row, void* workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    moe_status_t st = ep_region_args(E, n_ranks, n_sources, cap);
    if (st != MOE_OK)
        return st;
    if (T < 0 || k < 1 || (int64_t)T * k > INT32_MAX || source < 0 || source >= n_sources)
        return MOE_ERR_INVALID;
    if (k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)cap < moe_ep_capacity(T, E, k, n_ranks))
        return MOE_ERR_INVALID;
    if (!region_counts || (T > 0 && (!topk_idx || !send_row)))
        return MOE_ERR_INVALID;
    st = check_pack_args(x, x_dtype, T, H, k, send_row, x_dtype, regions, nullptr);
    if (st != MOE_OK)
        return st;
    if (!workspace || workspace_bytes < moe_dispatch_workspace_bytes(T, E, k))
        return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return MOE_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = hist_plan(R);
    const Workspace ws = carve_workspace(workspace, T, E, k);
    EpSend ep;
    ep.counts = region_counts;
    ep.source = source;
    ep.sources = n_sources;
    ep.cap = cap;
    ep.L = E / n_ranks;
    if (lp_fits(T, E)) {
        moe_dispatch_out_t o = {};
        o.recv = regions;
        o.token_row = send_row;
        launch_layout_pack(x, x_dtype, T, H, E, k, topk_idx, &x_dtype, &o, CountOutputs{}, stream,
                           &ep);
        return launch_status();
    }
    const int64_t x_bytes = (int64_t)T * H * (int64_t)dtype_size(x_dtype);
    launch_hist(topk_idx, R, E, ws, plan, make_prefetch(x, x_bytes, ws, 0, 3), stream);
    const WindowPlan wp = window_plan(plan, (int64_t)H * (int64_t)dtype_size(x_dtype), k);
    const CountOutputs none = {};
    launch_scan_rows(topk_idx, (int32_t)R, k, E, send_row, nullptr, none, &ep, ws, plan, wp,
                     make_prefetch(x, x_bytes, ws, 1, 3), make_prefetch(x, x_bytes, ws, 2, 3),
                     stream);
    launch_pack(x, x_dtype, T, H, k, send_row, ws.list, &wp, x_dtype, regions, nullptr,
                (int64_t)n_ranks * n_sources * cap, stream);
    return launch_status();
}

static moe_status_t ep_rank_args(moe_dtype_t dtype, int32_t H, int32_t E, int32_t n_ranks,
                                 int32_t n_sources, int32_t cap, const void* a, const void* b)
{
    moe_status_t st = ep_region_args(E, n_ranks, n_sources, cap);
    if (st != MOE_OK)
        return st;
    if (H < 1)
        return MOE_ERR_INVALID;
    if (!is_wide(dtype) || ((int64_t)H * (int64_t)dtype_size(dtype)) % 16 != 0)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)n_sources * (E / n_ranks) > kMaxEpSegments)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned(a, 16) || !aligned(b, 16))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static void launch_copy_rows(int DIR, const void* src, void* dst, moe_dtype_t dtype, int32_t H,
                             const int32_t* map, const int32_t* n_rows, int64_t max_rows,
                             int64_t row_limit, hipStream_t stream)
{
    const int32_t cpr = (int32_t)((int64_t)H * (int64_t)dtype_size(dtype) / 16);
    const int32_t pieces = (int32_t)ceil_div(cpr, 64);
    // grid-stride: at most 4096 workgroups (65536 wavefronts, eight rounds); the row count is only
    // known on the device, so a grid sized for max_rows would mostly start idle wavefronts. At the
    // prefill batch over 8 sources (about 4096 of 32768 possible rows a rank, 14 pieces a row)
    // receive and return take 27.3 and 22.5 us with 2048 workgroups, 26.9 and 22.0 with 4096,
    // 29.4 and 24.3 with 8192, 46.7 and 41.5 with one workgroup per 16 possible pieces
    int64_t blocks = ceil_div(max_rows * pieces, kPackWaves);
    blocks = blocks < 1 ? 1 : blocks > 4096 ? 4096 : blocks;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    if (DIR == COPY_GATHER)
        k_copy_rows<COPY_GATHER><<<(unsigned)blocks, 64 * kPackWaves, 0, stream>>>(
            s, d, cpr, pieces, map, n_rows, max_rows, row_limit);
    else
        k_copy_rows<COPY_SCATTER><<<(unsigned)blocks, 64 * kPackWaves, 0, stream>>>(
            s, d, cpr, pieces, map, n_rows, max_rows, row_limit);
}

moe_status_t moe_ep_recv(const void* regions, moe_dtype_t dtype, int32_t H, int32_t E,
                         int32_t n_ranks, int32_t rank, int32_t n_sources, int32_t cap,
                         const int32_t* region_counts, void* grouped, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* grouped_src, hipStream_t stream)
{
    moe_status_t st = ep_rank_args(dtype, H, E, n_ranks, n_sources, cap, regions, grouped);
    if (st != MOE_OK)
        return st;
    if (rank < 0 || rank >= n_ranks)
        return MOE_ERR_INVALID;
    if (!region_counts || !expert_counts || !expert_offsets ||
        (cap > 0 && (!regions || !grouped || !grouped_src)))
        return MOE_ERR_INVALID;
    const int32_t L = E / n_ranks;
    int64_t plan_blocks = ceil_div((int64_t)n_sources * cap, 4 * kGroupThreads);
    plan_blocks = plan_blocks < 1 ? 1 : plan_blocks > 64 ? 64 : plan_blocks;
    k_ep_recv_plan<<<(unsigned)plan_blocks, kGroupThreads, 0, stream>>>(
        region_counts, rank, n_sources, L, cap, expert_counts, expert_offsets, grouped_src);
    if (cap > 0)
        launch_copy_rows(COPY_GATHER, regions, grouped, dtype, H, grouped_src, expert_offsets + L,
                         (int64_t)n_sources * cap, (int64_t)n_ranks * n_sources * cap, stream);
    return launch_status();
}

moe_status_t moe_ep_return(const void* y_grouped, moe_dtype_t dtype, int32_t H, int32_t E,
                           int32_t n_ranks, int32_t n_sources, int32_t cap,
                           const int32_t* grouped_src, const int32_t* expert_offsets,
                           void* returns, hipStream_t stream)
{
    moe_status_t st = ep_rank_args(dtype, H, E, n_ranks, n_sources, cap, y_grouped, returns);
    if (st != MOE_OK)
        return st;
    if (cap == 0)
        return MOE_OK;
    if (!y_grouped || !grouped_src || !expert_offsets || !returns)
        return MOE_ERR_INVALID;
    launch_copy_rows(COPY_SCATTER, y_grouped, returns, dtype, H, grouped_src,
                     expert_offsets + E / n_ranks, (int64_t)n_sources * cap,
                     (int64_t)n_ranks * n_sources * cap, stream);
    return launch_status();
}

moe_status_t moe_ep_partial_rows(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                                 int32_t n_ranks, int32_t source, int32_t n_sources, int32_t pcap,
                                 int32_t* part_row, int32_t* part_counts, hipStream_t stream)
{
    moe_status_t st = ep_region_args(E, n_ranks, n_sources, pcap);
    if (st != MOE_OK)
        return st;
    if (T < 0 || k < 1 || pcap < T || source < 0 || source >= n_sources ||
        (int64_t)T * n_ranks > INT32_MAX || (int64_t)T * k > INT32_MAX)
        return MOE_ERR_INVALID;
    if (!part_counts || (T > 0 && (!topk_idx || !part_row)))
        return MOE_ERR_INVALID;
    k_ep_partial_rows<<<(unsigned)n_ranks, kGroupThreads, 0, stream>>>(
        topk_idx, T, k, E / n_ranks, n_sources, source, pcap, n_ranks, part_row, part_counts);
    return launch_status();
}

size_t moe_ep_reduce_workspace_bytes(int32_t n_sources, int32_t cap)
{
    if (n_sources < 1 || cap < 0)
        return 0;
    return align_up((size_t)n_sources * (size_t)(cap > 0 ? cap : 1) * sizeof(int32_t), 256);
}

moe_status_t moe_ep_reduce(const void* y_grouped, moe_dtype_t dtype, int32_t H, int32_t E,
                           int32_t n_ranks, int32_t rank, int32_t n_sources, int32_t cap,
                           const int32_t* grouped_src, int32_t T, int32_t k,
                           const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                           const int32_t* part_row, int32_t pcap, void* partials, void* workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    moe_status_t st = ep_rank_args(dtype, H, E, n_ranks, n_sources, cap, y_grouped, partials);
    if (st != MOE_OK)
        return st;
    st = ep_region_args(E, n_ranks, n_sources, pcap);
    if (st != MOE_OK)
        return st;
    if (rank < 0 || rank >= n_ranks || T < 0 || k < 1 || pcap < T ||
        (int64_t)n_sources * T * (k > n_ranks ? k : n_ranks) > INT32_MAX)
        return MOE_ERR_INVALID;
    if (H % 8 != 0)
        return MOE_ERR_UNSUPPORTED;
    const int64_t tokens = (int64_t)n_sources * T;
    if (tokens == 0 || cap == 0)
        return MOE_OK;
    if (!y_grouped || !grouped_src || !topk_idx || !topk_w || !send_row || !part_row ||
        !partials)
        return MOE_ERR_INVALID;
    if (!workspace || workspace_bytes < moe_ep_reduce_workspace_bytes(n_sources, cap))
        return MOE_ERR_WORKSPACE;
    int32_t* inv = static_cast<int32_t*>(workspace);
    const int64_t nreg = (int64_t)n_sources * cap;
    const int64_t base = (int64_t)rank * nreg;
    int64_t blocks = ceil_div(nreg, kThreads);
    blocks = blocks > 4096 ? 4096 : blocks;
    k_ep_invert<<<(unsigned)blocks, kThreads, 0, stream>>>(grouped_src, nreg, base, inv);
    const int32_t nseg = (int32_t)ceil_div(H / 8, 64);
    const dim3 grid((unsigned)ceil_div(tokens * nseg, kCombineWaves));
    const int64_t part_limit = (int64_t)n_ranks * n_sources * pcap;
    if (dtype == MOE_BF16)
        k_ep_reduce<uint16_t><<<grid, 64 * kCombineWaves, 0, stream>>>(
            static_cast<const uint16_t*>(y_grouped), H, nseg, tokens, k, E / n_ranks, n_ranks,
            rank, base, nreg, topk_idx, topk_w, send_row, part_row, inv, part_limit,
            static_cast<uint16_t*>(partials));
    else
        k_ep_reduce<float><<<grid, 64 * kCombineWaves, 0, stream>>>(
            static_cast<const float*>(y_grouped), H, nseg, tokens, k, E / n_ranks, n_ranks, rank,
            base, nreg, topk_idx, topk_w, send_row, part_row, inv, part_limit,
            static_cast<float*>(partials));
    return launch_status();
}

moe_status_t moe_ep_combine_reduced(const void* partials, moe_dtype_t dtype, int32_t T, int32_t H,
                                    int32_t n_ranks, const int32_t* part_row,
                                    int32_t partial_rows, void* out, moe_dtype_t out_dtype,
                                    hipStream_t stream)
{
    if (T < 0 || H < 1 || n_ranks < 1 || partial_rows < 0 || (int64_t)T * n_ranks > INT32_MAX)
        return MOE_ERR_INVALID;
    if (!is_wide(dtype) || !is_wide(out_dtype) || H % 8 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (T > 0 && (!partials || !part_row || !out))
        return MOE_ERR_INVALID;
    if (!aligned(partials, 16) || !aligned(out, 16))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    const int32_t nseg = (int32_t)ceil_div(H / 8, 64);
    const dim3 grid((unsigned)ceil_div((int64_t)T * nseg, kCombineWaves));
    const dim3 block(64 * kCombineWaves);
#define MOE_FINISH(YT, OT)                                                                        \
    k_ep_finish<YT, OT><<<grid, block, 0, stream>>>(static_cast<const YT*>(partials), T, H, nseg,  \
                                                    n_ranks, part_row, partial_rows,             \
                                                    static_cast<OT*>(out))
    if (dtype == MOE_BF16 && out_dtype == MOE_BF16)
        MOE_FINISH(uint16_t, uint16_t);
    else if (dtype == MOE_BF16)
        MOE_FINISH(uint16_t, float);
    else if (out_dtype == MOE_BF16)
        MOE_FINISH(float, uint16_t);
    else
        MOE_FINISH(float, float);
#undef MOE_FINISH
    return launch_status();
}

moe_status_t moe_ep_combine(const void* returns, moe_dtype_t y_dtype, int32_t T, int32_t H,
                            int32_t k, const int32_t* send_row, const float* topk_w,
                            int32_t region_rows, void* out, moe_dtype_t out_dtype,
                            hipStream_t stream)
{
    return combine_checked(returns, y_dtype, T, H, k, send_row, topk_w, out, out_dtype,
                           region_rows, stream);
}

}  // extern "C"
