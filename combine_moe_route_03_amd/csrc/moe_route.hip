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
//   k_route_topk      one wavefront per token, k rounds of a wave-wide 64-bit max;
//   k_layout_hist     per block of items: stable in-block ranks from LDS bit masks, and per-block
//                     expert histograms (no atomics decide a position);
//   k_layout_finalize per block: expert totals and offsets (scan in LDS), the block's base inside
//                     every expert, then token_row / row_token;
//   k_pack_copy       x row read once, written to its k rows with 16-byte non-temporal stores;
//   k_pack_fp8        same, quantising 1x128 blocks to e4m3 with an fp32 absmax/448 scale;
//   k_combine         gathers the k rows of a token with 16-byte loads, fp32 weighted sum.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "moe_route.h"

namespace {

constexpr int kThreads = 256;            // 4 wavefronts of 64 lanes
constexpr int kWaves = kThreads / 64;
constexpr int kMaxLayoutBlocks = 64;     // bound on per-block histograms the finalize pass scans
constexpr int kTargetBlocks = 2048;      // >= 8 workgroups per CU on 256 CUs for the row kernels

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
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    const uint32_t lo = __shfl_xor((int)(uint32_t)v, mask, 64);
    const uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), mask, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int mask)
{
    return __longlong_as_double((long long)shfl_xor_u64((uint64_t)__double_as_longlong(v), mask));
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

// One wavefront per token. Lane l holds experts l, l+64, ... (coalesced). Each of the k rounds
// takes the wave-wide maximum key, records it in lane j and removes it from its owner lane.
// The weights use double-precision exp and division, rounded once to fp32.
template <int PL>
__global__ __launch_bounds__(kThreads) void k_route_topk(const float* __restrict__ logits,
                                                         int32_t T, int32_t E, int32_t k,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const float* l = logits + t * E;
    uint64_t key[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) {
        const int e = lane + 64 * p;
        key[p] = (e < E) ? route_key(l[e], e) : 0ull;
    }
    int my_id = 0;
    float my_logit = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int p = 1; p < PL; ++p)
            best = key[p] > best ? key[p] : best;
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) {
            const uint64_t o = shfl_xor_u64(best, m);
            best = o > best ? o : best;
        }
        const int id = (int)(~(uint32_t)best);
#pragma unroll
        for (int p = 0; p < PL; ++p)
            if (lane + 64 * p == id)
                key[p] = 0ull;
        if (lane == j) {
            my_id = id;
            my_logit = route_key_logit(best);
        }
    }
    const double top = (double)__shfl(my_logit, 0, 64);
    const double ex = (lane < k) ? exp((double)my_logit - top) : 0.0;
    double sum = ex;
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        sum += shfl_xor_f64(sum, m);
    if (lane < k) {
        topk_idx[t * k + lane] = my_id;
        topk_w[t * k + lane] = (float)(ex / sum);
    }
}

// --------------------------------------------------------------------------------- layout --
// Items are the (token, slot) pairs in index order i = t*k + j. Block b owns the contiguous items
// [b*rows_per_block, (b+1)*rows_per_block) and walks them 256 at a time. For each group of 256,
// every item sets its lane bit in the LDS mask of (its wave, its expert); its rank among the
// block's items of the same expert is then
//   run[e] + (bits of e in lower waves) + (bits of e in lower lanes of its own wave),
// which keeps index order without any atomic deciding a position. The first item of each expert
// in the group then advances run[e] and clears the masks.
// LDS: masks [kWaves][E] u64, run [E] u32.
__global__ __launch_bounds__(kThreads) void k_layout_hist(const int32_t* __restrict__ topk_idx,
                                                          int32_t R, int32_t E,
                                                          int32_t rows_per_block,
                                                          uint32_t* __restrict__ hist,
                                                          uint32_t* __restrict__ local_rank)
{
    extern __shared__ uint64_t lds_u64[];
    uint64_t* mask = lds_u64;
    uint32_t* run = reinterpret_cast<uint32_t*>(mask + kWaves * E);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < kWaves * E; i += kThreads)
        mask[i] = 0ull;
    for (int i = tid; i < E; i += kThreads)
        run[i] = 0u;
    __syncthreads();
    const uint64_t lower_lanes = (1ull << lane) - 1ull;
    const int64_t first = (int64_t)blockIdx.x * rows_per_block;
    for (int c = 0; c < rows_per_block; c += kThreads) {
        const int64_t i = first + c + tid;
        int e = -1;
        if (i < R) {
            e = topk_idx[i];
            if ((uint32_t)e >= (uint32_t)E)
                e = -1;                                  // outside [0, E): no row
        }
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
        if (i < R)
            local_rank[i] = rank;
    }
    for (int i = tid; i < E; i += kThreads)
        hist[(int64_t)blockIdx.x * E + i] = run[i];
}

// Exclusive scan of one value per thread over the 256 threads of the block; returns the prefix
// and writes the block total to *total. `scratch` holds kWaves words of LDS.
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
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t s = scratch[w];
        base += (w < wave) ? s : 0u;
        all += s;
    }
    *total = all;
    return base + x - v;
}

// Every block rebuilds the expert totals and offsets from the per-block histograms (a few KB,
// served by L2), takes its own base inside every expert, and turns its items' local ranks into
// rows. Block 0 also writes the counts and offsets. LDS: base [E], offsets [E] u32.
__global__ __launch_bounds__(kThreads) void k_layout_finalize(
    const int32_t* __restrict__ topk_idx, int32_t R, int32_t k, int32_t E, int32_t N,
    int32_t rows_per_block, int32_t nblk, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ local_rank, int32_t* __restrict__ expert_counts,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ token_row,
    int32_t* __restrict__ row_token)
{
    extern __shared__ uint32_t lds_u32[];
    uint32_t* base = lds_u32;          // rows of expert e in blocks before this one
    uint32_t* offs = lds_u32 + E;      // expert totals, then their exclusive scan
    __shared__ uint32_t scratch[kWaves];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    for (int e = tid; e < E; e += kThreads) {
        uint32_t before = 0u, total = 0u;
        for (int bb = 0; bb < nblk; ++bb) {
            const uint32_t v = hist[(int64_t)bb * E + e];
            before += (bb < b) ? v : 0u;
            total += v;
        }
        base[e] = before;
        offs[e] = total;
        if (b == 0)
            expert_counts[e] = (int32_t)total;
    }
    __syncthreads();
    // exclusive scan of the totals: thread tid owns the contiguous experts [lo, hi)
    const int span = (E + kThreads - 1) / kThreads;
    const int lo = min(E, tid * span), hi = min(E, lo + span);
    uint32_t mine = 0u;
    for (int e = lo; e < hi; ++e)
        mine += offs[e];
    uint32_t grand = 0u;
    uint32_t run = block_exclusive_scan(mine, scratch, &grand);
    for (int e = lo; e < hi; ++e) {
        const uint32_t c = offs[e];
        offs[e] = run;
        run += c;
    }
    __syncthreads();
    if (b == 0) {
        const int epr = E / N;
        for (int e = tid; e < E; e += kThreads)
            expert_offsets[e] = (int32_t)offs[e];
        for (int r = tid; r < N; r += kThreads) {
            const uint32_t o0 = offs[r * epr];
            const uint32_t o1 = (r + 1 < N) ? offs[(r + 1) * epr] : grand;
            rank_offsets[r] = (int32_t)o0;
            rank_counts[r] = (int32_t)(o1 - o0);
        }
        if (tid == 0) {
            expert_offsets[E] = (int32_t)grand;
            rank_offsets[N] = (int32_t)grand;
        }
    }
    const int64_t i0 = (int64_t)b * rows_per_block;
    const int64_t i1 = min((int64_t)R, i0 + rows_per_block);
    for (int64_t i = i0 + tid; i < i1; i += kThreads) {
        const int e = topk_idx[i];
        if ((uint32_t)e < (uint32_t)E) {
            const uint32_t row = offs[e] + base[e] + local_rank[i];
            token_row[i] = (int32_t)row;
            row_token[row] = (int32_t)(i / k);
        } else {
            token_row[i] = -1;
        }
    }
}

// ----------------------------------------------------------------------------------- packing --
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Block (t, s) copies 16-byte chunks [s*cpb, (s+1)*cpb) of row t of x to the k rows of token t.
// The chunks are loaded once into registers (U per thread per pass) and stored k times with
// non-temporal stores: the receive buffer is consumed by another kernel, not re-read here.
template <int U>
__global__ __launch_bounds__(kThreads) void k_pack_copy(const u32x4* __restrict__ x, int32_t k,
                                                        int32_t R, int32_t chunks_per_row,
                                                        int32_t chunks_per_block,
                                                        const int32_t* __restrict__ token_row,
                                                        u32x4* __restrict__ recv)
{
    const int64_t t = blockIdx.x;
    const int c0 = blockIdx.y * chunks_per_block;
    const int c1 = min(chunks_per_row, c0 + chunks_per_block);
    const u32x4* src = x + t * chunks_per_row;
    for (int cb = c0 + (int)threadIdx.x; cb < c1; cb += kThreads * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + u * kThreads;
            if (c < c1)
                v[u] = __builtin_nontemporal_load(src + c);
        }
        for (int j = 0; j < k; ++j) {
            const int row = token_row[t * k + j];
            if ((uint32_t)row >= (uint32_t)R)
                continue;
            u32x4* dst = recv + (int64_t)row * chunks_per_row;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = cb + u * kThreads;
                if (c < c1)
                    __builtin_nontemporal_store(v[u], dst + c);
            }
        }
    }
}

// fp8 packing. A chunk is 8 elements; 16 consecutive lanes hold the 128 elements of one scale
// block (chunk ranges start at multiples of 16 chunks, so groups never straddle a block).
template <typename XT>
struct Load8;

template <>
struct Load8<float> {
    static __device__ __forceinline__ void run(const float* p, float (&v)[8])
    {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
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
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
};

template <typename XT>
__global__ __launch_bounds__(kThreads) void k_pack_fp8(const XT* __restrict__ x, int32_t H,
                                                       int32_t k, int32_t R,
                                                       int32_t chunks_per_block,
                                                       const int32_t* __restrict__ token_row,
                                                       uint8_t* __restrict__ recv,
                                                       float* __restrict__ recv_scales)
{
    const int64_t t = blockIdx.x;
    const int chunks_per_row = H / 8;
    const int nb = H / 128;
    const int c0 = blockIdx.y * chunks_per_block;
    const int c1 = min(chunks_per_row, c0 + chunks_per_block);
    for (int cb = c0; cb < c1; cb += kThreads) {       // uniform trip count: shuffles see all lanes
        const int c = cb + (int)threadIdx.x;
        const bool active = c < c1;
        float v[8];
        if (active) {
            Load8<XT>::run(x + t * H + (int64_t)c * 8, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = 0.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int m = 8; m > 0; m >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;   // correctly rounded division
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = f32_to_e4m3(v[i] / s);
        u32x2 packed;
        packed.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        packed.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
        if (!active)
            continue;
        for (int j = 0; j < k; ++j) {
            const int row = token_row[t * k + j];
            if ((uint32_t)row >= (uint32_t)R)
                continue;
            __builtin_nontemporal_store(
                packed, reinterpret_cast<u32x2*>(recv + (int64_t)row * H) + c);
            if ((threadIdx.x & 15) == 0)
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
        *reinterpret_cast<u32x4*>(p) = o;
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
        reinterpret_cast<u32x4*>(p)[0] = a;
        reinterpret_cast<u32x4*>(p)[1] = b;
    }
};

// Block (t, s) produces chunks [s*cpb, (s+1)*cpb) (8 elements each) of out[t]. KC is k when it is
// a compile-time constant (all k loads issued before the first multiply-add), else 0.
template <typename YT, typename OT, int KC>
__global__ __launch_bounds__(kThreads) void k_combine(const YT* __restrict__ y, int32_t H,
                                                      int32_t k_rt, int32_t R,
                                                      int32_t chunks_per_block,
                                                      const int32_t* __restrict__ token_row,
                                                      const float* __restrict__ topk_w,
                                                      OT* __restrict__ out)
{
    const int k = KC > 0 ? KC : k_rt;
    const int64_t t = blockIdx.x;
    const int chunks_per_row = H / 8;
    const int c0 = blockIdx.y * chunks_per_block;
    const int c1 = min(chunks_per_row, c0 + chunks_per_block);
    for (int c = c0 + (int)threadIdx.x; c < c1; c += kThreads) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = 0.0f;
        if constexpr (KC > 0) {
            Y8<YT> v[KC];
            float w[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int row = token_row[t * KC + j];
                w[j] = topk_w[t * KC + j];
                if ((uint32_t)row < (uint32_t)R)
                    v[j].load(y + (int64_t)row * H + (int64_t)c * 8);
                else
                    w[j] = 0.0f, v[j] = Y8<YT>{};
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
                v.load(y + (int64_t)row * H + (int64_t)c * 8);
                v.fma_into(topk_w[t * k + j], acc);
            }
        }
        Store8<OT>::run(out + t * H + (int64_t)c * 8, acc);
    }
}

// ------------------------------------------------------------------------------ host helpers --
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t dtype_size(moe_dtype_t d) { return d == MOE_F32 ? 4 : d == MOE_BF16 ? 2 : 1; }

inline bool is_wide(moe_dtype_t d) { return d == MOE_F32 || d == MOE_BF16; }

struct LayoutPlan {
    int32_t rows_per_block;
    int32_t nblk;
};

// Items per layout block: a multiple of 256, large enough that at most kMaxLayoutBlocks blocks
// exist (the finalize pass of every block reads all histograms).
inline LayoutPlan layout_plan(int64_t R)
{
    const int64_t per = kThreads * (int64_t)kMaxLayoutBlocks;
    const int64_t groups = R > 0 ? (R + per - 1) / per : 1;
    LayoutPlan p;
    p.rows_per_block = (int32_t)(groups * kThreads);
    p.nblk = (int32_t)((R + p.rows_per_block - 1) / p.rows_per_block);
    return p;
}

// Splits of a row across blocks so that T * splits reaches kTargetBlocks, with each split a
// multiple of `align` chunks and at least 64 chunks long.
inline int32_t chunks_per_block(int32_t T, int32_t chunks_per_row, int32_t align)
{
    int64_t splits = (kTargetBlocks + (int64_t)T - 1) / T;
    const int64_t max_splits = (chunks_per_row + 63) / 64;
    if (splits > max_splits)
        splits = max_splits;
    if (splits > 65535)                     // grid y limit
        splits = 65535;
    if (splits < 1)
        splits = 1;
    int64_t cpb = (chunks_per_row + splits - 1) / splits;
    cpb = (cpb + align - 1) / align * align;
    return (int32_t)cpb;
}

inline moe_status_t launch_status()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

inline size_t hist_bytes(int64_t R, int32_t E)
{
    return align_up((size_t)layout_plan(R).nblk * (size_t)E * sizeof(uint32_t), 256);
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
    if ((int64_t)H * (int64_t)dtype_size(x_dtype) / 16 > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t launch_layout(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                           int32_t n_ranks, const moe_dispatch_out_t* out, void* workspace,
                           hipStream_t stream)
{
    const int64_t R = (int64_t)T * k;
    const LayoutPlan plan = layout_plan(R);
    uint32_t* hist = static_cast<uint32_t*>(workspace);
    uint32_t* local_rank =
        reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + hist_bytes(R, E));
    if (plan.nblk > 0) {
        const size_t lds = (size_t)kWaves * E * sizeof(uint64_t) + (size_t)E * sizeof(uint32_t);
        k_layout_hist<<<plan.nblk, kThreads, lds, stream>>>(topk_idx, (int32_t)R, E,
                                                            plan.rows_per_block, hist,
                                                            local_rank);
    }
    const size_t lds2 = 2 * (size_t)E * sizeof(uint32_t);
    k_layout_finalize<<<plan.nblk > 0 ? plan.nblk : 1, kThreads, lds2, stream>>>(
        topk_idx, (int32_t)R, k, E, n_ranks, plan.rows_per_block, plan.nblk, hist, local_rank,
        out->expert_counts, out->expert_offsets, out->rank_counts, out->rank_offsets,
        out->token_row, out->row_token);
    return launch_status();
}

moe_status_t launch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H, int32_t k,
                         const int32_t* token_row, moe_dtype_t payload_dtype, void* recv,
                         float* recv_scales, hipStream_t stream)
{
    if (T == 0)
        return MOE_OK;
    const int32_t R = T * k;
    if (payload_dtype != MOE_FP8_E4M3) {
        const int32_t cpr = (int32_t)((int64_t)H * (int64_t)dtype_size(x_dtype) / 16);
        const int32_t cpb = chunks_per_block(T, cpr, 1);
        const dim3 grid(T, (cpr + cpb - 1) / cpb);
        k_pack_copy<4><<<grid, kThreads, 0, stream>>>(static_cast<const u32x4*>(x), k, R, cpr,
                                                      cpb, token_row, static_cast<u32x4*>(recv));
    } else {
        const int32_t cpr = H / 8;
        const int32_t cpb = chunks_per_block(T, cpr, 16);
        const dim3 grid(T, (cpr + cpb - 1) / cpb);
        if (x_dtype == MOE_F32)
            k_pack_fp8<float><<<grid, kThreads, 0, stream>>>(
                static_cast<const float*>(x), H, k, R, cpb, token_row,
                static_cast<uint8_t*>(recv), recv_scales);
        else
            k_pack_fp8<uint16_t><<<grid, kThreads, 0, stream>>>(
                static_cast<const uint16_t*>(x), H, k, R, cpb, token_row,
                static_cast<uint8_t*>(recv), recv_scales);
    }
    return launch_status();
}

template <typename YT, typename OT>
void launch_combine_typed(const void* y, int32_t T, int32_t H, int32_t k,
                          const int32_t* token_row, const float* topk_w, void* out,
                          hipStream_t stream)
{
    const int32_t R = T * k;
    const int32_t cpr = H / 8;
    const int32_t cpb = chunks_per_block(T, cpr, 1);
    const dim3 grid(T, (cpr + cpb - 1) / cpb);
    const YT* yp = static_cast<const YT*>(y);
    OT* op = static_cast<OT*>(out);
    switch (k) {
    case 1: k_combine<YT, OT, 1><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    case 2: k_combine<YT, OT, 2><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    case 4: k_combine<YT, OT, 4><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    case 6: k_combine<YT, OT, 6><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    case 8: k_combine<YT, OT, 8><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    default: k_combine<YT, OT, 0><<<grid, kThreads, 0, stream>>>(yp, H, k, R, cpb, token_row, topk_w, op); break;
    }
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
    const dim3 grid((T + kWaves - 1) / kWaves);
    if (pl <= 1)
        k_route_topk<1><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (pl <= 2)
        k_route_topk<2><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (pl <= 4)
        k_route_topk<4><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (pl <= 6)
        k_route_topk<6><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (pl <= 8)
        k_route_topk<8><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else
        k_route_topk<16><<<grid, kThreads, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    return launch_status();
}

size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k)
{
    if (T < 0 || E < 1 || k < 1 || (int64_t)T * k > INT32_MAX)
        return 0;
    const int64_t R = (int64_t)T * k;
    return hist_bytes(R, E) + align_up((size_t)(R > 0 ? R : 1) * sizeof(uint32_t), 256);
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
    return launch_layout(topk_idx, T, k, E, n_ranks, out, workspace, stream);
}

moe_status_t moe_dispatch_pack(const void* x, moe_dtype_t x_dtype, int32_t T, int32_t H,
                               int32_t k, const int32_t* token_row, moe_dtype_t payload_dtype,
                               void* recv, float* recv_scales, hipStream_t stream)
{
    moe_status_t st =
        check_pack_args(x, x_dtype, T, H, k, token_row, payload_dtype, recv, recv_scales);
    if (st != MOE_OK)
        return st;
    return launch_pack(x, x_dtype, T, H, k, token_row, payload_dtype, recv, recv_scales, stream);
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
    st = launch_layout(topk_idx, T, k, E, n_ranks, out, workspace, stream);
    if (st != MOE_OK)
        return st;
    return launch_pack(x, x_dtype, T, H, k, out->token_row, payload_dtype, out->recv,
                       out->recv_scales, stream);
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
