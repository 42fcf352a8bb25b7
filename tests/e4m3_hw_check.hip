// Exhaustive checks behind the fp8 quantiser's fast path (test helper, built by build() into
// tests/libe4m3_hw_check.so; no part of the routing library).
//
// 1. The gfx950 conversion v_cvt_pk_fp8_f32 (round to nearest even), with the magnitude bits kept
//    and the sign taken from the input, against an e4m3fn encoder written here from the format
//    definition as threshold counting: the code of a magnitude a is the number of midpoints
//    between consecutive finite codes that lie below a, a tie going to the even code, and 126
//    (448) at most; NaN gives the NaN code 0x7F with the input's sign. Every fp32 pattern with
//    |d| < 464, and every NaN pattern, is compared.
// 2. The quotient used for blocks with a normal scale: r = 1/s correctly rounded, q0 = |v|*r,
//    q = q0 + (|v|*2^j - q0*(s*2^j)) * (r*2^-j) with 2^j = 2^(127 - exponent of amax), sign of v;
//    its code against the code of the correctly rounded fp32 quotient v/s, for every pair of bf16
//    values (v, amax) with |v| <= amax, amax finite and not 0, s = amax/448 normal, amax < 2^127.
// 3. The same comparison for 2^32 pseudo-random fp32 pairs (v, amax) of the fast path (full 24-bit
//    significands, amax over the whole range that gives a normal s, v from the same binade as amax
//    down to 40 binades below it and into the subnormals), drawn from a counter-based hash of the
//    pair's index (splitmix64's finaliser).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ float e4m3_value(uint32_t c)   // finite positive codes 0..126
{
    const uint32_t e = c >> 3, m = c & 7u;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
}

__device__ uint32_t e4m3_def(float d)
{
    const uint32_t sign = (__float_as_uint(d) >> 24) & 0x80u;
    if (d != d)
        return sign | 0x7Fu;
    const float a = fabsf(d);
    uint32_t c = 0;
    bool tie = false;
    for (uint32_t i = 0; i < 126u; ++i) {
        const float mid = 0.5f * (e4m3_value(i) + e4m3_value(i + 1));   // exact in fp32
        c += mid < a ? 1u : 0u;
        tie = tie || mid == a;
    }
    if (tie && (c & 1u))
        c += 1u;                            // a sits on the midpoint above code c: the even one
    return sign | c;
}

__device__ uint32_t e4m3_hw(float d)
{
    const uint32_t c = __builtin_amdgcn_cvt_pk_fp8_f32(d, 0.0f, 0, false) & 0xFFu;
    return (c & 0x7Fu) | ((__float_as_uint(d) >> 24) & 0x80u);
}

__device__ float fast_quotient(float v, float s, float amax)
{
    const uint32_t ea = __float_as_uint(amax) >> 23;
    const float r = 1.0f / s;
    const float up = __uint_as_float((254u - ea) << 23);
    const float down = __uint_as_float(ea << 23);
    const float a = fabsf(v);
    const float q0 = a * r;
    return copysignf(fmaf(fmaf(-q0, s * up, a * up), r * down, q0), v);
}

__device__ uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// counts: [0] encoder inputs, [1] encoder mismatches, [2] bf16 quotient pairs, [3] their code
// mismatches, [4] random fp32 pairs, [5] their code mismatches
__global__ void k_check(unsigned long long* counts)
{
    const uint64_t n = 1ull << 32;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long c0 = 0, c1 = 0, c2 = 0, c3 = 0, c4 = 0, c5 = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t u = (uint32_t)i;
        const float d = __uint_as_float(u);
        if (d != d || fabsf(d) < 464.0f) {
            ++c0;
            c1 += e4m3_hw(d) != e4m3_def(d) ? 1u : 0u;
        }
        const float v = __uint_as_float((u & 0xFFFFu) << 16);
        const float amax = fabsf(__uint_as_float(u & 0xFFFF0000u));
        if (amax > 0.0f && amax < 0x1p127f && fabsf(v) <= amax) {
            const float s = amax / 448.0f;
            if (s >= 0x1p-126f) {
                ++c2;
                c3 += e4m3_hw(fast_quotient(v, s, amax)) != e4m3_def(v / s) ? 1u : 0u;
            }
        }
        const uint64_t z = mix64(i);
        const uint32_t ea = 10u + (uint32_t)(z % 243u);                     // amax in [2^-117, 2^126)
        const float ra = __uint_as_float((ea << 23) | (uint32_t)((z >> 8) & 0x7FFFFFu));
        const uint32_t drop = (uint32_t)((z >> 32) % 41u);
        const uint32_t ev = ea > drop ? ea - drop : 0u;                      // 0: a subnormal v
        float rv = __uint_as_float(((uint32_t)(z >> 63) << 31) | (ev << 23) |
                                   (uint32_t)((z >> 36) & 0x7FFFFFu));
        if (fabsf(rv) > ra)
            rv = copysignf(ra, rv);
        const float rs = ra / 448.0f;
        if (rs >= 0x1p-126f) {
            ++c4;
            c5 += e4m3_hw(fast_quotient(rv, rs, ra)) != e4m3_def(rv / rs) ? 1u : 0u;
        }
    }
    // one atomic per wavefront and counter
    for (int off = 32; off > 0; off >>= 1) {
        c0 += __shfl_down(c0, off, 64);
        c1 += __shfl_down(c1, off, 64);
        c2 += __shfl_down(c2, off, 64);
        c3 += __shfl_down(c3, off, 64);
        c4 += __shfl_down(c4, off, 64);
        c5 += __shfl_down(c5, off, 64);
    }
    if ((threadIdx.x & 63) == 0) {
        atomicAdd(&counts[0], c0);
        atomicAdd(&counts[1], c1);
        atomicAdd(&counts[2], c2);
        atomicAdd(&counts[3], c3);
        atomicAdd(&counts[4], c4);
        atomicAdd(&counts[5], c5);
    }
}

}  // namespace

// Runs the three checks on the current device; writes the six counts to host memory. Returns 0,
// or the HIP error code.
extern "C" int e4m3_hw_check(unsigned long long* host_counts)
{
    unsigned long long* d = nullptr;
    hipError_t err = hipMalloc(&d, 6 * sizeof(unsigned long long));
    if (err != hipSuccess)
        return (int)err;
    err = hipMemset(d, 0, 6 * sizeof(unsigned long long));
    if (err == hipSuccess) {
        k_check<<<16384, 256>>>(d);
        err = hipGetLastError();
    }
    if (err == hipSuccess)
        err = hipDeviceSynchronize();
    if (err == hipSuccess)
        err = hipMemcpy(host_counts, d, 6 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    const hipError_t err2 = hipFree(d);
    return (int)(err != hipSuccess ? err : err2);
}
