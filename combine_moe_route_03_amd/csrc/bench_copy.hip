// bench_copy.hip -- a plain 16-byte streaming copy, used only by the benchmark: it is the practical
// HBM ceiling on the same GPU, and the known-size kernel against which the HBM byte counters are
// calibrated. Not part of the routing library.
#include <hip/hip_runtime.h>

#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte non-temporal load and store per thread; consecutive lanes touch consecutive chunks.
__global__ __launch_bounds__(256) void k_stream_copy16(const u32x4* __restrict__ src,
                                                       u32x4* __restrict__ dst, int64_t n16)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

extern "C" int bench_stream_copy16(const void* src, void* dst, int64_t bytes, hipStream_t stream)
{
    if (!src || !dst || bytes < 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16)
        return 1;
    const int64_t n16 = bytes / 16;
    if (n16 == 0)
        return 0;
    const int64_t blocks = (n16 + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        return 1;
    k_stream_copy16<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<const u32x4*>(src),
                                                          static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
