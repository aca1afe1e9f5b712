// Packing of uint8 codes into per-row least-significant-bit-first bitstreams
// (the layout the product kernels consume as stored), and the split-K
// partial-sum reduction.
#include "qmm_kernels.hpp"

namespace qmm {
namespace {

// One thread per output word: word w of row n holds stream bits
// [32w, 32w + 32), i.e. parts of codes floor(32w/B) .. floor((32w+31)/B).
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes,
                                                   uint32_t *__restrict__ packed, int N, int K)
{
    const size_t wpr = (size_t)K * BITS / 32;
    const size_t total = (size_t)N * wpr;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t n = idx / wpr;
        const int w = (int)(idx % wpr);
        const int bit0 = 32 * w;
        const int k0 = bit0 / BITS, k1 = (bit0 + 31) / BITS;
        const uint8_t *row = codes + n * (size_t)K;
        uint32_t word = 0;
        for (int k = k0; k <= k1; ++k) {
            const uint32_t code = row[k] & mask;
            const int off = k * BITS - bit0;
            word |= off >= 0 ? (code << off) : (code >> (-off));
        }
        packed[idx] = word;
    }
}

// y[i] = sum over z = 0 .. S-1, in that order, of partials[z*count + i].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partials,
                                                            float *__restrict__ y, int S,
                                                            size_t count)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x) {
        float s = partials[i];
        for (int z = 1; z < S; ++z)
            s += partials[(size_t)z * count + i];
        y[i] = s;
    }
}

// y[i] = 0 for i < count (the launches that add two K halves into y start
// from it; a kernel rather than a memset, so that graph replays stay exact).
__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ y, size_t count)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
        y[i] = 0.f;
}

// Number of positions i < count where the 32-bit words a[i] and b[i]
// differ, written to *mismatches by one workgroup (no atomics, no clearing).
__global__ __launch_bounds__(256) void compare_words_kernel(const uint32_t *__restrict__ a,
                                                            const uint32_t *__restrict__ b,
                                                            size_t count, uint32_t *mismatches)
{
    __shared__ uint32_t part[256 / 64];
    uint32_t n = 0;
    for (size_t i = threadIdx.x; i < count; i += blockDim.x)
        n += a[i] != b[i] ? 1u : 0u;
    for (int d = 32; d >= 1; d /= 2)
        n += __shfl_xor(n, d);
    if (threadIdx.x % 64 == 0)
        part[threadIdx.x / 64] = n;
    __syncthreads();
    if (threadIdx.x == 0)
        *mismatches = part[0] + part[1] + part[2] + part[3];
}

unsigned grid_for(size_t work, unsigned threads)
{
    const size_t blocks = (work + threads - 1) / threads;
    return (unsigned)(blocks < 65536 ? (blocks ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_pack(const uint8_t *codes, uint32_t *packed, int N, int K, int bits,
                       hipStream_t stream)
{
    const size_t total = (size_t)N * K * bits / 32;
    const dim3 grid(grid_for(total, 256)), block(256);
    switch (bits) {
    case 2: hipLaunchKernelGGL(pack_kernel<2>, grid, block, 0, stream, codes, packed, N, K); break;
    case 3: hipLaunchKernelGGL(pack_kernel<3>, grid, block, 0, stream, codes, packed, N, K); break;
    case 4: hipLaunchKernelGGL(pack_kernel<4>, grid, block, 0, stream, codes, packed, N, K); break;
    case 5: hipLaunchKernelGGL(pack_kernel<5>, grid, block, 0, stream, codes, packed, N, K); break;
    case 6: hipLaunchKernelGGL(pack_kernel<6>, grid, block, 0, stream, codes, packed, N, K); break;
    case 8: hipLaunchKernelGGL(pack_kernel<8>, grid, block, 0, stream, codes, packed, N, K); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *partials, float *y, int split, size_t count,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for(count, 256)), dim3(256), 0, stream,
                       partials, y, split, count);
    return hipGetLastError();
}

hipError_t launch_zero(float *y, size_t count, hipStream_t stream)
{
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(count, 256)), dim3(256), 0, stream, y, count);
    return hipGetLastError();
}

hipError_t launch_compare_words(const uint32_t *a, const uint32_t *b, size_t count, uint32_t *mismatches,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(compare_words_kernel, dim3(1), dim3(256), 0, stream, a, b, count, mismatches);
    return hipGetLastError();
}

}  // namespace qmm
