// Streaming-read kernel: reads a buffer once with the 16-byte non-temporal
// loads the product kernels use for packed codes, and nothing else, so its
// time is the read ceiling those kernels are measured against (a one-row
// product streams its weight bytes once and writes almost nothing).
//
// Every thread issues all of its loads before using any of them, and a
// workgroup covers one contiguous span, so the whole buffer is requested
// about as fast as the chip can issue; each workgroup writes the XOR of its
// words to its own sink word (no atomics, no cross-workgroup ordering), which
// keeps the loads live and lets a test check that every byte was read.
//
// Shape: many small workgroups (256 threads, two 16-byte loads per thread,
// 8 KiB each) finish and are replaced continuously, which kept the most
// bytes in flight of the shapes measured over 55.7 MB (us per call): 2 loads
// x 256 threads 9.8, 2 x 512 9.9, 16 x 256 10.2, 1 x 256 10.8, 4 x 128 10.9,
// 1 x 1024 13.4; workgroups in XCD-contiguous order changed nothing.
#include "qmm_device.hpp"
#include "qmm_kernels.hpp"

namespace qmm {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadLoads = 2;  // 16-byte loads per thread
constexpr size_t kReadSpan = (size_t)kReadThreads * kReadLoads;  // 16-byte units per workgroup

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4 *src, size_t units,
                                                                    uint32_t *sink)
{
    __shared__ uint32_t part[kReadThreads / kWave];
    const size_t base = (size_t)blockIdx.x * kReadSpan + threadIdx.x;
    u32x4 v[kReadLoads];
#pragma unroll
    for (int j = 0; j < kReadLoads; ++j) {
        const size_t u = base + (size_t)j * kReadThreads;
        v[j] = u < units ? __builtin_nontemporal_load(src + u) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < kReadLoads; ++j)
        acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
#pragma unroll
    for (int d = kWave / 2; d >= 1; d /= 2)
        acc ^= __shfl_xor(acc, d);
    if (threadIdx.x % kWave == 0)
        part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < kReadThreads / kWave; ++k)
            w ^= part[k];
        sink[blockIdx.x] = w;
    }
}

}  // namespace

size_t stream_read_sink_words(size_t bytes)
{
    const size_t units = bytes / 16;
    return (units + kReadSpan - 1) / kReadSpan;
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    const size_t units = bytes / 16;
    const size_t blocks = stream_read_sink_words(bytes);
    if (blocks == 0 || blocks > 0x7FFFFFFFu)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream,
                       reinterpret_cast<const u32x4 *>(src), units, sink);
    return hipGetLastError();
}

}  // namespace qmm
