// Kernel launchers (one translation unit per kernel family) and the
// parameters shared between the host dispatcher and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

constexpr int kMaxProj = 4;  // projections sharing x in one fused launch

// One weight matrix with its output: codes, scales, biases, y [M, N].
struct Proj {
    const uint32_t *wq;
    const uint16_t *scales;
    const uint16_t *biases;
    float *y;
    int N;
};

// Arguments of one product launch. `y` receives either the final result
// (split == 1) or slice z's partial product at y + z*y_slice_stride
// (split > 1). M is the number of activation rows of this launch; the
// multi-row kernel takes at most 16 and the host walks larger M in 16-row
// steps.
//
// Fused launches (nproj >= 2, split == 1) run several projections of the
// same x: projection p owns the 16-row tiles [tile0[p], tile0[p+1]) of the
// launch, its rows padded to whole tiles, and N is 16 * tile0[nproj]. Every
// kernel works in 16-row tiles (a workgroup or a K-part wave owns whole
// tiles), so each tile belongs to one projection.
struct ProductArgs {
    const uint16_t *x;
    const uint32_t *wq;
    const uint16_t *scales;
    const uint16_t *biases;
    float *y;
    int M, K, N;
    int split;               // number of K slices (grid z); 1 = whole K
    size_t y_slice_stride;   // elements between consecutive slices' partials in y
    int nproj;               // 0 or 1: the single projection above
    int tile0[kMaxProj + 1];
    Proj proj[kMaxProj];
};

// The projection that owns 16-row tile t of a launch, and t's index inside it.
struct Slab {
    Proj p;
    int tile;
};

__host__ __device__ __forceinline__ Slab slab_of_tile(const ProductArgs &a, int t)
{
    if (a.nproj <= 1)
        return Slab{Proj{a.wq, a.scales, a.biases, a.y, a.N}, t};
    int q = 0;
#pragma unroll
    for (int j = 1; j < kMaxProj; ++j)
        q = (j < a.nproj && t >= a.tile0[j]) ? j : q;
    return Slab{a.proj[q], t - a.tile0[q]};
}

// Rows [m0, m0 + count) of a launch: x and every output advance by m0 rows.
inline ProductArgs rows_of(const ProductArgs &a, int m0, int count)
{
    ProductArgs b = a;
    b.M = count;
    b.x = a.x + (size_t)m0 * a.K;
    if (a.y)  // NULL in fused launches, whose outputs are the projections'
        b.y = a.y + (size_t)m0 * a.N;
    for (int j = 0; j < a.nproj && j < kMaxProj; ++j)
        b.proj[j].y = a.proj[j].y + (size_t)m0 * a.proj[j].N;
    return b;
}

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cu_count();

// Each launcher returns a hipError_t from the launch (hipSuccess, or the
// runtime's error) and hipErrorInvalidValue for an unsupported (bits, G).
hipError_t launch_pack(const uint8_t *codes, uint32_t *packed, int N, int K, int bits,
                       hipStream_t stream);
// bf16: x, scales and biases are bf16 bit patterns instead of fp16.
hipError_t launch_qmv(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream);
// bf16: x, scales and biases are bf16 bit patterns (M >= 3 per launch).
hipError_t launch_mfma(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream);
bool mfma_supported(int bits, int G);  // whether launch_mfma handles (bits, G)
// Register-resident multi-row kernel: whether it can run `a` (split included)
// and its launcher (hipErrorInvalidValue when it cannot).
bool mfma_xr_supported(const ProductArgs &a, int bits, int G);
// bf16: x, scales and biases are bf16 bit patterns (single-projection launches only).
hipError_t launch_mfma_xr(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream);
// Tiled (MFMA-native) weight layout: whether the product on it supports
// the shape (bits 2, 4, 8; K*bits a multiple of 512; K/G a multiple of 4;
// parts that fit), the repack from the standard layout (N padded to whole
// 16-row tiles with zeros) and the product (a.wq = tiled codes, a.scales =
// tiled (s, b) words; 16 rows per launch at most).
bool tiled_supported(const ProductArgs &a, int bits, int G);
hipError_t launch_repack_tiled(const uint32_t *wq, const uint16_t *scales, const uint16_t *biases, uint8_t *tw,
                               uint32_t *tsb, int N, int K, int bits, int G, hipStream_t stream);
hipError_t launch_mfma_tiled(const ProductArgs &a, int bits, int G, hipStream_t stream);
// Streaming read of `bytes` (a multiple of 16) at `src` (16-byte aligned):
// one sink word per workgroup, stream_read_sink_words(bytes) in all.
size_t stream_read_sink_words(size_t bytes);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
// *mismatches = number of i < count with a[i] != b[i] (32-bit words).
hipError_t launch_compare_words(const uint32_t *a, const uint32_t *b, size_t count, uint32_t *mismatches,
                                hipStream_t stream);
hipError_t launch_splitk_reduce(const float *partials, float *y, int split, size_t count,
                                hipStream_t stream);
hipError_t launch_zero(float *y, size_t count, hipStream_t stream);  // y[0 .. count) = 0

// Group range [begin, end) of K slice z when Kg groups are split into S
// slices: floor(Kg/S) groups each, one more for the first Kg mod S slices.
__host__ __device__ inline void slice_groups(int Kg, int S, int z, int &begin, int &end)
{
    const int base = Kg / S, extra = Kg % S;
    begin = z * base + (z < extra ? z : extra);
    end = begin + base + (z < extra ? 1 : 0);
}

}  // namespace qmm
