// Kernel launchers (one translation unit per kernel family) and the
// parameters shared between the host dispatcher and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

// Arguments of one product launch. `y` receives either the final result
// (split == 1) or slice z's partial product at y + z*y_slice_stride
// (split > 1). M is the number of activation rows of this launch; the
// multi-row kernel takes at most 16 and the host walks larger M in 16-row
// steps.
struct ProductArgs {
    const uint16_t *x;
    const uint32_t *wq;
    const uint16_t *scales;
    const uint16_t *biases;
    float *y;
    int M, K, N;
    int split;               // number of K slices (grid z); 1 = whole K
    size_t y_slice_stride;   // elements between consecutive slices' partials in y
};

// Each launcher returns a hipError_t from the launch (hipSuccess, or the
// runtime's error) and hipErrorInvalidValue for an unsupported (bits, G).
hipError_t launch_pack(const uint8_t *codes, uint32_t *packed, int N, int K, int bits,
                       hipStream_t stream);
hipError_t launch_qmv(const ProductArgs &a, int bits, int G, hipStream_t stream);
hipError_t launch_mfma(const ProductArgs &a, int bits, int G, hipStream_t stream);
// Register-resident multi-row kernel: whether it can run `a` (split included)
// and its launcher (hipErrorInvalidValue when it cannot).
bool mfma_xr_supported(const ProductArgs &a, int bits, int G);
hipError_t launch_mfma_xr(const ProductArgs &a, int bits, int G, hipStream_t stream);
hipError_t launch_splitk_reduce(const float *partials, float *y, int split, size_t count,
                                hipStream_t stream);

// Group range [begin, end) of K slice z when Kg groups are split into S
// slices: floor(Kg/S) groups each, one more for the first Kg mod S slices.
__host__ __device__ inline void slice_groups(int Kg, int S, int z, int &begin, int &end)
{
    const int base = Kg / S, extra = Kg % S;
    begin = z * base + (z < extra ? z : extra);
    end = begin + base + (z < extra ? 1 : 0);
}

}  // namespace qmm
