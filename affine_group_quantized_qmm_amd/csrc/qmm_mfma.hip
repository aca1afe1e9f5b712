// Multi-row product (M = 2..16 activation rows) on the gfx950 matrix cores.
//
// The verify blocks of speculative decoding multiply a few rows by the same
// packed weights. The vmlx-swift pull request #565 page (commit "LaneQMM")
// runs a tensor-op matmul directly over the raw affine codes with the
// dequantization applied after the dot product, so the cost stays nearly flat
// from 1 to 16 rows; its row-batching commit notes that addressing each
// verify row as a separate one-row call streamed a large projection once per
// row. Here every weight byte is read once per call for all rows.
//
// Operands of one v_mfma_f32_16x16x32_f16 (lane = 16*c + i, c = 0..3):
//   A (activations): lane (c, i) holds 8 values of activation row i,
//   B (codes):       lane (c, i) holds 8 codes of weight row n0 + i,
//   C (fp32):        lane (c, i) holds rows 4c..4c+3 of output column n0 + i.
// Each lane block c supplies codes c*G/4 .. c*G/4 + G/4 - 1 of a group, so
// one MFMA (G = 32) or G/32 accumulating MFMAs contract exactly one group,
// after which the fp32 epilogue acc += s*P + b*XS applies that group's scale
// and bias. The group sums XS come from one more MFMA against a ones operand,
// which leaves them in exactly the C layout.
//
// Weight loads. When a lane block's chunk is one or two words (4-bit codes
// with G = 32, 8-bit codes with G = 32) a direct chunk load would be 4 or 8
// bytes per lane; instead the wave walks its K range in steps of 4 groups,
// lane block c loads all of group g0 + c of its row with 16-byte loads, and a
// 4x4 transpose across the lane blocks (v_permlane32_swap + v_permlane16_swap,
// 4 swaps per chunk word) hands every lane block its own chunk of the 4
// groups. For larger chunks each lane loads its chunk of one group directly
// and shifts it to a bit-0 start. A ring of PD register stages keeps several
// steps of loads in flight.
//
// Activations are small and cache resident; each lane loads its 8 values per
// MFMA straight from global memory and permutes them in registers to the
// pair order of the code unpack.
//
// A workgroup of WAVES waves owns 16*NB weight rows; each wave takes one
// share of the K range (or of the split-K slice) and the partial tiles are
// summed in a fixed order through LDS.
#include "qmm_device.hpp"
#include "qmm_kernels.hpp"

namespace qmm {
namespace {

template <int BITS, int G>
struct Geometry {
    static constexpr int T = G / 32;               // MFMAs per group
    static constexpr int CH = G / 4;               // codes per lane block per group
    static constexpr int CHB = CH * BITS;          // bits per lane block
    static constexpr int NWG = G * BITS / 32;      // words per group
    // Transposed loads when a lane block's chunk is at most two words: lane
    // block c loads all of group g0 + c (16 or 32 bytes), the transpose
    // deals out the chunks. Steps then cover 4 groups.
    static constexpr bool kTranspose = CHB <= 64 && NWG % 4 == 0;
    static constexpr int SG = kTranspose ? 4 : 1;  // groups per step
    static constexpr int UNIT = NWG / 4;           // words per chunk (transposed path)
    static constexpr int LOAD_ALIGN = gcd_int(4 * NWG, 16);
    // Direct chunk loads: words per lane and the largest sub-word shift.
    static constexpr int max_shift()
    {
        int m = 0;
        for (int c = 0; c < 4; ++c)
            m = (c * CHB) % 32 > m ? (c * CHB) % 32 : m;
        return m;
    }
    static constexpr int RMAX = max_shift();
    static constexpr int NW = kTranspose ? NWG : (RMAX + CHB + 31) / 32;  // words loaded per lane
    static constexpr int NWC = (CHB + 31) / 32;                          // chunk words after shift
    static constexpr int CHUNK_ALIGN = RMAX == 0 ? gcd_int(4 * NWC, 16) : 4;
    // Steps kept in flight: about 2 KB of codes per 16-row block.
    static constexpr int PD = kTranspose ? 2 : (NWC <= 2 ? 4 : (NWC <= 4 ? 3 : 2));
    static constexpr bool fits()
    {
        if (kTranspose)
            return true;
        for (int c = 0; c < 4; ++c)
            if ((c * CHB) / 32 + NW > NWG)
                return false;
        return true;
    }
};

// The 8 activations of one MFMA K-block in the unpack's pair order.
template <int BITS>
__device__ __forceinline__ half8_t to_pair_order(half8_t v)
{
    if constexpr (pair_dist(BITS) == 4)
        return __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
    else
        return __builtin_shufflevector(v, v, 0, 2, 1, 3, 4, 6, 5, 7);
}

// 4x4 transpose across the four 16-lane rows of a wave: on entry register t
// of lane row c holds V[c][t]; on exit register t holds V[t][c].
__device__ __forceinline__ void transpose4(uint32_t &w0, uint32_t &w1, uint32_t &w2, uint32_t &w3)
{
    const auto a02 = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
    const auto a13 = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
    const auto o01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
    const auto o23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
    w0 = o01[0];
    w1 = o01[1];
    w2 = o23[0];
    w3 = o23[1];
}

template <int BITS, int G, int NB, int WAVES>
__global__ __launch_bounds__(WAVES *kWave) void mfma_kernel(const ProductArgs a)
{
    using Geo = Geometry<BITS, G>;
    constexpr int T = Geo::T;
    constexpr int CH = Geo::CH;
    constexpr int NW = Geo::NW;
    constexpr int NWC = Geo::NWC;
    constexpr int NWG = Geo::NWG;
    constexpr int SG = Geo::SG;
    constexpr int PD = Geo::PD;

    __shared__ float4_t partial[WAVES][NB][kWave];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane / 16, i = lane % 16;
    const int M = a.M, K = a.K, N = a.N, Kg = K / G;
    const size_t wpr = (size_t)K * BITS / 32;
    const int nbase = blockIdx.x * 16 * NB;

    int sb = 0, se = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, sb, se);
    int wb, we;
    slice_groups(se - sb, WAVES, wave, wb, we);
    wb += sb;
    we += sb;
    const int nsteps = (we - wb + SG - 1) / SG;

    // Weight row of block nb for this lane (clamped so every load stays in bounds).
    int row[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        row[nb] = min(nbase + nb * 16 + i, N - 1);
    // Lanes of activation rows i >= M read row M-1 instead: A rows >= M only
    // reach output rows >= M, which are never stored.
    const uint16_t *xrow = a.x + (size_t)min(i, M - 1) * K + c * CH;
    const int chunk_word = (c * Geo::CHB) / 32;   // direct path
    const int chunk_shift = (c * Geo::CHB) % 32;  // direct path

    half8_t ones;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ones[e] = (_Float16)1.0f;

    float4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = float4_t{0.f, 0.f, 0.f, 0.f};

    // One step of loads: SG groups of NB weight blocks, their scales and
    // biases and activations. Scales and biases stay raw 16-bit values until
    // they are used, so nothing consumes a load right after it is issued.
    // On the transposed path lane block c holds the scale and bias of group
    // g0 + c; the compute step gathers all four across the lane blocks.
    struct Stage {
        uint32_t w[NB][NW];
        uint16_t s[NB], b[NB];
        half8_t x[SG][T];
    };

    // Loads of one step. Every load is unconditional: steps past the wave's
    // range are clamped to its last step (cache hits, never used), so the
    // compiler can keep the ring of stages in flight.
    auto load = [&](Stage &st, int step) {
        const int g0 = wb + min(step, nsteps - 1) * SG;
        const int gsb = Geo::kTranspose ? min(g0 + c, we - 1) : g0;  // group of this lane's s, b
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const size_t rowbase = (size_t)row[nb] * wpr;
            if constexpr (Geo::kTranspose)
                load_words<NW, Geo::LOAD_ALIGN>(a.wq + rowbase + (size_t)gsb * NWG, st.w[nb]);
            else
                load_words<NW, Geo::CHUNK_ALIGN>(a.wq + rowbase + (size_t)g0 * NWG + chunk_word, st.w[nb]);
            const size_t sidx = (size_t)row[nb] * Kg + gsb;
            st.s[nb] = a.scales[sidx];
            st.b[nb] = a.biases[sidx];
        }
#pragma unroll
        for (int t = 0; t < SG; ++t) {
            const int g = min(g0 + t, we - 1);
#pragma unroll
            for (int h = 0; h < T; ++h)
                st.x[t][h] = *reinterpret_cast<const half8_t *>(xrow + (size_t)g * G + 8 * h);
        }
    };

    auto compute = [&](Stage &st, int step) {
        const int g0 = wb + step * SG;
        // (scale, bias) of group g0 + t for this lane's weight row
        uint32_t sb[NB][SG];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t own = (uint32_t)st.s[nb] | ((uint32_t)st.b[nb] << 16);
            if constexpr (Geo::kTranspose) {
#pragma unroll
                for (int t = 0; t < SG; ++t)
                    sb[nb][t] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * t + i) * 4, (int)own);
            } else {
                sb[nb][0] = own;
            }
        }
        // chunk[nb][t]: this lane block's chunk of group g0 + t of block nb, from bit 0
        uint32_t chunk[NB][SG][NWC];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if constexpr (Geo::kTranspose) {
#pragma unroll
                for (int u = 0; u < Geo::UNIT; ++u) {
                    uint32_t w0 = st.w[nb][0 * Geo::UNIT + u], w1 = st.w[nb][1 * Geo::UNIT + u];
                    uint32_t w2 = st.w[nb][2 * Geo::UNIT + u], w3 = st.w[nb][3 * Geo::UNIT + u];
                    transpose4(w0, w1, w2, w3);
                    chunk[nb][0][u] = w0;
                    chunk[nb][1][u] = w1;
                    chunk[nb][2][u] = w2;
                    chunk[nb][3][u] = w3;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NWC; ++j) {
                    if constexpr (Geo::RMAX == 0)
                        chunk[nb][0][j] = st.w[nb][j];
                    else
                        chunk[nb][0][j] = j + 1 < NW
                                              ? __builtin_amdgcn_alignbit(st.w[nb][j + 1], st.w[nb][j], chunk_shift)
                                              : (st.w[nb][j] >> chunk_shift);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < SG; ++t) {
            if (g0 + t < we) {  // wave-uniform
                half8_t A[T];
                float4_t xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < T; ++h) {
                    A[h] = to_pair_order<BITS>(st.x[t][h]);
                    xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[h], ones, xs, 0, 0, 0);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    half2_t q[CH / 2];
                    unpack_pairs<BITS, CH>(chunk[nb][t], q);
                    float4_t P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int h = 0; h < T; ++h) {
                        const half8_t B = {q[4 * h].x, q[4 * h].y, q[4 * h + 1].x, q[4 * h + 1].y,
                                           q[4 * h + 2].x, q[4 * h + 2].y, q[4 * h + 3].x, q[4 * h + 3].y};
                        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[h], B, P, 0, 0, 0);
                    }
                    const float s = half_bits_to_float((uint16_t)(sb[nb][t] & 0xffffu));
                    const float b = half_bits_to_float((uint16_t)(sb[nb][t] >> 16));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[nb][r] += s * P[r] + b * xs[r];
                }
            }
        }
    };

    if (nsteps > 0) {
        Stage ring[PD];
#pragma unroll
        for (int p = 0; p < PD; ++p)
            load(ring[p], p);
        // steady state: compute step s, then refill its stage with step s + PD
        int s0 = 0;
        for (; s0 + PD < nsteps; s0 += PD) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                compute(ring[p], s0 + p);
                load(ring[p], s0 + p + PD);
            }
        }
        // drain: the last (at most PD) steps are already loaded
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (s0 + p < nsteps)
                compute(ring[p], s0 + p);
    }

#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        partial[wave][nb][lane] = acc[nb];
    __syncthreads();

    for (int idx = threadIdx.x; idx < NB * kWave; idx += WAVES * kWave) {
        const int nb = idx / kWave, l = idx % kWave;
        float4_t sum = partial[0][nb][l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            sum += partial[w][nb][l];
        const int n = nbase + nb * 16 + l % 16;
        float *__restrict__ yout = a.y + (size_t)blockIdx.z * a.y_slice_stride;
        if (n < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * (l / 16) + r;
                if (m < M)
                    yout[(size_t)m * N + n] = sum[r];
            }
        }
    }
}

#ifndef QMM_MFMA_NB
#define QMM_MFMA_NB 4
#endif
#ifndef QMM_MFMA_WAVES
#define QMM_MFMA_WAVES 8
#endif

template <int BITS, int G>
hipError_t launch_mfma_t(const ProductArgs &a, hipStream_t stream)
{
    constexpr int NB = QMM_MFMA_NB, WAVES = QMM_MFMA_WAVES;
    static_assert(Geometry<BITS, G>::fits(), "lane chunk loads overrun the group");
    const int rows = 16 * NB;
    const dim3 grid((a.N + rows - 1) / rows, 1, a.split);
    hipLaunchKernelGGL((mfma_kernel<BITS, G, NB, WAVES>), grid, dim3(WAVES * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const ProductArgs &a, int bits, int G, hipStream_t stream)
{
#define QMM_MFMA_CASE(B, GG) \
    if (bits == B && G == GG) return launch_mfma_t<B, GG>(a, stream);
    QMM_MFMA_CASE(4, 32) QMM_MFMA_CASE(4, 64) QMM_MFMA_CASE(4, 128)
    QMM_MFMA_CASE(5, 32) QMM_MFMA_CASE(5, 64) QMM_MFMA_CASE(5, 128)
    QMM_MFMA_CASE(6, 32) QMM_MFMA_CASE(6, 64) QMM_MFMA_CASE(6, 128)
    QMM_MFMA_CASE(8, 32) QMM_MFMA_CASE(8, 64) QMM_MFMA_CASE(8, 128)
#undef QMM_MFMA_CASE
    return hipErrorInvalidValue;
}

}  // namespace qmm
