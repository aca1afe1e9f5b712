// One-row mat-vec (M = 1): y[n] = sum_g s[n,g] * (q[n,g,:] . x[g,:]) + b[n,g] * XS[g].
//
// The plain autoregressive decode step of the pages calls one quantized
// mat-vec per projection (vmlx-swift pull request #565 page, tiling-policy
// commit: below four rows the quantized mat-vec beats the lane matmul). At
// one row the weight stream is the whole cost, so the kernel is built around
// keeping many wide, coalesced loads of packed codes in flight:
//
//  * a workgroup of 4 waves owns 4*RPW output rows; each wave owns RPW rows;
//  * lane l of a wave takes groups l, l+64, ..., l+64*(SLOTS-1) of a row, so
//    every load instruction of a wave reads 64 consecutive groups, one
//    contiguous span of the row's stream (16-byte loads for 4-bit G = 32);
//  * the (row, slot) tasks of a wave form one fully unrolled sequence with a
//    ring of PD register stages: the loads of task t + PD are issued as soon
//    as task t is consumed, and the first PD tasks are issued before the
//    activations are staged, overlapping that latency;
//  * the activations of a K chunk are staged once per workgroup in LDS with
//    16-byte loads, permuted to the pair order of the code unpack, together
//    with their per-group sums XS;
//  * a group's codes are widened to exact fp16 pairs in registers and dotted
//    with v_dot2 (fp32 accumulation), then s*P + b*XS is added;
//  * each wave sums its lanes per row with DPP row rotations and readlanes.
#include "qmm_device.hpp"
#include "qmm_kernels.hpp"

namespace qmm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowsPerWave = 4;
constexpr int kMaxChunkK = 8192;  // activations staged per pass: at most 16 KB of fp16

// The 8 activations of an aligned 8-code run in the unpack's pair order.
template <int BITS>
__device__ __forceinline__ half8_t to_pair_order8(half8_t v)
{
    if constexpr (pair_dist(BITS) == 4)
        return __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
    else
        return __builtin_shufflevector(v, v, 0, 2, 1, 3, 4, 6, 5, 7);
}

template <int BITS, int G, int SLOTS, int RPW>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const ProductArgs a)
{
    constexpr int NWG = G * BITS / 32;        // words per group
    constexpr int NPAIR = G / 2;              // fp16 pairs per group
    constexpr int UPG = G / 8;                // 8-activation units per group
    constexpr int CHUNK_G = SLOTS * kWave;    // groups per staged chunk
    constexpr int ALIGN = gcd_int(4 * NWG, 16);
    constexpr int TASKS = RPW * SLOTS;
    constexpr int PD = TASKS < 2 * SLOTS ? TASKS : 2 * SLOTS;  // tasks in flight
    static_assert(CHUNK_G * G <= kMaxChunkK, "staged chunk too large");

    __shared__ half8_t xp[CHUNK_G * UPG];
    __shared__ float xsum[CHUNK_G];

    const int K = a.K, N = a.N, Kg = K / G;
    const size_t wpr = (size_t)K * BITS / 32;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int row0 = (blockIdx.x * kWaves + wave) * RPW;

    int gbeg = 0, gend = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, gbeg, gend);
    float *__restrict__ yout = a.y + (size_t)blockIdx.z * a.y_slice_stride;

    // Row of each task (clamped so loads stay in bounds; results of rows >= N are dropped).
    size_t rowoff[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
        rowoff[r] = (size_t)min(row0 + r, N - 1);

    float acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
        acc[r] = 0.f;

    // Scale and bias stay raw 16-bit values until they are used, so nothing
    // consumes a load right after it is issued.
    struct Stage {
        uint32_t w[NWG];
        uint16_t s, b;
    };
    Stage ring[PD];

    for (int g0 = gbeg; g0 < gend; g0 += CHUNK_G) {
        const int ng = min(CHUNK_G, gend - g0);

        // Every load is unconditional (lanes past the chunk re-read its last
        // group), so the compiler can keep the ring of stages in flight.
        auto load = [&](Stage &st, int task) {
            const int r = task / SLOTS, sl = task % SLOTS;
            const int g = g0 + min(lane + sl * kWave, ng - 1);
            load_words<NWG, ALIGN>(a.wq + rowoff[r] * wpr + (size_t)g * NWG, st.w);
            const size_t sidx = rowoff[r] * Kg + g;
            st.s = a.scales[sidx];
            st.b = a.biases[sidx];
        };

#pragma unroll
        for (int t = 0; t < PD; ++t)
            load(ring[t], t);

        __syncthreads();  // all waves are done reading the previous chunk
        for (int u = threadIdx.x; u < ng * UPG; u += kThreads) {
            const half8_t v = *reinterpret_cast<const half8_t *>(a.x + (size_t)g0 * G + 8 * u);
            xp[u] = to_pair_order8<BITS>(v);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s += (float)v[e];
#pragma unroll
            for (int off = 1; off < UPG; off *= 2)
                s += __shfl_xor(s, off);
            if (u % UPG == 0)
                xsum[u / UPG] = s;
        }
        __syncthreads();

#pragma unroll
        for (int t = 0; t < TASKS; ++t) {
            const int r = t / SLOTS, sl = t % SLOTS;
            Stage &st = ring[t % PD];
            if (sl * kWave < ng) {
                const int gl = lane + sl * kWave;
                const int glc = min(gl, ng - 1);
                half2_t q[NPAIR];
                unpack_pairs<BITS, G>(st.w, q);
                float P = 0.f;
#pragma unroll
                for (int u = 0; u < UPG; ++u) {
                    const half8_t xv = xp[glc * UPG + u];
                    P = __builtin_amdgcn_fdot2(q[4 * u + 0], half2_t{xv[0], xv[1]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 1], half2_t{xv[2], xv[3]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 2], half2_t{xv[4], xv[5]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 3], half2_t{xv[6], xv[7]}, P, false);
                }
                const float contrib = half_bits_to_float(st.s) * P + half_bits_to_float(st.b) * xsum[glc];
                acc[r] += gl < ng ? contrib : 0.f;
            }
            if (t + PD < TASKS)
                load(ring[t % PD], t + PD);
        }
    }

#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == 0 && row0 + r < N)
            yout[row0 + r] = v;
    }
}

template <int BITS, int G, int SLOTS>
hipError_t launch_qmv_slots(const ProductArgs &a, hipStream_t stream)
{
    constexpr int RPW = kRowsPerWave;
    const int rows_per_block = kWaves * RPW;
    const dim3 grid((a.N + rows_per_block - 1) / rows_per_block, 1, a.split);
    hipLaunchKernelGGL((qmv_kernel<BITS, G, SLOTS, RPW>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// Slots per lane: enough to cover the K range (or slice) in one staged chunk
// when it fits, capped by the chunk's LDS size.
template <int BITS, int G>
hipError_t launch_qmv_t(const ProductArgs &a, hipStream_t stream)
{
    constexpr int max_slots = kMaxChunkK / (kWave * G);
    const int Kg = a.K / G;
    const int slice = a.split > 1 ? (Kg + a.split - 1) / a.split : Kg;
    int slots = (slice + kWave - 1) / kWave;
    slots = slots < 1 ? 1 : (slots > max_slots ? max_slots : slots);
    if constexpr (max_slots >= 4)
        if (slots == 4) return launch_qmv_slots<BITS, G, 4>(a, stream);
    if constexpr (max_slots >= 3)
        if (slots == 3) return launch_qmv_slots<BITS, G, 3>(a, stream);
    if constexpr (max_slots >= 2)
        if (slots == 2) return launch_qmv_slots<BITS, G, 2>(a, stream);
    return launch_qmv_slots<BITS, G, 1>(a, stream);
}

}  // namespace

hipError_t launch_qmv(const ProductArgs &a, int bits, int G, hipStream_t stream)
{
#define QMM_QMV_CASE(B, GG) \
    if (bits == B && G == GG) return launch_qmv_t<B, GG>(a, stream);
    QMM_QMV_CASE(4, 32) QMM_QMV_CASE(4, 64) QMM_QMV_CASE(4, 128)
    QMM_QMV_CASE(5, 32) QMM_QMV_CASE(5, 64) QMM_QMV_CASE(5, 128)
    QMM_QMV_CASE(6, 32) QMM_QMV_CASE(6, 64) QMM_QMV_CASE(6, 128)
    QMM_QMV_CASE(8, 32) QMM_QMV_CASE(8, 64) QMM_QMV_CASE(8, 128)
#undef QMM_QMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace qmm
