// One-row mat-vec (M = 1): y[n] = sum_g s[n,g] * (q[n,g,:] . x[g,:]) + b[n,g] * XS[g].
//
// The plain autoregressive decode step of the pages calls one quantized
// mat-vec per projection (vmlx-swift pull request #565 page, tiling-policy
// commit: below four rows the quantized mat-vec beats the lane matmul). At
// one row the weight stream is the whole cost, so the kernel is built around
// keeping many wide, coalesced loads of packed codes in flight:
//
//  * a workgroup of 4 waves owns 4*RPW output rows; each wave owns RPW rows;
//  * LPR lanes (64 or 32) share a row: lane l takes row l / LPR of a row
//    group and groups l % LPR + LPR*s (s < SLOTS) of that row, so every load
//    instruction of a wave reads 64/LPR rows of LPR consecutive groups, whole
//    contiguous spans of the rows' streams (16-byte loads for 4-bit G = 32).
//    LPR = 32 covers group counts that are odd multiples of 32 without idle
//    lanes (160 groups: 5 slots of 32 instead of 3 slots of 64);
//  * the (row, slot) tasks of a wave form one fully unrolled sequence with a
//    ring of PD register stages: the loads of task t + PD are issued as soon
//    as task t is consumed, and the first PD tasks are issued before the
//    activations are staged, overlapping that latency;
//  * the activations of a K chunk are staged once per workgroup in LDS with
//    16-byte loads, permuted to the pair order of the code unpack, together
//    with their per-group sums XS, and so are the scales and biases of the
//    workgroup's rows (16-byte loads, one (scale, bias) pair per LDS word);
//    these loads are issued before the weight prefetch so that they head the
//    memory queue;
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
constexpr int kPrefetchRows = 1;  // rows of loads kept in flight per wave
constexpr int kMaxChunkK = 8192;  // activations staged per pass: at most 16 KB of fp16

template <int BITS, int G, int LPR, int SLOTS, int RPW, int PD_ROWS>
__global__ __launch_bounds__(kThreads) void qmv_kernel(const ProductArgs a)
{
    constexpr int NWG = G * BITS / 32;        // words per group
    constexpr int NPAIR = G / 2;              // fp16 pairs per group
    constexpr int UPG = G / 8;                // 8-activation units per group
    constexpr int RPI = kWave / LPR;          // rows per load instruction
    constexpr int RG = RPW / RPI;             // row groups per wave
    constexpr int CHUNK_G = SLOTS * LPR;      // groups per staged chunk
    constexpr int ALIGN = gcd_int(4 * NWG, 16);
    constexpr int TASKS = RG * SLOTS;
    constexpr int PD = TASKS < PD_ROWS * SLOTS ? TASKS : PD_ROWS * SLOTS;  // tasks in flight
    static_assert(RPW % RPI == 0, "a wave's rows come in whole row groups");
    constexpr int ROWS = kWaves * RPW;        // rows of the workgroup
    constexpr int XUNITS = CHUNK_G * UPG;                           // activation units per chunk
    constexpr int XPT = (XUNITS + kThreads - 1) / kThreads;         // ... per thread
    constexpr int SBU = ROWS * CHUNK_G / 8;                         // 8-group scale units per chunk
    constexpr int SPT = (SBU + kThreads - 1) / kThreads;            // ... per thread
    static_assert(CHUNK_G * G <= kMaxChunkK, "staged chunk too large");
    static_assert(CHUNK_G % 8 == 0, "chunks hold whole 8-group scale units");

    // Activations unit-major: xp[u][g] holds units u of group g, so the
    // 64 lanes of a wave (consecutive groups) read consecutive 16-byte units.
    __shared__ half8_t xp[UPG][CHUNK_G];
    __shared__ float xsum[CHUNK_G];
    __shared__ uint32_t sbl[ROWS][CHUNK_G];   // (scale, bias) fp16 pair per row and group

    const int K = a.K, N = a.N, Kg = K / G;
    const size_t wpr = (size_t)K * BITS / 32;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rho = lane / LPR, lam = lane % LPR;  // row within a row group, lane within the row
    const int wg_row0 = blockIdx.x * ROWS;
    const int row0 = wg_row0 + wave * RPW;

    int gbeg = 0, gend = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, gbeg, gend);
    float *__restrict__ yout = a.y + (size_t)blockIdx.z * a.y_slice_stride;
    // 16-byte scale/bias staging needs 8-group alignment of every row span
    const bool sb_vector = Kg % 8 == 0 && gbeg % 8 == 0 && gend % 8 == 0;

    // Rows of each row group: a wave-uniform base row and this lane's row
    // offset from it (clamped so loads stay in bounds; results of rows >= N
    // are dropped).
    size_t rowbase[RG];
    uint32_t rowlane[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int b = min(row0 + r * RPI, N - 1);
        rowbase[r] = (size_t)b;
        rowlane[r] = (uint32_t)(min(row0 + r * RPI + rho, N - 1) - b) * (uint32_t)(wpr * 4);
    }

    float acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r)
        acc[r] = 0.f;

    struct Stage {
        uint32_t w[NWG];
    };
    Stage ring[PD];

    for (int g0 = gbeg; g0 < gend; g0 += CHUNK_G) {
        const int ng = min(CHUNK_G, gend - g0);

        // 1. Activation and scale/bias loads first: they head the memory
        //    queue, so the workgroup can start computing as early as possible.
        half8_t xreg[XPT];
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int u = min((int)threadIdx.x + t * kThreads, ng * UPG - 1);
            xreg[t] = *reinterpret_cast<const half8_t *>(a.x + (size_t)g0 * G + 8 * u);
        }
        u32x4 sreg[SPT], breg[SPT];
        if (sb_vector) {
            // unit v: row v / (CHUNK_G/8), groups 8*(v % (CHUNK_G/8)) .. +8 of the chunk
#pragma unroll
            for (int t = 0; t < SPT; ++t) {
                const int v = min((int)threadIdx.x + t * kThreads, SBU - 1);
                const int r = v / (CHUNK_G / 8);
                const int gu = min(8 * (v % (CHUNK_G / 8)), ng - 8);
                const size_t off = (size_t)min(wg_row0 + r, N - 1) * Kg + g0 + gu;
                sreg[t] = *reinterpret_cast<const u32x4 *>(a.scales + off);
                breg[t] = *reinterpret_cast<const u32x4 *>(a.biases + off);
            }
        }

        // 2. Group of slot sl for this lane, relative to the chunk (lanes past
        //    the chunk re-read its last group), and the weight prefetch ring.
        //    Every weight load is unconditional, so the compiler can keep the
        //    ring in flight; addresses are a wave-uniform row base plus a
        //    32-bit lane offset.
        int lgroup[SLOTS];
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl)
            lgroup[sl] = min(lam + sl * LPR, ng - 1);
        auto load = [&](Stage &st, int task) {
            const int r = task / SLOTS, sl = task % SLOTS;
            const uint32_t *wbase = a.wq + rowbase[r] * wpr + (size_t)g0 * NWG;
            load_words<NWG, ALIGN>(byte_offset(wbase, rowlane[r] + (uint32_t)(lgroup[sl] * NWG * 4)), st.w);
        };
#pragma unroll
        for (int t = 0; t < PD; ++t)
            load(ring[t], t);

        // 3. Stage the chunk in LDS: activations in the unpack's pair order
        //    with their group sums, and one (scale, bias) pair per row and group.
        __syncthreads();  // all waves are done reading the previous chunk
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int u = (int)threadIdx.x + t * kThreads;
            const half8_t v = xreg[t];
            float s8 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                s8 += (float)v[e];
#pragma unroll
            for (int off = 1; off < UPG; off *= 2)
                s8 += __shfl_xor(s8, off);
            if (u < ng * UPG) {
                xp[u % UPG][u / UPG] = to_pair_order<BITS>(v);
                if (u % UPG == 0)
                    xsum[u / UPG] = s8;
            }
        }
        if (sb_vector) {
#pragma unroll
            for (int t = 0; t < SPT; ++t) {
                const int v = (int)threadIdx.x + t * kThreads;
                const int r = v / (CHUNK_G / 8);
                const int gu = 8 * (v % (CHUNK_G / 8));
                if (v < SBU && gu < ng) {
                    const u32x4 sv = sreg[t], bv = breg[t];
                    uint32_t *dst = &sbl[r][gu];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dst[2 * e] = __builtin_amdgcn_perm(bv[e], sv[e], 0x05040100u);      // (s_lo, b_lo)
                        dst[2 * e + 1] = __builtin_amdgcn_perm(bv[e], sv[e], 0x07060302u);  // (s_hi, b_hi)
                    }
                }
            }
        } else {
            for (int v = threadIdx.x; v < ROWS * ng; v += kThreads) {
                const int r = v / ng, gl = v % ng;
                const size_t off = (size_t)min(wg_row0 + r, N - 1) * Kg + g0 + gl;
                sbl[r][gl] = (uint32_t)a.scales[off] | ((uint32_t)a.biases[off] << 16);
            }
        }
        __syncthreads();

        // 4. The (row, slot) tasks in program order, refilling the ring.
#pragma unroll
        for (int t = 0; t < TASKS; ++t) {
            // keep tasks in program order (no hoisting of later tasks' work,
            // which would force early waits on their loads)
            __builtin_amdgcn_sched_barrier(0);
            const int r = t / SLOTS, sl = t % SLOTS;
            Stage &st = ring[t % PD];
#pragma unroll
            for (int j = 0; j < NWG; ++j)
                pin_register(st.w[j]);
            if (sl * LPR < ng) {
                const int gl = lam + sl * LPR;
                const int glc = min(gl, ng - 1);
                half2_t q[NPAIR];
                unpack_pairs<BITS, G>(st.w, q);
                float P = 0.f;
#pragma unroll
                for (int u = 0; u < UPG; ++u) {
                    const half8_t xv = xp[u][glc];
                    P = __builtin_amdgcn_fdot2(q[4 * u + 0], half2_t{xv[0], xv[1]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 1], half2_t{xv[2], xv[3]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 2], half2_t{xv[4], xv[5]}, P, false);
                    P = __builtin_amdgcn_fdot2(q[4 * u + 3], half2_t{xv[6], xv[7]}, P, false);
                }
                const uint32_t sb = sbl[wave * RPW + r * RPI + rho][glc];
                const float sc = half_bits_to_float((uint16_t)(sb & 0xffffu));
                const float bias = half_bits_to_float((uint16_t)(sb >> 16)) - CodeOffset<BITS>::value * sc;
                const float contrib = sc * P + bias * xsum[glc];
                acc[r] += gl < ng ? contrib : 0.f;
            }
            if (t + PD < TASKS)
                load(ring[t % PD], t + PD);
        }
    }

    // Row sums: a DPP sum inside each 16-lane row, then the 16-lane rows of
    // each of the RPI rows of a row group are added in order.
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int v = __builtin_bit_cast(int, row16_sum(acc[r]));
        float part[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            part[q] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(v, 16 * q));
#pragma unroll
        for (int p = 0; p < RPI; ++p) {
            constexpr int QPR = LPR / 16;  // 16-lane rows per output row
            float sum = part[p * QPR];
#pragma unroll
            for (int q = 1; q < QPR; ++q)
                sum += part[p * QPR + q];
            const int row = row0 + r * RPI + p;
            if (lane == 0 && row < N)
                yout[row] = sum;
        }
    }
}

template <int BITS, int G, int LPR, int SLOTS, int RPW = kRowsPerWave, int PD_ROWS = kPrefetchRows>
hipError_t launch_qmv_slots(const ProductArgs &a, hipStream_t stream)
{
    const int rows_per_block = kWaves * RPW;
    const dim3 grid((a.N + rows_per_block - 1) / rows_per_block, 1, a.split);
    hipLaunchKernelGGL((qmv_kernel<BITS, G, LPR, SLOTS, RPW, PD_ROWS>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// Lanes per row and slots per lane: enough slots to cover the K range (or
// slice) in one staged chunk when it fits, capped by the chunk's LDS size.
// With 32 lanes per row a wave's rows form two row groups, both kept in
// flight (measured: 12.7 us against 13.8 us with one in flight on the
// 5120 x 17408 4-bit projection).
// 32 lanes per row take group counts that leave more than half of a 64-lane
// slot idle (an odd number of 32-group slots covers them exactly); even
// numbers of 32-group slots are the 64-lane kernel.
template <int BITS, int G>
hipError_t launch_qmv_t(const ProductArgs &a, hipStream_t stream)
{
    constexpr int max_slots = kMaxChunkK / (kWave * G);
    const int Kg = a.K / G;
    const int slice = a.split > 1 ? (Kg + a.split - 1) / a.split : Kg;
    int slots = (slice + kWave - 1) / kWave;
    slots = slots < 1 ? 1 : (slots > max_slots ? max_slots : slots);
    const int half = (slice + 31) / 32;  // 32-group slots covering the slice
    if (slice <= max_slots * kWave && half % 2 == 1) {
        if (half == 1) return launch_qmv_slots<BITS, G, 32, 1, kRowsPerWave, 2>(a, stream);
        if constexpr (2 * max_slots >= 3)
            if (half == 3) return launch_qmv_slots<BITS, G, 32, 3, kRowsPerWave, 2>(a, stream);
        if constexpr (2 * max_slots >= 5)
            if (half == 5) return launch_qmv_slots<BITS, G, 32, 5, kRowsPerWave, 2>(a, stream);
        if constexpr (2 * max_slots >= 7)
            if (half == 7) return launch_qmv_slots<BITS, G, 32, 7, kRowsPerWave, 2>(a, stream);
    }
    if constexpr (max_slots >= 4)
        if (slots == 4) return launch_qmv_slots<BITS, G, 64, 4>(a, stream);
    if constexpr (max_slots >= 3)
        if (slots == 3) return launch_qmv_slots<BITS, G, 64, 3>(a, stream);
    if constexpr (max_slots >= 2)
        if (slots == 2) return launch_qmv_slots<BITS, G, 64, 2>(a, stream);
    return launch_qmv_slots<BITS, G, 64, 1>(a, stream);
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
