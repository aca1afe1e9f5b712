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
constexpr int kMaxChunkK = 8192;  // activations staged per pass: at most 16 KB of fp16 ...
constexpr int chunk_limit(int mr) { return mr == 1 ? kMaxChunkK : 2 * kMaxChunkK; }  // ... 32 KB for several rows

// MR: activation rows per launch (M <= MR). Every row runs exactly the
// arithmetic of the one-row launch (same lane-to-group map, same dot and
// epilogue sequence, same reduction tree), so with the same LPR each row of
// an MR-row result is bitwise equal to that row computed alone.
// BF16: x, scales and biases hold bf16 bit patterns (codes widened to bf16
// and dotted with v_dot2_f32_bf16) instead of fp16.
// WS: coalesced weight loads for groups wider than 16 bytes. A lane that
// loads its own group's bytes reads 16-byte pieces at the group stride, and
// such loads stream at about half the rate of contiguous ones (measured on
// the 5120 x 5120 8-bit G = 64 matrix with this kernel's grid: 9.5 against
// 5.3 us). With WS the lanes of a row load consecutive 16-byte pieces of the
// slot's span, write them to the wave's LDS region and read back their own
// group's words: the same words reach the same lane, so the results keep
// their bits. Needs 16-byte aligned rows and one K slice (the host checks).
template <int BITS, int G, int LPR, int SLOTS, int RPW, int PD_ROWS, int MR, bool BF16, bool WS = false>
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
    constexpr int XUNITS = CHUNK_G * UPG;                           // activation units per row and chunk
    constexpr int XPT = (MR * XUNITS + kThreads - 1) / kThreads;    // ... of all rows, per thread
    constexpr int SBU = ROWS * CHUNK_G / 8;                         // 8-group scale units per chunk
    constexpr int SPT = (SBU + kThreads - 1) / kThreads;            // ... per thread
    static_assert(MR * CHUNK_G * G <= chunk_limit(MR), "staged chunk too large");
    static_assert(CHUNK_G % 8 == 0, "chunks hold whole 8-group scale units");
    // WS geometry: 16-byte pieces per lane and task; a row's region holds the
    // slot's LPR groups, each padded to an odd number of 16-byte units when
    // whole units hold a group (so that lanes reading their groups spread over
    // the LDS banks)
    constexpr int GBY = 4 * NWG;                                   // bytes per group
    constexpr int NPC = (GBY + 15) / 16;
    constexpr int GU = GBY % 16 == 0 ? GBY / 16 : 0;               // whole units per group
    constexpr int GSTRIDE = GU ? 16 * (GU | 1) : GBY;              // region bytes per group
    constexpr int RUNITS = GU ? LPR * (GU | 1) : LPR * NPC;        // region units per row
    constexpr int RALIGN = gcd_int(GSTRIDE, 16);                   // alignment of a group in the region
    static_assert(!WS || GBY > 16, "coalesced loads are for groups wider than 16 bytes");

    // Activations unit-major: xp[m][u][g] holds unit u of group g of row m,
    // so the lanes of a row (consecutive groups) read consecutive 16-byte units.
    __shared__ half8_t xp[MR][UPG][CHUNK_G];
    __shared__ float xsum[MR][CHUNK_G];
    __shared__ uint32_t sbl[ROWS][CHUNK_G];   // (scale, bias) fp16 pair per row and group
    __shared__ u32x4 wst[WS ? kWaves * RPI * RUNITS : 1];  // WS: per wave, RPI rows of a slot's pieces

    static_assert(16 % ROWS == 0, "a workgroup owns a whole part of one 16-row tile");
    constexpr int TPW = 16 / ROWS;                     // workgroups per 16-row tile
    const Slab slab = slab_of_tile(a, blockIdx.x / TPW);  // the projection of this workgroup's tile
    const int K = a.K, N = slab.p.N, Kg = K / G;
    const size_t wpr = (size_t)K * BITS / 32;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rho = lane / LPR, lam = lane % LPR;  // row within a row group, lane within the row
    const int wg_row0 = slab.tile * 16 + (int)(blockIdx.x % TPW) * ROWS;
    const int row0 = wg_row0 + wave * RPW;

    int gbeg = 0, gend = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, gbeg, gend);
    float *__restrict__ yout = slab.p.y + (size_t)blockIdx.z * a.y_slice_stride;
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

    float acc[MR][RG];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < RG; ++r)
            acc[m][r] = 0.f;

    struct Stage {
        uint32_t w[WS ? 4 * NPC : NWG];
    };
    Stage ring[PD];

    for (int g0 = gbeg; g0 < gend; g0 += CHUNK_G) {
        const int ng = min(CHUNK_G, gend - g0);

        // 1. Activation and scale/bias loads first: they head the memory
        //    queue, so the workgroup can start computing as early as possible.
        // unit v: row v / XUNITS (rows past M re-read row M-1), unit v % XUNITS
        half8_t xreg[XPT];
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int v = min((int)threadIdx.x + t * kThreads, MR * XUNITS - 1);
            const int m = min(v / XUNITS, a.M - 1);
            const int u = min(v % XUNITS, ng * UPG - 1);
            xreg[t] = *reinterpret_cast<const half8_t *>(a.x + (size_t)m * K + (size_t)g0 * G + 8 * u);
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
                sreg[t] = *reinterpret_cast<const u32x4 *>(slab.p.scales + off);
                breg[t] = *reinterpret_cast<const u32x4 *>(slab.p.biases + off);
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
            const uint32_t *wbase = slab.p.wq + rowbase[r] * wpr + (size_t)g0 * NWG;
            if constexpr (WS) {
                // piece lam + LPR j of the slot's span, clamped to the chunk's last 16 bytes
                const uint32_t last = (uint32_t)(ng * GBY - 16);
#pragma unroll
                for (int j = 0; j < NPC; ++j) {
                    const uint32_t off = min((uint32_t)(sl * LPR * GBY + 16 * (lam + LPR * j)), last);
                    const u32x4 v = load_weight(reinterpret_cast<const u32x4 *>(
                        byte_offset(wbase, rowlane[r] + off)));
                    st.w[4 * j + 0] = v.x; st.w[4 * j + 1] = v.y; st.w[4 * j + 2] = v.z; st.w[4 * j + 3] = v.w;
                }
            } else {
                load_words<NWG, ALIGN>(byte_offset(wbase, rowlane[r] + (uint32_t)(lgroup[sl] * NWG * 4)), st.w);
            }
        };
#pragma unroll
        for (int t = 0; t < PD; ++t)
            load(ring[t], t);

        // 3. Stage the chunk in LDS: activations in the unpack's pair order
        //    with their group sums, and one (scale, bias) pair per row and group.
        __syncthreads();  // all waves are done reading the previous chunk
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int vv = (int)threadIdx.x + t * kThreads;
            const int m = vv / XUNITS, u = vv % XUNITS;
            const half8_t v = xreg[t];
            // sum of the unit's 8 activations (fp32 accumulation of pairs)
            float s8 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (BF16) {
                    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
                    s8 = __builtin_amdgcn_fdot2_f32_bf16(
                        __builtin_bit_cast(bf16x2_t, half2_t{v[2 * e], v[2 * e + 1]}), ones, s8, false);
                } else {
                    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
                    s8 = __builtin_amdgcn_fdot2(half2_t{v[2 * e], v[2 * e + 1]}, ones, s8, false);
                }
            }
            // the UPG units of a group sit in consecutive lanes
#pragma unroll
            for (int off = 1; off < UPG; off *= 2)
                s8 += __shfl_xor(s8, off);
            if (m < MR && u < ng * UPG) {
                xp[m][u % UPG][u / UPG] = BF16 ? to_pair_order_bf16<BITS>(v) : to_pair_order<BITS>(v);
                if (u % UPG == 0)
                    xsum[m][u / UPG] = s8;
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
                sbl[r][gl] = (uint32_t)slab.p.scales[off] | ((uint32_t)slab.p.biases[off] << 16);
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
            for (int j = 0; j < (WS ? 4 * NPC : NWG); ++j)
                pin_register(st.w[j]);
            uint32_t gw[NWG];  // this lane's group words
            if constexpr (WS) {
                // pieces to the wave's region, then this lane's group back
                uint8_t *region = reinterpret_cast<uint8_t *>(wst + (size_t)(wave * RPI + rho) * RUNITS);
                wave_lds_sync();  // the previous task's reads of the region are done
#pragma unroll
                for (int j = 0; j < NPC; ++j) {
                    const int q = lam + LPR * j;  // logical 16-byte piece of the span
                    const int phys = GU ? q + (q / GU) * ((GU | 1) - GU) : q;
                    *reinterpret_cast<u32x4 *>(region + 16 * phys) =
                        u32x4{st.w[4 * j], st.w[4 * j + 1], st.w[4 * j + 2], st.w[4 * j + 3]};
                }
                wave_lds_sync();  // other lanes' pieces are read below
                const int gi = min(lam + sl * LPR, ng - 1) - sl * LPR;  // group within the slot (clamped)
                const uint8_t *src = region + (size_t)max(gi, 0) * GSTRIDE;
                if constexpr (RALIGN >= 16 && NWG % 4 == 0) {
#pragma unroll
                    for (int k = 0; k < NWG / 4; ++k) {
                        const u32x4 v = reinterpret_cast<const u32x4 *>(src)[k];
                        gw[4 * k] = v.x; gw[4 * k + 1] = v.y; gw[4 * k + 2] = v.z; gw[4 * k + 3] = v.w;
                    }
                } else if constexpr (RALIGN >= 8 && NWG % 2 == 0) {
#pragma unroll
                    for (int k = 0; k < NWG / 2; ++k) {
                        const u32x2 v = reinterpret_cast<const u32x2 *>(src)[k];
                        gw[2 * k] = v.x; gw[2 * k + 1] = v.y;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < NWG; ++k)
                        gw[k] = reinterpret_cast<const uint32_t *>(src)[k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < NWG; ++k)
                    gw[k] = st.w[k];
            }
            if (sl * LPR < ng) {
                const int gl = lam + sl * LPR;
                const int glc = min(gl, ng - 1);
                const uint32_t sb = sbl[wave * RPW + r * RPI + rho][glc];
                // codes are widened to exact fp16 (or bf16) integers: v_dot2
                // loses precision on subnormal operands (see code_pair4_int)
                float sc, bias;
                if constexpr (BF16) {
                    sc = bf16_bits_to_float(sb & 0xffffu);
                    bias = bf16_bits_to_float(sb >> 16);
                } else {
                    sc = half_bits_to_float((uint16_t)(sb & 0xffffu));
                    bias = half_bits_to_float((uint16_t)(sb >> 16));
                }
                constexpr bool kTwoChains = !BF16 && BITS == 4;
                half2_t q[NPAIR];
                bf16x2_t qb[NPAIR];
                if constexpr (BF16)
                    unpack_pairs_bf16<BITS, G>(gw, qb);
                else if constexpr (BITS == 4)
                    unpack_pairs4_int<G>(gw, q);
                else
                    unpack_pairs<BITS, G>(gw, q);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    // two accumulators for 4-bit codes (even and odd pairs, two
                    // independent v_dot2 chains), added below
                    float Pa = 0.f, Pb = 0.f;
#pragma unroll
                    for (int u = 0; u < UPG; ++u) {
                        const half8_t xv = xp[m][u][glc];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const half2_t xe = {xv[2 * e], xv[2 * e + 1]};
                            if constexpr (BF16)
                                Pa = __builtin_amdgcn_fdot2_f32_bf16(qb[4 * u + e], __builtin_bit_cast(bf16x2_t, xe),
                                                                     Pa, false);
                            else if (kTwoChains && e % 2 == 1)
                                Pb = __builtin_amdgcn_fdot2(q[4 * u + e], xe, Pb, false);
                            else
                                Pa = __builtin_amdgcn_fdot2(q[4 * u + e], xe, Pa, false);
                        }
                    }
                    const float P = kTwoChains ? Pa + Pb : Pa;
                    // explicit fma: the same rounding in every instantiation
                    const float contrib = __builtin_fmaf(sc, P, bias * xsum[m][glc]);
                    acc[m][r] += gl < ng ? contrib : 0.f;
                }
            }
            if (t + PD < TASKS)
                load(ring[t % PD], t + PD);
        }
    }

    // Row sums: a DPP sum inside each 16-lane row, then the 16-lane rows of
    // each of the RPI rows of a row group are added in order.
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int v = __builtin_bit_cast(int, row16_sum(acc[m][r]));
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
                if (lane == 0 && row < N && m < a.M)
                    yout[(size_t)m * N + row] = sum;
            }
        }
    }
}

template <int BITS, int G, int LPR, int SLOTS, int RPW, int PD_ROWS, int MR, bool BF16>
hipError_t launch_qmv_slots(const ProductArgs &a, hipStream_t stream)
{
    const int rows_per_block = kWaves * RPW;
    const dim3 grid((a.N + rows_per_block - 1) / rows_per_block, 1, a.split);
    // Coalesced loads of wide groups (40 bytes and more): one-row fp16 launches
    // on 16-byte rows with few workgroups. Measured against the per-lane group
    // loads (us, 5120 x 5120 at M = 1): 8-bit G64 9.5 vs 12.4, 6-bit G64 8.5 vs
    // 9.2, 5-bit G64 8.4 vs 8.9, 8-bit G64 on 5120 x 1024 5.2 vs 6.0; with
    // groups of 20 to 32 bytes, or on the 5120 x 17408 projection (2176
    // workgroups), the staging costs about what it saves or more (5-bit G32
    // 8.2 vs 7.6, 4-bit G64 7.4 vs 7.1, 8-bit G32 on 5120 x 17408 22.0 vs 21.5).
    constexpr bool kWide = G * BITS / 8 >= 40 && MR == 1 && !BF16;
    if constexpr (kWide) {
        const long long wgs = (a.N + rows_per_block - 1) / rows_per_block;
        if (a.split == 1 && ((long long)a.K * BITS) % 128 == 0 && wgs <= 4LL * device_cu_count()) {
            hipLaunchKernelGGL((qmv_kernel<BITS, G, LPR, SLOTS, RPW, PD_ROWS, MR, BF16, true>), grid, dim3(kThreads), 0,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((qmv_kernel<BITS, G, LPR, SLOTS, RPW, PD_ROWS, MR, BF16>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// Lanes per row: 32 for group counts that leave more than half of a 64-lane
// slot idle (an odd number of 32-group slots covers them exactly), else 64.
// The choice depends on the K range only, so every row count takes the same
// lane map as the one-row launch. Slots per lane: enough to cover the range
// in one staged chunk when the chunk of all MR rows fits (chunk_limit(MR)
// activations), else as many as fit.
template <int BITS, int G>
int qmv_lanes_per_row(int slice)
{
    constexpr int max_slots1 = kMaxChunkK / (kWave * G);
    const int half = (slice + 31) / 32;
    return slice <= max_slots1 * kWave && half % 2 == 1 ? 32 : 64;
}

// Rows per wave: one row group (RPI rows: two with 32 lanes per row, one
// with 64) for the one- and two-row launches, four otherwise. The
// narrow form has two or four times more waves, each with a shorter chain
// of tasks: 12.0-12.7 us against 12.7-13.1 us on the 5120 x 17408 4-bit
// projection at M = 1, 9.4 against 11.2 us on a 5120 x 5120 5-bit one (320
// tiles: 1.25 waves per SIMD in the wide form). A row's arithmetic depends
// on the lane map only, so both forms give the same bits.
template <int BITS, int G, int LPR, int MR, int S, bool BF16>
hipError_t launch_qmv_upto(const ProductArgs &a, int slots, hipStream_t stream)
{
    // PD: with 32 lanes per row both row groups of a wave stay in flight
    // (measured: 12.7 us against 13.8 us with one on the 5120 x 17408 4-bit
    // projection at M = 1).
    // Two-row launches with 32 lanes per row take two row groups per wave,
    // one in flight at a time (half the workgroups, the same registers):
    // 15.9-16.4 us against 16.5-17.5 us on the 5120 x 17408 4-bit projection
    // (the one-row launch is faster with one row group per wave).
    constexpr bool kTwoGroups = MR == 2 && LPR == 32;
    constexpr int PDR = kTwoGroups ? 1 : LPR == 32 ? 2 : kPrefetchRows;
    constexpr int RPW = kTwoGroups ? 4 : MR <= 2 ? kWave / LPR : kRowsPerWave;
    if constexpr (S > 1) {
        if (slots < S)
            return launch_qmv_upto<BITS, G, LPR, MR, S - 1, BF16>(a, slots, stream);
    }
    return launch_qmv_slots<BITS, G, LPR, S, RPW, PDR, MR, BF16>(a, stream);
}

template <int BITS, int G, int MR, bool BF16>
hipError_t launch_qmv_rows(const ProductArgs &a, hipStream_t stream)
{
    const int Kg = a.K / G;
    const int slice = a.split > 1 ? (Kg + a.split - 1) / a.split : Kg;
    const int lpr = qmv_lanes_per_row<BITS, G>(slice);
    const int need = (slice + lpr - 1) / lpr;
    if (lpr == 32) {
        constexpr int max_s = chunk_limit(MR) / (MR * 32 * G);
        if constexpr (max_s >= 1)
            return launch_qmv_upto<BITS, G, 32, MR, (max_s < 8 ? max_s : 8), BF16>(a, need, stream);
    } else {
        constexpr int max_s = chunk_limit(MR) / (MR * 64 * G);
        if constexpr (max_s >= 1)
            return launch_qmv_upto<BITS, G, 64, MR, (max_s < 4 ? max_s : 4), BF16>(a, need, stream);
    }
    return hipErrorInvalidValue;
}

// Rows per launch that fit a one-slot chunk with this lane map.
template <int BITS, int G>
int qmv_max_rows(int lpr)
{
    int mr = 8;
    while (mr > 1 && chunk_limit(mr) / (mr * lpr * G) < 1)
        mr /= 2;
    return mr;
}

// Up to 8 rows (a.M <= 8), in as few launches as the chunk size allows.
template <int BITS, int G, bool BF16>
hipError_t launch_qmv_t(const ProductArgs &a, hipStream_t stream)
{
    const int Kg = a.K / G;
    const int slice = a.split > 1 ? (Kg + a.split - 1) / a.split : Kg;
    const int cap = qmv_max_rows<BITS, G>(qmv_lanes_per_row<BITS, G>(slice));
    for (int m0 = 0; m0 < a.M; m0 += cap) {
        const ProductArgs b = rows_of(a, m0, a.M - m0 < cap ? a.M - m0 : cap);
        hipError_t e;
        if (b.M <= 1) e = launch_qmv_rows<BITS, G, 1, BF16>(b, stream);
        else if (b.M <= 2) e = launch_qmv_rows<BITS, G, 2, BF16>(b, stream);
        else if (b.M <= 4) e = launch_qmv_rows<BITS, G, 4, BF16>(b, stream);
        else e = launch_qmv_rows<BITS, G, 8, BF16>(b, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_qmv(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream)
{
#define QMM_QMV_CASE(B, GG) \
    if (bits == B && G == GG) return bf16 ? launch_qmv_t<B, GG, true>(a, stream) : launch_qmv_t<B, GG, false>(a, stream);
    QMM_QMV_CASE(2, 32) QMM_QMV_CASE(2, 64) QMM_QMV_CASE(2, 128)
    QMM_QMV_CASE(3, 32) QMM_QMV_CASE(3, 64) QMM_QMV_CASE(3, 128)
    QMM_QMV_CASE(4, 32) QMM_QMV_CASE(4, 64) QMM_QMV_CASE(4, 128)
    QMM_QMV_CASE(5, 32) QMM_QMV_CASE(5, 64) QMM_QMV_CASE(5, 128)
    QMM_QMV_CASE(6, 32) QMM_QMV_CASE(6, 64) QMM_QMV_CASE(6, 128)
    QMM_QMV_CASE(8, 32) QMM_QMV_CASE(8, 64) QMM_QMV_CASE(8, 128)
#undef QMM_QMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace qmm
