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
// Lane block c supplies codes c*G/4 .. c*G/4 + G/4 - 1 of a group, so one
// MFMA (G = 32) or G/32 accumulating MFMAs contract exactly one group; the
// fp32 epilogue acc += s*P + b*XS then applies that group's scale and bias.
// The group sums XS come from one more MFMA against a ones operand, which
// leaves them in exactly the C layout.
//
// Activations. The workgroup stages the activations of a K chunk in LDS,
// already in A-operand layout and in the pair order of the code unpack, so
// a wave reads each A operand with one conflict-free ds_read_b128. Chunks
// are double-buffered: the global loads of chunk j+1 are issued when chunk j
// starts and written to LDS when it ends, so their latency hides behind the
// compute, and the barrier only waits for LDS traffic, never for the weight
// stream.
//
// Weights. When a lane block's chunk of a group is one or two words (4-bit
// or 8-bit codes with G = 32), lane block c loads all of group g0 + c of its
// row with 16- or 32-byte loads and a 4x4 transpose across the lane blocks
// (v_permlane32_swap + v_permlane16_swap) hands every lane block its chunk
// of the 4 groups; the scale and bias loaded by lane block c are gathered
// with ds_bpermute. Larger chunks are loaded directly per lane. A ring of PD
// register stages keeps several steps of loads in flight; every load is
// unconditional (steps past the end re-read the last step), so the compiler
// never has to drain the ring.
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
    static constexpr bool kTranspose = CHB <= 64 && NWG % 4 == 0;
    static constexpr int SG = kTranspose ? 4 : 1;  // groups per step
    static constexpr int UNIT = NWG / 4;           // words per chunk (transposed path)
    static constexpr int LOAD_ALIGN = gcd_int(4 * NWG, 16);
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

// Barrier for LDS hand-off only: orders this wave's LDS operations, not its
// outstanding global loads (which keep streaming across it).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Work split: a workgroup holds RT x KP waves. Wave (rt, kp) owns 16
// weight rows (row tile rt) and the kp-th of KP contiguous parts of the K
// range, so a 16-row tile is shared by KP waves and the grid has enough waves
// to cover latency; the KP partial tiles are summed through LDS in a fixed
// order at the end. The RT waves of a K part share its staged activations.
// SPC: steps per staged activation chunk. MR: activation rows staged and
// finished per launch (M <= MR <= 16).
#ifndef QMM_MFMA_WAVES_PER_SIMD
#define QMM_MFMA_WAVES_PER_SIMD 4
#endif

// BF16: x, scales and biases hold bf16 bit patterns; codes are widened to
// bf16 and contracted with v_mfma_f32_16x16x32_bf16.
template <int BITS, int G, int RT, int KP, int SPC, int PD, int MR, bool BF16>
__global__ __launch_bounds__(RT *KP *kWave) __attribute__((amdgpu_waves_per_eu(QMM_MFMA_WAVES_PER_SIMD)))
void mfma_kernel(const ProductArgs a)
{
    using Geo = Geometry<BITS, G>;
    constexpr int T = Geo::T;
    constexpr int CH = Geo::CH;
    constexpr int NW = Geo::NW;
    constexpr int NWC = Geo::NWC;
    constexpr int NWG = Geo::NWG;
    constexpr int SG = Geo::SG;
    constexpr int CG = SPC * SG;                                  // groups per chunk
    constexpr int KC = CG * G;                                    // activations per row per chunk
    constexpr int UNITS = 16 * KC / 8;                            // A units per part per chunk
    constexpr int THREADS = RT * KP * kWave;
    constexpr int UPR = KC / 8;                                   // units per row per chunk
    constexpr int PART_UNITS = MR * UPR;                          // units staged per part per chunk
    constexpr int STAGE_UNITS = KP * PART_UNITS;
    constexpr int UPT = (STAGE_UNITS + THREADS - 1) / THREADS;    // units per thread
    constexpr int RLIVE = MR < 4 ? MR : 4;                        // live C rows per lane
    static_assert(PD % (2 * SPC) == 0, "ring depth must cover whole pairs of chunks");
    constexpr int R = PD / SPC;                                   // chunks per ring turn (even)

    __shared__ half8_t xa[KP][2][UNITS];
    __shared__ float red[KP][RT][RLIVE][kWave];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rt = wave % RT, kp = wave / RT;
    const int c = lane / 16, i = lane % 16;
    const Slab slab = slab_of_tile(a, (int)blockIdx.x * RT + rt);  // the projection of this wave's tile
    const int M = a.M, K = a.K, N = slab.p.N, Kg = K / G;
    const size_t wpr = (size_t)K * BITS / 32;

    int gb = 0, ge = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, gb, ge);
    // this wave's K part [pb, pe); parts differ by at most one group
    int pb, pe;
    slice_groups(ge - gb, KP, kp, pb, pe);
    pb += gb;
    pe += gb;
    const int my_steps = (pe - pb + SG - 1) / SG;
    // loads past the end of the part re-read its last group (an empty part
    // re-reads a valid group of the slice and computes nothing)
    const int lo = min(pb, ge - 1), hi = max(lo, pe - 1);
    const int nchunks = ((ge - gb + KP - 1) / KP + CG - 1) / CG;  // same for every wave

    // weight row of this lane (clamped so every load stays in bounds)
    const size_t n = (size_t)min(slab.tile * 16 + i, N - 1);
    const uint32_t *wrow = slab.p.wq + n * wpr + (Geo::kTranspose ? (size_t)c * NWG : (size_t)((c * Geo::CHB) / 32));
    const uint16_t *srow = slab.p.scales + n * Kg + (Geo::kTranspose ? c : 0);
    const uint16_t *brow = slab.p.biases + n * Kg + (Geo::kTranspose ? c : 0);
    const int chunk_shift = (c * Geo::CHB) % 32;  // direct path

    // Activation staging: unit u is part p = u / PART_UNITS, row
    // m = (u % PART_UNITS) / UPR, 8 values at k = 8 * (u % UPR) of that part's
    // chunk; its A slot is ((gl*T + h)*4 + c)*16 + m of xa[p].
    half8_t xreg[UPT];
    auto stage_load = [&](int chunk) {
#pragma unroll
        for (int t = 0; t < UPT; ++t) {
            const int u = min((int)threadIdx.x + t * THREADS, STAGE_UNITS - 1);
            const int p = u / PART_UNITS, rem = u % PART_UNITS;
            const int m = min(rem / UPR, M - 1), k8 = rem % UPR;
            int qb, qe;
            slice_groups(ge - gb, KP, p, qb, qe);
            const int g = min(max(gb + qb + chunk * CG + (8 * k8) / G, gb), ge - 1);  // clamped: always a valid group
            xreg[t] = *reinterpret_cast<const half8_t *>(a.x + (size_t)m * K + (size_t)g * G + (8 * k8) % G);
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int t = 0; t < UPT; ++t) {
            const int u = (int)threadIdx.x + t * THREADS;
            if (STAGE_UNITS % THREADS == 0 || u < STAGE_UNITS) {
                const int p = u / PART_UNITS, rem = u % PART_UNITS;
                const int m = rem / UPR, k = 8 * (rem % UPR);
                const int gl = k / G, kg = k % G;
                const int cb = kg / CH, h = (kg % CH) / 8;
                xa[p][buf][((gl * T + h) * 4 + cb) * 16 + m] =
                    BF16 ? to_pair_order_bf16<BITS>(xreg[t]) : to_pair_order<BITS>(xreg[t]);
            }
        }
    };

    half8_t ones;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ones[e] = (_Float16)1.0f;
    bf16x8_t ones_bf16;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        ones_bf16[e] = (__bf16)1.0f;

    float acc[RLIVE];
#pragma unroll
    for (int r = 0; r < RLIVE; ++r)
        acc[r] = 0.f;

    struct Stage {
        uint32_t w[NW];
        uint32_t s, b;  // fp16 bit patterns, zero-extended
    };

    // Loads of one step. Every load is unconditional (steps past the end of
    // the part re-read its last group, cache hits that are never used), so
    // the compiler can keep the ring of stages in flight.
    auto load = [&](Stage &st, int step) {
        const int g0 = pb + step * SG;
        if constexpr (Geo::kTranspose) {
            // lane block c: group g0 + c
            const int gofs = min(max(g0 + c, lo), hi) - c;
            load_words<NW, Geo::LOAD_ALIGN>(wrow + (ptrdiff_t)gofs * NWG, st.w);
            st.s = srow[gofs];
            st.b = brow[gofs];
        } else {
            const int g = min(max(g0, lo), hi);
            load_words<NW, Geo::CHUNK_ALIGN>(wrow + (size_t)g * NWG, st.w);
            st.s = srow[g];
            st.b = brow[g];
        }
    };

    auto compute = [&](Stage &st, int step, int buf) {
        // Keep steps in program order and consume the stage here: hoisting
        // work on later stages would force waits on their loads.
        __builtin_amdgcn_sched_barrier(0);
        pin_register(st.s);
        pin_register(st.b);
#pragma unroll
        for (int j = 0; j < NW; ++j)
            pin_register(st.w[j]);
        const int g0 = pb + step * SG;
        const int gl0 = (step % SPC) * SG;  // first group of the step within its chunk
        uint32_t sb[SG];
        const uint32_t own = st.s | (st.b << 16);
        if constexpr (Geo::kTranspose) {
#pragma unroll
            for (int t = 0; t < SG; ++t)
                sb[t] = (uint32_t)__builtin_amdgcn_ds_bpermute((16 * t + i) * 4, (int)own);
        } else {
            sb[0] = own;
        }
        uint32_t chunk[SG][NWC];
        if constexpr (Geo::kTranspose) {
#pragma unroll
            for (int u = 0; u < Geo::UNIT; ++u) {
                uint32_t w0 = st.w[0 * Geo::UNIT + u], w1 = st.w[1 * Geo::UNIT + u];
                uint32_t w2 = st.w[2 * Geo::UNIT + u], w3 = st.w[3 * Geo::UNIT + u];
                transpose4(w0, w1, w2, w3);
                chunk[0][u] = w0;
                chunk[1][u] = w1;
                chunk[2][u] = w2;
                chunk[3][u] = w3;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NWC; ++j) {
                if constexpr (Geo::RMAX == 0)
                    chunk[0][j] = st.w[j];
                else
                    chunk[0][j] = j + 1 < NW ? __builtin_amdgcn_alignbit(st.w[j + 1], st.w[j], chunk_shift)
                                             : (st.w[j] >> chunk_shift);
            }
        }
#pragma unroll
        for (int t = 0; t < SG; ++t) {
            if (g0 + t < pe) {  // wave-uniform
                float4_t P = {0.f, 0.f, 0.f, 0.f}, XS = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BF16) {
                    bf16x2_t q[CH / 2];
                    unpack_pairs_bf16<BITS, CH>(chunk[t], q);
#pragma unroll
                    for (int h = 0; h < T; ++h) {
                        const bf16x8_t A = __builtin_bit_cast(
                            bf16x8_t, xa[kp][buf][(((gl0 + t) * T + h) * 4 + c) * 16 + i]);
                        XS = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ones_bf16, XS, 0, 0, 0);
                        const bf16x8_t B = {q[4 * h].x, q[4 * h].y, q[4 * h + 1].x, q[4 * h + 1].y,
                                            q[4 * h + 2].x, q[4 * h + 2].y, q[4 * h + 3].x, q[4 * h + 3].y};
                        P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, P, 0, 0, 0);
                    }
                } else {
                    half2_t q[CH / 2];
                    unpack_pairs<BITS, CH>(chunk[t], q);
#pragma unroll
                    for (int h = 0; h < T; ++h) {
                        const half8_t A = xa[kp][buf][(((gl0 + t) * T + h) * 4 + c) * 16 + i];
                        XS = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, ones, XS, 0, 0, 0);
                        const half8_t B = {q[4 * h].x, q[4 * h].y, q[4 * h + 1].x, q[4 * h + 1].y,
                                           q[4 * h + 2].x, q[4 * h + 2].y, q[4 * h + 3].x, q[4 * h + 3].y};
                        P = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, P, 0, 0, 0);
                    }
                }
                // the widened codes carry 1 / CodeScale (4-bit fp16 codes are
                // subnormals q * 2^-20); the scale takes it back
                float s, b;
                if constexpr (BF16) {
                    s = bf16_bits_to_float(sb[t] & 0xffffu);
                    b = bf16_bits_to_float(sb[t] >> 16);
                } else {
                    s = half_bits_to_float((uint16_t)(sb[t] & 0xffffu)) * CodeScale<BITS>::value;
                    b = half_bits_to_float((uint16_t)(sb[t] >> 16));
                }
#pragma unroll
                for (int r = 0; r < RLIVE; ++r)
                    acc[r] += s * P[r] + b * XS[r];
            }
        }
    };

    // prologue: chunk 0 in LDS, the first PD steps in flight
    stage_load(0);
    Stage ring[PD];
#pragma unroll
    for (int p = 0; p < PD; ++p)
        load(ring[p], p);
    stage_store(0);
    lds_barrier();

    for (int j0 = 0; j0 < nchunks; j0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = j0 + r;
            if (j >= nchunks)  // uniform over the workgroup
                break;
            stage_load(j + 1);
#pragma unroll
            for (int q = 0; q < SPC; ++q) {
                const int step = j * SPC + q;
                if (step < my_steps)
                    compute(ring[r * SPC + q], step, r & 1);
                load(ring[r * SPC + q], step + PD);
            }
            stage_store((r + 1) & 1);
            lds_barrier();
        }
    }

    // fixed-order sum of the KP partial tiles
#pragma unroll
    for (int r = 0; r < RLIVE; ++r)
        red[kp][rt][r][lane] = acc[r];
    __syncthreads();
    if (kp == 0) {
        const int col = slab.tile * 16 + i;
        float *__restrict__ yout = slab.p.y + (size_t)blockIdx.z * a.y_slice_stride;
#pragma unroll
        for (int r = 0; r < RLIVE; ++r) {
            float v = red[0][rt][r][lane];
#pragma unroll
            for (int p = 1; p < KP; ++p)
                v += red[p][rt][r][lane];
            const int m = 4 * c + r;
            if (col < N && m < M)
                yout[(size_t)m * N + col] = v;
        }
    }
}

#ifndef QMM_MFMA_RT
#define QMM_MFMA_RT 1
#endif
#ifndef QMM_MFMA_KP
#define QMM_MFMA_KP 4
#endif

// Steps per staged chunk: at least 128 activations per row (4 KB of LDS per
// K part and buffer).
template <int BITS, int G>
constexpr int default_spc()
{
    return (128 / G) / Geometry<BITS, G>::SG > 0 ? (128 / G) / Geometry<BITS, G>::SG : 1;
}

// Ring depth: two chunks, and at least four steps.
template <int BITS, int G>
constexpr int default_pd()
{
    return 2 * default_spc<BITS, G>() * (default_spc<BITS, G>() < 2 ? 2 : 1);
}

template <int BITS, int G, int MR, bool BF16, int RT = QMM_MFMA_RT, int KP = QMM_MFMA_KP,
          int SPC = default_spc<BITS, G>(), int PD = default_pd<BITS, G>()>
hipError_t launch_mfma_rows(const ProductArgs &a, hipStream_t stream)
{
    static_assert(Geometry<BITS, G>::fits(), "lane chunk loads overrun the group");
    const int rows = 16 * RT;
    const dim3 grid((a.N + rows - 1) / rows, 1, a.split);
    hipLaunchKernelGGL((mfma_kernel<BITS, G, RT, KP, SPC, PD, MR, BF16>), grid, dim3(RT * KP * kWave), 0, stream, a);
    return hipGetLastError();
}

// Row tiles per workgroup: one up to four rows, two from eight rows on
// (measured on the 17408 x 5120 4-bit projection: 41.7 / 46.8 / 57.3 us at
// M = 4 / 8 / 16 with one, 47.0 / 43.9 / 48.0 with two).
template <int BITS, int G>
hipError_t launch_mfma_t(const ProductArgs &a, bool bf16, hipStream_t stream)
{
    if (bf16) {  // bf16 takes this kernel from three rows on only
        if (a.M <= 4) return launch_mfma_rows<BITS, G, 4, true, 1>(a, stream);
        if (a.M <= 8) return launch_mfma_rows<BITS, G, 8, true, 2>(a, stream);
        return launch_mfma_rows<BITS, G, 16, true, 2>(a, stream);
    }
    if (a.M <= 1) return launch_mfma_rows<BITS, G, 1, false, 1>(a, stream);
    if (a.M <= 2) return launch_mfma_rows<BITS, G, 2, false, 1>(a, stream);
    if (a.M <= 4) return launch_mfma_rows<BITS, G, 4, false, 1>(a, stream);
    if (a.M <= 8) return launch_mfma_rows<BITS, G, 8, false, 2>(a, stream);
    return launch_mfma_rows<BITS, G, 16, false, 2>(a, stream);
}

}  // namespace

// Every (bits, G) whose lane chunks can be loaded without reading past their
// group; 3-bit codes at G = 32 cannot (a 24-bit chunk straddles words and
// the last lane block would need the next group's word).
bool mfma_supported(int bits, int G)
{
#define QMM_MFMA_FITS(B, GG) \
    if (bits == B && G == GG) return Geometry<B, GG>::fits();
    QMM_MFMA_FITS(2, 32) QMM_MFMA_FITS(2, 64) QMM_MFMA_FITS(2, 128)
    QMM_MFMA_FITS(3, 32) QMM_MFMA_FITS(3, 64) QMM_MFMA_FITS(3, 128)
    QMM_MFMA_FITS(4, 32) QMM_MFMA_FITS(4, 64) QMM_MFMA_FITS(4, 128)
    QMM_MFMA_FITS(5, 32) QMM_MFMA_FITS(5, 64) QMM_MFMA_FITS(5, 128)
    QMM_MFMA_FITS(6, 32) QMM_MFMA_FITS(6, 64) QMM_MFMA_FITS(6, 128)
    QMM_MFMA_FITS(8, 32) QMM_MFMA_FITS(8, 64) QMM_MFMA_FITS(8, 128)
#undef QMM_MFMA_FITS
    return false;
}

hipError_t launch_mfma(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream)
{
#define QMM_MFMA_CASE(B, GG) \
    if (bits == B && G == GG) return launch_mfma_t<B, GG>(a, bf16, stream);
    QMM_MFMA_CASE(2, 32) QMM_MFMA_CASE(2, 64) QMM_MFMA_CASE(2, 128)
    QMM_MFMA_CASE(3, 64) QMM_MFMA_CASE(3, 128)
    QMM_MFMA_CASE(4, 32) QMM_MFMA_CASE(4, 64) QMM_MFMA_CASE(4, 128)
    QMM_MFMA_CASE(5, 32) QMM_MFMA_CASE(5, 64) QMM_MFMA_CASE(5, 128)
    QMM_MFMA_CASE(6, 32) QMM_MFMA_CASE(6, 64) QMM_MFMA_CASE(6, 128)
    QMM_MFMA_CASE(8, 32) QMM_MFMA_CASE(8, 64) QMM_MFMA_CASE(8, 128)
#undef QMM_MFMA_CASE
    return hipErrorInvalidValue;
}

}  // namespace qmm
