// Multi-row product (M = 2..16 activation rows) on the gfx950 matrix cores,
// with each wave's share of the activations held in registers.
//
// The vmlx-swift pull request #565 page (commit "LaneQMM") contracts the raw
// affine codes with a tensor-op matmul and applies the group scale and bias
// after the dot product; this kernel does the same with
// v_mfma_f32_16x16x32_f16 (lane = 16*c + i, c = 0..3):
//   A (activations): lane (c, i) holds 8 values of activation row i,
//   B (codes):       lane (c, i) holds 8 codes of weight row n0 + i,
//   C (fp32):        lane (c, i) holds rows 4c..4c+3 of output column n0 + i.
// Lane block c supplies codes c*G/4 .. c*G/4 + G/4 - 1 of a group, so G/32
// accumulating MFMAs contract exactly one group into P_g, and the fp32
// epilogue acc += s[n][g] * P_g applies that group's scale. The bias term
// sum_g b[n][g] * XS[m][g] (XS: the activations' group sums) is itself a
// small product over groups: one v_mfma_f32_16x16x4_f32 per quad of groups,
// from group sums computed once per launch.
//
// Work split. A workgroup of KP waves walks a contiguous range of 16-row
// tiles. Wave kp owns the kp-th of KP parts of the K range (at most 768
// activations per row, 640 for 8-bit codes) and loads its A operands once,
// into registers, for the whole launch. The KP partial tiles wait in LDS
// and are summed in a fixed part order after every batch of tiles (one
// barrier per batch), so results do not depend on timing. When K does not
// fit KP parts, each wave walks several parts in turn (passes): at each pass
// it reloads its activations and group sums and streams the workgroup's
// tiles again over the next K range, and each tile's running sum waits in
// LDS until the last pass writes y.
//
// Weights. Every lane of a 16-byte load reads a consecutive piece of one
// weight row, so one load instruction covers whole row segments (the 16 rows
// x segment-bytes block of a tile and part), which is the access shape that
// streams from HBM at full rate. The wave writes the block to its own LDS
// region and reads back each lane's chunk in the MFMA B layout; the tile's
// scales and biases go the same way, interleaved as (s | b << 16) words. The
// loads of the tile NST ahead (one register stage) are issued as soon as the
// current one is in LDS, so they stream while it is computed.
#include <atomic>

#include "qmm_device.hpp"
#include "qmm_kernels.hpp"

#include <type_traits>

namespace qmm {
namespace {

constexpr int kXrMaxParts = 8;    // waves (K parts) per workgroup
constexpr size_t kXrLdsLimit = 160 * 1024;  // LDS of one CU
#ifndef XR_MAX_PASSES
#define XR_MAX_PASSES 8
#endif
constexpr int kXrMaxPasses = XR_MAX_PASSES;  // K parts per wave (activations reloaded between them)
constexpr int kXrBatchMax = 6;    // tiles whose partial sums are reduced after one barrier, at most

// Activations per row held by one wave (XC: 640 or 768, i.e. 80 or 96
// registers of A operands; 640 for 8-bit codes, and 512 in the tiled
// layout's 8-bit variant). The host takes the first variant of a width whose
// parts fit the workgroup (plan_xr_any).
//
// Tiles of loads in flight per wave (register stages): one. A stage's
// registers are free again as soon as its tile is in LDS, so the next
// tile's loads stream during the computation even with one stage; more
// stages only make the first burst of requests larger, and every wave's
// first tile then lands later in it. Measured on the 5120 x 17408 4-bit
// projection: 22.1 / 23.6 us (M = 4 / 16) with three stages, 20.6 / 22.6 with
// two, 18.4 / 21.4 with one.
#ifndef XR_STD_STAGES
#define XR_STD_STAGES 1
#endif
constexpr int xr_stages_sbw(int, int, int) { return XR_STD_STAGES; }

template <int BITS, int G, int XC>
struct XrGeo {
    static constexpr int T = G / 32;                         // MFMAs per group
    static constexpr int CH = G / 4;                         // codes per lane block per group
    static constexpr int CHB = CH * BITS;                    // bits per lane block (multiple of 8)
    static constexpr int GB = G * BITS / 8;                  // bytes per group (multiple of 4)
    static constexpr int XG = XC / G;                        // groups per part, at most
    static constexpr int GRAN = 16 / gcd_int(GB, 16);        // part starts: multiples of GRAN groups
    static constexpr int NI = (XG * GB + 63) / 64;           // 16-byte loads per lane per tile
    static constexpr int LSTR = XG * GB + 16;                // LDS bytes per weight row
    static constexpr int XQ = (XG + 3) / 4;                  // group quads per part
    static constexpr int SBSTR = 4 * XQ + ((XQ % 2) ? 0 : 4); // LDS words per scale/bias row: 16-byte rows, odd quad count
    static constexpr int max_shift()
    {
        int m = 0;
        for (int c = 0; c < 4; ++c)
            m = (c * CHB) % 32 > m ? (c * CHB) % 32 : m;
        return m;
    }
    static constexpr int SHIFT = max_shift();
    static constexpr int NWR = (SHIFT + CHB + 31) / 32;      // LDS words read per lane block
    static constexpr int NWC = (CHB + 31) / 32;              // chunk words after the shift
    static_assert(CHB % 8 == 0 && GB % 4 == 0, "chunks must start on byte boundaries");
    static_assert(LSTR % 16 == 0, "weight rows must keep 16-byte LDS alignment");
};

struct XrArgs {
    ProductArgs p;
    int gran;    // part boundary granularity in groups
    int ntiles;  // 16-row tiles of N
    int npass;   // K passes: wave kp owns parts kp, KP + kp, 2 KP + kp, ... of the slice
    int batch;   // tiles whose partial sums are reduced after one barrier
    int nbuf;    // partial-sum buffers: 1 when one batch holds every tile of a workgroup's one pass, else 2
    int add;     // the two K slices (grid z) add into a zeroed y instead of writing partials
};

// Group range [pb, pe) of part kp: the slice [gb, ge) cut into KP parts of
// whole granules of `gran` groups (the last granule may be short).
__host__ __device__ inline void part_range(int gb, int ge, int KP, int kp, int gran, int &pb, int &pe)
{
    const int nu = (ge - gb + gran - 1) / gran;
    int ub, ue;
    slice_groups(nu, KP, kp, ub, ue);
    pb = gb + ub * gran < ge ? gb + ub * gran : ge;
    pe = gb + ue * gran < ge ? gb + ue * gran : ge;
}

// Dynamic LDS of one workgroup of KP waves: per wave a weight tile region
// (16 x LSTR bytes) and a scale/bias region (16 x SBSTR words), at least as
// large as the group-sum scratch of the start (XG x 64 floats), then `nbuf`
// buffers of `batch` tiles of partial sums (XrArgs).
// (The tiled-layout variant keeps its weights in registers: only the group-
// sum scratch.)
template <int BITS, int G, int XC, bool TILED = false>
__host__ __device__ constexpr size_t xr_wave_lds()
{
    using Geo = XrGeo<BITS, G, XC>;
    const size_t run = TILED ? 0 : 16 * (size_t)Geo::LSTR + 16 * 4 * (size_t)Geo::SBSTR;
    const size_t xs = (size_t)Geo::XG * 4 * 16 * sizeof(float);
    return run > xs ? run : xs;
}
template <int BITS, int G, int XC, bool TILED = false>
__host__ __device__ constexpr size_t xr_lds_bytes(int KP, int batch, int nbuf)
{
    return (size_t)KP * xr_wave_lds<BITS, G, XC, TILED>() + (size_t)nbuf * batch * KP * 4 * kWave * sizeof(float);
}

// Tiled (MFMA-native) layout, for codes whose lane chunk (the G/4 codes lane
// block c takes of a group: G*bits/32 bytes) is a whole number of 16-bit
// halves: 2, 4 and 8 bits. Per 16-row tile t, lane L = 16c + i owns the
// stream of row 16t + i's chunks c of groups 0, 1, 2, ..., cut into 16-byte
// units; unit u of lane L of tile t sits at byte ((t*UB + u)*64 + L)*16,
// UB = K*bits/512. Scales and biases: word (s | b << 16) of row 16t + i and
// group g at word ((t*Kg/4 + g/4)*16 + i)*4 + g%4. Rows past N hold zeros.
template <int BITS, int G>
__host__ __device__ constexpr int tiled_chunk_bytes() { return G * BITS / 32; }

// SBW: bytes per scale/bias load (4: two groups per load, 2: one group).
// NST: tiles of loads in flight per wave (register stages).
// FUSED: the launch runs several projections (tile -> projection lookup).
// TILED: weights in the tiled layout above (a.wq: codes, a.scales: the
// (s, b) words); each lane loads its MFMA operands directly and nothing of
// the weights goes through LDS.
// BF16: x, scales and biases hold bf16 bit patterns; codes are widened to
// bf16 and contracted with v_mfma_f32_16x16x32_bf16.
// MP: K passes (xa.npass parts per wave, activations reloaded between them,
// later passes adding into y); single-pass variants compile the loop away.
template <int BITS, int G, int XC, int SBW, int NST, bool FUSED, bool TILED = false, bool BF16 = false,
          bool MP = false>
__global__ __launch_bounds__(kXrMaxParts *kWave) void mfma_xr_kernel(const XrArgs xa)
{
    static_assert(!(TILED && BF16), "the tiled layout is fp16 only");
    using Geo = XrGeo<BITS, G, XC>;
    // factor between the accumulated sums and y (see CodeScale)
    constexpr float kOutScale = BF16 ? 1.0f : CodeScale<BITS>::value;
    constexpr int CB = tiled_chunk_bytes<BITS, G>();       // tiled: bytes per lane chunk
    constexpr int NIT = (Geo::XG * CB + 15) / 16;          // tiled: 16-byte code loads per lane per tile
    constexpr int T = Geo::T, CH = Geo::CH, GB = Geo::GB, XG = Geo::XG, NI = Geo::NI;
    constexpr int LSTR = Geo::LSTR, SBSTR = Geo::SBSTR, NWR = Geo::NWR, NWC = Geo::NWC;
    constexpr int SBE = SBW / 2;                             // groups per scale/bias load
    constexpr int NS = (16 * XG / SBE + 63) / 64;            // scale (and bias) loads per lane per tile

    extern __shared__ __align__(16) uint8_t xr_lds[];

    const ProductArgs &a = xa.p;
    const int lane = threadIdx.x % kWave;
    const int kp = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int KP = blockDim.x / kWave;
    uint8_t *const wmy = xr_lds + (size_t)kp * xr_wave_lds<BITS, G, XC, TILED>();
    uint32_t *const sbmy = reinterpret_cast<uint32_t *>(wmy + 16 * LSTR);
    // red[buf][slot][part][r][lane]
    float *const red = reinterpret_cast<float *>(xr_lds + (size_t)KP * xr_wave_lds<BITS, G, XC, TILED>());
    auto red_at = [&](int buf, int slot, int part, int r) -> float & {
        return red[(((size_t)(buf * xa.batch + slot) * KP + part) * 4 + r) * kWave + lane];
    };
    // multi-pass: the running sums of the workgroup's tiles between passes,
    // accl[tile - t0][r][lane], each word read and written by one thread only
    float *const accl = red + (size_t)xa.nbuf * xa.batch * KP * 4 * kWave;
    const int c = lane / 16, i = lane % 16;
    const int M = a.M, K = a.K, Kg = K / G;
    // projection of a tile; single-projection launches skip the lookup
    auto slab_at = [&](int t) -> Slab {
        if constexpr (FUSED)
            return slab_of_tile(a, t);
        else
            return Slab{Proj{a.wq, a.scales, a.biases, a.y, a.N}, t};
    };
    const uint32_t RB = (uint32_t)K * BITS / 8;  // bytes per weight row

    int gb = 0, ge = Kg;
    if (a.split > 1)
        slice_groups(Kg, a.split, blockIdx.z, gb, ge);
    const int npass = (TILED || !MP) ? 1 : xa.npass;

    // tiles of this workgroup
    const int t0 = (int)(((long long)blockIdx.x * xa.ntiles) / gridDim.x);
    const int t1 = (int)(((long long)(blockIdx.x + 1) * xa.ntiles) / gridDim.x);
    const int batch = xa.batch;
    const int nbatch = (t1 - t0 + batch - 1) / batch;  // barriers per pass

    // This wave's K part of the current pass, [pb, pe) (ng >= 1: the host never
    // makes empty parts), and the per-lane load geometry of that part. Weight
    // unit u (16 bytes) is row u / U, column u % U of the tile's 16 x (ng*GB)
    // block.
    int pb, pe, ng;
    int wr[NI];
    uint32_t wcol[NI], wl[NI];
    int sr[NS], scol[NS];
    auto set_part = [&](int pass) {
        part_range(gb, ge, KP * npass, pass * KP + kp, xa.gran, pb, pe);
        ng = pe - pb;
        const int U = ng * GB / 16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int u = min(64 * j + lane, 16 * U - 1);
            wr[j] = u / U;
            wcol[j] = (uint32_t)pb * GB + (uint32_t)(u % U) * 16;
            wl[j] = (uint32_t)wr[j] * LSTR + (uint32_t)(u % U) * 16;
        }
        const int V = ng / SBE;  // scale/bias units per row (ng is a multiple of SBE)
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int e = min(64 * j + lane, 16 * V - 1);
            sr[j] = e / V;
            scol[j] = e % V;
        }
    };
    set_part(0);

    struct StageStd {
        u32x4 w[NI];
        uint32_t s[NS], b[NS];
    };
    struct StageTiled {
        u32x4 w[NIT];
        u32x4 sb[Geo::XQ];
    };
    using Stage = std::conditional_t<TILED, StageTiled, StageStd>;
    // tiled: this part's first 16-byte unit and group quad, and their counts
    // (parts start on whole units and quads)
    const uint32_t UB = (uint32_t)K * BITS / 512;
    const int u0 = pb * CB / 16, nu_part = max(ng * CB / 16, 1);
    const int q0 = pb / 4, nq = max(ng / 4, 1);
    // Loads of one tile. Past the workgroup's last tile every lane reads the
    // first 16 bytes of that tile instead (one cache line, never used), so
    // the loads stay unconditional without streaming a tile twice.
    auto issue = [&](Stage &st, int tile) {
        // a per-lane mask instead of a branch on `past`: a branch around
        // loads makes the compiler drain every load in flight
        uint32_t keep = tile >= t1 ? 0u : ~0u;
        pin_register(keep);
        if constexpr (TILED) {
            const int tc = min(tile, t1 - 1);
            const uint8_t *tw = reinterpret_cast<const uint8_t *>(a.wq) + (size_t)tc * UB * 1024;
#pragma unroll
            for (int j = 0; j < NIT; ++j) {
                const uint32_t off = ((uint32_t)((u0 + min(j, nu_part - 1)) * 64 + lane) * 16) & keep;
                st.w[j] = load_weight(reinterpret_cast<const u32x4 *>(tw + off));
            }
            const uint32_t *tsb = reinterpret_cast<const uint32_t *>(a.scales) + (size_t)tc * (Kg / 4) * 64;
#pragma unroll
            for (int u = 0; u < Geo::XQ; ++u) {
                const uint32_t off = ((uint32_t)((q0 + min(u, nq - 1)) * 16 + i) * 4) & keep;
                st.sb[u] = *reinterpret_cast<const u32x4 *>(tsb + off);
            }
        } else {
            const Slab sl = slab_at(min(tile, t1 - 1));
            const int rmax = sl.p.N - 1 - sl.tile * 16;  // rows past N re-read row N-1
            const uint8_t *wt = reinterpret_cast<const uint8_t *>(sl.p.wq) + (size_t)sl.tile * 16 * RB;
    #pragma unroll
            for (int j = 0; j < NI; ++j) {
                const uint32_t off = ((uint32_t)min(wr[j], rmax) * RB + wcol[j]) & keep;
                st.w[j] = load_weight(reinterpret_cast<const u32x4 *>(wt + off));
            }
            const size_t sbase = (size_t)sl.tile * 16 * Kg + pb;
    #pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint32_t off = ((uint32_t)min(sr[j], rmax) * Kg + scol[j] * SBE) & keep;
                if constexpr (SBW == 4) {
                    st.s[j] = *reinterpret_cast<const uint32_t *>(sl.p.scales + sbase + off);
                    st.b[j] = *reinterpret_cast<const uint32_t *>(sl.p.biases + sbase + off);
                } else {
                    st.s[j] = sl.p.scales[sbase + off];
                    st.b[j] = sl.p.biases[sbase + off];
                }
            }
        }
    };
    auto stage_to_lds = [&](StageStd &st) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
            *reinterpret_cast<u32x4 *>(wmy + wl[j]) = st.w[j];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            uint32_t *row = sbmy + sr[j] * SBSTR + scol[j] * SBE;
            if constexpr (SBW == 4) {
                row[0] = __builtin_amdgcn_perm(st.b[j], st.s[j], 0x05040100u);
                row[1] = __builtin_amdgcn_perm(st.b[j], st.s[j], 0x07060302u);
            } else {
                row[0] = st.s[j] | (st.b[j] << 16);
            }
        }
    };

    // A operands of the current part: lane (c, i) holds activation row
    // min(i, M-1) (rows past M repeat the last row and are never stored).
    // Group sums XS[row i][group 4u + c] of the part, as the A operand of one
    // fp32 MFMA per group quad (the bias term sum_g b[n][g] XS[m][g]).
    half8_t xr[XG][T];
    float xsa[Geo::XQ];
    Stage st[NST];
    // Start of a pass: the part's activations, the first NST tiles' loads
    // (issued after the activation loads, so that the loop always finds its
    // stages in the same order of age), and the part's group sums. Lane block
    // c sums its quarter of every group with v_dot2 against (1, 1); the
    // quarters meet in the wave's LDS region (sized for them, and free at the
    // start of a pass) and are added in lane-block order.
    // The A operand of lane (c, i) is 16 bytes of row i; loaded that way, one
    // instruction touches 16 rows in 16-byte pieces and the activations take
    // 2.5 times as long to arrive as with row-contiguous loads (measured on
    // the 16 x 5120 activations of 218 workgroups of 8 waves). So lane
    // 4r + p loads piece p of row r, and the lanes are then permuted to the
    // MFMA layout (lane 16c + i takes lane 4i + c's 16 bytes): the same data
    // per lane, four ds_bpermute per 16 bytes.
    const int ldr = lane / 4, ldp = lane % 4;          // row and piece this lane loads
    const int from = (4 * i + c) * 4;                  // byte address of the source lane
    // Issue priority. Waves kp and kp + 4 share a SIMD, and the arbiter
    // favours the older one: left alone, the second wave starts 0.3 us later,
    // falls 2.5 us behind by the last tile, and the workgroup's final barrier
    // waits for it. So the second wave takes the higher priority while it
    // loads its activations, and from the first tile on the two take turns,
    // tile by tile (17.6 against 19.0 us at M = 4, 17.7 against 18.3 at M = 16
    // on the 5120 x 17408 projection, medians of six runs).
    auto begin_pass = [&]() {
        if (kp >= 4)
            __builtin_amdgcn_s_setprio(1);
        const uint16_t *xrow = a.x + (size_t)min(ldr, M - 1) * K;
        half8_t raw[XG][T];
#pragma unroll
        for (int g = 0; g < XG; ++g) {
            const int gg = min(pb + g, pe - 1);  // groups past the part re-read its last group
#pragma unroll
            for (int h = 0; h < T; ++h)
                raw[g][h] = *reinterpret_cast<const half8_t *>(xrow + (size_t)gg * G + ldp * CH + 8 * h);
        }
#pragma unroll
        for (int g = 0; g < XG; ++g) {
#pragma unroll
            for (int h = 0; h < T; ++h) {
                const u32x4 w = __builtin_bit_cast(u32x4, raw[g][h]);
                const u32x4 m = {(uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)w.x),
                                 (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)w.y),
                                 (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)w.z),
                                 (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)w.w)};
                const half8_t v = __builtin_bit_cast(half8_t, m);
                xr[g][h] = BF16 ? to_pair_order_bf16<BITS>(v) : to_pair_order<BITS>(v);
            }
        }
#pragma unroll
        for (int k = 0; k < NST; ++k)
            issue(st[k], t0 + k);

        float *xsl = reinterpret_cast<float *>(wmy);
        const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
        wave_lds_sync();  // the previous pass's reads of the region are done
#pragma unroll
        for (int g = 0; g < XG; ++g) {
            float ps = 0.f;
#pragma unroll
            for (int h = 0; h < T; ++h)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const half2_t xe = {xr[g][h][e], xr[g][h][e + 1]};
                    if constexpr (BF16) {
                        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
                        ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xe), ones, ps, false);
                    } else {
                        ps = __builtin_amdgcn_fdot2(xe, one2, ps, false);
                    }
                }
            xsl[(g * 4 + c) * 16 + i] = ps;
        }
        wave_lds_sync();  // the quarters written by the other lane blocks are read below
#pragma unroll
        for (int u = 0; u < Geo::XQ; ++u) {
            const int g = 4 * u + c;
            float v = 0.f;
            if (g < ng) {
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    v += xsl[(g * 4 + cc) * 16 + i];
            }
            xsa[u] = v;
        }
        wave_lds_sync();  // the scratch is rewritten below (zeroed words, staged tiles)
        // scale/bias words of groups past the part stay zero: those groups
        // (computed in whole quads) contribute nothing
        if constexpr (!TILED)
            for (int e = lane; e < 16 * SBSTR; e += kWave)
                sbmy[e] = 0u;
    };

    const int chunk_byte = c * (Geo::CHB / 8);
    const int chunk_shift = 8 * (chunk_byte % 4);
    const uint8_t *wrow_lds = wmy + i * LSTR + (chunk_byte & ~3);
    const uint32_t *sbrow = sbmy + i * SBSTR;

    int pass = 0;
    auto process = [&](Stage &sk, int tile) {
        __builtin_amdgcn_sched_barrier(0);
        if ((((tile - t0) + (kp >> 2)) & 1) != 0)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        if constexpr (!TILED) {
            wave_lds_sync();  // the previous tile's reads of the region are done
            stage_to_lds(sk);
            wave_lds_sync();  // other lanes read the staged rows below
            // the stage's registers are free again: start the loads NST tiles ahead
            issue(sk, tile + NST);
        }
        if (tile >= t1) {  // uniform over the workgroup: a round's tail past the range
            if constexpr (TILED)
                issue(sk, tile + NST);
            return;
        }
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < Geo::XQ; ++u) {
            if (4 * u < ng) {  // wave-uniform
                // the quad's MFMAs first, so their latency overlaps
                float4_t P[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int g = 4 * u + t;
                    P[t] = float4_t{0.f, 0.f, 0.f, 0.f};
                    if (g < XG) {  // compile-time after unrolling
                        uint32_t chunk[NWC];
                        if constexpr (TILED) {
                            // group g's chunk: bytes g*CB .. g*CB+CB-1 of the lane's part stream
#pragma unroll
                            for (int w = 0; w < NWC; ++w) {
                                const int d = (g * CB) / 4 + w;  // compile-time
                                const uint32_t v = sk.w[d / 4][d % 4];
                                chunk[w] = CB >= 4 ? v : (v >> (8 * ((g * CB) % 4)));
                            }
                        } else {
                            uint32_t raw[NWR];
#pragma unroll
                            for (int w = 0; w < NWR; ++w)
                                raw[w] = *reinterpret_cast<const uint32_t *>(wrow_lds + g * GB + 4 * w);
#pragma unroll
                            for (int w = 0; w < NWC; ++w) {
                                if constexpr (Geo::SHIFT == 0)
                                    chunk[w] = raw[w];
                                else
                                    chunk[w] = w + 1 < NWR ? __builtin_amdgcn_alignbit(raw[w + 1], raw[w], chunk_shift)
                                                           : (raw[w] >> chunk_shift);
                            }
                        }
                        if constexpr (BF16) {
                            bf16x2_t q[CH / 2];
                            unpack_pairs_bf16<BITS, CH>(chunk, q);
#pragma unroll
                            for (int h = 0; h < T; ++h) {
                                const bf16x8_t B = {q[4 * h].x, q[4 * h].y, q[4 * h + 1].x, q[4 * h + 1].y,
                                                    q[4 * h + 2].x, q[4 * h + 2].y, q[4 * h + 3].x, q[4 * h + 3].y};
                                P[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8_t, xr[g][h]), B, P[t], 0, 0, 0);
                            }
                        } else {
                            half2_t q[CH / 2];
                            unpack_pairs<BITS, CH>(chunk, q);
#pragma unroll
                            for (int h = 0; h < T; ++h) {
                                const half8_t B = {q[4 * h].x, q[4 * h].y, q[4 * h + 1].x, q[4 * h + 1].y,
                                                   q[4 * h + 2].x, q[4 * h + 2].y, q[4 * h + 3].x, q[4 * h + 3].y};
                                P[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xr[g][h], B, P[t], 0, 0, 0);
                            }
                        }
                    }
                }
                // bias term of the quad: one fp32 MFMA over its 4 groups
                uint32_t sbo;
                u32x4 sbq;
                if constexpr (TILED) {
                    sbq = sk.sb[u];
                    sbo = c == 0 ? sbq[0] : c == 1 ? sbq[1] : c == 2 ? sbq[2] : sbq[3];
                } else {
                    sbo = sbrow[4 * u + c];
                    sbq = *reinterpret_cast<const u32x4 *>(sbrow + 4 * u);
                }
                // acc carries the factor 1 / kOutScale of the widened codes
                // (4-bit fp16 codes are subnormals q * 2^-20), so the bias
                // enters scaled by it (exact: a power of two)
                float bo;
                if constexpr (BF16)
                    bo = bf16_bits_to_float(sbo >> 16);
                else
                    bo = half_bits_to_float((uint16_t)(sbo >> 16)) * CodeScale<BITS>::inverse;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xsa[u], bo, acc, 0, 0, 0);
                // scale term: acc += s[n][g] * P_g
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (4 * u + t < XG) {
                        const float sg = BF16 ? bf16_bits_to_float(sbq[t] & 0xffffu)
                                              : half_bits_to_float((uint16_t)(sbq[t] & 0xffffu));
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[r] = __builtin_fmaf(sg, P[t][r], acc[r]);
                    }
                }
            }
        }
        // Partial sums wait in LDS; after every `batch` tiles (and the last)
        // one barrier, then wave p sums slot p's KP partials in part order.
        const int lt = tile - t0;
        // batches are counted across passes, so the two partial-sum buffers
        // keep alternating at a pass boundary
        const int buf = (pass * nbatch + lt / batch) & (xa.nbuf - 1), slot = lt % batch;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red_at(buf, slot, kp, r) = acc[r];
        if (slot == batch - 1 || tile == t1 - 1) {  // uniform over the workgroup
            __syncthreads();
            const int first = tile - slot;
            for (int sl = kp; sl <= slot; sl += KP) {
                const Slab ts = slab_at(first + sl);
                const int col = ts.tile * 16 + i, N = ts.p.N;
                float *__restrict__ yout = ts.p.y + (size_t)blockIdx.z * a.y_slice_stride;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o;
                    if (!MP && !xa.add && KP % 2 == 0) {
                        // the two halves of the parts summed apart and then
                        // added: the bits of an additive two-slice launch over
                        // the same parts, (0 + a) + b (kOutScale is a power of
                        // two, so the products are exact)
                        float va = red_at(buf, sl, 0, r), vb = red_at(buf, sl, KP / 2, r);
                        for (int p = 1; p < KP / 2; ++p) {
                            va += red_at(buf, sl, p, r);
                            vb += red_at(buf, sl, KP / 2 + p, r);
                        }
                        o = va * kOutScale + vb * kOutScale;
                    } else {
                        float v = red_at(buf, sl, 0, r);
                        for (int p = 1; p < KP; ++p)
                            v += red_at(buf, sl, p, r);
                        o = v * kOutScale;
                    }
                    const int m = 4 * c + r;
                    if constexpr (MP) {
                        // the running sum of the earlier passes, kept by this thread
                        float &run = accl[((size_t)(first + sl - t0) * 4 + r) * kWave + lane];
                        if (pass > 0)
                            o += run;
                        if (pass + 1 < npass) {
                            run = o;
                            continue;
                        }
                    }
                    if (col < N && m < M) {
                        if (xa.add)  // exactly two addends on +0: the same sum in either order
                            atomicAdd(&yout[(size_t)m * N + col], o);
                        else
                            yout[(size_t)m * N + col] = o;
                    }
                }
            }
        }
        if constexpr (TILED)  // the stage's registers are consumed: the loads NST tiles ahead
            issue(sk, tile + NST);
    };

    // Rounds of NST tiles, one per stage. Every round stages and reloads all
    // NST stages (tiles past the range load one cache line and are not
    // computed), so no path around a stage's loads reaches the back edge and
    // the waits stay per stage.
    for (pass = 0; pass < npass; ++pass) {
        if (pass > 0)
            set_part(pass);
        begin_pass();
        for (int t = t0; t < t1; t += NST) {
#pragma unroll
            for (int k = 0; k < NST; ++k)
                process(st[k], t + k);
        }
    }
}

struct XrPlan {
    int KP, gran, sbw;
    int npass;  // K passes (parts per wave)
};

// More than 64 KB of dynamic LDS must be allowed per kernel: set the limit
// of `fns` once per device (bit d of `done` records device d; two threads
// racing both set it, which is harmless).
hipError_t allow_dynamic_lds(const void *const *fns, int count, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = 0;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit)
        return hipSuccess;
    for (int k = 0; k < count; ++k) {
        const hipError_t e = hipFuncSetAttribute(fns[k], hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess)
            return e;
    }
    done.fetch_or(bit, std::memory_order_release);
    return hipSuccess;
}

// Workgroups of a launch: two waves per SIMD fit, so 8 / KP workgroups per
// CU, shared by the K slices, at most one per tile, and then as few as give
// every workgroup the same number of tiles (the launch takes as long as its
// longest tile run; fewer workgroups on it contend less for HBM: 20.7 against
// 21.0 us at M = 16 on the 5120 x 17408 projection, 218 workgroups of 5 tiles
// against 256 of 4 or 5).
int xr_grid_x(const ProductArgs &a, int KP, int npass)
{
    const int ntiles = (a.N + 15) / 16;
    const int per_cu = kXrMaxParts / KP;
    const long long want = ((long long)device_cu_count() * per_cu + a.split - 1) / a.split;
    const int gx = (int)(want < ntiles ? want : ntiles);
    const int per = (ntiles + gx - 1) / gx;
    return (ntiles + per - 1) / per;
}

// Grid, barrier batch and LDS of a launch: one batch holds every tile of a
// workgroup's pass when that fits (one barrier per pass, and a single
// partial-sum buffer when there is one pass), else batches of up to
// kXrBatchMax tiles in two alternating buffers, smaller while the LDS does
// not fit. Multi-pass launches also keep each tile's running sum (4 x 64
// floats) in LDS between passes. Measured on the 5120 x 17408 projection
// (218 workgroups of 5 tiles): 19.8-20.1 us at M = 16 with one barrier per
// workgroup against 20.6-21.3 with barriers after every 4 tiles.
struct XrShape {
    int gx, batch, nbuf;
    size_t lds;
};
template <int BITS, int G, int XC, bool TILED = false>
bool xr_shape(const ProductArgs &a, int KP, int npass, int gx, XrShape &sh)
{
    const int ntiles = (a.N + 15) / 16;
    const int tpw = (ntiles + gx - 1) / gx;
    const size_t run = npass > 1 ? (size_t)tpw * 4 * kWave * sizeof(float) : 0;
    for (int b = tpw < kXrBatchMax ? tpw : kXrBatchMax; b >= 1; --b) {
        const int nbuf = npass == 1 && tpw <= b ? 1 : 2;
        const size_t lds = xr_lds_bytes<BITS, G, XC, TILED>(KP, b, nbuf) + run;
        if (lds <= kXrLdsLimit) {
            sh = XrShape{gx, b, nbuf, lds};
            return true;
        }
    }
    return false;
}

// The register-resident kernel needs: whole 16-byte rows of packed codes,
// K slices starting on a granule, at most kXrMaxParts parts of at most
// XC activations each, and no empty part.
template <int BITS, int G, int XC>
bool plan_xr(const ProductArgs &a, XrPlan &plan, int max_pass = 1)
{
    using Geo = XrGeo<BITS, G, XC>;
    const int Kg = a.K / G;
    if (((long long)a.K * BITS) % 128 != 0)
        return false;
    const int sbw = Kg % 2 == 0 ? 4 : 2;
    const int gran = sbw == 4 ? Geo::GRAN * 2 / gcd_int(Geo::GRAN, 2) : Geo::GRAN;
    const int S = a.split;
    int lmin = Kg, lmax = 0;
    for (int z = 0; z < S; ++z) {
        int b, e;
        slice_groups(Kg, S, z, b, e);
        if (b % gran != 0)
            return false;
        lmin = e - b < lmin ? e - b : lmin;
        lmax = e - b > lmax ? e - b : lmax;
    }
    const int per_part = Geo::XG / gran;  // granules per part
    if (per_part < 1)
        return false;
    const int nu_max = (lmax + gran - 1) / gran, nu_min = (lmin + gran - 1) / gran;
    // parts of at most per_part granules: KP waves, each walking npass of them
    const int parts = (nu_max + per_part - 1) / per_part;
    const int npass = (parts + kXrMaxParts - 1) / kXrMaxParts;
    if (npass > max_pass)
        return false;
    const int KP = (parts + npass - 1) / npass;
    const int total = KP * npass;
    if (total > nu_min)
        return false;
    // a part whose granule count is at its maximum must still fit
    if (((nu_max + total - 1) / total) * gran > Geo::XG)
        return false;
    XrShape sh;
    if (!xr_shape<BITS, G, XC>(a, KP, npass, xr_grid_x(a, KP, npass), sh))
        return false;
    plan = XrPlan{KP, gran, sbw, npass};
    return true;
}

// Variants of a width, preferred first: fewer activation registers leave
// room for more tiles in flight; the longer parts take longer K. 8-bit codes
// take 640-activation parts (their 40 registers of weight loads per tile
// leave no room for 768); the tiled layout keeps 512 for them (its loads
// stay in registers through the computation).
template <int BITS>
constexpr int xr_small_codes() { return 640; }
template <int BITS>
constexpr int xr_large_codes() { return BITS == 8 ? 640 : 768; }
template <int BITS>
constexpr int xr_tiled_small_codes() { return BITS == 8 ? 512 : 640; }
template <int BITS>
constexpr int xr_tiled_large_codes() { return BITS == 8 ? 512 : 768; }
#ifndef XR_MP_WIDE
#define XR_MP_WIDE 1
#endif
// Parts of the multi-pass variants (several K parts per wave).
template <int BITS>
constexpr int xr_pass_codes() { return XR_MP_WIDE && BITS <= 4 ? xr_large_codes<BITS>() : xr_small_codes<BITS>(); }

template <int BITS, int G, int XC, bool BF16>
hipError_t launch_xr_variant(const ProductArgs &a, const XrPlan &plan, hipStream_t stream, bool add = false)
{
    XrShape sh;
    if (!xr_shape<BITS, G, XC>(a, plan.KP, plan.npass, xr_grid_x(a, plan.KP, plan.npass), sh))
        return hipErrorInvalidValue;  // excluded by plan_xr
    XrArgs xa{a, plan.gran, (a.N + 15) / 16, plan.npass, sh.batch, sh.nbuf, add ? 1 : 0};
    const dim3 grid(sh.gx, 1, a.split), block(plan.KP * kWave);
    const size_t lds = sh.lds;
    constexpr int NST4 = xr_stages_sbw(BITS, XC, 4), NST2 = xr_stages_sbw(BITS, XC, 2);
    // bf16 launches are single-projection only (no fused bf16 entry point)
    const bool fused = !BF16 && a.nproj >= 2;
    // more than 64 KB of dynamic LDS must be allowed per kernel, once
    static std::atomic<uint64_t> allowed{0};
    {
        const int cap = (int)kXrLdsLimit;
        constexpr bool kMP = XC == xr_pass_codes<BITS>();  // multi-pass variants exist for one width only
        const void *fns[8] = {
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 4, NST4, false, false, BF16>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 2, NST2, false, false, BF16>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 4, NST4, !BF16, false, BF16>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 2, NST2, !BF16, false, BF16>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 4, NST4, false, false, BF16, kMP>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 2, NST2, false, false, BF16, kMP>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 4, NST4, !BF16, false, BF16, kMP>),
            reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 2, NST2, !BF16, false, BF16, kMP>)};
        const hipError_t e = allow_dynamic_lds(fns, 8, cap, allowed);
        if (e != hipSuccess)
            return e;
    }
    if (plan.npass > 1) {  // multi-pass plans take the narrow parts (plan_xr_any)
        if constexpr (XC == xr_pass_codes<BITS>()) {
            if (plan.sbw == 4) {
                if (fused)
                    hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 4, NST4, !BF16, false, BF16, true>), grid, block,
                                       lds, stream, xa);
                else
                    hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 4, NST4, false, false, BF16, true>), grid, block,
                                       lds, stream, xa);
            } else {
                if (fused)
                    hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 2, NST2, !BF16, false, BF16, true>), grid, block,
                                       lds, stream, xa);
                else
                    hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 2, NST2, false, false, BF16, true>), grid, block,
                                       lds, stream, xa);
            }
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (plan.sbw == 4) {
        if (fused)
            hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 4, NST4, !BF16, false, BF16>), grid, block, lds, stream, xa);
        else
            hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 4, NST4, false, false, BF16>), grid, block, lds, stream, xa);
    } else {
        if (fused)
            hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 2, NST2, !BF16, false, BF16>), grid, block, lds, stream, xa);
        else
            hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 2, NST2, false, false, BF16>), grid, block, lds, stream, xa);
    }
    return hipGetLastError();
}


template <int BITS, int G>
bool plan_xr_any(const ProductArgs &a, XrPlan &plan, int &xc)
{
    if (plan_xr<BITS, G, xr_small_codes<BITS>()>(a, plan)) {
        xc = xr_small_codes<BITS>();
        return true;
    }
    if (plan_xr<BITS, G, xr_large_codes<BITS>()>(a, plan)) {
        xc = xr_large_codes<BITS>();
        return true;
    }
    // K too long for one pass: the narrow parts, several per wave
    if (plan_xr<BITS, G, xr_pass_codes<BITS>()>(a, plan, kXrMaxPasses)) {
        xc = xr_pass_codes<BITS>();
        return true;
    }
    return false;
}

// Whether a one-pass, one-slice plan and a one-pass, two-slice plan of the
// same variant cut K into the same parts (slice z's parts being parts
// z*KP/2 .. z*KP/2 + KP/2 - 1 of the one slice).
template <int G>
bool xr_same_parts(const ProductArgs &a, const XrPlan &one, int xc1, const XrPlan &two, int xc2)
{
    if (xc1 != xc2 || one.npass != 1 || two.npass != 1 || one.KP != 2 * two.KP || one.gran != two.gran ||
        one.sbw != two.sbw)
        return false;
    const int Kg = a.K / G;
    for (int z = 0; z < 2; ++z) {
        int gb, ge;
        slice_groups(Kg, 2, z, gb, ge);
        for (int kp = 0; kp < two.KP; ++kp) {
            int b1, e1, b2, e2;
            part_range(0, Kg, one.KP, z * two.KP + kp, one.gran, b1, e1);
            part_range(gb, ge, two.KP, kp, two.gran, b2, e2);
            if (b1 != b2 || e1 != e2)
                return false;
        }
    }
    return true;
}

template <int BITS, int G, bool BF16>
hipError_t launch_xr_t(const ProductArgs &a, hipStream_t stream, bool &done)
{
    XrPlan plan;
    int xc = 0;
    done = plan_xr_any<BITS, G>(a, plan, xc);
    if (!done)
        return hipSuccess;
    // Two half-K slices on twice the workgroups, each adding its tiles into y
    // (zeroed first); exactly two addends reach each output, so the result
    // does not depend on their order.
    //  * Long K (several passes per wave in one slice): 26.6 against 30.2 us
    //    on the 17408 x 5120 4-bit projection at M = 16.
    //  * Small N, when the one-slice grid leaves at least half the CUs idle:
    //    the halves' workgroups still get a CU each and every chain is half as
    //    long (8.7 against 9.5 us at N = 1024 and K = 5120, 9.3 against 10.4
    //    for 8-bit G64 codes at N = 2048; M = 16). Taken only where the halves
    //    cut K into the one-slice launch's parts, whose epilogue sums the two
    //    halves of its parts apart: both launches then give the same bits,
    //    so fused and separate calls agree whichever of the two they take.
    const bool small_n = plan.npass == 1 && plan.KP % 2 == 0 && 2 * xr_grid_x(a, plan.KP, 1) <= device_cu_count();
    if ((plan.npass > 1 || small_n) && a.split == 1) {
        ProductArgs h = a;
        h.split = 2;
        h.y_slice_stride = 0;
        XrPlan hp;
        int hxc = 0;
        if (plan_xr_any<BITS, G>(h, hp, hxc) && (plan.npass > 1 || xr_same_parts<G>(a, plan, xc, hp, hxc))) {
            for (int j = 0; j < (a.nproj >= 2 ? a.nproj : 1); ++j) {
                const Proj &pj = a.nproj >= 2 ? a.proj[j] : Proj{a.wq, a.scales, a.biases, a.y, a.N};
                const hipError_t e = launch_zero(pj.y, (size_t)a.M * pj.N, stream);
                if (e != hipSuccess)
                    return e;
            }
            if (hxc == xr_small_codes<BITS>())
                return launch_xr_variant<BITS, G, xr_small_codes<BITS>(), BF16>(h, hp, stream, true);
            if constexpr (xr_large_codes<BITS>() != xr_small_codes<BITS>())
                return launch_xr_variant<BITS, G, xr_large_codes<BITS>(), BF16>(h, hp, stream, true);
            return hipErrorInvalidValue;
        }
    }
    if (xc == xr_small_codes<BITS>())
        return launch_xr_variant<BITS, G, xr_small_codes<BITS>(), BF16>(a, plan, stream);
    if constexpr (xr_large_codes<BITS>() != xr_small_codes<BITS>())
        return launch_xr_variant<BITS, G, xr_large_codes<BITS>(), BF16>(a, plan, stream);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Tiled layout: repack and the product on it.
// ---------------------------------------------------------------------------

// One thread per output byte of the tiled codes: byte p of unit u of lane
// L = 16c + i of tile t is byte (16u + p) of that lane's stream, i.e. byte
// (16u + p) % CB of group g = (16u + p) / CB's chunk c of row 16t + i, whose
// codes start at stream bit (g*G + c*G/4)*BITS of the row.
template <int BITS, int G>
__global__ __launch_bounds__(256) void repack_codes_kernel(const uint32_t *__restrict__ wq,
                                                           uint8_t *__restrict__ out, int N, int K,
                                                           size_t total)
{
    constexpr int CB = tiled_chunk_bytes<BITS, G>();
    const uint32_t UB = (uint32_t)K * BITS / 512;
    const size_t wpr = (size_t)K * BITS / 32;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int p = (int)(idx % 16);
        const int L = (int)((idx / 16) % 64);
        const size_t tu = idx / 1024;  // t * UB + u
        const size_t t = tu / UB;
        const int u = (int)(tu % UB);
        const int c = L / 16, i = L % 16;
        const size_t n = t * 16 + i;
        uint8_t v = 0;
        if (n < (size_t)N) {
            const int sb = 16 * u + p;  // byte of the lane stream
            const int g = sb / CB;
            const size_t bit = ((size_t)g * G + (size_t)c * (G / 4)) * BITS + (size_t)(sb % CB) * 8;
            const uint32_t *row = wq + n * wpr;
            v = (uint8_t)((row[bit / 32] >> (bit % 32)) & 0xffu);  // 8-bit aligned: never straddles words
        }
        out[idx] = v;
    }
}

// One thread per output word of the tiled (s, b) words.
__global__ __launch_bounds__(256) void repack_sb_kernel(const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ biases,
                                                        uint32_t *__restrict__ out, int N, int Kg,
                                                        size_t total)
{
    const int Kq = Kg / 4;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int e = (int)(idx % 4);
        const int i = (int)((idx / 4) % 16);
        const size_t tq = idx / 64;  // t * Kq + q
        const size_t t = tq / Kq;
        const int g = (int)(tq % Kq) * 4 + e;
        const size_t n = t * 16 + i;
        uint32_t v = 0;
        if (n < (size_t)N)
            v = (uint32_t)scales[n * Kg + g] | ((uint32_t)biases[n * Kg + g] << 16);
        out[idx] = v;
    }
}

template <int BITS, int G>
hipError_t launch_repack_t(const uint32_t *wq, const uint16_t *scales, const uint16_t *biases,
                           uint8_t *tw, uint32_t *tsb, int N, int K, hipStream_t stream)
{
    const size_t tiles = ((size_t)N + 15) / 16;
    const size_t wbytes = tiles * 16 * (size_t)K * BITS / 8;
    const size_t sbwords = tiles * 16 * (size_t)(K / G);
    auto grid = [](size_t work) {
        const size_t b = (work + 255) / 256;
        return dim3((unsigned)(b < 65536 ? (b ? b : 1) : 65536));
    };
    hipLaunchKernelGGL((repack_codes_kernel<BITS, G>), grid(wbytes), dim3(256), 0, stream, wq, tw, N, K, wbytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(repack_sb_kernel, grid(sbwords), dim3(256), 0, stream, scales, biases, tsb, N, K / G,
                       sbwords);
    return hipGetLastError();
}

// The product on tiled weights: parts must start on whole 16-byte units of
// the lane streams and on whole group quads.
template <int BITS, int G, int XC>
bool plan_xr_tiled(const ProductArgs &a, XrPlan &plan)
{
    using Geo = XrGeo<BITS, G, XC>;
    constexpr int CB = tiled_chunk_bytes<BITS, G>();
    const int Kg = a.K / G;
    if (((long long)a.K * BITS) % 512 != 0 || Kg % 4 != 0 || a.split != 1)
        return false;
    const int gran = CB >= 4 ? 4 : 16 / CB;
    const int per_part = Geo::XG / gran;
    if (per_part < 1)
        return false;
    const int nu = Kg / gran;
    const int KP = (nu + per_part - 1) / per_part;
    if (KP > kXrMaxParts || KP > nu || ((nu + KP - 1) / KP) * gran > Geo::XG)
        return false;
    plan = XrPlan{KP, gran, 4, 1};
    return true;
}

#ifndef XR_TILED_NST3
#define XR_TILED_NST3 2
#endif
// Register stages of the tiled variant: three while the stages and the
// activation registers stay within 200 VGPRs, else two.
template <int BITS, int G, int XC>
constexpr int xr_tiled_stages()
{
    using Geo = XrGeo<BITS, G, XC>;
    constexpr int per_stage = 4 * ((Geo::XG * tiled_chunk_bytes<BITS, G>() + 15) / 16 + Geo::XQ);
    return 3 * per_stage + 4 * Geo::XG * Geo::T <= 200 ? XR_TILED_NST3 : 2;
}

template <int BITS, int G, int XC>
hipError_t launch_xr_tiled_variant(const ProductArgs &a, const XrPlan &plan, hipStream_t stream)
{
    const int ntiles = (a.N + 15) / 16;
    const int per_cu = kXrMaxParts / plan.KP;
    const long long want = (long long)device_cu_count() * per_cu;
    const int gx = (int)(want < ntiles ? want : ntiles);
    XrShape sh;
    if (!xr_shape<BITS, G, XC, true>(a, plan.KP, 1, gx, sh))
        return hipErrorInvalidValue;
    XrArgs xa{a, plan.gran, ntiles, 1, sh.batch, sh.nbuf};
    const size_t lds = sh.lds;
    constexpr int NST = xr_tiled_stages<BITS, G, XC>();
    static std::atomic<uint64_t> allowed{0};
    {
        const void *fns[1] = {reinterpret_cast<const void *>(&mfma_xr_kernel<BITS, G, XC, 4, NST, false, true>)};
        const hipError_t e = allow_dynamic_lds(fns, 1, (int)kXrLdsLimit, allowed);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((mfma_xr_kernel<BITS, G, XC, 4, NST, false, true>), dim3(gx), dim3(plan.KP * kWave), lds,
                       stream, xa);
    return hipGetLastError();
}

template <int BITS, int G>
hipError_t launch_xr_tiled_t(const ProductArgs &a, hipStream_t stream, bool &done)
{
    XrPlan plan;
    done = true;
    if (plan_xr_tiled<BITS, G, xr_tiled_small_codes<BITS>()>(a, plan))
        return launch_xr_tiled_variant<BITS, G, xr_tiled_small_codes<BITS>()>(a, plan, stream);
    if constexpr (xr_tiled_large_codes<BITS>() != xr_tiled_small_codes<BITS>()) {
        if (plan_xr_tiled<BITS, G, xr_tiled_large_codes<BITS>()>(a, plan))
            return launch_xr_tiled_variant<BITS, G, xr_tiled_large_codes<BITS>()>(a, plan, stream);
    }
    done = false;
    return hipSuccess;
}

template <int BITS, int G>
bool tiled_supported_t(const ProductArgs &a)
{
    XrPlan plan;
    if (plan_xr_tiled<BITS, G, xr_tiled_small_codes<BITS>()>(a, plan))
        return true;
    return plan_xr_tiled<BITS, G, xr_tiled_large_codes<BITS>()>(a, plan);
}

}  // namespace

bool mfma_xr_supported(const ProductArgs &a, int bits, int G)
{
    XrPlan plan;
    int xc;
#define QMM_XR_CASE(B, GG) \
    if (bits == B && G == GG) return plan_xr_any<B, GG>(a, plan, xc);
    QMM_XR_CASE(2, 32) QMM_XR_CASE(2, 64) QMM_XR_CASE(2, 128)
    QMM_XR_CASE(3, 32) QMM_XR_CASE(3, 64) QMM_XR_CASE(3, 128)
    QMM_XR_CASE(4, 32) QMM_XR_CASE(4, 64) QMM_XR_CASE(4, 128)
    QMM_XR_CASE(5, 32) QMM_XR_CASE(5, 64) QMM_XR_CASE(5, 128)
    QMM_XR_CASE(6, 32) QMM_XR_CASE(6, 64) QMM_XR_CASE(6, 128)
    QMM_XR_CASE(8, 32) QMM_XR_CASE(8, 64) QMM_XR_CASE(8, 128)
#undef QMM_XR_CASE
    return false;
}

hipError_t launch_mfma_xr(const ProductArgs &a, int bits, int G, bool bf16, hipStream_t stream)
{
    bool done = false;
    hipError_t e = hipErrorInvalidValue;
    if (bf16 && a.nproj >= 2)
        return hipErrorInvalidValue;
#define QMM_XR_CASE(B, GG) \
    if (bits == B && G == GG) \
        e = bf16 ? launch_xr_t<B, GG, true>(a, stream, done) : launch_xr_t<B, GG, false>(a, stream, done);
    QMM_XR_CASE(2, 32) QMM_XR_CASE(2, 64) QMM_XR_CASE(2, 128)
    QMM_XR_CASE(3, 32) QMM_XR_CASE(3, 64) QMM_XR_CASE(3, 128)
    QMM_XR_CASE(4, 32) QMM_XR_CASE(4, 64) QMM_XR_CASE(4, 128)
    QMM_XR_CASE(5, 32) QMM_XR_CASE(5, 64) QMM_XR_CASE(5, 128)
    QMM_XR_CASE(6, 32) QMM_XR_CASE(6, 64) QMM_XR_CASE(6, 128)
    QMM_XR_CASE(8, 32) QMM_XR_CASE(8, 64) QMM_XR_CASE(8, 128)
#undef QMM_XR_CASE
    if (e == hipSuccess && !done)
        return hipErrorInvalidValue;
    return e;
}

#define QMM_TILED_CASES(X) \
    X(2, 32) X(2, 64) X(2, 128) X(4, 32) X(4, 64) X(4, 128) X(8, 32) X(8, 64) X(8, 128)

bool tiled_supported(const ProductArgs &a, int bits, int G)
{
#define QMM_TS(B, GG) \
    if (bits == B && G == GG) return tiled_supported_t<B, GG>(a);
    QMM_TILED_CASES(QMM_TS)
#undef QMM_TS
    return false;
}

hipError_t launch_repack_tiled(const uint32_t *wq, const uint16_t *scales, const uint16_t *biases, uint8_t *tw,
                               uint32_t *tsb, int N, int K, int bits, int G, hipStream_t stream)
{
#define QMM_RP(B, GG) \
    if (bits == B && G == GG) return launch_repack_t<B, GG>(wq, scales, biases, tw, tsb, N, K, stream);
    QMM_TILED_CASES(QMM_RP)
#undef QMM_RP
    return hipErrorInvalidValue;
}

hipError_t launch_mfma_tiled(const ProductArgs &a, int bits, int G, hipStream_t stream)
{
    bool done = false;
    hipError_t e = hipErrorInvalidValue;
#define QMM_TL(B, GG) \
    if (bits == B && G == GG) e = launch_xr_tiled_t<B, GG>(a, stream, done);
    QMM_TILED_CASES(QMM_TL)
#undef QMM_TL
    if (e == hipSuccess && !done)
        return hipErrorInvalidValue;
    return e;
}

}  // namespace qmm
