// Device-side building blocks shared by the gfx950 kernels: vector types,
// the in-register code unpack/widen path, the activation permutation that
// matches it, and wavefront reductions.
//
// The unpack follows the factored evaluation of the vmlx-swift pull request
// #565 page, commit "LaneQMM": raw b-bit codes are widened to exact fp16
// integers and multiplied with the activations; the scale and bias are
// applied to the group's dot product afterwards (C += s*P + b*XS). The same
// page's qwen_mixed_qmv commit attributes a compute-bound one-row mat-vec to
// inner loops with run-time bounds that cannot unroll; every loop bound and
// bit offset here is a compile-time constant of (bits, G).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qmm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------------------
// Pairing of codes into fp16 pairs.
//
// A 32-bit window of the bitstream holds two codes, one in each 16-bit half,
// each entirely inside the half's 10 fraction bits at offset o (o + bits <= 10).
// OR-ing the exponent of 2^(10-o) into that half turns the bits into the fp16
// number 2^(10-o) + code exactly; subtracting 2^(10-o) then leaves the code
// as an exact fp16 integer. One window, one mask-or and one packed subtract
// give two codes.
//
// Codes are paired (i, i+d) inside blocks of 2d consecutive codes, with d
// chosen per width so that code i+d always lands in the upper half of a
// window whose lower half holds code i:
//   bits 2: d = 4 ( 8 bits apart)   bits 3: d = 4 (12 bits apart)
//   bits 4: d = 4 (16 bits apart)   bits 5: d = 4 (20 bits apart)
//   bits 6: d = 2 (12 bits apart)   bits 8: d = 2 (16 bits apart)
// Pair P of a run of codes therefore holds codes lo(P) and lo(P) + d, and
// the activations are stored in the same pair order ("permuted order").
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int pair_dist(int bits) { return bits <= 5 ? 4 : 2; }

// Index (within a run of codes starting at a block boundary) of the lower
// code of pair P, and of the code at permuted position `pos`.
__host__ __device__ constexpr int pair_lo(int bits, int P)
{
    return 2 * pair_dist(bits) * (P / pair_dist(bits)) + P % pair_dist(bits);
}
__host__ __device__ constexpr int perm_code(int bits, int pos)
{
    return pair_lo(bits, pos / 2) + ((pos & 1) ? pair_dist(bits) : 0);
}

// Offset of the lower code inside the lower half: within the allowed range,
// prefer one that puts the window start on a byte boundary.
__host__ __device__ constexpr int pair_lo_offset(int bits, int p_lo)
{
    const int D = bits * pair_dist(bits) - 16;      // o_hi - o_lo
    const int lo_min = D < 0 ? -D : 0;
    const int lo_max = (10 - bits) - (D > 0 ? D : 0);
    for (int o = lo_min; o <= lo_max; ++o)
        if (((p_lo - o) % 8 + 8) % 8 == 0)
            return o;
    return lo_min;
}

__host__ __device__ constexpr uint32_t half_pow2_bits(int e) { return (uint32_t)(15 + e) << 10; }

// 32-bit window of the stream starting at bit S (S may be negative: the
// bits below 0 read as zero). The words hold the stream from bit 0.
template <int S, int NW>
__device__ __forceinline__ uint32_t stream_window(const uint32_t (&w)[NW])
{
    if constexpr (S < 0) {
        return w[0] << (-S);
    } else {
        constexpr int j = S / 32, r = S % 32;
        static_assert(j < NW, "window starts past the loaded words");
        if constexpr (r == 0)
            return w[j];
        else if constexpr (j + 1 < NW)
            return __builtin_amdgcn_alignbit(w[j + 1], w[j], r);
        else
            return w[j] >> r;
    }
}

// fp16 pair (code lo(P), code lo(P)+d) of a run of codes stored from bit 0 of w.
template <int BITS, int P, int NW>
__device__ __forceinline__ half2_t code_pair(const uint32_t (&w)[NW])
{
    constexpr int d = pair_dist(BITS);
    constexpr int i = pair_lo(BITS, P);
    constexpr int p_lo = BITS * i;
    constexpr int o_lo = pair_lo_offset(BITS, p_lo);
    constexpr int o_hi = o_lo + BITS * d - 16;
    static_assert(o_lo >= 0 && o_lo + BITS <= 10, "low code does not fit the fraction");
    static_assert(o_hi >= 0 && o_hi + BITS <= 10, "high code does not fit the fraction");
    static_assert(BITS * (i + d) + BITS <= 32 * NW, "pair reads past the loaded words");
    constexpr uint32_t code_mask = (1u << BITS) - 1u;
    constexpr uint32_t mask = (code_mask << o_lo) | (code_mask << (16 + o_hi));
    constexpr uint32_t magic = half_pow2_bits(10 - o_lo) | (half_pow2_bits(10 - o_hi) << 16);
    const uint32_t win = stream_window<p_lo - o_lo>(w);
    const half2_t v = __builtin_bit_cast(half2_t, (win & mask) | magic);
    const half2_t off = {(_Float16)(float)(1 << (10 - o_lo)), (_Float16)(float)(1 << (10 - o_hi))};
    return v - off;
}

// v_and_or_b32 (x & mask) | magic. The compiler does not fuse the two
// operations when both constants are literals, so it is written out.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
    return r;
}

// 4-bit codes take a cheaper route that needs no exponent at all: a 16-bit
// half whose exponent field is zero is the fp16 subnormal (fraction) * 2^-24,
// so a code moved to bits 4..7 of its half, with every other bit cleared,
// is exactly q * 2^-20. Each pair costs one shift (none for P = 1) and one
// mask: three shifts and four ands per word, and no constant to remove
// afterwards. The matrix cores and v_dot2 multiply fp16 subnormals exactly
// (no flush to zero on gfx950), so the group dot product comes out as
// 2^-20 * P; the epilogue multiplies by CodeScale<4>::value = 2^20 (a power of
// two, so no rounding is added).
template <int P>
__device__ __forceinline__ half2_t code_pair4(uint32_t word)
{
    constexpr uint32_t mask = 0x00F000F0u;          // bits 4..7 of each half
    uint32_t v;
    if constexpr (P == 0)
        v = word << 4;
    else if constexpr (P == 1)
        v = word;
    else if constexpr (P == 2)
        v = word >> 4;
    else
        v = word >> 8;
    return __builtin_bit_cast(half2_t, v & mask);
}

// The subnormal form suits the matrix cores only. v_dot2_f32_f16 accumulates
// products of subnormal operands with reduced precision (tens of ulps on
// gfx950, measured), so the v_dot2 kernels widen 4-bit codes to normal fp16
// integers instead: pairs 0 and 2 of a word (bits 0..3 of each half, from
// the word and the word shifted by 8) become 1024 + q under the exponent of
// 2^10, pairs 1 and 3 (bits 4..7) become 64 + q under 2^6, and one packed
// subtract removes the constant exactly. One shift, four v_and_or_b32 and
// four v_pk_add_f16 per word; the codes come out as exact integers (scale 1).
template <int P>
__device__ __forceinline__ half2_t code_pair4_int(uint32_t word, uint32_t word_hi)
{
    constexpr bool low = P % 2 == 0;
    constexpr uint32_t mask = low ? 0x000F000Fu : 0x00F000F0u;
    constexpr uint32_t magic = low ? 0x64006400u : 0x54005400u;  // 2^10 or 2^6 in each half
    const half2_t v = __builtin_bit_cast(half2_t, and_or(P < 2 ? word : word_hi, mask, magic));
    const _Float16 off = low ? (_Float16)1024.0f : (_Float16)64.0f;
    return v - half2_t{off, off};
}

// Factor that turns a widened-code dot product into the true one.
template <int BITS>
struct CodeScale {
    static constexpr float value = BITS == 4 ? 1048576.0f : 1.0f;          // 2^20
    static constexpr float inverse = BITS == 4 ? 1.0f / 1048576.0f : 1.0f; // 2^-20
};

// The 8 activations of one MFMA K-block (8 consecutive codes of a lane's
// chunk) rearranged into the pair order of unpack_pairs.
template <int BITS>
__device__ __forceinline__ half8_t to_pair_order(half8_t v)
{
    if constexpr (pair_dist(BITS) == 4)
        return __builtin_shufflevector(v, v, 0, 4, 1, 5, 2, 6, 3, 7);
    else
        return __builtin_shufflevector(v, v, 0, 2, 1, 3, 4, 6, 5, 7);
}

template <int BITS, int NW, int... Ps>
__device__ __forceinline__ void unpack_pairs_impl(const uint32_t (&w)[NW], half2_t *out,
                                                  std::integer_sequence<int, Ps...>)
{
    if constexpr (BITS == 4)
        ((out[Ps] = code_pair4<Ps % 4>(w[Ps / 4])), ...);
    else
        ((out[Ps] = code_pair<BITS, Ps>(w)), ...);
}

// 4-bit codes as exact fp16 integers for v_dot2 (code_pair4_int): pair P of
// word j is out[4j + P], in the pair order of unpack_pairs.
template <int NCODES, int NW>
__device__ __forceinline__ void unpack_pairs4_int(const uint32_t (&w)[NW], half2_t (&out)[NCODES / 2])
{
    static_assert(NCODES == 8 * NW, "one word per 8 codes");
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const uint32_t hi = w[j] >> 8;
        out[4 * j + 0] = code_pair4_int<0>(w[j], hi);
        out[4 * j + 1] = code_pair4_int<1>(w[j], hi);
        out[4 * j + 2] = code_pair4_int<2>(w[j], hi);
        out[4 * j + 3] = code_pair4_int<3>(w[j], hi);
    }
}

// Widen NCODES codes (stored from bit 0 of w) into NCODES/2 fp16 pairs in
// pair order: exact integers for 2, 3, 5, 6 and 8 bits, q * 2^-20 for 4 bits.
template <int BITS, int NCODES, int NW>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[NW], half2_t (&out)[NCODES / 2])
{
    static_assert(NCODES % (2 * pair_dist(BITS)) == 0, "runs must hold whole pairing blocks");
    unpack_pairs_impl<BITS, NW>(w, out, std::make_integer_sequence<int, NCODES / 2>{});
}

// ---------------------------------------------------------------------------
// bf16 widening (activations, scales and biases in bf16).
//
// A bf16 number has 7 fraction bits and no exponent trick leaves a code
// without an offset except a subnormal, whose products with bf16 activations
// would fall among the fp32 subnormals. Codes are therefore converted
// exactly: each code becomes an fp32 integer and two of them are packed to
// bf16 with round-to-nearest (exact, every code is an integer below 2^8).
// For 4-bit codes the nibbles are first split into the bytes of two words
// (codes 0, 2, 4, 6 and 1, 3, 5, 7), so that every code converts with one
// v_cvt_f32_ubyte; other widths extract each code with a bit-field read.
// Pairs hold consecutive codes (2i, 2i + 1) and the activations keep their
// natural order.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Code k of a run of codes stored from bit 0 of w.
template <int BITS, int K, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW])
{
    static_assert(K * BITS + BITS <= 32 * NW, "code past the loaded words");
    return stream_window<K * BITS>(w) & ((1u << BITS) - 1u);
}

// Pair P (codes 2P, 2P + 1) of the 8 codes of a 4-bit word, from the word's
// even nibbles (lo = w & 0x0F0F0F0F) and odd nibbles (hi = (w >> 4) & ...).
template <int P>
__device__ __forceinline__ bf16x2_t code_pair4_bf16(uint32_t lo, uint32_t hi)
{
    const float a = (float)((lo >> (8 * P)) & 0xffu);
    const float b = (float)((hi >> (8 * P)) & 0xffu);
    return bf16x2_t{(__bf16)a, (__bf16)b};
}

template <int BITS, int NW, int... Ps>
__device__ __forceinline__ void unpack_pairs_bf16_impl(const uint32_t (&w)[NW], bf16x2_t *out,
                                                       std::integer_sequence<int, Ps...>)
{
    if constexpr (BITS == 4) {
        uint32_t lo[NW], hi[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            lo[j] = w[j] & 0x0F0F0F0Fu;
            hi[j] = (w[j] >> 4) & 0x0F0F0F0Fu;
        }
        ((out[Ps] = code_pair4_bf16<Ps % 4>(lo[Ps / 4], hi[Ps / 4])), ...);
    } else {
        ((out[Ps] = bf16x2_t{(__bf16)(float)code_at<BITS, 2 * Ps>(w),
                             (__bf16)(float)code_at<BITS, 2 * Ps + 1>(w)}), ...);
    }
}

// Widen NCODES codes into NCODES/2 bf16 pairs of exact integers in natural
// order.
template <int BITS, int NCODES, int NW>
__device__ __forceinline__ void unpack_pairs_bf16(const uint32_t (&w)[NW], bf16x2_t (&out)[NCODES / 2])
{
    static_assert(NCODES % 8 == 0, "runs of whole 8-code units");
    unpack_pairs_bf16_impl<BITS, NW>(w, out, std::make_integer_sequence<int, NCODES / 2>{});
}

// The 8 activations of a unit (bf16 bit patterns) in the order of
// unpack_pairs_bf16: natural order.
template <int BITS>
__device__ __forceinline__ half8_t to_pair_order_bf16(half8_t v)
{
    return v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16)
{
    return __builtin_bit_cast(float, h16 << 16);
}

// ---------------------------------------------------------------------------
// Loads of NW consecutive words with a known byte alignment. Packed weights
// are read once per call, so the loads carry the non-temporal hint unless
// QMM_WEIGHT_LOADS_NT is defined to 0.
// ---------------------------------------------------------------------------
#ifndef QMM_WEIGHT_LOADS_NT
#define QMM_WEIGHT_LOADS_NT 1
#endif

template <typename T>
__device__ __forceinline__ T load_weight(const T *p)
{
#if QMM_WEIGHT_LOADS_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

template <int NW, int ALIGN>
__device__ __forceinline__ void load_words(const uint32_t *__restrict__ p, uint32_t (&w)[NW])
{
    if constexpr (ALIGN >= 16 && NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = load_weight(reinterpret_cast<const u32x4 *>(p) + i);
            w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if constexpr (ALIGN >= 8 && NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) {
            const u32x2 v = load_weight(reinterpret_cast<const u32x2 *>(p) + i);
            w[2 * i + 0] = v.x; w[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i)
            w[i] = load_weight(p + i);
    }
}

__host__ __device__ constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// Empty asm that claims to modify v: nothing computed from v can be moved
// above this point. Used where a register stage is consumed, so that work on
// loads still in flight is not hoisted (which would force an early wait).
template <typename T>
__device__ __forceinline__ void pin_register(T &v)
{
    asm volatile("" : "+v"(v));
}

// Lanes of one wave that hand data to each other through LDS (one lane
// writes, other lanes of the same wave read, or a region is rewritten after
// other lanes read it) need no workgroup barrier: a wave's LDS instructions
// execute in program order. What they need is that the compiler keeps that
// order: in the per-thread memory model those accesses look unrelated
// (other lanes' addresses, and different types for the same bytes), so it
// could otherwise move them past each other. The wavefront-scope fences and
// the wave barrier pin every LDS access on its side; they emit no wait.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// base + a 32-bit byte offset: with a wave-uniform base this maps onto the
// scalar-base + 32-bit vector-offset addressing of global loads.
template <typename T>
__device__ __forceinline__ const T *byte_offset(const T *base, uint32_t bytes)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + bytes);
}

// ---------------------------------------------------------------------------
// Wavefront (64-lane) reductions.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x124>(v);  // row_ror:4
    v += dpp_f32<0x128>(v);  // row_ror:8
    return v;
}

// Sum over all 64 lanes, returned to every lane (a wave-uniform value).
__device__ __forceinline__ float wave_sum(float v)
{
    v = row16_sum(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

}  // namespace qmm
