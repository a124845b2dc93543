// FP4 E2M1 / E4M3 codec pieces shared by the append kernels and the decode
// kernel that appends the step's new token itself.
//
// Number formats ("Quantising the KV cache", numerics-explained, Code
// section): E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with the sign in bit 3
// of the nibble; E4M3 (OCP FN) scales, bias 7, largest finite 448, smallest
// subnormal 2^-9.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"

namespace fp4kv {
namespace quant {

// E4M3 code of y >= 0 (finite), rounded to nearest even, saturating at 448.
// Subnormal range (y < 2^-6): the grid is 2^-9, so the code is rint(y * 512),
// exact because the product is exact and rint rounds half to even; 8 carries
// into the smallest normal, whose code is also 8.  Normal range: round the
// f32 significand to 3 bits (add half an ulp minus one, plus the kept LSB),
// then rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code_rne_sat(float y)
{
    if (y >= 448.0f)
        return 126u;
    if (y < 0.015625f)
        return static_cast<uint32_t>(__builtin_rintf(y * 512.0f));
    const uint32_t b = __float_as_uint(y);
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
    return r - (120u << 3);
}

// Value of an E4M3 magnitude code (the sign bit is ignored; 0x7F decodes to
// 480 instead of NaN so that never-written slots stay finite).
__device__ __forceinline__ float e4m3_value(uint32_t code)
{
    code &= 0x7Fu;
    return code < 8u ? static_cast<float>(code) * 0.001953125f
                     : __uint_as_float((code + (120u << 3)) << 20);
}

// Signed E2M1 value of a nibble (bit 3 sign, bits 2-1 exponent with bias 1,
// bit 0 mantissa).  Codes 2..7 map onto f32 by placing the 3 bits under an
// exponent offset of 126; code 1 is the subnormal 0.5 and code 0 is zero.
__device__ __forceinline__ float e2m1_value(uint32_t nib)
{
    const uint32_t c = nib & 7u;
    uint32_t bits = (c + 252u - (c == 1u ? 1u : 0u)) << 22;
    bits = c ? bits : 0u;
    return __uint_as_float(bits | ((nib & 8u) << 28));
}

// The quotient x / s rounded once to fp32, without a division per element:
// q = x * r with r ~ 1/s (the hardware reciprocal, within 1 ulp, once per
// block), then one Newton step with the exact residual, q - (q*s - x)*r, in
// two FMAs.  The residual is exact (q*s has at most 28 significant bits and
// lies within a few ulps of x), so the result is within about 2^-44
// (relative) of the exact quotient.  A bf16 x over an
// E4M3 s is either exactly an E2M1 rounding midpoint (0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5) or at least 2^-8 (relative) away from every one, so the
// corrected quotient rounds to the same E2M1 code as the exact one, ties
// included (an exact midpoint comes out exactly).  The plain product x * r
// does not: with s = 1.875 * 2^k it overshoots the ties at 1.25, 2.5 and 5.
// Checked on the CPU for every bf16 value and every scale; within a block
// |x| / s stays below 9 (s is rounded from amax / 6), so nothing overflows.
__device__ __forceinline__ float quotient(float x, float s, float r)
{
    const float q = x * r;
    return __builtin_fmaf(-__builtin_fmaf(q, s, -x), r, q);
}

// Channels 2i, 2i+1 (the dword w of two bf16 values) into byte I of d.
template <int I>
__device__ __forceinline__ uint32_t pack_pair(uint32_t d, uint32_t w, float s, float r)
{
    const float x0 = __uint_as_float(w << 16);
    const float x1 = __uint_as_float(w & 0xFFFF0000u);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, quotient(x0, s, r), quotient(x1, s, r), 1.0f, I);
}

// Quantise one block of 16 bf16 values held as 8 dwords (low half = even
// channel).  Returns the 16 nibbles packed low-to-high (channel 2i in the low
// nibble of byte i) and the scale code.  The E2M1 rounding (nearest, ties to
// even, saturating at 6, sign kept) is the hardware conversion, two values
// per instruction, applied to the exactly rounding quotient above with a
// unit scale (the conversion would use only the exponent of a scale).
__device__ __forceinline__ void quantize_block16(const uint32_t w[8], uint32_t &lo, uint32_t &hi,
                                                 uint32_t &scale_code)
{
    // bf16 magnitudes as unsigned 16-bit integers order like the values:
    // two channels per packed max
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m2 = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    const uint32_t amax = max(static_cast<uint32_t>(m2.x), static_cast<uint32_t>(m2.y));
    // amax / 6 in correctly rounded fp32 gives the same E4M3 code as the exact
    // quotient for every bf16 amax (checked exhaustively against the oracle).
    // It is formed without a division: q = amax * RN(1/6), then one Newton
    // step with the exact residual, which rounds correctly (Markstein's
    // condition: a correctly rounded reciprocal; also checked for every bf16).
    const float a = __uint_as_float(amax << 16);
    constexpr float kSixth = 0x1.555556p-3f;            // RN(1/6)
    const float q6 = a * kSixth;
    uint32_t sc = e4m3_code_rne_sat(__builtin_fmaf(__builtin_fmaf(-q6, 6.0f, a), kSixth, q6));
    sc = sc ? sc : 1u;                                  // zero scale -> smallest subnormal
    scale_code = sc;
    const float s = e4m3_value(sc);
    const float r = __builtin_amdgcn_rcpf(s);
    lo = pack_pair<0>(0u, w[0], s, r);
    lo = pack_pair<1>(lo, w[1], s, r);
    lo = pack_pair<2>(lo, w[2], s, r);
    lo = pack_pair<3>(lo, w[3], s, r);
    hi = pack_pair<0>(0u, w[4], s, r);
    hi = pack_pair<1>(hi, w[5], s, r);
    hi = pack_pair<2>(hi, w[6], s, r);
    hi = pack_pair<3>(hi, w[7], s, r);
}

// -------------------------------------------------------- quantise / append

// Page-local placement of V.  Codes: the page's 64 tokens form 4 slices of
// 16; row (slice, channel) is 8 bytes and byte b holds tokens 2b (low nibble)
// and 2b + 1 (high nibble) of the slice.  Scales: row (slice, 16-channel
// block) is 16 bytes, one per token of the slice.
template <int D>
__device__ __forceinline__ int v_code_row(int t, int c) { return ((t >> 4) * D + c) * 8; }
template <int D>
__device__ __forceinline__ int v_scale_byte(int t, int blk) { return ((t >> 4) * (D / 16) + blk) * 16 + (t & 15); }

__device__ __forceinline__ void load_block16(const uint16_t *src, uint32_t w[8])
{
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
    const uint4 x0 = p[0], x1 = p[1];
    w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
    w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
}

// E4M3 code of |x| / s, rounded to nearest even and saturating at 448
// ("Quantising the KV cache", Concept section, results table: FP8 E4M3
// with one scale per tensor; rounding as the page's encoder does it).  The
// fp32 quotient is correctly rounded, so it lies on the same side of every
// E4M3 rounding midpoint as the exact quotient, except that it can land
// exactly on one; then the sign of q*s - |x|, exact in one FMA, decides.
// The bound on s (2^-64 .. 2^64, checked on the host) keeps that FMA's
// result away from underflow.
__device__ __forceinline__ uint32_t fp8_code(uint32_t bits16, float s)
{
    const float x = __uint_as_float((bits16 & 0x7FFFu) << 16);
    const float q = x / s;
    uint32_t c;
    if (!(q < 448.0f)) {
        c = 126u;
    } else {
        c = e4m3_code_rne_sat(q);
        uint32_t lo;
        bool mid;
        if (q < 0.015625f) {                            // subnormal grid 2^-9
            const float t = q * 512.0f;                 // exact
            const float f = __builtin_floorf(t);
            lo = static_cast<uint32_t>(f);
            mid = t - f == 0.5f;
        } else {
            const uint32_t b = __float_as_uint(q);
            lo = (b >> 20) - (120u << 3);               // truncated: the lower neighbour
            mid = (b & 0xFFFFFu) == 0x80000u;
        }
        if (mid) {
            const float r = __builtin_fmaf(q, s, -x);
            c = r > 0.0f ? lo : (r < 0.0f ? lo + 1u : c);
        }
    }
    return c | ((bits16 >> 8) & 0x80u);
}

// ---- fp16 scales (FP8 with a scale per token; the sweep's formats)

__device__ __forceinline__ float fp16_value(uint32_t code)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(code)));
}

// fp16 code of amax / div (div a positive integer of at most 9 significant
// bits: an integer format's qmax, or 448 for E4M3 elements): nearest even,
// saturating at 65504, and the smallest subnormal (code 1) in place of zero.
// The correctly rounded fp32 quotient lies on the same side of every fp16
// midpoint (an fp32 number) as the exact one, or on it; then the sign of
// mid * div - amax, exact in one FMA, decides.
__device__ __forceinline__ uint32_t fp16_scale_code(float amax, float div)
{
    const float q = amax / div;
    uint32_t code;
    if (!(q < 65504.0f)) {
        code = 0x7BFFu;
    } else {
        code = __builtin_bit_cast(uint16_t, static_cast<_Float16>(q));
        const float f = fp16_value(code);
        if (f != q) {
            const uint32_t other = q > f ? code + 1u : code - 1u;   // the neighbour on q's side
            const float mid = 0.5f * (f + fp16_value(other));
            if (q == mid) {
                const float r = __builtin_fmaf(mid, div, -amax);   // sign of mid * div - amax
                if (r > 0.0f)
                    code = code < other ? code : other;
                else if (r < 0.0f)
                    code = code > other ? code : other;
            }
        }
    }
    return code == 0u ? 1u : code;
}

// The fp16 scale code of one token's row of one KV head (E4M3 elements:
// amax / 448) from its 16-channel blocks, one block per lane in NB
// consecutive, NB-aligned lanes that all take part: the block maxima (as
// bf16 magnitude bits, which order like the values) meet by lane shuffles.
template <int NB>
__device__ __forceinline__ uint32_t row_scale_code_e4m3(const uint32_t w[8])
{
    uint32_t am = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        am = lo > am ? lo : am;
        am = hi > am ? hi : am;
    }
#pragma unroll
    for (int o = 1; o < NB; o <<= 1) {
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), o));
        am = other > am ? other : am;
    }
    return fp16_scale_code(__uint_as_float(am << 16), 448.0f);
}

// ---- the decode step's own token, appended inside the decode kernel

// Quantise one token's K and V rows of one KV head (bf16, D channels each)
// and store them at page offset `off` of the (page, KV head) block at `base`,
// with one wave: lanes 0 .. D/16-1 take the K blocks, the next D/16 lanes the
// V blocks (FP8 with per-token scales: each group also finds its row's
// scale and its first lane stores it).  The caller guarantees that no other thread writes this block
// during the kernel, so the FP4 V nibbles (two tokens per byte) are placed
// by a plain read-modify-write of their dwords.
template <int D, bool FP8>
__device__ __forceinline__ void append_token_in_wave(const CacheGeom &g, const uint16_t *k_row,
                                                     const uint16_t *v_row, uint8_t *base, int off, int lane)
{
    constexpr int NB = D / 16;
    if (lane >= 2 * NB)
        return;
    const bool is_v = lane >= NB;
    const int blk = is_v ? lane - NB : lane;
    uint32_t w[8];
    load_block16((is_v ? v_row : k_row) + 16 * blk, w);
    if constexpr (FP8) {
        float s = is_v ? g.v_scale : g.k_scale;
        if (g.token_scales) {
            // the K lanes and the V lanes are two NB-lane groups
            const uint32_t sc = row_scale_code_e4m3<NB>(w);
            s = fp16_value(sc);
            if (blk == 0)
                *reinterpret_cast<uint16_t *>(base + (is_v ? g.v_scales_off : g.k_scales_off) + 2 * off) =
                    static_cast<uint16_t>(sc);
        }
        uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            c[i >> 2] |= fp8_code(bits, s) << (8 * (i & 3));
        }
        if (!is_v) {
            *reinterpret_cast<uint4 *>(base + g.k_codes_off + off * D + 16 * blk) = make_uint4(c[0], c[1], c[2], c[3]);
        } else {
            uint8_t *vrow = base + g.v_codes_off + ((((off >> 4) * 2 + ((off >> 3) & 1)) * D + 16 * blk) * 8) + (off & 7);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                vrow[8 * i] = static_cast<uint8_t>(c[i >> 2] >> (8 * (i & 3)));
        }
    } else {
        uint32_t lo, hi, sc;
        quantize_block16(w, lo, hi, sc);
        if (!is_v) {
            *reinterpret_cast<uint2 *>(base + g.k_codes_off + off * (D / 2) + 8 * blk) = make_uint2(lo, hi);
            base[g.k_scales_off + off * (D / 16) + blk] = static_cast<uint8_t>(sc);
        } else {
            const int shift = 4 * (off & 7);
            const int word = ((off & 15) >> 3) * 4;
            uint32_t *dw[16];
            uint32_t cur[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                dw[i] = reinterpret_cast<uint32_t *>(base + g.v_codes_off + v_code_row<D>(off, 16 * blk + i) + word);
                cur[i] = *dw[i];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t nib = ((i < 8 ? lo : hi) >> (4 * (i & 7))) & 0xFu;
                *dw[i] = (cur[i] & ~(0xFu << shift)) | (nib << shift);
            }
            base[g.v_scales_off + v_scale_byte<D>(off, blk)] = static_cast<uint8_t>(sc);
        }
    }
}

}  // namespace quant
}  // namespace fp4kv
