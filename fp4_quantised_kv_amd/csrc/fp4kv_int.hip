// KV formats of the bit-width sweep: quantisers (per token, per channel) and
// a matrix-core decode attention over their codes.
//
// ("Quantising the KV cache", Concept section, results table: INT8, INT4 and
// INT2 with one scale per token, or K per channel and V per token; Maths
// section: one FP16 scale per group.  "KV Cache Quantisation", Common
// questions: FP8 scale granularities.)  The pages give no encoder for these;
// the symmetric nearest-even integer rule and the FP8 E4M3 rule used here are
// spelled out in fp4kv_int.h.  A template's FMT is the ABI's element format
// (2, 4, 8, 16 or FP4KV_INT_FP8_E4M3); BITS is its width in the codes.
//
// Exact rounding.  Both roundings (amax / qmax to fp16, |x| / scale to an
// integer) start from the correctly rounded fp32 quotient.  Every rounding
// boundary (an fp16 midpoint, an integer + 1/2) is an fp32 number, so the
// fp32 quotient lies on the same side of it as the exact quotient, or on it;
// in that last case the sign of boundary * divisor - dividend, exact in one
// FMA, says on which side the exact quotient lies.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_int.h"
#include "fp4kv_internal.h"
#include "fp4kv_merge.h"
#include "fp4kv_mfma_util.h"
#include "fp4kv_quant.h"

namespace fp4kv {
namespace {

constexpr int kE4M3 = FP4KV_INT_FP8_E4M3;
constexpr int fmt_bits(int fmt) { return fmt == kE4M3 ? 8 : fmt; }
constexpr int fmt_max(int fmt) { return fmt == kE4M3 ? 448 : (1 << (fmt - 1)) - 1; }   // divisor of amax

__device__ __forceinline__ float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

using quant::fp16_value;

// fp16 code of amax / qmax (qmax = 127, 7, 1 or 448): nearest even,
// saturating at 65504, and the smallest subnormal in place of zero.
__device__ __forceinline__ uint32_t int_scale_code(float amax, int qmax)
{
    return quant::fp16_scale_code(amax, static_cast<float>(qmax));
}

// sign(x) * nearest-even integer of |x| / s, capped at qmax.
__device__ __forceinline__ int int_code(uint32_t bits16, float s, int qmax)
{
    const float ax = bf16_value(bits16 & 0x7FFFu);
    const float q = ax / s;
    float r;
    if (!(q < static_cast<float>(qmax) + 0.5f)) {
        r = static_cast<float>(qmax);
    } else {
        r = rintf(q);
        const float fl = floorf(q);
        if (q - fl == 0.5f) {
            const float e = fmaf(q, s, -ax);                         // sign of q * s - |x|
            if (e > 0.0f)
                r = fl;
            else if (e < 0.0f)
                r = fl + 1.0f;
        }
    }
    const int c = static_cast<int>(r);
    return (bits16 & 0x8000u) ? -c : c;
}

__device__ __forceinline__ void load_row16(const uint16_t *src, uint32_t w[8])
{
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
    const uint4 x0 = p[0], x1 = p[1];
    w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
    w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
}

__device__ __forceinline__ uint32_t half16(const uint32_t w[8], int c)
{
    return (c & 1) ? (w[c >> 1] >> 16) : (w[c >> 1] & 0xFFFFu);
}

// 16 codes of BITS bits, packed little-endian (channel 16*blk + i in field i),
// stored at dst (16 * BITS / 8 bytes).
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t *dst, const int c[16])
{
    constexpr uint32_t mask = (1u << BITS) - 1u;
    constexpr int per = 32 / BITS;                      // codes per dword
    uint32_t d[16 * BITS / 32];
#pragma unroll
    for (int k = 0; k < 16 * BITS / 32; ++k) {
        d[k] = 0u;
#pragma unroll
        for (int n = 0; n < per; ++n)
            d[k] |= (static_cast<uint32_t>(c[k * per + n]) & mask) << (BITS * n);
    }
    if constexpr (BITS == 8)
        *reinterpret_cast<uint4 *>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
    else if constexpr (BITS == 4)
        *reinterpret_cast<uint2 *>(dst) = make_uint2(d[0], d[1]);
    else
        *reinterpret_cast<uint32_t *>(dst) = d[0];
}

// ------------------------------------------------------------- quantisers

// One thread per (sequence, token, KV head, 16-channel block).  The D/16
// threads of a row are consecutive lanes of one wave; they exchange their
// block maxima by lane shuffles.  BITS 16 copies the bf16 row to its
// head-major place.
template <int D, int FMT>
__global__ __launch_bounds__(256) void int_quantize_token(const uint16_t *__restrict__ x,
                                                          uint8_t *__restrict__ codes,
                                                          uint16_t *__restrict__ scales,
                                                          int64_t n_rows, int64_t T, int H)
{
    constexpr int NB = D / 16;
    constexpr int BITS = fmt_bits(FMT);
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool valid = idx < n_rows * NB;
    const int blk = static_cast<int>(idx % NB);
    const int64_t row = idx / NB;                       // (b * T + t) * H + h
    const int h = static_cast<int>(row % H);
    const int64_t bt = row / H;
    const int64_t t = bt % T, b = bt / T;
    const int64_t orow = (b * H + h) * T + t;           // head-major row
    uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (valid)
        load_row16(x + row * D + 16 * blk, w);
    if constexpr (BITS == 16) {
        if (valid) {
            uint4 *dst = reinterpret_cast<uint4 *>(codes + orow * (2 * D) + 32 * blk);
            dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
        return;
    } else {
        constexpr int qmax = fmt_max(FMT);
        uint32_t am = 0u;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint32_t m = half16(w, c) & 0x7FFFu;
            am = m > am ? m : am;
        }
#pragma unroll
        for (int o = 1; o < NB; o <<= 1) {               // every lane takes part, valid or not
            const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), o));
            am = other > am ? other : am;
        }
        if (!valid)
            return;
        const uint32_t sc = int_scale_code(bf16_value(am), qmax);
        const float s = fp16_value(sc);
        int c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            c[i] = FMT == kE4M3 ? static_cast<int>(quant::fp8_code(half16(w, i), s)) : int_code(half16(w, i), s, qmax);
        store_codes<BITS>(codes + orow * (D * BITS / 8) + blk * (2 * BITS), c);
        if (blk == 0)
            scales[orow] = static_cast<uint16_t>(sc);
    }
}

// Per-channel scales: one workgroup per (KV head, sequence) scans the T
// tokens; thread (token lane, channel pair) keeps the two channels' maxima,
// then the token lanes are merged in LDS.
template <int D>
__global__ __launch_bounds__(256) void int_channel_scales(const uint16_t *__restrict__ x,
                                                          uint16_t *__restrict__ scales, int64_t T,
                                                          int qmax)
{
    constexpr int CP = D / 2;                           // channel pairs
    constexpr int TL = 256 / CP;                        // token lanes
    const int h = blockIdx.x, H = gridDim.x;
    const int64_t b = blockIdx.y;
    const int cp = threadIdx.x % CP, tl = threadIdx.x / CP;
    const int64_t stride = static_cast<int64_t>(H) * D / 2;   // dwords per token
    const uint32_t *src = reinterpret_cast<const uint32_t *>(x + (b * T * H + h) * D) + cp;
    uint32_t lo = 0u, hi = 0u;
    int64_t t = tl;
    for (; t + 3 * TL < T; t += 4 * TL) {               // four loads in flight
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = src[(t + i * TL) * stride];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l = v[i] & 0x7FFFu, u = (v[i] >> 16) & 0x7FFFu;
            lo = l > lo ? l : lo;
            hi = u > hi ? u : hi;
        }
    }
    for (; t < T; t += TL) {
        const uint32_t v = src[t * stride];
        const uint32_t l = v & 0x7FFFu, u = (v >> 16) & 0x7FFFu;
        lo = l > lo ? l : lo;
        hi = u > hi ? u : hi;
    }
    __shared__ uint32_t red[TL][D];
    red[tl][2 * cp] = lo;
    red[tl][2 * cp + 1] = hi;
    __syncthreads();
    if (threadIdx.x < D) {
        uint32_t am = 0u;
#pragma unroll
        for (int i = 0; i < TL; ++i)
            am = red[i][threadIdx.x] > am ? red[i][threadIdx.x] : am;
        scales[(b * H + h) * D + threadIdx.x] = static_cast<uint16_t>(int_scale_code(bf16_value(am), qmax));
    }
}

// Codes with per-channel scales: one thread per (sequence, token, KV head,
// 16-channel block), reading the block's 16 channel scales.
template <int D, int FMT>
__global__ __launch_bounds__(256) void int_quantize_channel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ scales,
                                                            uint8_t *__restrict__ codes,
                                                            int64_t n_rows, int64_t T, int H)
{
    constexpr int NB = D / 16;
    constexpr int BITS = fmt_bits(FMT);
    constexpr int qmax = fmt_max(FMT);
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n_rows * NB)
        return;
    const int blk = static_cast<int>(idx % NB);
    const int64_t row = idx / NB;
    const int h = static_cast<int>(row % H);
    const int64_t bt = row / H;
    const int64_t t = bt % T, b = bt / T;
    uint32_t w[8], sw[8];
    load_row16(x + row * D + 16 * blk, w);
    load_row16(scales + (b * H + h) * D + 16 * blk, sw);
    int c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float s = fp16_value(half16(sw, i));
        c[i] = FMT == kE4M3 ? static_cast<int>(quant::fp8_code(half16(w, i), s)) : int_code(half16(w, i), s, qmax);
    }
    store_codes<BITS>(codes + ((b * H + h) * T + t) * (D * BITS / 8) + blk * (2 * BITS), c);
}

// ------------------------------------------------------------------ decode
//
// One workgroup per (KV head, sequence, split), four waves; wave w takes
// the split's token blocks w, w + 4, ... of TOK tokens.  Per block:
//   scores  S^T = K q^T on v_mfma_f32_16x16x32_bf16, one 16-token tile at a
//           time: A = 16 K rows (lane: row l%16, 8 channels of MFMA kk --
//           a quarter row per lane group l/16, or for bf16 channels 32kk +
//           8*(l/16) .. +7), B = the group's query rows (head l%16, the
//           same channels); the lane gets the scores of tokens 4*(l/16) + e
//           (e = 0..3) of the tile for head l%16;
//   softmax online, base 2, with a lazily moved reference maximum;
//   values  O^T += V^T P^T per 32 tokens (two tiles): A = V^T (row m =
//           channel (D/16)*m + j of MFMA j; k = the 8 tokens whose scores
//           the lane holds), B = those 8 probabilities of head l%16 -- the
//           lane's own score registers, so no data moves between the two
//           products; the lane accumulates head l%16 over channels
//           (l/16)*D/4 .. +D/4-1.
// Stored values reach the matrix cores exactly as bf16: bf16 as stored; an
// E4M3 code by the hardware conversion; an INT8 code as a signed byte
// converted to fp32 and truncated to bf16 (8 significant bits: exact).  INT4
// and INT2 codes take the hardware FP8 conversions too: a code c is made
// unsigned, u = c + 8 (INT4) or c + 2 (INT2), one per byte, and the byte
// read as E4M3 (INT4) or E5M2 (INT2), whose codes 0..15 and 0..3 stand for
// exactly u * 2^-9 and u * 2^-16 (the subnormals and the lowest binade are
// evenly spaced); the offset comes off afterwards as a multiple of the
// query's (or probabilities') sum, taken through the same operands.  The
// query is bf16 already; with per-channel K scales the exact fp32 product
// q * s is split into three bf16 terms (8 + 8 + 8 significant bits cover its
// 19).  The probabilities (times a per-token V scale) enter as hi + lo bf16
// terms, ~2^-15 relative.  Products are exact and accumulate in fp32.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int D, int FMT>
struct MfmaShape {
    static constexpr int BITS = fmt_bits(FMT);
    static constexpr int TOK = BITS == 16 || FMT == 8 ? 32 : 64;   // tokens per wave block
    static constexpr int NT = TOK / 16;                 // score tiles per block
    static constexpr int NS = TOK / 32;                 // value steps per block
    static constexpr int ROW = D * BITS / 8;            // bytes per token row
    static constexpr int KW = ROW / 16;                 // K dwords per lane per tile (a quarter row)
    static constexpr int VB = ROW / 16;                 // V bytes per lane per token
    static constexpr int VW = VB >= 4 ? VB / 4 : 1;     // ... in dwords
    static constexpr int KK = D / 32;                   // score MFMAs per tile
    static constexpr int NJ = D / 16;                   // value MFMAs per step
    // a stored code c reaches the matrix cores as (c + kOffset) / kCodeScale
    static constexpr float kCodeScale = BITS == 4 ? 512.0f : BITS == 2 ? 65536.0f : 1.0f;
    static constexpr float kOffset = BITS == 4 ? 8.0f : BITS == 2 ? 2.0f : 0.0f;
};

// Order of the 8 channels (of a lane's 8 consecutive ones) in the k slots of
// a score MFMA: the order the conversions below produce them in.
template <int FMT>
__device__ __forceinline__ constexpr int k_slot_channel(int k)
{
    return fmt_bits(FMT) == 4 ? (k < 4 ? 2 * k : 2 * (k - 4) + 1)
         : fmt_bits(FMT) == 2 ? (k & 1 ? 4 + (k >> 1) : k >> 1) : k;
}

// Two fp32 values truncated to bf16, a in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

__device__ __forceinline__ float sbyte(uint32_t w, int i)
{
    return static_cast<float>(static_cast<int8_t>(w >> (8 * i)));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}

// Bytes 0, 1 (HI: 2, 3) of w as E4M3 / E5M2 values, a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <bool HI>
__device__ __forceinline__ uint32_t bf8_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}

// A operand of score MFMA kk: the lane's 8 channels of its token, from the
// lane's K dwords kw, as bf16 pairs in the order k_slot_channel gives.
template <int FMT, int KW>
__device__ __forceinline__ bf16x8_t k_op(const uint32_t (&kw)[KW], int kk)
{
    constexpr int BITS = fmt_bits(FMT);
    if constexpr (BITS == 16) {
        return as_bf16x8(kw[4 * kk], kw[4 * kk + 1], kw[4 * kk + 2], kw[4 * kk + 3]);
    } else if constexpr (FMT == kE4M3) {
        const uint32_t x = kw[2 * kk], y = kw[2 * kk + 1];
        return as_bf16x8(fp8_pair<false>(x), fp8_pair<true>(x), fp8_pair<false>(y), fp8_pair<true>(y));
    } else if constexpr (BITS == 8) {
        const uint32_t x = kw[2 * kk], y = kw[2 * kk + 1];
        return as_bf16x8(bf16_pair(sbyte(x, 0), sbyte(x, 1)), bf16_pair(sbyte(x, 2), sbyte(x, 3)),
                         bf16_pair(sbyte(y, 0), sbyte(y, 1)), bf16_pair(sbyte(y, 2), sbyte(y, 3)));
    } else if constexpr (BITS == 4) {
        // channel 2i in the low nibble of byte i, 2i + 1 in the high
        const uint32_t x = kw[kk] ^ 0x88888888u;
        const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        return as_bf16x8(fp8_pair<false>(lo), fp8_pair<true>(lo), fp8_pair<false>(hi), fp8_pair<true>(hi));
    } else {
        // channel 4i + n in bits 2n, 2n + 1 of byte i; MFMA kk takes bytes
        // 0, 1 (kk even) or 2, 3 of its dword
        const uint32_t x = kw[kk >> 1] ^ 0xAAAAAAAAu;
        const uint32_t e0 = x & 0x03030303u, e1 = (x >> 2) & 0x03030303u;
        const uint32_t e2 = (x >> 4) & 0x03030303u, e3 = (x >> 6) & 0x03030303u;
        if (kk & 1)
            return as_bf16x8(bf8_pair<true>(e0), bf8_pair<true>(e1), bf8_pair<true>(e2), bf8_pair<true>(e3));
        return as_bf16x8(bf8_pair<false>(e0), bf8_pair<false>(e1), bf8_pair<false>(e2), bf8_pair<false>(e3));
    }
}

// Value MFMAs come in groups of four, converted together: group g, member
// jj is MFMA (channel) v_mfma_index(g, jj).  For INT2 a group takes the
// channels of two 2-bit fields of each byte, n = 2g, 2g + 1, from both
// halves of the token words (channels n and 4 + n); otherwise 4g + jj.
template <int FMT, int NJ>
__device__ __forceinline__ constexpr int v_mfma_index(int g, int jj)
{
    return fmt_bits(FMT) == 2 && NJ == 8 ? (jj & 1) + 2 * g + 4 * (jj >> 1) : 4 * g + jj;
}

// A operands of value MFMA group g of one step: v[jj][i] = channel
// v_mfma_index(g, jj) of the lane's tokens 2i and 2i + 1 (token 2i low).
// vw[k]: token k's VW dwords (the lane's NJ channels, VB bytes, low-aligned).
template <int FMT, int NJ, int VW>
__device__ __forceinline__ void v_ops(const uint32_t (&vw)[8][VW], int g, uint32_t (&v)[4][4])
{
    constexpr int BITS = fmt_bits(FMT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t *a = vw[2 * i], *b = vw[2 * i + 1];
        if constexpr (BITS == 16) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * g + jj;
                v[jj][i] = __builtin_amdgcn_perm(b[j >> 1], a[j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
            }
        } else if constexpr (FMT == kE4M3) {
            const uint32_t y0 = __builtin_amdgcn_perm(b[g], a[g], 0x05010400u);   // a0 b0 a1 b1
            const uint32_t y1 = __builtin_amdgcn_perm(b[g], a[g], 0x07030602u);   // a2 b2 a3 b3
            v[0][i] = fp8_pair<false>(y0);
            v[1][i] = fp8_pair<true>(y0);
            v[2][i] = fp8_pair<false>(y1);
            v[3][i] = fp8_pair<true>(y1);
        } else if constexpr (BITS == 8) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                v[jj][i] = bf16_pair(sbyte(a[g], jj), sbyte(b[g], jj));
        } else if constexpr (BITS == 4) {
            // bytes 2g, 2g + 1 of the two tokens interleaved, then split
            // into nibbles: channels 4g .. 4g + 3
            const uint32_t y = __builtin_amdgcn_perm(b[0], a[0], g ? 0x07030602u : 0x05010400u) ^ 0x88888888u;
            const uint32_t lo = y & 0x0F0F0F0Fu, hi = (y >> 4) & 0x0F0F0F0Fu;
            v[0][i] = fp8_pair<false>(lo);
            v[1][i] = fp8_pair<false>(hi);
            v[2][i] = fp8_pair<true>(lo);
            v[3][i] = fp8_pair<true>(hi);
        } else {
            const uint32_t y = __builtin_amdgcn_perm(b[0], a[0], 0x05010400u) ^ 0xAAAAAAAAu;
            if constexpr (NJ == 8) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const uint32_t e = (y >> (2 * (2 * g + m))) & 0x03030303u;   // channels n, 4 + n
                    v[m][i] = bf8_pair<false>(e);
                    v[2 + m][i] = bf8_pair<true>(e);
                }
            } else {
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    v[n][i] = bf8_pair<false>((y >> (2 * n)) & 0x03030303u);
            }
        }
    }
}

// N dwords from p (16-byte aligned when N >= 4), non-temporal: the cache is
// read once per call.
template <int N>
__device__ __forceinline__ void load_words(const uint8_t *p, uint32_t (&w)[N])
{
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p) + i);
            w[4 * i] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
        }
    } else if constexpr (N == 2) {
        const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        w[0] = x[0]; w[1] = x[1];
    } else {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    }
}

// VB (< 4) bytes into the low bits of a dword.
template <int VB>
__device__ __forceinline__ uint32_t load_small(const uint8_t *p)
{
    if constexpr (VB == 2)
        return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
    else
        return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float quad_sum(float x)
{
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <int D, int FMT, bool KCH>
__global__ __launch_bounds__(256) void int_decode_mfma(IntDecodeArgs a)
{
    using S = MfmaShape<D, FMT>;
    constexpr int BITS = S::BITS, TOK = S::TOK, NT = S::NT, NS = S::NS, ROW = S::ROW;
    constexpr int KW = S::KW, VB = S::VB, VW = S::VW, KK = S::KK, NJ = S::NJ;
    constexpr bool kScales = BITS != 16;
    constexpr int AREA = merge_area_bytes<D>();
    __shared__ __align__(16) uint8_t areas[kWavesPerGroup][AREA];
    // per-token factors of a block: K (softmax scale times the token's K
    // scale) and V (the token's V scale), fp32
    __shared__ __align__(16) float tok_f[kWavesPerGroup][2][64];

    const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, quad = lane >> 4;        // MFMA column (head / row), lane group
    const int G = a.group;
    const int64_t T = a.tokens;
    const int64_t t_begin = static_cast<int64_t>(split) * a.chunks_per_split * 256;
    const int64_t t_end = t_begin + static_cast<int64_t>(a.chunks_per_split) * 256 < T
                              ? t_begin + static_cast<int64_t>(a.chunks_per_split) * 256 : T;
    const int64_t kvh = static_cast<int64_t>(b) * a.num_kv_heads + h;
    const int64_t head_row0 = kvh * T;                 // first row of (b, h)
    static_assert(kScales || !KCH, "bf16 has no scales");
    constexpr bool k_tok = kScales && !KCH;
    const bool v_tok = kScales && !a.v_per_channel;

    // Channels of score MFMA kk in lane group `quad`: 32kk + 8quad .. +7 for
    // bf16 (so that one 16-byte load of each lane reads 64 contiguous bytes
    // of a row per group of four lanes), else a quarter row, quad*D/4 + 8kk
    // .. +7 (the lane's codes of all kk in one or two loads).
    auto k_chan = [&](int kk) { return BITS == 16 ? 32 * kk + 8 * quad : quad * (D / 4) + 8 * kk; };

    // B operands of the scores: head `col`'s channels k_chan(kk) .. +7 in
    // the order of the K operand's slots, as 1 (bf16 query) or 3 (query
    // times per-channel K scale) bf16 terms; and the column's query sum
    constexpr int QT = KCH ? 3 : 1;
    bf16x8_t qop[QT][KK];
    float qsum = 0.0f;
    {
        const bool live = col < G;
        const uint16_t *qrow = a.q + (static_cast<int64_t>(b) * a.num_q_heads + h * G + (live ? col : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint4 x = live ? *reinterpret_cast<const uint4 *>(qrow + k_chan(kk)) : make_uint4(0u, 0u, 0u, 0u);
            const uint32_t qw[4] = {x.x, x.y, x.z, x.w};
            float qv[8];                                // channel order
#pragma unroll
            for (int c = 0; c < 8; ++c)
                qv[c] = bf16_value((qw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);
            if constexpr (KCH) {
                const uint4 sv = *reinterpret_cast<const uint4 *>(a.k_scales + kvh * D + k_chan(kk));
                const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    qv[c] *= fp16_value((sw[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);   // exact in fp32
            }
            uint32_t t0[4], t1[4], t2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p[2], r1[2], r2[2];
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    p[n] = qv[k_slot_channel<FMT>(2 * i + n)];
                    r1[n] = p[n] - __uint_as_float(__float_as_uint(p[n]) & 0xFFFF0000u);
                    r2[n] = r1[n] - __uint_as_float(__float_as_uint(r1[n]) & 0xFFFF0000u);
                }
                t0[i] = bf16_pair(p[0], p[1]);
                t1[i] = bf16_pair(r1[0], r1[1]);
                t2[i] = bf16_pair(r2[0], r2[1]);
            }
            qop[0][kk] = as_bf16x8(t0[0], t0[1], t0[2], t0[3]);
            if constexpr (KCH) {
                qop[1][kk] = as_bf16x8(t1[0], t1[1], t1[2], t1[3]);
                qop[2][kk] = as_bf16x8(t2[0], t2[1], t2[2], t2[3]);
            }
            if constexpr (S::kOffset != 0.0f) {
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    qsum += qv[c];
            }
        }
    }
    // a score's offset term, (kOffset / kCodeScale) * sum of the column's query
    const float kcorr = S::kOffset != 0.0f ? quad_sum(qsum) * (S::kOffset / S::kCodeScale) : 0.0f;
    const float zscale = a.scale_log2e * S::kCodeScale;

    // the lane's byte offsets within a block (rows relative to the block's
    // first token; a load's row adds a constant), and its column in row 0
    // for rows past the end
    const uint32_t kcol = BITS == 16 ? 16 * quad : quad * (ROW / 4);
    const uint32_t vcol = col * VB;
    const uint32_t klane = col * ROW + kcol;
    const uint32_t vlane = 4 * quad * ROW + vcol;

    float m_ref = -INFINITY, lsum = 0.0f;
    float4_t acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float4_t pacc = {0.0f, 0.0f, 0.0f, 0.0f};          // sum of the weights as the value MFMAs see them
    constexpr uint32_t kOneBf16x2 = 0x3F803F80u;
    const bf16x8_t ones = as_bf16x8(kOneBf16x2, kOneBf16x2, kOneBf16x2, kOneBf16x2);
    float *kf_lds = tok_f[wave][0];
    float *vf_lds = tok_f[wave][1];

    for (int64_t it0 = t_begin + static_cast<int64_t>(wave) * TOK; it0 < t_end;
         it0 += static_cast<int64_t>(kWavesPerGroup) * TOK) {
        const int valid = t_end - it0 < TOK ? static_cast<int>(t_end - it0) : TOK;
        const bool full = valid == TOK;
        const uint8_t *kb = a.k_codes + (head_row0 + it0) * ROW;
        const uint8_t *vb = a.v_codes + (head_row0 + it0) * ROW;
        // ---- loads, the per-token scales first (their results are needed
        // first; vector loads complete in order), then K, then V
        uint16_t ksc = 0, vsc = 0;
        if constexpr (kScales) {
            const bool ok = lane < valid;             // valid <= TOK <= 64
            if (k_tok && ok)
                ksc = a.k_scales[head_row0 + it0 + lane];
            if (v_tok && ok)
                vsc = a.v_scales[head_row0 + it0 + lane];
        }
        uint32_t kw[NT][KW];
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) {
            const uint8_t *p = kb + (full || 16 * tl + col < valid ? klane + 16 * tl * ROW : kcol);
            if constexpr (BITS == 16) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    uint32_t w4[4];
                    load_words<4>(p + 64 * kk, w4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        kw[tl][4 * kk + i] = w4[i];
                }
            } else {
                load_words<KW>(p, kw[tl]);
            }
        }
        uint32_t vw[NS][8][VW];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int rc = 32 * s + (k < 4 ? k : 12 + k);     // the row less 4 * quad
                const uint8_t *p = vb + (full || 4 * quad + rc < valid ? vlane + rc * ROW : vcol);
                if constexpr (VB >= 4)
                    load_words<VW>(p, vw[s][k]);
                else
                    vw[s][k][0] = load_small<VB>(p);
            }
        if constexpr (kScales) {
            if (k_tok)
                kf_lds[lane] = zscale * fp16_value(ksc);
            if (v_tok)
                vf_lds[lane] = fp16_value(vsc);
        }

        // ---- scores
        float z[NT][4];
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) {
            float4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t kop = k_op<FMT, KW>(kw[tl], kk);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[0][kk], s4, 0, 0, 0);
                if constexpr (KCH) {
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[1][kk], s4, 0, 0, 0);
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[2][kk], s4, 0, 0, 0);
                }
            }
            if constexpr (k_tok) {
                const float4_t f = *reinterpret_cast<const float4_t *>(kf_lds + 16 * tl + 4 * quad);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z[tl][e] = (s4[e] - kcorr) * f[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z[tl][e] = (s4[e] - kcorr) * zscale;
            }
        }
        if (!full) {                                    // tokens past the end score -inf
#pragma unroll
            for (int tl = 0; tl < NT; ++tl)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z[tl][e] = 16 * tl + 4 * quad + e < valid ? z[tl][e] : -INFINITY;
        }

        // ---- online softmax: reference max moved only when exceeded by 8
        float mx = z[0][0];
#pragma unroll
        for (int tl = 0; tl < NT; ++tl)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = fmaxf(mx, z[tl][e]);
        mx = mfma::xor_max(mx);
        const bool move = mx > m_ref + mfma::kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m_new = move ? mx : m_ref;
            const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
            m_ref = m_new;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[j] *= alpha;
            pacc *= alpha;
            lsum *= alpha;
        }
        float pv[NT][4];
#pragma unroll
        for (int tl = 0; tl < NT; ++tl) {
            float4_t sv = {1.0f, 1.0f, 1.0f, 1.0f};
            if (v_tok)
                sv = *reinterpret_cast<const float4_t *>(vf_lds + 16 * tl + 4 * quad);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = __builtin_amdgcn_exp2f(z[tl][e] - m_ref);
                lsum += p;
                pv[tl][e] = p * sv[e];
            }
        }

        // ---- values, 32 tokens (tiles 2s, 2s + 1) per step
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint32_t ph[4], pl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = pv[2 * s + (i >> 1)][2 * (i & 1)], x1 = pv[2 * s + (i >> 1)][2 * (i & 1) + 1];
                ph[i] = bf16_pair(x0, x1);
                pl[i] = bf16_pair(x0 - __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u),
                                  x1 - __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u));
            }
            const bf16x8_t phi = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
            const bf16x8_t plo = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
            for (int g = 0; g < NJ / 4; ++g) {
                uint32_t vo[4][4];
                v_ops<FMT, NJ, VW>(vw[s], g, vo);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = v_mfma_index<FMT, NJ>(g, jj);
                    const bf16x8_t vop = as_bf16x8(vo[jj][0], vo[jj][1], vo[jj][2], vo[jj][3]);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, acc[j], 0, 0, 0);
                }
            }
            if constexpr (S::kOffset != 0.0f) {
                pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phi, pacc, 0, 0, 0);
                pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, plo, pacc, 0, 0, 0);
            }
        }
    }

    // ---- the wave's state into its area: head `col`, channels
    // quad*D/4 + (D/16)*e + j; the offset term, the code scale and
    // per-channel V scales come off here
    lsum = quad_sum(lsum);
    const MergeArea<D> ar(areas[wave]);
    float *orow = ar.row(col) + quad * (D / 4);
    const bool v_chan = kScales && a.v_per_channel;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float off = pacc[e] * (S::kOffset / S::kCodeScale);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = NJ * e + j;
            const float f = v_chan ? fp16_value(a.v_scales[kvh * D + quad * (D / 4) + c]) * S::kCodeScale
                                   : S::kCodeScale;
            orow[c] = (acc[j][e] - off) * f;
        }
    }
    if (quad == 0) {
        ar.ml[2 * col] = m_ref;
        ar.ml[2 * col + 1] = lsum;
    }
    DecodeArgs ma{};
    ma.group = G;
    ma.q_tokens = 1;
    ma.partials = a.splits;
    ma.num_q_heads = a.num_q_heads;
    ma.ws_o = a.ws_o;
    ma.ws_ml = a.ws_ml;
    merge_waves_and_store<D>([&](int w) { return MergeArea<D>(areas[w]); }, ma, b, h, split);
}

template <int D, int FMT>
hipError_t quantize_for(const IntQuantArgs &q, hipStream_t stream)
{
    const int64_t rows = q.batch * q.tokens * q.num_kv_heads;
    const int64_t threads = rows * (D / 16);
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (FMT == 16 || !q.per_channel) {
        int_quantize_token<D, FMT><<<grid, 256, 0, stream>>>(q.x, q.codes, q.scales, rows, q.tokens,
                                                             q.num_kv_heads);
        return hipGetLastError();
    }
    if constexpr (FMT != 16) {
        const dim3 sgrid(q.num_kv_heads, static_cast<unsigned>(q.batch));
        int_channel_scales<D><<<sgrid, 256, 0, stream>>>(q.x, q.scales, q.tokens, fmt_max(FMT));
        int_quantize_channel<D, FMT><<<grid, 256, 0, stream>>>(q.x, q.scales, q.codes, rows, q.tokens,
                                                               q.num_kv_heads);
    }
    return hipGetLastError();
}

template <int D>
hipError_t quantize_d(const IntQuantArgs &q, hipStream_t stream)
{
    switch (q.bits) {
    case 2: return quantize_for<D, 2>(q, stream);
    case 4: return quantize_for<D, 4>(q, stream);
    case 8: return quantize_for<D, 8>(q, stream);
    case kE4M3: return quantize_for<D, kE4M3>(q, stream);
    default: return quantize_for<D, 16>(q, stream);
    }
}

template <int D, int FMT>
hipError_t decode_for(const IntDecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.num_kv_heads, a.batch, a.splits);
    if constexpr (FMT == 16) {
        int_decode_mfma<D, FMT, false><<<grid, kGroupThreads, 0, stream>>>(a);
    } else {
        if (a.k_per_channel)
            int_decode_mfma<D, FMT, true><<<grid, kGroupThreads, 0, stream>>>(a);
        else
            int_decode_mfma<D, FMT, false><<<grid, kGroupThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <int D>
hipError_t decode_d(const IntDecodeArgs &a, hipStream_t stream)
{
    switch (a.bits) {
    case 2: return decode_for<D, 2>(a, stream);
    case 4: return decode_for<D, 4>(a, stream);
    case 8: return decode_for<D, 8>(a, stream);
    case kE4M3: return decode_for<D, kE4M3>(a, stream);
    default: return decode_for<D, 16>(a, stream);
    }
}

}  // namespace

hipError_t launch_int_quantize(const IntQuantArgs &q, hipStream_t stream)
{
    return q.head_dim == 64 ? quantize_d<64>(q, stream) : quantize_d<128>(q, stream);
}

hipError_t launch_int_decode(const IntDecodeArgs &a, hipStream_t stream)
{
    const hipError_t e = a.head_dim == 64 ? decode_d<64>(a, stream) : decode_d<128>(a, stream);
    if (e != hipSuccess)
        return e;
    return launch_decode_combine(a.ws_o, a.ws_ml, a.batch, a.num_q_heads, a.splits, a.head_dim, a.out, stream);
}

}  // namespace fp4kv
