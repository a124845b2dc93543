// KV formats of the bit-width sweep: quantisers (per token, per channel) and
// a vector-ALU decode attention over their codes.
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
#include "fp4kv_quant.h"

namespace fp4kv {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

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

// A wave attends over 64 * TPL consecutive tokens per iteration; GM query
// rows (the group, padded) per KV head; the split is a whole number of
// 256-token chunks.
template <int GM>
struct IntTile {
    static constexpr int TPL = 32 / GM;                 // tokens per lane in the score phase
    static constexpr int kTokens = 64 * TPL;            // tokens per wave iteration
    static constexpr int kPBytes = kTokens * GM * 4;    // weights [kTokens][GM] fp32
};

template <int D>
constexpr int int_wave_area_bytes()
{
    return merge_area_bytes<D>() > 8192 ? merge_area_bytes<D>() : 8192;
}

// Field n (of 32 / BITS per dword) of dword w as a float.  A two's-
// complement field is read as offset binary: flipping its top bit gives
// code + 2^(BITS-1) as an unsigned number, converted exactly and then
// lowered by `off` = 2^(BITS-1).  `off` comes from opaque_offset() so that
// the compiler keeps the subtraction in floating point: folded back into a
// sign-extended byte it becomes a conversion that reads negative bytes as
// large unsigned numbers.  An E4M3 byte converts exactly in hardware (a pair
// per instruction; scale 1).
template <int FMT>
__device__ __forceinline__ float field_value(uint32_t w, int n, float off)
{
    constexpr int BITS = fmt_bits(FMT);
    if constexpr (FMT == kE4M3) {
        const float2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w >> (16 * (n >> 1)), 1.0f, false);
        return (n & 1) ? p[1] : p[0];
    } else if constexpr (BITS == 16) {
        return __uint_as_float(n ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        constexpr uint32_t top = BITS == 8 ? 0x80808080u : BITS == 4 ? 0x88888888u : 0xAAAAAAAAu;
        const uint32_t u = ((w ^ top) >> (BITS * n)) & ((1u << BITS) - 1u);
        return static_cast<float>(u) - off;
    }
}

template <int BITS>
__device__ __forceinline__ float opaque_offset()
{
    float off;
    asm("v_mov_b32 %0, %1" : "=v"(off) : "v"(static_cast<float>(BITS == 16 ? 0 : 1 << (BITS - 1))));
    return off;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

template <int D, int FMT, int GM>
__global__ __launch_bounds__(256) void int_decode_split(IntDecodeArgs a)
{
    constexpr int BITS = fmt_bits(FMT);
    using Tile = IntTile<GM>;
    constexpr int TPL = Tile::TPL;
    constexpr int ROW = D * BITS / 8;                   // bytes per token row
    constexpr int PIECES = ROW / 16;
    constexpr int PER = 32 / BITS;                      // channels per dword
    constexpr int SUB = PER < 4 ? PER : 4;              // channels converted together
    constexpr int CPL = D / 64;                         // channels per lane in the PV phase
    constexpr int AREA = int_wave_area_bytes<D>();
    static_assert(Tile::kPBytes <= AREA, "weights fit the wave's area");

    __shared__ __align__(16) float qs[GM][D];
    __shared__ __align__(16) uint8_t areas[kWavesPerGroup][AREA];

    const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = a.group;
    const int64_t T = a.tokens;
    const int64_t t_begin = static_cast<int64_t>(split) * a.chunks_per_split * 256;
    const int64_t t_end = t_begin + static_cast<int64_t>(a.chunks_per_split) * 256 < T
                              ? t_begin + static_cast<int64_t>(a.chunks_per_split) * 256 : T;
    const int64_t head_row0 = (static_cast<int64_t>(b) * a.num_kv_heads + h) * T;   // first row of (b, h)

    // query rows, pre-scaled into base 2 (and by the per-channel K scales)
    for (int i = threadIdx.x; i < GM * D; i += kGroupThreads) {
        const int g = i / D, c = i % D;
        float v = 0.0f;
        if (g < G) {
            v = bf16_value(a.q[(static_cast<int64_t>(b) * a.num_q_heads + h * G + g) * D + c]) * a.scale_log2e;
            if (BITS != 16 && a.k_per_channel)
                v *= fp16_value(a.k_scales[(static_cast<int64_t>(b) * a.num_kv_heads + h) * D + c]);
        }
        qs[g][c] = v;
    }
    __syncthreads();

    float m[GM], l[GM], o[GM][CPL];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            o[g][c] = 0.0f;
    }
    float *pw = reinterpret_cast<float *>(areas[wave]);     // weights [kTokens][GM]
    const float off = opaque_offset<BITS>();

    for (int64_t it0 = t_begin + static_cast<int64_t>(wave) * Tile::kTokens; it0 < t_end;
         it0 += static_cast<int64_t>(kWavesPerGroup) * Tile::kTokens) {
        // ---- scores: lane owns tokens it0 + 64 j + lane
        float acc[TPL][GM];
        bool ok[TPL];
        const uint8_t *krow[TPL];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int64_t t = it0 + 64 * j + lane;
            ok[j] = t < t_end;
            krow[j] = a.k_codes + (head_row0 + (ok[j] ? t : it0)) * ROW;
#pragma unroll
            for (int g = 0; g < GM; ++g)
                acc[j][g] = 0.0f;
        }
        for (int p = 0; p < PIECES; ++p) {
            uint4 piece[TPL];
#pragma unroll
            for (int j = 0; j < TPL; ++j)
                piece[j] = *reinterpret_cast<const uint4 *>(krow[j] + 16 * p);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // channels of dword k in runs of SUB: each run's values are
                // converted once and meet the GM query rows' matching floats
#pragma unroll
                for (int n0 = 0; n0 < PER; n0 += SUB) {
                    const int c0 = (16 * p + 4 * k) * 8 / BITS + n0;
                    float val[TPL][SUB];
#pragma unroll
                    for (int j = 0; j < TPL; ++j) {
                        const uint32_t w = k == 0 ? piece[j].x : k == 1 ? piece[j].y : k == 2 ? piece[j].z : piece[j].w;
#pragma unroll
                        for (int n = 0; n < SUB; ++n)
                            val[j][n] = field_value<FMT>(w, n0 + n, off);
                    }
#pragma unroll
                    for (int g = 0; g < GM; ++g) {
#pragma unroll
                        for (int n = 0; n < SUB; ++n) {
                            const float qv = qs[g][c0 + n];
#pragma unroll
                            for (int j = 0; j < TPL; ++j)
                                acc[j][g] = fmaf(qv, val[j][n], acc[j][g]);
                        }
                    }
                    // keep the next run's query reads from being hoisted
                    // here (with short rows they would all be live at once)
                    asm volatile("" ::: "memory");
                }
            }
        }
        // per-token K scale; tokens past the end score -inf
        float z[TPL][GM];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int64_t t = it0 + 64 * j + lane;
            const float sk = (BITS == 16 || a.k_per_channel) ? 1.0f
                                                             : fp16_value(a.k_scales[head_row0 + (ok[j] ? t : it0)]);
#pragma unroll
            for (int g = 0; g < GM; ++g)
                z[j][g] = ok[j] ? acc[j][g] * sk : -INFINITY;
        }
        // ---- online softmax (base 2); the first token of the iteration is valid
        float sv[TPL];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int64_t t = it0 + 64 * j + lane;
            sv[j] = (BITS == 16 || a.v_per_channel) ? 1.0f
                                                    : fp16_value(a.v_scales[head_row0 + (ok[j] ? t : it0)]);
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            float mx = z[0][g];
#pragma unroll
            for (int j = 1; j < TPL; ++j)
                mx = fmaxf(mx, z[j][g]);
            const float m_new = fmaxf(m[g], wave_max(mx));
            const float alpha = exp2f(m[g] - m_new);
            m[g] = m_new;
            float ls = 0.0f;
#pragma unroll
            for (int j = 0; j < TPL; ++j) {
                const float pj = exp2f(z[j][g] - m_new);
                ls += pj;
                pw[(64 * j + lane) * GM + g] = pj * sv[j];
            }
            l[g] = fmaf(l[g], alpha, ls);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                o[g][c] *= alpha;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the weights are in LDS for every lane

        // ---- values: lane owns channels CPL*lane .. CPL*lane + CPL-1
        const int n_tok = t_end - it0 < Tile::kTokens ? static_cast<int>(t_end - it0) : Tile::kTokens;
        const int bit0 = lane * CPL * BITS;
        const uint8_t *vbase = a.v_codes + (head_row0 + it0) * ROW + 4 * (bit0 >> 5);
        const int shift = bit0 & 31;
        int i = 0;
        for (; i + 8 <= n_tok; i += 8) {
            uint32_t w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                w[u] = *reinterpret_cast<const uint32_t *>(vbase + static_cast<int64_t>(i + u) * ROW);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float v[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    v[c] = field_value<FMT>(BITS == 16 ? w[u] : (w[u] >> shift), BITS == 16 ? (shift >> 4) + c : c, off);
                const float *pr = pw + (i + u) * GM;
#pragma unroll
                for (int g = 0; g < GM; ++g) {
                    const float pg = pr[g];
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        o[g][c] = fmaf(pg, v[c], o[g][c]);
                }
            }
        }
        for (; i < n_tok; ++i) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(vbase + static_cast<int64_t>(i) * ROW);
            float v[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                v[c] = field_value<FMT>(BITS == 16 ? w : (w >> shift), BITS == 16 ? (shift >> 4) + c : c, off);
            const float *pr = pw + i * GM;
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                const float pg = pr[g];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    o[g][c] = fmaf(pg, v[c], o[g][c]);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // weight reads done before the next writes
    }

    // per-channel V scales multiply the outputs
    if (BITS != 16 && a.v_per_channel) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float s = fp16_value(a.v_scales[(static_cast<int64_t>(b) * a.num_kv_heads + h) * D + CPL * lane + c]);
#pragma unroll
            for (int g = 0; g < GM; ++g)
                o[g][c] *= s;
        }
    }
    // the wave's state into its area (the weights are no longer needed)
    const MergeArea<D> ar(areas[wave]);
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        const float lsum = wave_sum(l[g]);
        if (g < 16) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                ar.row(g)[CPL * lane + c] = o[g][c];
            if (lane == 0) {
                ar.ml[2 * g] = m[g];
                ar.ml[2 * g + 1] = lsum;
            }
        }
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
    if (a.group <= 8)
        int_decode_split<D, FMT, 8><<<grid, kGroupThreads, 0, stream>>>(a);
    else
        int_decode_split<D, FMT, 16><<<grid, kGroupThreads, 0, stream>>>(a);
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
