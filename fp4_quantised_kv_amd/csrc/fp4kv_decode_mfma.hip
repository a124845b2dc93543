// Split-K decode attention on the CDNA4 matrix cores (v_mfma_f32_16x16x32_f16).
//
// Workgroups of four waves per (4 context chunks, KV head, sequence); each
// wave attends over one chunk and the four results are merged in LDS into
// one partial.  For each 64-token page of its chunk, a wave computes:
//
//   scores  S^T[token][query] = K^ Q^T as four 16-token tiles.  The A operand
//           is the page's K codes, converted two at a time by the hardware FP4
//           conversion (scale 1: the instruction applies only the exponent of
//           a scale) and multiplied by the token's E4M3 scale in packed fp16;
//           E2M1 x E4M3 products have at most 6 significant bits, so every
//           dequantised value is exact in fp16.  The B operand is the group's
//           query rows (up to 16; missing rows are zero), converted to fp16
//           after multiplying by a power of two that puts the largest |q|
//           just under 2^15 (exact for bf16 inputs, undone on the scores).
//   softmax the C layout gives each lane one query column and 16 of the page's
//           tokens; the running max per query is a lane max plus two
//           cross-lane steps.  The reference max is only moved when the page
//           max exceeds it by more than 8 (base 2), so the accumulators are
//           rescaled rarely and probabilities stay below 2^8.
//   values  O^T[channel][query] += V^T P^T.  The 16 tokens a lane holds in the
//           score tiles are exactly the 16 consecutive tokens it needs as the
//           B operand of the value product, so P needs no data movement.  V is
//           stored channel-pair-major, so a lane's 16 tokens of one channel
//           pair are one 16-byte load; conversion gives (even, odd) pairs per
//           token, which are regrouped into per-channel token pairs and scaled
//           by the per-token scales.  P enters as two fp16 parts (hi + lo),
//           each multiplied on the matrix cores, so the probabilities keep
//           ~21 significant bits.  The softmax denominator is one more
//           product, of P with a ones matrix, so it sums exactly the
//           probabilities used for the values.
//
// Page-local token order of score tile a, row r: token 16*(r/4) + 4*a + r%4,
// so the C-layout lane (query n, row group jj) holds tokens 16*jj + 0..15.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"
#include "fp4kv_merge.h"
#include "fp4kv_mfma_util.h"

namespace fp4kv {
namespace {

using namespace mfma;

// 8 consecutive channels of one token (one code dword) times one scale.
__device__ __forceinline__ half8_t k_operand(uint32_t w, half2_t s)
{
    return cat(fp4x2<0>(w), fp4x2<1>(w), fp4x2<2>(w), fp4x2<3>(w)) *
           __builtin_shufflevector(s, s, 0, 1, 0, 1, 0, 1, 0, 1);
}

// K operands of one page as a lane holds them: score tile t, code dwords i
// (channels jj*D/4 + 8i .. +7 of the tile's token) and the two (D = 128) or
// one (D = 64, repeated) scale bytes of those channels.
template <int D>
struct KRegs {
    static constexpr int KW = D / 32;
    uint32_t kw[4][KW];
    uint32_t ks[4];
};

// V operands of one page: pair block u (pair 16u + col), tokens 16jj .. +15:
// code bytes and the scale bytes of that pair's 16-channel block.
template <int D>
struct VRegs {
    static constexpr int NU = D / 32;
    uint4 vw[NU];
    uint4 vs[NU];
};

// Scores and online softmax of one page of which the lane's query column
// sees the tokens lo .. valid-1 (page-local); leaves the probabilities as the
// value product's B operands (hi and lo parts for the two 32-token halves).
template <int D>
__device__ __forceinline__ void scores_phase(const KRegs<D> &r, int lo, int valid, const half8_t (&qf)[D / 32],
                                             float zscale, int jj, SplitState<D> &st, half8_t (&pf)[2],
                                             half8_t (&pl)[2])
{
    constexpr int KW = KRegs<D>::KW;
    float z[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const half2_t s = fp8x2<false>(r.ks[t]);          // (scale of first 16 channels, of next 16)
        float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            const half2_t si = (KW == 4 && i >= 2) ? __builtin_shufflevector(s, s, 1, 1)
                                                   : __builtin_shufflevector(s, s, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(r.kw[t][i], si), qf[i], sacc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            z[t][e] = sacc[e];                          // scaled inside the exponent below
    }
    if (valid < kPage || lo > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 16 * jj + 4 * t + e;
                z[t][e] = (tok < valid && tok >= lo) ? z[t][e] : -INFINITY;
            }
    }

    softmax_tiles<D, 4>(z, st, zscale, pf, pl);
}

// Value accumulation of pair blocks [u0, u0 + N) of one page: tile (u,
// parity) rows are channels 32u + 2*row + parity.  A lane holds, for its
// channels c = 32u + 2*col and c + 1, the code dwords of tokens 16jj + 0..7
// and + 8..15 (two tokens per byte, in token order), and the fp16 scales of
// those 16 tokens (sv[u][half]); each conversion yields two consecutive
// tokens of one channel, exactly an MFMA operand pair.
template <int D, int N>
__device__ __forceinline__ void values_phase(int u0, const uint4 (&vw)[N], const half8_t (&sv)[N][2],
                                             const half8_t (&pf)[2], const half8_t (&pl)[2], SplitState<D> &st)
{
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const uint32_t cw[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
        float4_t &ae = st.acc[2 * (u0 + u)];
        float4_t &ao = st.acc[2 * (u0 + u) + 1];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint32_t we = cw[kt], wo = cw[2 + kt];
            const half8_t ev = cat(fp4x2<0>(we), fp4x2<1>(we), fp4x2<2>(we), fp4x2<3>(we)) * sv[u][kt];
            const half8_t od = cat(fp4x2<0>(wo), fp4x2<1>(wo), fp4x2<2>(wo), fp4x2<3>(wo)) * sv[u][kt];
            ae = __builtin_amdgcn_mfma_f32_16x16x32_f16(ev, pf[kt], ae, 0, 0, 0);
            ae = __builtin_amdgcn_mfma_f32_16x16x32_f16(ev, pl[kt], ae, 0, 0, 0);
            ao = __builtin_amdgcn_mfma_f32_16x16x32_f16(od, pf[kt], ao, 0, 0, 0);
            ao = __builtin_amdgcn_mfma_f32_16x16x32_f16(od, pl[kt], ao, 0, 0, 0);
        }
    }
}

// fp16 scales of a lane's 16 tokens (16jj + 0..15) from their 16 E4M3 bytes,
// zero for tokens at or past `valid` so never-written slots add exact zeros.
__device__ __forceinline__ void v_scales(uint4 raw, int valid, int jj, half8_t (&sv)[2])
{
    if (valid < kPage) {
        raw.x = keep_valid_bytes(raw.x, 16 * jj + 0, valid);
        raw.y = keep_valid_bytes(raw.y, 16 * jj + 4, valid);
        raw.z = keep_valid_bytes(raw.z, 16 * jj + 8, valid);
        raw.w = keep_valid_bytes(raw.w, 16 * jj + 12, valid);
    }
    sv[0] = cat(fp8x2<false>(raw.x), fp8x2<true>(raw.x), fp8x2<false>(raw.y), fp8x2<true>(raw.y));
    sv[1] = cat(fp8x2<false>(raw.z), fp8x2<true>(raw.z), fp8x2<false>(raw.w), fp8x2<true>(raw.w));
}

// Direct loads: every operand straight from global memory into registers.
template <int D>
__device__ __forceinline__ void load_k_direct(const uint8_t *blk, const CacheGeom &g, int col, int jj, KRegs<D> &r)
{
    constexpr int NB = D / 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int tok = tile_token(t, col);
        const uint8_t *krow = blk + g.k_codes_off + tok * (D / 2) + jj * (D / 8);
        if constexpr (KRegs<D>::KW == 4) {
            const uint4 x = *reinterpret_cast<const uint4 *>(krow);
            r.kw[t][0] = x.x; r.kw[t][1] = x.y; r.kw[t][2] = x.z; r.kw[t][3] = x.w;
            r.ks[t] = *reinterpret_cast<const uint16_t *>(blk + g.k_scales_off + tok * NB + 2 * jj);
        } else {
            const uint2 x = *reinterpret_cast<const uint2 *>(krow);
            r.kw[t][0] = x.x; r.kw[t][1] = x.y;
            const uint32_t s1 = blk[g.k_scales_off + tok * NB + jj];
            r.ks[t] = s1 | (s1 << 8);
        }
    }
}

// V codes: row (slice jj, channel c) of 8 bytes at (jj*D + c)*8; V scales:
// row (slice jj, block) of 16 bytes at (jj*D/16 + block)*16.
template <int D>
__device__ __forceinline__ void load_v_direct(const uint8_t *blk, const CacheGeom &g, int col, int jj, VRegs<D> &r)
{
#pragma unroll
    for (int u = 0; u < VRegs<D>::NU; ++u) {
        const int c = 32 * u + 2 * col;
        r.vw[u] = *reinterpret_cast<const uint4 *>(blk + g.v_codes_off + (jj * D + c) * 8);
        r.vs[u] = *reinterpret_cast<const uint4 *>(blk + g.v_scales_off + (jj * (D / 16) + (c >> 4)) * 16);
    }
}

// Staged loads for D = 128: direct-to-LDS copies issued a phase ahead of the
// arithmetic, so that no registers are held while the copies are in flight.
// K and V have separate LDS slots, so the next page's K copy can start as
// soon as this page's K operands are in registers, and likewise for V.  All
// copies are 16 bytes per lane; the two scale planes of a page travel in one
// instruction with the K codes.
//   K slot [0, 4096): tile t at t*1024, lane l's 16 code bytes at l*16;
//          [4096, 4608): the page's K scale plane [64 tokens][8] in 16-byte
//          pieces of two tokens, piece p stored at k_scale_piece(p);
//          [4608, 5120): its V scale plane [4 slices][8 blocks][16].
//   V slot [0, 4096): pair block u at u*1024, lane l at l*16;
//          [4096, 5120): the page's V scales in fp16, converted once per page
//          during the K phase (each lane converts 8), 32-byte block b (slice
//          b/8, channel block b%8, 16 tokens) stored at v_scale_block(b).
// The two permutations keep the scale reads free of LDS bank conflicts: the
// lanes reading one score tile's K scales (two tokens per piece, pieces
// 8q + 2t + {0, 1} for q = 0..3) and the lanes reading one pair block's V
// scales (blocks 8*slice + 2u + {0, 1}) land on distinct banks instead of
// on blocks 128 or 256 bytes apart.
constexpr int kKSlotBytes = 5120;
constexpr int kVSlotBytes = 5120;
constexpr int kCopiesK = 5;               // direct-to-LDS instructions per K copy
constexpr int kCopiesV = 4;               // ... per V copy

__device__ __forceinline__ uint32_t k_scale_piece(uint32_t p) { return p ^ (2u * ((p >> 3) & 3u)); }
__device__ __forceinline__ uint32_t v_scale_block(uint32_t b) { return b ^ (2u * ((b >> 3) & 3u)); }

struct StageOffsets {
    uint32_t k, s, v;                     // per-lane byte offsets inside a block: tile/block 0, scales
};

__device__ __forceinline__ StageOffsets stage_offsets(const CacheGeom &g, int lane, int col, int jj)
{
    StageOffsets o;
    const uint32_t tok0 = static_cast<uint32_t>(tile_token(0, col));
    o.k = static_cast<uint32_t>(g.k_codes_off) + tok0 * 64u + jj * 16u;
    // lanes 0..31: the K scale plane (lane l fetches the piece stored at
    // position l; k_scale_piece is its own inverse), lanes 32..63: the V
    // scale plane
    o.s = lane < 32 ? static_cast<uint32_t>(g.k_scales_off) + k_scale_piece(static_cast<uint32_t>(lane)) * 16u
                    : static_cast<uint32_t>(g.v_scales_off) + (lane & 31) * 16u;
    o.v = static_cast<uint32_t>(g.v_codes_off) + (jj * 128u + 2u * col) * 8u;
    return o;
}

// Tile t's token rows are 4t past tile 0's (+256 bytes of K codes); V pair
// block u is 32 channels (256 bytes) past block 0.
__device__ __forceinline__ void stage_k(const uint8_t *blk, const StageOffsets &o, uint8_t *slot)
{
    const uint8_t *k = blk + o.k;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds(k + 256 * t, slot + t * 1024, 16, 0, kStream);
    __builtin_amdgcn_global_load_lds(blk + o.s, slot + 4096, 16, 0, kStream);
}

__device__ __forceinline__ void stage_v(const uint8_t *blk, const StageOffsets &o, uint8_t *slot)
{
    const uint8_t *v = blk + o.v;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_global_load_lds(v + 256 * u, slot + u * 1024, 16, 0, kStream);
}

__device__ __forceinline__ void read_k(const uint8_t *slot, int lane, int col, int jj, KRegs<128> &r)
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint4 x = *reinterpret_cast<const uint4 *>(slot + t * 1024 + lane * 16);
        r.kw[t][0] = x.x; r.kw[t][1] = x.y; r.kw[t][2] = x.z; r.kw[t][3] = x.w;
        const uint32_t tok = static_cast<uint32_t>(tile_token(t, col));
        r.ks[t] = *reinterpret_cast<const uint16_t *>(slot + 4096 + k_scale_piece(tok >> 1) * 16 + (tok & 1) * 8 +
                                                      2 * jj);
    }
}

// V scales of the page in the K slot -> fp16 in the V slot: lane l takes
// bytes 8l .. 8l+7 of the plane, i.e. tokens 16*(l/16) + 8*(l%2) + 0..7;
// scales of tokens at or past `valid` become zero, so never-written slots
// add exact zeros.
__device__ __forceinline__ void convert_v_scales(const uint8_t *kslot, uint8_t *vslot, int lane, int valid)
{
    uint2 raw = *reinterpret_cast<const uint2 *>(kslot + 4608 + lane * 8);
    if (valid < kPage) {
        const int t0 = 16 * (lane >> 4) + 8 * (lane & 1);
        raw.x = keep_valid_bytes(raw.x, t0, valid);
        raw.y = keep_valid_bytes(raw.y, t0 + 4, valid);
    }
    const half8_t h = cat(fp8x2<false>(raw.x), fp8x2<true>(raw.x), fp8x2<false>(raw.y), fp8x2<true>(raw.y));
    *reinterpret_cast<half8_t *>(vslot + 4096 + v_scale_block(lane >> 1) * 32 + (lane & 1) * 16) = h;
}

template <int N>
__device__ __forceinline__ void read_v(const uint8_t *slot, int u0, int lane, int col, int jj, uint4 (&vw)[N],
                                       half8_t (&sv)[N][2])
{
#pragma unroll
    for (int u = 0; u < N; ++u) {
        vw[u] = *reinterpret_cast<const uint4 *>(slot + (u0 + u) * 1024 + lane * 16);
        const half8_t *sp = reinterpret_cast<const half8_t *>(
            slot + 4096 + v_scale_block(static_cast<uint32_t>(jj * 8 + 2 * (u0 + u) + (col >> 3))) * 32);
        sv[u][0] = sp[0];
        sv[u][1] = sp[1];
    }
}

// The page loop of the staged kernel.  The slots are restrict-qualified so
// that the compiler knows the direct-to-LDS copies into one never alias
// reads of the other; without that it waits for every copy in flight before
// any LDS read, and the next page's K copy would stall this page's V reads.
// On entry `ids` holds the page ids of pages p0 .. p0+63 (one per lane) and
// the copies of page p0 (id `pid`) have been issued, K then V, if it is live.
template <int D>
__device__ __forceinline__ void staged_pages(uint8_t *__restrict__ kslot, uint8_t *__restrict__ vslot,
                                             const DecodeArgs &a, const StageOffsets &so, int lane, int col,
                                             int jj, int h, int p0, int p1, int len, int shortfall, int first,
                                             const int32_t *ptab, int ids, int pid, const half8_t (&qf)[D / 32],
                                             float zscale, SplitState<D> &st)
{
    const CacheGeom &g = a.geom;
    auto live_page = [&](int id) { return id >= 0 && id < g.num_pages; };   // others are skipped
    auto block_of = [&](int id) {
        return a.cache + static_cast<int64_t>(id) * g.page_stride + h * g.head_stride;
    };
    half8_t pf[2], pl[2];
    int base = p0;
    for (int pg = p0; pg < p1; ++pg) {
        const int nxt = pg + 1;
        if (nxt < p1 && nxt - base == 64) {
            base = nxt;
            ids = (base + lane < p1) ? ptab[base + lane] : -1;
            wait_vmem_at_most<0>();
        }
        const int pid_next = nxt < p1 ? __builtin_amdgcn_readlane(ids, nxt - base) : -1;
        const bool cur = live_page(pid), next = live_page(pid_next);
        const int valid = min(kPage, len - pg * kPage);

        // K: outstanding now are this page's K then V copies
        if (cur)
            wait_vmem_at_most<kCopiesV>();
        convert_v_scales(kslot, vslot, lane, valid);   // the V slot's fp16 plane is free since the last page
        KRegs<D> kr;
        read_k(kslot, lane, col, jj, kr);
        __builtin_amdgcn_s_waitcnt(kWaitLds);
        if (next)
            stage_k(block_of(pid_next), so, kslot);
        if (cur)
            scores_phase<D>(kr, first - pg * kPage, min(kPage, len - pg * kPage - shortfall), qf, zscale, jj, st,
                            pf, pl);

        // V: outstanding now are this page's V then the next page's K
        // copies.  One pair block at a time keeps few registers live.
        if (next)
            wait_vmem_at_most<kCopiesK>();
        else
            wait_vmem_at_most<0>();
        uint4 vw[1];
        half8_t sv[1][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            read_v<1>(vslot, u, lane, col, jj, vw, sv);
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            if (u == 3 && next)
                stage_v(block_of(pid_next), so, vslot);
            if (cur)
                values_phase<D, 1>(u, vw, sv, pf, pl, st);
        }
        pid = pid_next;
    }
}

// ---- one workgroup per (KV head, sequence, partial)

template <int D, bool STAGED, bool APPEND>
__global__ __launch_bounds__(kGroupThreads) void decode_split_mfma(DecodeArgs a)
{
    static_assert(merge_area_bytes<D>() <= 16 * D * 4 + 128, "merge area layout");
    static_assert(8 * D * 4 + 128 <= kKSlotBytes && 8 * D * 4 <= kVSlotBytes, "merge area must fit the slots");
    static_assert(kWavesPerGroup * (kKSlotBytes + kVSlotBytes) <= 40 * 1024, "four workgroups per CU");

    // separate LDS objects for K and V, so the copies into one never wait on
    // reads of the other
    __shared__ __attribute__((aligned(16))) uint8_t kslots[kWavesPerGroup][kKSlotBytes];
    __shared__ __attribute__((aligned(16))) uint8_t vslots[kWavesPerGroup][kVSlotBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps the page loop scalar
    const int col = lane & 15;            // query column / tile row
    const int jj = lane >> 4;             // lane group
    const CacheGeom &g = a.geom;

    // grid (KV head, sequence, partial): the partial index varies slowest, so
    // the chunks nearest the start of every sequence (never empty) are
    // dispatched first, and consecutive workgroups -- which the hardware
    // deals round-robin to the XCDs -- belong to different KV heads.  Every
    // independent load is issued before any is waited on.
    Chunk c = chunk_start(a, blockIdx.x, blockIdx.y, blockIdx.z, wave);
    int ids = STAGED ? chunk_ids(a, c, wave, lane) : -1;
    uint32_t qbits[D / 8];
    load_q_bits<D>(a, c.b, c.h, col, jj, qbits);
    // the length is read only now: issued earlier, its scalar load would
    // join the wait for the kernel arguments the loads above need, and
    // delay them by a memory round trip (an empty workgroup leaves them
    // unused)
    __builtin_amdgcn_sched_barrier(0);
    chunk_clamp(a, c);
    if constexpr (STAGED)
        ids = chunk_ids_moved(a, c, wave, lane, ids);
    if (!a.out && group_chunks_empty(a, c, wave)) {
        mark_partial_empty(a, c.b, c.h, c.part);
        return;
    }
    half8_t qf[D / 32];
    float zscale;
    make_q_operand<D>(qbits, a.scale_log2e, qf, zscale);

    if constexpr (APPEND)
        append_if_last_chunk<D, false>(a, c, lane);

    const int shortfall = column_shortfall(a, col);
    const int first = column_first_token(a, c.len, shortfall);
    SplitState<D> st;
    init_state(st);
    if constexpr (STAGED) {
        // the query and page-id loads were in flight together, so converting
        // the query before the first page's copies costs no extra wait
        const StageOffsets so = stage_offsets(g, lane, col, jj);
        const int pid = c.p0 < c.p1 ? __builtin_amdgcn_readlane(ids, 0) : -1;
        if (pid >= 0 && pid < g.num_pages) {
            const uint8_t *blk = a.cache + static_cast<int64_t>(pid) * g.page_stride + c.h * g.head_stride;
            stage_k(blk, so, kslots[wave]);
            stage_v(blk, so, vslots[wave]);
        } else if (APPEND) {
            // no first page: the page loop issues the next page's copy before
            // its first wait, so the token's stores must complete here
            wait_vmem_at_most<0>();
        }
        staged_pages<D>(kslots[wave], vslots[wave], a, so, lane, col, jj, c.h, c.p0, c.p1, c.len, shortfall, first,
                        c.ptab, ids, pid, qf, zscale, st);
    } else {
        half8_t pf[2], pl[2];
        for (int pg = c.p0; pg < c.p1; ++pg) {
            const int id = c.ptab[pg];
            if (id < 0 || id >= g.num_pages)            // skipped, like the staged loop
                continue;
            const uint8_t *blk = a.cache + static_cast<int64_t>(id) * g.page_stride + c.h * g.head_stride;
            const int valid = min(kPage, c.len - pg * kPage);
            KRegs<D> kr;
            VRegs<D> vr;
            load_k_direct<D>(blk, g, col, jj, kr);
            load_v_direct<D>(blk, g, col, jj, vr);
            scores_phase<D>(kr, first - pg * kPage, min(kPage, c.len - pg * kPage - shortfall), qf, zscale, jj,
                            st, pf, pl);
            half8_t sv[VRegs<D>::NU][2];
#pragma unroll
            for (int u = 0; u < VRegs<D>::NU; ++u)
                v_scales(vr.vs[u], valid, jj, sv[u]);
            values_phase<D, VRegs<D>::NU>(0, vr.vw, sv, pf, pl, st);
        }
    }

    auto area = [&](int w) { return MergeArea<D>(kslots[w], vslots[w]); };
    state_to_area<D>(area(wave), st, col, jj, query_columns(a));
    merge_waves_and_store<D>(area, a, c.b, c.h, c.part);
}

}  // namespace

hipError_t launch_split_mfma(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.geom.num_kv_heads, a.batch, a.partials);
    if (a.geom.head_dim == 64) {
        decode_split_mfma<64, false, false><<<grid, kGroupThreads, 0, stream>>>(a);
    } else if (a.staged) {
        if (a.k_new)
            decode_split_mfma<128, true, true><<<grid, kGroupThreads, 0, stream>>>(a);
        else
            decode_split_mfma<128, true, false><<<grid, kGroupThreads, 0, stream>>>(a);
    } else {
        decode_split_mfma<128, false, false><<<grid, kGroupThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace fp4kv
