// Merge of the running states of a workgroup's waves into one partial result.
//
// A decode workgroup has kWavesPerGroup waves; wave w attends over context
// chunk 4 * part + w, part being the workgroup's partial index.  Each wave
// leaves, in its own LDS area, its unnormalised outputs o_w[q][c] (16 query
// rows x D channels, fp32) and its (m_w[q], l_w[q]) pairs (base-2 running
// max and sum).  The workgroup then
// writes one partial per query row, relative to M = max_w m_w:
//   o = sum_w o_w 2^(m_w - M),  l = sum_w l_w 2^(m_w - M),  m = M,
// or (m, l, o) = (-inf, 0, 0) when every wave was empty.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "fp4kv_internal.h"

namespace fp4kv {

constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = 64 * kWavesPerGroup;

// Context chunk k (wave k % 4 of partial k / 4) holds chunk_pages(a, k)
// pages from chunk_first_page(a, k); the chunks tile the context in order:
// lead_chunks chunks of lead_pages, then chunks of tail_pages.  The grid's
// partial index varies slowest, so the long chunks are dispatched first and
// the workgroups that start last -- in a grid of many more workgroups than
// the GPU holds at once -- are short ones: fewer slots idle while the grid
// drains.
__device__ __forceinline__ int chunk_first_page(const DecodeArgs &a, int k)
{
    return k < a.lead_chunks ? k * a.lead_pages
                             : a.lead_chunks * a.lead_pages + (k - a.lead_chunks) * a.tail_pages;
}

__device__ __forceinline__ int chunk_pages(const DecodeArgs &a, int k)
{
    return k < a.lead_chunks ? a.lead_pages : a.tail_pages;
}

template <int D>
constexpr int merge_area_bytes() { return 16 * D * 4 + 16 * 2 * 4; }

// The area of one wave: outputs of query rows 0..7 and the (max, sum) pairs
// [16][2] in the first block, outputs of rows 8..15 in the second.
template <int D>
struct MergeArea {
    float *lo, *hi, *ml;
    __device__ MergeArea(uint8_t *first, uint8_t *second)
        : lo(reinterpret_cast<float *>(first)), hi(reinterpret_cast<float *>(second)), ml(lo + 8 * D) {}
    // one contiguous area of merge_area_bytes<D>()
    __device__ explicit MergeArea(uint8_t *base) : MergeArea(base, base + 8 * D * 4 + 16 * 2 * 4) {}
    __device__ float *row(int q) const { return q < 8 ? lo + q * D : hi + (q - 8) * D; }
};

// Call with every thread of the workgroup, after each wave has filled its
// area; area(w) gives wave w's area.  With a.out set (one partial per row)
// the rows are written to a.out as final outputs instead of partials.  Area row q is query token q / G, head
// h*G + q % G of the group; its partial goes to row
// (q / G) * num_q_heads + h*G + q % G of ws_o[b][part] and ws_ml[b][part],
// so with one query token a workgroup's G rows are one contiguous block of
// G*D floats (and of G (m, l) pairs), written with 16-byte stores.
template <int D, typename AreaOf>
__device__ __forceinline__ void merge_waves_and_store(AreaOf area, const DecodeArgs &a, int b, int h, int part)
{
    __syncthreads();
    const int G = a.group;
    const int S = a.q_tokens > 1 ? a.q_tokens : 1;
    const int64_t row0 = (static_cast<int64_t>(b) * a.partials + part) * S * a.num_q_heads + static_cast<int64_t>(h) * G;
    for (int idx = threadIdx.x; idx < S * G * (D / 4); idx += kGroupThreads) {
        const int q = idx / (D / 4), c = 4 * (idx % (D / 4));
        const int64_t row = row0 + static_cast<int64_t>(q / G) * a.num_q_heads + q % G;
        float mw[kWavesPerGroup];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWavesPerGroup; ++w) {
            mw[w] = area(w).ml[2 * q];
            M = fmaxf(M, mw[w]);
        }
        float4 O = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float L = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWavesPerGroup; ++w) {
                if (mw[w] == -INFINITY)
                    continue;
                const MergeArea<D> ar = area(w);
                const float wt = exp2f(mw[w] - M);
                const float4 x = *reinterpret_cast<const float4 *>(ar.row(q) + c);
                O.x = fmaf(x.x, wt, O.x);
                O.y = fmaf(x.y, wt, O.y);
                O.z = fmaf(x.z, wt, O.z);
                O.w = fmaf(x.w, wt, O.w);
                L = fmaf(ar.ml[2 * q + 1], wt, L);
            }
        }
        if (a.out) {
            // the only partial of its rows: the final output, normalised as
            // the combine would (with one partial its weight is exactly 1)
            const float inv = L > 0.0f ? 1.0f / L : 0.0f;
            *reinterpret_cast<float4 *>(a.out + row * D + c) = make_float4(O.x * inv, O.y * inv, O.z * inv, O.w * inv);
        } else {
            *reinterpret_cast<float4 *>(a.ws_o + row * D + c) = O;
            if (c == 0)
                *reinterpret_cast<float2 *>(a.ws_ml + row * 2) = make_float2(M, L);
        }
    }
}

}  // namespace fp4kv
