// Row-dot helpers and constants shared by the score stream and the Reindex
// scorer (gfx950, wave64): a key row of RW = 256*VPR values (Hk heads of Di
// channels), stored as fp32 or as E4M3FN bytes, dotted with the query row
// held in registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace csa2 {
namespace {

constexpr int kHistBins = 4096;      // first-level digit: top 12 bits of the key
constexpr int kDigitShift = 20;
constexpr int kStreamThreads32 = 256;   // score stream workgroup (fp32 keys)
constexpr int kStreamThreads8 = 512;    // score stream workgroup (E4M3 keys)
constexpr int kRowsPerWG = 4096;     // score stream: rows per workgroup (fp32 keys)
constexpr int kRowsPerWG8 = 8192;    // score stream: rows per workgroup (E4M3 keys)
constexpr int kStreamNB8 = 2;        // E4M3 stream: 16 KB sub-blocks per wave iteration

// Lane-resident slice of the query vector: chunk j of lane l holds floats
// [4(l + 64 j), 4(l + 64 j) + 4) of the RW = 256*VPR-float query row.  With
// one shared key head (Hk == 1) the query heads are summed first.
template <int VPR>
__device__ __forceinline__ void load_qvec(const float* __restrict__ qI, int q, int Hi, int Hk,
                                          int Di, float4 (&qv)[VPR]) {
    const int lane = lane_id();
    if (Hk == Hi) {
        const float4* p = reinterpret_cast<const float4*>(qI + (size_t)q * Hi * Di);
#pragma unroll
        for (int j = 0; j < VPR; ++j) qv[j] = p[lane + 64 * j];
    } else {
#pragma unroll
        for (int j = 0; j < VPR; ++j) {
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int h = 0; h < Hi; ++h) {
                float4 v = reinterpret_cast<const float4*>(qI + ((size_t)q * Hi + h) * Di)[lane + 64 * j];
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
            qv[j] = s;
        }
    }
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Streaming load of one float4 of a key row: each key byte is read once, so
// the load is marked nontemporal (no reuse expected in the caches).
__device__ __forceinline__ float4 load_stream(const float* p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Sums 8 per-lane partials across the wave (transpose-reduction): returns in
// every lane the full sum of partial (lane >> 3) & 7.  After the xor-32/16/8
// steps lane l holds a partial of row (l>>3)&7 summed over 8 lanes; xor-4/2/1
// completes it.
__device__ __forceinline__ float reduce8(float (&a)[8]) {
    const int lane = lane_id();
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float send = b5 ? a[i] : a[i + 4];
        float keep = b5 ? a[i + 4] : a[i];
        a[i] = keep + __shfl_xor(send, 32);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float send = b4 ? a[i] : a[i + 2];
        float keep = b4 ? a[i + 2] : a[i];
        a[i] = keep + __shfl_xor(send, 16);
    }
    {
        float send = b3 ? a[0] : a[1];
        float keep = b3 ? a[1] : a[0];
        a[0] = keep + __shfl_xor(send, 8);
    }
    a[0] += __shfl_xor(a[0], 4);
    a[0] += __shfl_xor(a[0], 2);
    a[0] += __shfl_xor(a[0], 1);
    return a[0];
}

// Dot products of the query with ROWS key rows (all loads issued first).
// Returns in out[h] the full sum of row 8h + ((lane >> 3) & 7).  Invalid
// rows (ok[i] false) read nothing.
template <int VPR, int ROWS>
__device__ __forceinline__ void dot_rows(const float* const (&rows)[ROWS], const bool (&ok)[ROWS],
                                         const float4 (&qv)[VPR], float (&out)[ROWS / 8]) {
    const int lane = lane_id();
    float4 k[ROWS][VPR];
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
#pragma unroll
        for (int j = 0; j < VPR; ++j)
            k[i][j] = ok[i] ? load_stream(rows[i] + 4 * (lane + 64 * j))
                            : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int h = 0; h < ROWS / 8; ++h) {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < VPR; ++j) {
                const float4 x = k[8 * h + i][j];
                s += qv[j].x * x.x + qv[j].y * x.y + qv[j].z * x.z + qv[j].w * x.w;
            }
            a[i] = s;
        }
        out[h] = reduce8(a);
    }
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- E4M3 rows
//
// Key rows of RB = 256 * VPR E4M3FN bytes are read by 16 lanes each, four
// rows per load instruction: lane l serves row (l >> 4) of a group of four
// and the 16-byte columns 16 (l & 15) + 256 j, j < VPR, of that row.  A wave
// iteration covers G = 16 / VPR such groups (16 KB).  The per-lane partial
// sums of the G groups are reduced over the 16 lanes of each row by a
// transposition through DPP lane permutations (row mirror, half-row mirror,
// quad permutes), so that lane l ends with the full sum of row
// 4 (((l & 15) >> (4 - log2 G))) + (l >> 4) of the iteration.

// Lane-resident query slice for this layout: qv[j][m] = floats
// [256 j + 16 (l & 15) + 4 m, +4) of the query row (heads summed when the
// key head is shared, Hk == 1).
template <int VPR>
__device__ __forceinline__ void load_qvec16(const float* __restrict__ qI, int q, int Hi, int Hk,
                                            int Di, float4 (&qv)[VPR][4]) {
    const int u = lane_id() & 15;
#pragma unroll
    for (int j = 0; j < VPR; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int c = 64 * j + 4 * u + m;   // float4 index within the row
            if (Hk == Hi) {
                qv[j][m] = reinterpret_cast<const float4*>(qI + (size_t)q * Hi * Di)[c];
            } else {
                float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int h = 0; h < Hi; ++h) {
                    const float4 v = reinterpret_cast<const float4*>(qI + ((size_t)q * Hi + h) * Di)[c];
                    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
                }
                qv[j][m] = s;
            }
        }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// One transposition step: N values per lane become N/2, each the sum over
// this lane and its partner (lane ^ mask, as the DPP control CTRL permutes);
// lanes with bit SB set keep the upper half of the indices.
template <int N, int CTRL, int SB>
__device__ __forceinline__ void tstep(float (&a)[16]) {
    const bool up = (lane_id() >> SB) & 1;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = up ? a[i] : a[i + N / 2];
        const float keep = up ? a[i + N / 2] : a[i];
        a[i] = keep + dpp_f32<CTRL>(send);
    }
}

constexpr int kDppRowMirror = 0x140;       // lane i <- lane 15 - i (xor 15 in a row of 16)
constexpr int kDppHalfMirror = 0x141;      // lane i <- lane 7 - i  (xor 7 in a half row)
constexpr int kDppXor2 = 0x4E;             // quad_perm [2,3,0,1]
constexpr int kDppXor1 = 0xB1;             // quad_perm [1,0,3,2]

template <int G>
constexpr int log2_groups() { return G == 16 ? 4 : G == 8 ? 3 : G == 4 ? 2 : G == 2 ? 1 : 0; }

// Sum of a[g] over the 16 lanes of this lane's row, for g = the group this
// lane ends with ((l & 15) >> (4 - log2 G)); the masks 15, 7, 2, 1 span all
// 16 lanes, the steps past log2 G are plain butterflies.
template <int G>
__device__ __forceinline__ float reduce16(float (&a)[16]) {
    constexpr int L = log2_groups<G>();
    if constexpr (L >= 1) tstep<G, kDppRowMirror, 3>(a);
    if constexpr (L >= 2) tstep<G / 2, kDppHalfMirror, 2>(a);
    if constexpr (L >= 3) tstep<G / 4, kDppXor2, 1>(a);
    if constexpr (L >= 4) tstep<G / 8, kDppXor1, 0>(a);
    if constexpr (L < 1) a[0] += dpp_f32<kDppRowMirror>(a[0]);
    if constexpr (L < 2) a[0] += dpp_f32<kDppHalfMirror>(a[0]);
    if constexpr (L < 3) a[0] += dpp_f32<kDppXor2>(a[0]);
    if constexpr (L < 4) a[0] += dpp_f32<kDppXor1>(a[0]);
    return a[0];
}

// Dot products of the query slice with this lane's NB x G rows: grow[b][g]
// points at byte 16 (l & 15) of the row this lane reads in group g of
// sub-block b.  All NB x G loads are issued before the first product.
// out[b] = the full sum of the row of sub-block b named above.
template <int VPR, int G, int NB>
__device__ __forceinline__ void dot_rows16(const uint8_t* const (&grow)[NB][G],
                                           const float4 (&qv)[VPR][4], float (&out)[NB]) {
    u32x4v w[NB][G][VPR];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < VPR; ++j)
                w[b][g][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4v*>(grow[b][g] + 256 * j));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float a[16];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < VPR; ++j)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float2 lo = fp8x2_to_f32<false>(w[b][g][j][m]);
                    const float2 hi = fp8x2_to_f32<true>(w[b][g][j][m]);
                    s += qv[j][m].x * lo.x + qv[j][m].y * lo.y + qv[j][m].z * hi.x +
                         qv[j][m].w * hi.y;
                }
            a[g] = s;
        }
        out[b] = reduce16<G>(a);
    }
}

}  // namespace
}  // namespace csa2
