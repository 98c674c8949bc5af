// Row-dot helpers and constants shared by the score stream and the Reindex
// scorer (gfx950, wave64): a key row of RW = 256*VPR floats (Hk heads of Di
// channels) dotted with the query row held in registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace csa2 {
namespace {

constexpr int kHistBins = 4096;      // first-level digit: top 12 bits of the key
constexpr int kDigitShift = 20;
constexpr int kStreamThreads = 512;
constexpr int kRowsPerWG = 2048;     // score stream: rows per workgroup

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

}  // namespace
}  // namespace csa2
