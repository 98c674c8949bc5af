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
constexpr int kStreamThreads = 512;
constexpr int kRowsPerWG = 2048;     // score stream: rows per workgroup

// Float4 chunk j of lane l's slice of a key row.  fp32 keys: chunk l + 64 j
// (each load instruction covers 1 KB of the row); E4M3 keys: chunk VPR l + j,
// so that a lane's 4 VPR key bytes are contiguous (one dword / dwordx2 /
// dwordx4 load per row).
template <int VPR, bool BYTES>
__device__ __forceinline__ int qchunk(int lane, int j) {
    return BYTES ? VPR * lane + j : lane + 64 * j;
}

// Lane-resident slice of the query vector, in the key layout's chunk order
// (qchunk).  With one shared key head (Hk == 1) the query heads are summed
// first.
template <int VPR, bool BYTES = false>
__device__ __forceinline__ void load_qvec(const float* __restrict__ qI, int q, int Hi, int Hk,
                                          int Di, float4 (&qv)[VPR]) {
    const int lane = lane_id();
    if (Hk == Hi) {
        const float4* p = reinterpret_cast<const float4*>(qI + (size_t)q * Hi * Di);
#pragma unroll
        for (int j = 0; j < VPR; ++j) qv[j] = p[qchunk<VPR, BYTES>(lane, j)];
    } else {
#pragma unroll
        for (int j = 0; j < VPR; ++j) {
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int h = 0; h < Hi; ++h) {
                float4 v = reinterpret_cast<const float4*>(qI + ((size_t)q * Hi + h) * Di)
                    [qchunk<VPR, BYTES>(lane, j)];
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

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Streaming load of a lane's 4*VPR contiguous E4M3 key bytes (nontemporal,
// as for fp32 keys).
template <int VPR>
__device__ __forceinline__ void load_stream8(const uint8_t* p, uint32_t (&w)[VPR]) {
    if constexpr (VPR == 1) {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (VPR == 2) {
        const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
        w[0] = v[0]; w[1] = v[1];
    } else {
        const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    }
}

// E4M3 key rows: the same dot products, each key byte decoded to fp32 by the
// gfx950 OCP FP8 conversion (exact) before the multiply.  Lane l reads bytes
// [4 VPR l, 4 VPR (l + 1)) of each row, matching load_qvec<VPR, true>.
template <int VPR, int ROWS>
__device__ __forceinline__ void dot_rows(const uint8_t* const (&rows)[ROWS], const bool (&ok)[ROWS],
                                         const float4 (&qv)[VPR], float (&out)[ROWS / 8]) {
    const int lane = lane_id();
    uint32_t k[ROWS][VPR];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        if (ok[i]) {
            load_stream8<VPR>(rows[i] + 4 * VPR * lane, k[i]);
        } else {
#pragma unroll
            for (int j = 0; j < VPR; ++j) k[i][j] = 0u;
        }
    }
#pragma unroll
    for (int h = 0; h < ROWS / 8; ++h) {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < VPR; ++j) {
                const float2 lo = fp8x2_to_f32<false>(k[8 * h + i][j]);
                const float2 hi = fp8x2_to_f32<true>(k[8 * h + i][j]);
                s += qv[j].x * lo.x + qv[j].y * lo.y + qv[j].z * hi.x + qv[j].w * hi.y;
            }
            a[i] = s;
        }
        out[h] = reduce8(a);
    }
}

// Rows per wave and gather round: the same bytes in flight for both key
// formats (a 2 KB fp32 row holds as many bytes as four E4M3 rows).
template <int VPR, typename KT>
constexpr int stream_rows() {
    return sizeof(KT) == 1 ? (VPR >= 4 ? 32 : 64) : (VPR >= 4 ? 8 : 16);
}

}  // namespace
}  // namespace csa2
