// Score stream of the CSA2 Full-mode indexer (gfx950): one pass over every
// visible key row at HBM speed, writing each score's order-preserving key
// and the first-level histograms the selection starts from.
//
// Method (jaehun.me review of arXiv 2609.19969, section "2) CSA2"): a Full
// layer scores every visible compressed entry with its indexer; the score is
// the sum over indexer heads of the query head dotted with the key row.  Key
// rows are fp32 (k_score_stream) or, in the compact cache, one E4M3FN byte
// per value (k_score_stream_e4m3).
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"

namespace csa2 {
namespace {

// End of a score-stream workgroup: its keys (staged in LDS) are written out
// as whole lines and its 16-bit LDS bin counts added to the query's
// histograms.
template <int NT>
__device__ __forceinline__ void stream_flush(int q, int r0, int r1, bool pool, int bs_log2,
                                             const uint32_t* s_ke, const uint32_t* s_kb,
                                             const uint32_t* s_he, const uint32_t* s_hb,
                                             uint32_t* __restrict__ krow,
                                             uint32_t* __restrict__ bkeys, int64_t bstride,
                                             uint32_t* __restrict__ hist_e,
                                             uint32_t* __restrict__ hist_b) {
    __syncthreads();
    // r0 and the key strides are multiples of 4 (64): whole 16-byte stores
    // (nontemporal: the keys are read once, by the select, and stay out of
    // the way of the row stream), a scalar tail for the last workgroup of a row
    typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
    const int nk = r1 - r0;
    for (int i = 4 * threadIdx.x; i < nk; i += 4 * NT) {
        if (i + 4 <= nk)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4s*>(s_ke + i),
                                        reinterpret_cast<u32x4s*>(krow + r0 + i));
        else
            for (int x = i; x < nk; ++x) krow[r0 + x] = s_ke[x];
    }
    if (pool) {
        const int b0 = r0 >> bs_log2, nb = ((r1 - 1) >> bs_log2) - b0 + 1;
        uint32_t* brow = bkeys + (size_t)q * bstride + b0;
        for (int i = 4 * threadIdx.x; i < nb; i += 4 * NT) {
            if (i + 4 <= nb)
                *reinterpret_cast<uint4*>(brow + i) = *reinterpret_cast<const uint4*>(s_kb + i);
            else
                for (int x = i; x < nb; ++x) brow[x] = s_kb[x];
        }
    }
    for (int i = threadIdx.x; i < kHistBins; i += NT) {
        const uint32_t sh = (i & 1) << 4;
        const uint32_t ce = (s_he[i >> 1] >> sh) & 0xFFFFu;
        if (ce) atomicAdd(&hist_e[(size_t)q * kHistBins + i], ce);
        if (pool) {
            const uint32_t cb = (s_hb[i >> 1] >> sh) & 0xFFFFu;
            if (cb) atomicAdd(&hist_b[(size_t)q * kHistBins + i], cb);
        }
    }
}

template <int VPR>
__global__ __launch_bounds__(kStreamThreads32) void k_score_stream(
    const float* __restrict__ qI, const float* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_nvis, int Hi, int Hk, int Di, uint32_t* __restrict__ keys,
    int64_t kstride, uint32_t* __restrict__ hist_e, uint32_t* __restrict__ bkeys,
    int64_t bstride, int bs_log2, int block_sum, uint32_t* __restrict__ hist_b, int rpw,
    int max_nvis) {
    // 16-bit bin counters, two per word (a workgroup sees at most
    // kRowsPerWG keys).  Three 4-wave workgroups of 4,096 rows (48 KB of LDS
    // each) fill the twelve wave slots the registers allow per CU; a sweep
    // over 256/512 threads and 1,024-4,096 rows per workgroup chose this
    __shared__ uint32_t s_he[kHistBins / 2];
    __shared__ uint32_t s_hb[kHistBins / 2];
    // this workgroup's keys, written out as whole lines at the end
    __shared__ __attribute__((aligned(16))) uint32_t s_ke[kRowsPerWG];
    __shared__ __attribute__((aligned(16))) uint32_t s_kb[kRowsPerWG];
    constexpr int RW = 256 * VPR;
    constexpr int kStreamRows = VPR >= 4 ? 8 : 16;   // rows per wave iteration (32 KB of 2 KB rows)
    const int q = blockIdx.y;
    const int nvis = min(q_nvis[q], max_nvis);   // a larger q_nvis counts as max_nvis
    const int r0 = blockIdx.x * rpw;   // rpw <= kRowsPerWG, a multiple of 64
    if (r0 >= nvis) return;
    const int r1 = min(nvis, r0 + rpw);
    const bool pool = bkeys != nullptr;
    for (int i = threadIdx.x; i < kHistBins / 2; i += kStreamThreads32) { s_he[i] = 0; s_hb[i] = 0; }
    __syncthreads();

    float4 qv[VPR];
    load_qvec<VPR>(qI, q, Hi, Hk, Di, qv);
    const int64_t row0 = seq_row_off[q_seq ? q_seq[q] : 0];
    const float* kb = kI + row0 * RW;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int myrow = (lane >> 3) & 7;
    const uint32_t bmask = (1u << bs_log2) - 1u;
    uint32_t* krow = keys + (size_t)q * kstride;

    for (int g0 = r0 + kStreamRows * wave; g0 < r1; g0 += kStreamRows * (kStreamThreads32 / kWave)) {
        const float* rows[kStreamRows];
        bool ok[kStreamRows];
#pragma unroll
        for (int i = 0; i < kStreamRows; ++i) {
            ok[i] = g0 + i < r1;
            rows[i] = kb + (int64_t)(g0 + i) * RW;
        }
        float sc[kStreamRows / 8];
        dot_rows<VPR, kStreamRows>(rows, ok, qv, sc);
#pragma unroll
        for (int hh = 0; hh < kStreamRows / 8; ++hh) {
            const int row = g0 + 8 * hh + myrow;
            const bool valid = row < r1;
            const uint32_t k = ord_key(sc[hh]);
            if ((lane & 7) == 0 && valid) {
                s_ke[row - r0] = k;
                const uint32_t d = k >> kDigitShift;
                atomicAdd(&s_he[d >> 1], 1u << ((d & 1u) << 4));
            }
            if (pool) {
                // rows 8 hh + 0..7 sit in lanes that differ in bits 3..5
                uint32_t bk;
                if (block_sum) {
                    float bsum = valid ? sc[hh] : 0.f;
                    if (bs_log2 >= 1) bsum += __shfl_xor(bsum, 8);
                    if (bs_log2 >= 2) bsum += __shfl_xor(bsum, 16);
                    if (bs_log2 >= 3) bsum += __shfl_xor(bsum, 32);
                    bk = ord_key(bsum);
                } else {
                    bk = valid ? k : 0u;
                    if (bs_log2 >= 1) bk = max(bk, (uint32_t)__shfl_xor(bk, 8));
                    if (bs_log2 >= 2) bk = max(bk, (uint32_t)__shfl_xor(bk, 16));
                    if (bs_log2 >= 3) bk = max(bk, (uint32_t)__shfl_xor(bk, 32));
                }
                if ((lane & 7) == 0 && valid && ((uint32_t)myrow & bmask) == 0) {
                    s_kb[(row - r0) >> bs_log2] = bk;
                    const uint32_t d = bk >> kDigitShift;
                    atomicAdd(&s_hb[d >> 1], 1u << ((d & 1u) << 4));
                }
            }
        }
    }
    stream_flush<kStreamThreads32>(q, r0, r1, pool, bs_log2, s_ke, s_kb, s_he, s_hb, krow, bkeys, bstride, hist_e,
                 hist_b);
}

// The stream over E4M3 key rows (RB = 256 * VPR bytes): 16 lanes per row,
// four rows per load instruction, G = 16 / VPR groups of four rows (16 KB) per
// sub-block and NB sub-blocks per wave iteration (see dot_rows16).  Rows past
// the workgroup's last one are read as that last row again and discarded, so
// no load is predicated.
template <int VPR, int NB>
__global__ __launch_bounds__(kStreamThreads8) void k_score_stream_e4m3(
    const float* __restrict__ qI, const uint8_t* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_nvis, int Hi, int Hk, int Di, uint32_t* __restrict__ keys,
    int64_t kstride, uint32_t* __restrict__ hist_e, uint32_t* __restrict__ bkeys,
    int64_t bstride, int bs_log2, int block_sum, uint32_t* __restrict__ hist_b, int rpw,
    int max_nvis) {
    __shared__ uint32_t s_he[kHistBins / 2];
    __shared__ uint32_t s_hb[kHistBins / 2];
    __shared__ __attribute__((aligned(16))) uint32_t s_ke[kRowsPerWG8];
    __shared__ __attribute__((aligned(16))) uint32_t s_kb[kRowsPerWG8];
    constexpr int RB = 256 * VPR;
    constexpr int G = 16 / VPR;
    constexpr int RPB = 4 * G;                            // rows per sub-block
    constexpr int RPI = NB * RPB;                         // rows per wave iteration
    constexpr int GSH = 4 - log2_groups<G>();             // lane bits below the group index
    const int q = blockIdx.y;
    const int nvis = min(q_nvis[q], max_nvis);
    const int r0 = blockIdx.x * rpw;   // rpw <= kRowsPerWG8, a multiple of 64
    if (r0 >= nvis) return;
    const int r1 = min(nvis, r0 + rpw);
    const bool pool = bkeys != nullptr;
    for (int i = threadIdx.x; i < kHistBins / 2; i += kStreamThreads8) { s_he[i] = 0; s_hb[i] = 0; }
    __syncthreads();

    float4 qv[VPR][4];
    load_qvec16<VPR>(qI, q, Hi, Hk, Di, qv);
    const int64_t row0 = seq_row_off[q_seq ? q_seq[q] : 0];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int rq = lane >> 4;                             // row within a group of four
    const int mg = (lane & 15) >> GSH;                    // group whose sum this lane ends with
    const int myrow = 4 * mg + rq;                        // row of that sum within a sub-block
    const bool writer = (lane & ((1 << GSH) - 1)) == 0;
    const uint8_t* kl = kI + row0 * RB + 16 * (lane & 15);
    const uint32_t bmask = (1u << bs_log2) - 1u;
    uint32_t* krow = keys + (size_t)q * kstride;

    for (int g0 = r0 + RPI * wave; g0 < r1; g0 += RPI * (kStreamThreads8 / kWave)) {
        const uint8_t* grow[NB][G];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < G; ++g)
                grow[b][g] = kl + (int64_t)min(g0 + RPB * b + 4 * g + rq, r1 - 1) * RB;
        float sc[NB];
        dot_rows16<VPR, G, NB>(grow, qv, sc);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int row = g0 + RPB * b + myrow;
            const bool valid = row < r1;
            const uint32_t k = ord_key(sc[b]);
            if (writer && valid) {
                s_ke[row - r0] = k;
                const uint32_t d = k >> kDigitShift;
                atomicAdd(&s_he[d >> 1], 1u << ((d & 1u) << 4));
            }
        }
    }
    if (pool) {
        // block keys from the row keys staged in LDS: block bi covers rows
        // [bi << bs_log2, (bi + 1) << bs_log2) of this workgroup's range
        // (ranges start on whole blocks: rpw is a multiple of 8); for
        // the maximum, the rows past the last valid one read as 0, below
        // every real key
        const int nk = r1 - r0, nb = (nk + (int)bmask) >> bs_log2;
        if (threadIdx.x < 8 && nk + (int)threadIdx.x < ((nk + 7) & ~7)) s_ke[nk + threadIdx.x] = 0u;
        __syncthreads();
        for (int bi = threadIdx.x; bi < nb; bi += kStreamThreads8) {
            const int i0 = bi << bs_log2;
            uint32_t bk = 0u;
            if (block_sum) {
                // the scores back from their keys, summed in row order over
                // the block's valid rows
                float bsum = 0.f;
                for (int i = i0; i < min(nk, i0 + (1 << bs_log2)); ++i)
                    bsum += ord_key_to_f32(s_ke[i]);
                bk = ord_key(bsum);
            } else if (bs_log2 >= 2) {
                for (int i = i0; i < i0 + (1 << bs_log2); i += 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(s_ke + i);
                    bk = max(bk, max(max(v.x, v.y), max(v.z, v.w)));
                }
            } else {
                for (int i = i0; i < i0 + (1 << bs_log2); ++i) bk = max(bk, s_ke[i]);
            }
            s_kb[bi] = bk;
            const uint32_t d = bk >> kDigitShift;
            atomicAdd(&s_hb[d >> 1], 1u << ((d & 1u) << 4));
        }
    }
    stream_flush<kStreamThreads8>(q, r0, r1, pool, bs_log2, s_ke, s_kb, s_he, s_hb, krow, bkeys, bstride, hist_e,
                 hist_b);
}

}  // namespace

int launch_score_stream(int vpr, bool e4m3, int max_nvis, int Q, hipStream_t s,
                        const float* qI, const void* kI, const int64_t* seq_row_off,
                        const int32_t* q_seq, const int32_t* q_nvis, int Hi, int Hk, int Di,
                        uint32_t* keys, int64_t kstride, uint32_t* hist_e, uint32_t* bkeys,
                        int64_t bstride, int bs_log2, int block_sum, uint32_t* hist_b) {
    // rows per workgroup: the tuned maximum for large launches; small ones
    // (few queries, short rows) are cut into more workgroups, about 512
    // (fp32) or 256 (E4M3, two per CU) in all, of at least 64 rows
    const int rmax = e4m3 ? kRowsPerWG8 : kRowsPerWG;
    const int64_t want = ((int64_t)Q * max_nvis + (e4m3 ? 255 : 511)) / (e4m3 ? 256 : 512);
    const int rpw = (int)std::min<int64_t>(rmax, std::max<int64_t>(64, (want + 63) / 64 * 64));
    const dim3 grid((max_nvis + rpw - 1) / rpw, Q);
    const dim3 block(e4m3 ? kStreamThreads8 : kStreamThreads32);
#define CSA2_STREAM(KERNEL, KT, NAME)                                                         \
    CSA2_LAUNCH(NAME, KERNEL, grid, block, s, qI, static_cast<const KT*>(kI),                \
                seq_row_off, q_seq, q_nvis, Hi, Hk, Di, keys, kstride, hist_e, bkeys, bstride,\
                bs_log2, block_sum, hist_b, rpw, max_nvis)
    if (e4m3)
        return vpr == 1 ? CSA2_STREAM((k_score_stream_e4m3<1, kStreamNB8>), uint8_t,
                                      "score_stream_e4m3")
               : vpr == 2 ? CSA2_STREAM((k_score_stream_e4m3<2, kStreamNB8>), uint8_t,
                                        "score_stream_e4m3")
                          : CSA2_STREAM((k_score_stream_e4m3<4, kStreamNB8>), uint8_t,
                                        "score_stream_e4m3");
    return vpr == 1   ? CSA2_STREAM(k_score_stream<1>, float, "score_stream")
           : vpr == 2 ? CSA2_STREAM(k_score_stream<2>, float, "score_stream")
                      : CSA2_STREAM(k_score_stream<4>, float, "score_stream");
#undef CSA2_STREAM
}

}  // namespace csa2
