// Score stream of the CSA2 Full-mode indexer (gfx950): one pass over every
// visible key row at HBM speed, writing each score's order-preserving key
// and the first-level histograms the selection starts from.
//
// Method (jaehun.me review of arXiv 2609.19969, section "2) CSA2"): a Full
// layer scores every visible compressed entry with its indexer; the score is
// the sum over indexer heads of the query head dotted with the key row.  Key
// rows are fp32 or, in the compact cache, one E4M3FN byte per value.
#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"

namespace csa2 {
namespace {

template <int VPR, typename KT>
__global__ __launch_bounds__(kStreamThreads) void k_score_stream(
    const float* __restrict__ qI, const KT* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_nvis, int Hi, int Hk, int Di, uint32_t* __restrict__ keys,
    int64_t kstride, uint32_t* __restrict__ hist_e, uint32_t* __restrict__ bkeys,
    int64_t bstride, int bs_log2, uint32_t* __restrict__ hist_b) {
    // 16-bit bin counters, two per word (a workgroup sees at most
    // kRowsPerWG keys), so that four workgroups fit a CU's LDS
    __shared__ uint32_t s_he[kHistBins / 2];
    __shared__ uint32_t s_hb[kHistBins / 2];
    // this workgroup's keys, written out as whole lines at the end
    __shared__ __attribute__((aligned(16))) uint32_t s_ke[kRowsPerWG];
    __shared__ __attribute__((aligned(16))) uint32_t s_kb[kRowsPerWG];
    constexpr int RW = 256 * VPR;
    constexpr int kStreamRows = stream_rows<VPR, KT>();   // rows per wave iteration
    const int q = blockIdx.y;
    const int nvis = min(q_nvis[q], (int)kstride);   // q_nvis <= max_nvis <= kstride
    const int r0 = blockIdx.x * kRowsPerWG;
    if (r0 >= nvis) return;
    const int r1 = min(nvis, r0 + kRowsPerWG);
    const bool pool = bkeys != nullptr;
    for (int i = threadIdx.x; i < kHistBins / 2; i += kStreamThreads) { s_he[i] = 0; s_hb[i] = 0; }
    __syncthreads();

    float4 qv[VPR];
    load_qvec<VPR, sizeof(KT) == 1>(qI, q, Hi, Hk, Di, qv);
    const int64_t row0 = seq_row_off[q_seq ? q_seq[q] : 0];
    const KT* kb = kI + row0 * RW;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int myrow = (lane >> 3) & 7;
    const uint32_t bmask = (1u << bs_log2) - 1u;
    uint32_t* krow = keys + (size_t)q * kstride;

    for (int g0 = r0 + kStreamRows * wave; g0 < r1; g0 += kStreamRows * (kStreamThreads / kWave)) {
        const KT* rows[kStreamRows];
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
                uint32_t bk = valid ? k : 0u;
                if (bs_log2 >= 1) bk = max(bk, (uint32_t)__shfl_xor(bk, 8));
                if (bs_log2 >= 2) bk = max(bk, (uint32_t)__shfl_xor(bk, 16));
                if (bs_log2 >= 3) bk = max(bk, (uint32_t)__shfl_xor(bk, 32));
                if ((lane & 7) == 0 && valid && ((uint32_t)myrow & bmask) == 0) {
                    s_kb[(row - r0) >> bs_log2] = bk;
                    const uint32_t d = bk >> kDigitShift;
                    atomicAdd(&s_hb[d >> 1], 1u << ((d & 1u) << 4));
                }
            }
        }
    }
    __syncthreads();
    // r0 and the key strides are multiples of 4 (64): whole uint4 stores,
    // a scalar tail for the last workgroup of a row
    const int nk = r1 - r0;
    for (int i = 4 * threadIdx.x; i < nk; i += 4 * kStreamThreads) {
        if (i + 4 <= nk)
            *reinterpret_cast<uint4*>(krow + r0 + i) = *reinterpret_cast<const uint4*>(s_ke + i);
        else
            for (int x = i; x < nk; ++x) krow[r0 + x] = s_ke[x];
    }
    if (pool) {
        const int b0 = r0 >> bs_log2, nb = ((r1 - 1) >> bs_log2) - b0 + 1;
        uint32_t* brow = bkeys + (size_t)q * bstride + b0;
        for (int i = 4 * threadIdx.x; i < nb; i += 4 * kStreamThreads) {
            if (i + 4 <= nb)
                *reinterpret_cast<uint4*>(brow + i) = *reinterpret_cast<const uint4*>(s_kb + i);
            else
                for (int x = i; x < nb; ++x) brow[x] = s_kb[x];
        }
    }
    for (int i = threadIdx.x; i < kHistBins; i += kStreamThreads) {
        const uint32_t sh = (i & 1) << 4;
        const uint32_t ce = (s_he[i >> 1] >> sh) & 0xFFFFu;
        if (ce) atomicAdd(&hist_e[(size_t)q * kHistBins + i], ce);
        if (pool) {
            const uint32_t cb = (s_hb[i >> 1] >> sh) & 0xFFFFu;
            if (cb) atomicAdd(&hist_b[(size_t)q * kHistBins + i], cb);
        }
    }
}

}  // namespace

int launch_score_stream(int vpr, bool e4m3, dim3 grid, hipStream_t s, const float* qI,
                        const void* kI, const int64_t* seq_row_off, const int32_t* q_seq,
                        const int32_t* q_nvis, int Hi, int Hk, int Di, uint32_t* keys,
                        int64_t kstride, uint32_t* hist_e, uint32_t* bkeys, int64_t bstride,
                        int bs_log2, uint32_t* hist_b) {
#define CSA2_STREAM(V, KT, NAME)                                                              \
    CSA2_LAUNCH(NAME, (k_score_stream<V, KT>), grid, dim3(kStreamThreads), s, qI,             \
                static_cast<const KT*>(kI), seq_row_off, q_seq, q_nvis, Hi, Hk, Di, keys,     \
                kstride, hist_e, bkeys, bstride, bs_log2, hist_b)
    if (e4m3)
        return vpr == 1   ? CSA2_STREAM(1, uint8_t, "score_stream_e4m3")
               : vpr == 2 ? CSA2_STREAM(2, uint8_t, "score_stream_e4m3")
                          : CSA2_STREAM(4, uint8_t, "score_stream_e4m3");
    return vpr == 1   ? CSA2_STREAM(1, float, "score_stream")
           : vpr == 2 ? CSA2_STREAM(2, float, "score_stream")
                      : CSA2_STREAM(4, float, "score_stream");
#undef CSA2_STREAM
}

}  // namespace csa2
