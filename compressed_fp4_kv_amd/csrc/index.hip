// Full-mode indexer (score stream + exact Top-K + candidate pool) and the
// Reindex step of CSA2, for gfx950.
//
// Method (jaehun.me review of arXiv 2609.19969, section "2) CSA2" and the
// worked example of the modes): a Full layer scores every visible compressed
// entry with its indexer and keeps the Top-K; the decoder's first Full layer
// also keeps the best 2,048 blocks of 8 positions as a candidate pool; a
// Reindex layer rescores only the pool with its own indexer query.
//
// Structure on the GPU
//   1. k_score_stream (stream.hip): one pass over the key rows at HBM speed.  A wave
//      takes 8 rows at a time (each lane holds 2 float4 of every 2 KB row,
//      fully coalesced), dots them with the query held in registers and
//      reduces the 8 sums across the wave with a transpose-reduction.  The
//      order-preserving uint32 key of each score goes to workspace, together
//      with a 4096-bin histogram of its top 12 bits (LDS, flushed once per
//      workgroup) and, for the pool, the block maximum and its histogram.
//   2. k_filter: the histogram gives the bin holding the K-th key; entries
//      above it are certain winners, entries in it are candidates (their
//      composite key score|~index goes to a short list); one atomic per
//      workgroup and list.
//   3. k_finalize: one workgroup per query selects the remaining winners
//      among the candidates (direct ranking, or a register-resident 64-bit
//      radix select) and writes the K winners in index order.  If the
//      candidate bin holds more than 16,384 entries (degenerate score
//      distributions) it falls back to an exact select over the whole row.
//   (Kernel boundaries order the phases: a grid-wide "last workgroup" hand-
//   off would need agent-scope fences, which write back L2 on this part.)
//   Reindex: k_reindex_score gathers the pool rows (8 contiguous 2 KB rows
//   per block) with the same 8-row dot and writes one 4-byte score key per
//   candidate; k_reindex_select rebuilds the <= 16,384 composite keys of a
//   query from them and the pool row, and selects in one workgroup.
#include <limits.h>

#include <algorithm>

#include <mutex>

#include "common.hpp"
#include "internal.hpp"
#include "rowdot.hpp"

namespace csa2 {
namespace {

constexpr int kCandCap = 16384;      // candidates a selecting workgroup holds
constexpr int kSelThreads = 1024;
constexpr int kSelItems = kCandCap / kSelThreads;
constexpr int kSelElems = 16384;    // filter: keys per workgroup (64 per thread)
constexpr int kFilterLoads = kSelElems / (4 * 256);   // uint4 loads per thread
constexpr int kRankMax = 4096;      // candidates held in LDS by the one-workgroup selects
constexpr int kRankDirect = 512;    // up to this many candidates are ranked directly
constexpr int kLdsCandItems = kRankMax / kSelThreads;  // per thread, radix path
constexpr int kSmallRow = 65536;    // rows up to this length are selected by one workgroup
constexpr int kRowRegs = kSmallRow / (4 * kSelThreads);   // uint4 per thread for a whole row
constexpr int kReindexPerWG = 256;   // reindex: candidates per workgroup
constexpr int kReindexThreads = 256;

__global__ void k_zero_u32(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ------------------------------------------------------------ selects

// Radix select over NT*IPT register-resident 64-bit keys (0 = empty slot;
// non-empty keys distinct): returns T such that exactly `k` keys are >= T.
// 1 <= k <= number of non-empty keys.
// Digits are taken from bit `top_shift` down; bits above top_shift + 8 must
// already be equal across all keys.  Stops early once the chosen digit's
// bucket holds exactly the keys still wanted.  Once the score word (bits
// 32-63) is resolved, the keys tied on it (at most kTieCap) are ranked
// directly by their index word instead of taking four more radix passes:
// with integer scores the K-th score is usually shared by a few keys.
constexpr int kTieCap = 1024;

template <int NT, int IPT>
__device__ uint64_t block_select_kth(const uint64_t (&it)[IPT], uint32_t k, uint32_t* s_hist,
                                     uint32_t* s_dig, int top_shift) {
    uint64_t prefix = 0, mask = 0;
    uint32_t want = k;
    if (top_shift < 56) {
        // common high bits: take them from any non-empty key
        uint64_t any = 0;
#pragma unroll
        for (int j = 0; j < IPT; ++j) any = it[j] ? it[j] : any;
        if (threadIdx.x == 0) s_dig[0] = 0;
        __syncthreads();
        if (any) { s_dig[0] = (uint32_t)(any >> 32); }
        __syncthreads();
        const uint64_t hi_mask = ~((1ull << (top_shift + 8)) - 1ull);
        prefix = ((uint64_t)s_dig[0] << 32) & hi_mask;
        mask = hi_mask;
        __syncthreads();
    }
    for (int shift = top_shift; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += NT) s_hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint64_t v = it[j];
            const bool m = v != 0 && (v & mask) == prefix;
            const uint32_t d = (uint32_t)(v >> shift) & 255u;
            // one atomic per wave when all matching lanes share the digit
            const uint64_t mm = __ballot(m);
            if (mm) {
                const int lead = __builtin_ctzll(mm);
                const uint32_t d0 = __shfl(d, lead);
                const uint64_t same = __ballot(m && d == d0);
                if (same == mm) {
                    if (lane_id() == lead) atomicAdd(&s_hist[d0], (uint32_t)__popcll(mm));
                } else if (m) {
                    atomicAdd(&s_hist[d], 1u);
                }
            }
        }
        __syncthreads();
        find_digit_256(s_hist, want, s_dig);
        const uint32_t d = s_dig[0], above = s_dig[1];
        const uint32_t bucket = s_hist[d];
        __syncthreads();
        prefix |= (uint64_t)d << shift;
        mask |= 0xFFull << shift;
        want -= above;
        if (bucket == want) break;   // every key of this bucket is selected
        if (shift == 32 && bucket <= (uint32_t)kTieCap) {
            // the bucket's keys share the K-th score; their index words are
            // distinct, and the want-th largest has exactly want - 1 above it
            __shared__ uint32_t s_tie[kTieCap];
            __shared__ uint32_t s_nt;
            if (threadIdx.x == 0) s_nt = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < IPT; ++j)
                if (it[j] != 0 && (it[j] & mask) == prefix)
                    s_tie[atomicAdd(&s_nt, 1u)] = (uint32_t)it[j];
            __syncthreads();
            for (int i = threadIdx.x; i < (int)bucket; i += NT) {
                const uint32_t v = s_tie[i];
                uint32_t r = 0;
                for (int x = 0; x < (int)bucket; ++x) r += s_tie[x] > v;
                if (r == want - 1u) s_dig[0] = v;
            }
            __syncthreads();
            prefix |= (uint64_t)s_dig[0];
            __syncthreads();
            break;
        }
    }
    return prefix;
}

// Exact Top-K over a whole row of uint32 keys (n > K) by one workgroup,
// written in ascending index order: radix-select the K-th key value T, then
// an ordered pass keeps every key > T and the lowest-index ties of T.
template <int NT>
__device__ void select_global_row(const uint32_t* __restrict__ keys, int n, int K,
                                  int32_t* __restrict__ out, uint32_t* s_hist, uint32_t* s_dig,
                                  uint32_t* s_tmp) {
    uint32_t prefix = 0, mask = 0, want = (uint32_t)K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += NT) s_hist[i] = 0u;
        __syncthreads();
        for (int base = 0; base < n; base += NT) {
            const int i = base + threadIdx.x;
            const uint32_t v = i < n ? keys[i] : 0u;
            const bool m = i < n && (v & mask) == prefix;
            const uint32_t d = (v >> shift) & 255u;
            const uint64_t mm = __ballot(m);
            if (mm) {
                const int lead = __builtin_ctzll(mm);
                const uint32_t d0 = __shfl(d, lead);
                const uint64_t same = __ballot(m && d == d0);
                if (same == mm) {
                    if (lane_id() == lead) atomicAdd(&s_hist[d0], (uint32_t)__popcll(mm));
                } else if (m) {
                    atomicAdd(&s_hist[d], 1u);
                }
            }
        }
        __syncthreads();
        find_digit_256(s_hist, want, s_dig);
        const uint32_t d = s_dig[0], above = s_dig[1];
        __syncthreads();
        prefix |= d << shift;
        mask |= 0xFFu << shift;
        want -= above;
    }
    const uint32_t T = prefix, need = want;  // keys > T: K - need of them
    uint32_t tie_run = 0, sel_run = 0;
    for (int base = 0; base < n; base += NT) {
        const int i = base + threadIdx.x;
        const uint32_t v = i < n ? keys[i] : 0u;
        const bool eq = i < n && v == T, gt = i < n && v > T;
        uint32_t tie_tot, sel_tot;
        const uint32_t tie_ex = block_exclusive_sum<NT>(eq ? 1u : 0u, s_tmp, tie_tot);
        const bool sel = gt || (eq && tie_run + tie_ex < need);
        const uint32_t sel_ex = block_exclusive_sum<NT>(sel ? 1u : 0u, s_tmp, sel_tot);
        if (sel && sel_run + sel_ex < (uint32_t)K) out[sel_run + sel_ex] = i;
        tie_run += tie_tot;
        sel_run += sel_tot;
    }
    for (int i = (int)sel_run + threadIdx.x; i < K; i += NT) out[i] = -1;
}

// Writes the `count` distinct non-negative indices of s_list (unordered,
// 16-byte aligned, room for 4 pad slots after them) to o in ascending order
// and pads the K slots with -1, with NT threads.  Lists of up to
// min(128, NT): each index is written at its rank among all of them.  Longer
// ones: a counting sort into NT buckets spread evenly over [min, max] of the
// list, then each index is placed by its rank inside its bucket (ranking a
// list of 512 against itself costs about three times as long).
template <int NT = kSelThreads>
__device__ void rank_and_write(int32_t* s_list, int count, int K, int32_t* __restrict__ o) {
    constexpr int NB = NT;
    __shared__ uint32_t s_start[NB + 1];
    __shared__ uint32_t s_cur[NB];
    __shared__ int32_t s_srt[CSA2_MAX_TOPK];
    __shared__ int32_t s_mm[2 * (NT / kWave)];
    __shared__ uint32_t s_scan[NT / kWave + 1];
    if (count <= (NT < 128 ? NT : 128)) {
        // rank = #{smaller indices}, each element's comparisons split over
        // NT / count threads whose partial counts add up in LDS
        if (count == 0) {
            for (int i = threadIdx.x; i < K; i += NT) o[i] = -1;
            return;
        }
        for (int i = threadIdx.x; i < count; i += NT) s_cur[i] = 0u;
        if (threadIdx.x < 4) s_list[count + threadIdx.x] = INT_MAX;   // never smaller
        __syncthreads();
        const int P = NT / count, i = threadIdx.x % count, part = threadIdx.x / count;
        if (part < P) {
            const int n4 = (count + 3) / 4, chunk = (n4 + P - 1) / P;
            const int j0 = part * chunk, j1 = min(n4, j0 + chunk);
            const int4* l4 = reinterpret_cast<const int4*>(s_list);
            const int32_t e = s_list[i];
            uint32_t r = 0;
#pragma unroll 4
            for (int j = j0; j < j1; ++j) {
                const int4 v = l4[j];
                r += (v.x < e) + (v.y < e) + (v.z < e) + (v.w < e);
            }
            if (r) atomicAdd(&s_cur[i], r);
        }
        __syncthreads();
        for (int i = threadIdx.x; i < count; i += NT) o[s_cur[i]] = s_list[i];
    } else {
        // range of the list
        int32_t mn = INT_MAX, mx = 0;
        for (int i = threadIdx.x; i < count; i += NT) {
            mn = min(mn, s_list[i]);
            mx = max(mx, s_list[i]);
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            mn = min(mn, __shfl_xor(mn, off));
            mx = max(mx, __shfl_xor(mx, off));
        }
        const int wid = threadIdx.x / kWave;
        if (lane_id() == 0) { s_mm[2 * wid] = mn; s_mm[2 * wid + 1] = mx; }
        s_cur[threadIdx.x] = 0u;
        __syncthreads();
        mn = INT_MAX; mx = 0;
        for (int w = 0; w < NT / kWave; ++w) {
            mn = min(mn, s_mm[2 * w]);
            mx = max(mx, s_mm[2 * w + 1]);
        }
        // bucket(e) is non-decreasing in e
        const float scale = (float)NB / ((float)(mx - mn) + 1.0f);
        auto bucket = [&](int32_t e) { return min(NB - 1, (int)((float)(e - mn) * scale)); };
        for (int i = threadIdx.x; i < count; i += NT) atomicAdd(&s_cur[bucket(s_list[i])], 1u);
        __syncthreads();
        const uint32_t c = s_cur[threadIdx.x];
        uint32_t tot;
        const uint32_t ex = block_exclusive_sum<NT>(c, s_scan, tot);
        s_start[threadIdx.x] = ex;
        s_cur[threadIdx.x] = ex;
        if (threadIdx.x == NB - 1) s_start[NB] = ex + c;
        __syncthreads();
        for (int i = threadIdx.x; i < count; i += NT) {
            const int32_t e = s_list[i];
            s_srt[atomicAdd(&s_cur[bucket(e)], 1u)] = e;
        }
        __syncthreads();
        for (int p = threadIdx.x; p < count; p += NT) {
            const int32_t e = s_srt[p];
            const int bk = bucket(e);
            const int lo = (int)s_start[bk], hi = (int)s_start[bk + 1];
            int r = 0;
            for (int j = lo; j < hi; ++j) r += s_srt[j] < e;
            o[lo + r] = e;
        }
    }
    for (int i = count + threadIdx.x; i < K; i += NT) o[i] = -1;
}

// Appends to s_out[NA ..] the indices of the `need` best of the NC distinct
// candidate keys in s_cand (1 <= need <= NC <= kRankMax, 16-byte aligned, one
// pad slot after them): direct ranking when
// NC <= kRankDirect, else a register-resident radix select whose digits
// start at bit top_shift (48 when the candidates share their top 8 bits, as
// keys of one first-level bin do; 56 for any candidates).  Ends with a
// barrier.
__device__ void pick_lds_candidates(uint64_t* s_cand, uint32_t NC, uint32_t need, uint32_t NA,
                                    int32_t* s_out, uint32_t* s_hist, uint32_t* s_dig,
                                    uint32_t* s_count, int top_shift = 48) {
    if (NC <= (uint32_t)kRankDirect) {
        // candidate i has rank r = #{larger candidates}; the best `need` ranks
        // win.  Each candidate's comparisons are split over kSelThreads / NC
        // threads whose partial counts add up in LDS.
        __shared__ uint32_t s_rank[kRankDirect];
        for (int i = threadIdx.x; i < (int)NC; i += kSelThreads) s_rank[i] = 0u;
        if (threadIdx.x == 0) s_cand[NC] = 0ull;   // pad: never larger
        __syncthreads();
        const int n = (int)NC;
        const int P = kSelThreads / n, i = threadIdx.x % n, part = threadIdx.x / n;
        if (part < P) {
            const int n2 = (n + 1) / 2, chunk = (n2 + P - 1) / P;
            const int j0 = part * chunk, j1 = min(n2, j0 + chunk);
            const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(s_cand);
            const uint64_t ci = s_cand[i];
            uint32_t r = 0;
#pragma unroll 4
            for (int j = j0; j < j1; ++j) {
                const ulonglong2 w = c2[j];
                r += (w.x > ci) + (w.y > ci);
            }
            if (r) atomicAdd(&s_rank[i], r);
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kSelThreads)
            if (s_rank[i] < need) s_out[NA + s_rank[i]] = (int32_t)comp_idx(s_cand[i]);
    } else {
        uint64_t it[kLdsCandItems];
#pragma unroll
        for (int j = 0; j < kLdsCandItems; ++j) {
            const uint32_t i = threadIdx.x + j * kSelThreads;
            it[j] = i < NC ? s_cand[i] : 0ull;
        }
        const uint64_t T =
            block_select_kth<kSelThreads, kLdsCandItems>(it, need, s_hist, s_dig, top_shift);
        if (threadIdx.x == 0) *s_count = NA;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kLdsCandItems; ++j) {
            if (it[j] != 0 && it[j] >= T) {
                const uint32_t pos = atomicAdd(s_count, 1u);
                if (pos < NA + need) s_out[pos] = (int32_t)comp_idx(it[j]);
            }
        }
    }
    __syncthreads();
}

// Filter of one key row per query (entries or blocks): every workgroup
// classifies kSelElems keys against the bin b1 that holds the K-th largest
// key (from the first-level histogram).  Keys above b1 are winners, keys in
// b1 are candidates (composite key score|~index); both lists grow by one
// atomic per workgroup.  cnt[2q + 0/1]: winners, candidates (zeroed first).
__global__ __launch_bounds__(256) void k_filter(const uint32_t* __restrict__ keys, int64_t stride,
                                                const int32_t* __restrict__ q_nvis, int nmax,
                                                int bs_log2,
                                                int K, const uint32_t* __restrict__ hist,
                                                uint32_t* __restrict__ cnt,
                                                int32_t* __restrict__ above,
                                                uint64_t* __restrict__ cand) {
    __shared__ uint32_t s_tmp[256 / kWave + 3];
    __shared__ uint32_t s_bc[2];
    const int q = blockIdx.y;
    const int nvis = q_nvis[q];
    const int n = min((nvis + (1 << bs_log2) - 1) >> bs_log2, nmax);
    const int e0 = blockIdx.x * kSelElems;
    if (n <= K || e0 >= n) return;
    // the keys (coalesced uint4 loads) are in flight during the bin search
    const uint32_t* row = keys + (size_t)q * stride;
    uint32_t kk[4 * kFilterLoads];
#pragma unroll
    for (int j = 0; j < kFilterLoads; ++j) {
        const int e = e0 + 4 * (threadIdx.x + 256 * j);
        const uint4 v = e < n ? *reinterpret_cast<const uint4*>(row + e) : make_uint4(0, 0, 0, 0);
        kk[4 * j] = v.x; kk[4 * j + 1] = v.y; kk[4 * j + 2] = v.z; kk[4 * j + 3] = v.w;
    }
    uint32_t b1, nabove;
    find_digit_4096<256>(hist + (size_t)q * kHistBins, (uint32_t)K, s_tmp, b1, nabove);
    uint32_t na = 0, nc = 0;
#pragma unroll
    for (int i = 0; i < 4 * kFilterLoads; ++i) {
        const int e = e0 + 4 * (threadIdx.x + 256 * (i >> 2)) + (i & 3);
        const uint32_t d = kk[i] >> kDigitShift;
        na += e < n && d > b1;
        nc += e < n && d == b1;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_sum<256>((na << 16) | nc, s_tmp, tot);
    if (threadIdx.x == 0) {
        s_bc[0] = (tot >> 16) ? atomicAdd(&cnt[2 * q], tot >> 16) : 0u;
        s_bc[1] = (tot & 0xFFFFu) ? atomicAdd(&cnt[2 * q + 1], tot & 0xFFFFu) : 0u;
    }
    __syncthreads();
    uint32_t pa = s_bc[0] + (ex >> 16), pc = s_bc[1] + (ex & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 4 * kFilterLoads; ++i) {
        const int e = e0 + 4 * (threadIdx.x + 256 * (i >> 2)) + (i & 3);
        const uint32_t d = kk[i] >> kDigitShift;
        if (e < n && d > b1) {
            if (pa < (uint32_t)K) above[(size_t)q * K + pa] = e;
            ++pa;
        } else if (e < n && d == b1) {
            if (pc < (uint32_t)kCandCap) cand[(size_t)q * kCandCap + pc] = comp_key(kk[i], (uint32_t)e);
            ++pc;
        }
    }
}

// Final selection, one workgroup per query: picks the K - #winners best
// candidates -- by direct ranking when there are at most kRankDirect of them,
// else by a register-resident radix select, else (more than kCandCap:
// degenerate ties) by an exact select over the whole row -- and writes the K
// indices in ascending order.
__global__ __launch_bounds__(kSelThreads) void k_finalize(
    const uint32_t* __restrict__ keys, int64_t stride, const int32_t* __restrict__ q_nvis,
    int nmax, int bs_log2, int K, const uint32_t* __restrict__ cnt, const int32_t* __restrict__ above,
    const uint64_t* __restrict__ cand, int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) int32_t s_out[CSA2_MAX_TOPK + 4];
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[kRankDirect + 2];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[kSelThreads / kWave + 3];
    __shared__ uint32_t s_count;
    const int q = blockIdx.x;
    const int nvis = q_nvis[q];
    const int n = min((nvis + (1 << bs_log2) - 1) >> bs_log2, nmax);
    int32_t* o = out + (size_t)q * K;
    if (n <= K) {  // everything is selected
        for (int i = threadIdx.x; i < K; i += kSelThreads) o[i] = i < n ? i : -1;
        return;
    }
    const uint32_t NA = min(cnt[2 * q], (uint32_t)K - 1u);
    const uint32_t NC = cnt[2 * q + 1];
    const uint32_t need = (uint32_t)K - NA;
    if (NC > (uint32_t)kCandCap) {
        select_global_row<kSelThreads>(keys + (size_t)q * stride, n, K, o, s_hist, s_dig, s_tmp);
        return;
    }
    for (int i = threadIdx.x; i < (int)NA; i += kSelThreads) s_out[i] = above[(size_t)q * K + i];
    if (NC <= (uint32_t)kRankDirect) {
        for (int i = threadIdx.x; i < (int)NC; i += kSelThreads) s_cand[i] = cand[(size_t)q * kCandCap + i];
        pick_lds_candidates(s_cand, NC, need, NA, s_out, s_hist, s_dig, &s_count);
    } else {
        uint64_t it[kSelItems];
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            const uint32_t i = threadIdx.x + j * kSelThreads;
            it[j] = i < NC ? cand[(size_t)q * kCandCap + i] : 0ull;
        }
        const uint64_t T = block_select_kth<kSelThreads, kSelItems>(it, need, s_hist, s_dig, 48);
        if (threadIdx.x == 0) s_count = NA;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            if (it[j] != 0 && it[j] >= T) {
                const uint32_t pos = atomicAdd(&s_count, 1u);
                if (pos < (uint32_t)K) s_out[pos] = (int32_t)comp_idx(it[j]);
            }
        }
        __syncthreads();
    }
    rank_and_write(s_out, K, K, o);
}

// The K-th largest of the non-zero 32-bit values held IPT per thread (ties
// allowed; 1 <= K <= their number), by 8-bit radix passes from the top:
// returns thr and sets `need` so that the K largest are every value > thr and
// the first `need` values == thr (in any fixed order).  A pass whose chosen
// bucket holds exactly the values still wanted ends the search: then every
// value >= the bucket's lower bound is taken (thr = bound - 1, need = 0).
//   With last_shift > 0 the passes stop at that digit: then (unless a pass
// ended the search) thr is the lower bound of the last bucket (its low bits
// zero), and the K largest are among the values >= thr.
template <int NT, int IPT>
__device__ int64_t block_kth_u32(const uint32_t (&it)[IPT], uint32_t K, uint32_t* s_hist,
                                 uint32_t* s_dig, uint32_t& need, int last_shift = 0) {
    uint32_t prefix = 0, mask = 0, want = K;
    for (int shift = 24; shift >= last_shift; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += NT) s_hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const uint32_t v = it[j];
            const bool m = v != 0u && (v & mask) == prefix;
            const uint32_t d = (v >> shift) & 255u;
            // one atomic per wave when all matching lanes share the digit
            const uint64_t mm = __ballot(m);
            if (mm) {
                const int lead = __builtin_ctzll(mm);
                const uint32_t d0 = (uint32_t)__shfl((int)d, lead);
                const uint64_t same = __ballot(m && d == d0);
                if (same == mm) {
                    if (lane_id() == lead) atomicAdd(&s_hist[d0], (uint32_t)__popcll(mm));
                } else if (m) {
                    atomicAdd(&s_hist[d], 1u);
                }
            }
        }
        __syncthreads();
        find_digit_256(s_hist, want, s_dig);
        const uint32_t d = s_dig[0], above = s_dig[1];
        const uint32_t bucket = s_hist[d];
        __syncthreads();
        prefix |= d << shift;
        mask |= 0xFFu << shift;
        want -= above;
        if (bucket == want) {
            need = 0u;
            return (int64_t)prefix - 1;
        }
    }
    need = want;
    return (int64_t)prefix;
}

// A whole row of n <= kSmallRow keys in registers: thread t holds keys
// 4 (t + 1024 j) .. +3 in v[j], 0 past the row (no real key is 0).
__device__ __forceinline__ void load_row_regs(const uint32_t* __restrict__ row, int n,
                                              uint4 (&v)[kRowRegs]) {
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) {
        const int e = 4 * ((int)threadIdx.x + kSelThreads * j);
        uint4 x = e + 3 < n ? *reinterpret_cast<const uint4*>(row + e) : make_uint4(0, 0, 0, 0);
        if (e + 3 >= n && e < n) {
            x.x = row[e];
            x.y = e + 1 < n ? row[e + 1] : 0u;
            x.z = e + 2 < n ? row[e + 2] : 0u;
        }
        v[j] = x;
    }
}

// Exact Top-K of a row held as load_row_regs leaves it, given a threshold
// T >= 1: when between K and kRankMax keys are >= T, writes the K best
// indices to o in ascending order and returns true; otherwise writes nothing
// and returns false (uniformly).  The keys >= T go to LDS in index order
// (slot j of lane l of wave w holds indices 4 (64 w + l + 1024 j) + x, so
// (j, w, l, x) order is index order: offsets within a wave from ballots,
// wave offsets from one scan over (slot, wave) counts); a radix select over
// their 32-bit values finds the K-th value and how many of its ties to take;
// one block scan then puts every key above it, and the first such ties in
// index order, at its output slot.  s_wbase holds kRowRegs * 16 words.
__device__ __forceinline__ bool select_row_regs(const uint4 (&v)[kRowRegs], uint32_t tord, int K,
                                int32_t* __restrict__ o, uint64_t* s_cand, uint32_t* s_wbase,
                                uint32_t* s_hist, uint32_t* s_dig, uint32_t* s_tmp) {
    const int wv = threadIdx.x / kWave, ln = lane_id();
    uint32_t inwave[kRowRegs];
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) {
        const uint64_t b0 = __ballot(v[j].x >= tord), b1 = __ballot(v[j].y >= tord);
        const uint64_t b2 = __ballot(v[j].z >= tord), b3 = __ballot(v[j].w >= tord);
        inwave[j] = (uint32_t)(lanes_below(b0) + lanes_below(b1) + lanes_below(b2) + lanes_below(b3));
        if (ln == 0) s_wbase[j * (kSelThreads / kWave) + wv] =
            (uint32_t)(__popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3));
    }
    __syncthreads();
    if (wv == 0) {   // exclusive scan of the 256 (slot, wave) counts, 4 per lane
        uint32_t c[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) { c[k] = s_wbase[4 * ln + k]; sum += c[k]; }
        uint32_t incl = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)incl, off);
            if (ln >= off) incl += y;
        }
        uint32_t run = incl - sum;
#pragma unroll
        for (int k = 0; k < 4; ++k) { s_wbase[4 * ln + k] = run; run += c[k]; }
        if (ln == kWave - 1) s_dig[1] = incl;
    }
    __syncthreads();
    const uint32_t total = s_dig[1];
    if (total < (uint32_t)K || total > (uint32_t)kRankMax) return false;
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) {
        uint32_t at = s_wbase[j * (kSelThreads / kWave) + wv] + inwave[j];
        const uint32_t e = 4u * (threadIdx.x + kSelThreads * j);
        const uint32_t kk[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int x = 0; x < 4; ++x)
            if (kk[x] >= tord) s_cand[at++] = comp_key(kk[x], e + x);
    }
    __syncthreads();
    uint32_t it[kLdsCandItems];
#pragma unroll
    for (int k = 0; k < kLdsCandItems; ++k) {
        const uint32_t c = kLdsCandItems * threadIdx.x + k;
        it[k] = c < total ? (uint32_t)(s_cand[c] >> 32) : 0u;
    }
    uint32_t need;
    const int64_t thr = block_kth_u32<kSelThreads, kLdsCandItems>(it, (uint32_t)K, s_hist, s_dig, need);
    uint32_t na = 0, nt = 0;
#pragma unroll
    for (int k = 0; k < kLdsCandItems; ++k) {
        na += (it[k] != 0u && (int64_t)it[k] > thr) ? 1u : 0u;
        nt += (it[k] != 0u && (int64_t)it[k] == thr) ? 1u : 0u;
    }
    uint32_t tot2;
    const uint32_t pre = block_exclusive_sum<kSelThreads>((na << 16) | nt, s_tmp, tot2);
    uint32_t ab = pre >> 16, ti = pre & 0xFFFFu;
#pragma unroll
    for (int k = 0; k < kLdsCandItems; ++k) {
        const uint32_t c = kLdsCandItems * threadIdx.x + k;
        const bool above = it[k] != 0u && (int64_t)it[k] > thr;
        const bool tie = it[k] != 0u && (int64_t)it[k] == thr;
        if (above || (tie && ti < need)) o[ab + min(ti, need)] = (int32_t)comp_idx(s_cand[c]);
        ab += above ? 1u : 0u;
        ti += tie ? 1u : 0u;
    }
    return true;
}

// Top-K of one key row per query by a single workgroup (rows of at most
// kSmallRow keys: the c1 entry rows, the pool's block rows): the bin b1 of
// the K-th key comes from the first-level histogram, so the keys at or above
// b1's lower bound are the candidates; the row is read once into registers
// and select_row_regs picks the K best of them.  More than kRankMax such keys
// (degenerate score distributions) falls back to the exact whole-row select.
// Replaces the filter + finalize pair where one workgroup can read the row.
__global__ __launch_bounds__(kSelThreads) void k_select_small(
    const uint32_t* __restrict__ keys, int64_t stride, const int32_t* __restrict__ q_nvis,
    int nmax, int bs_log2, int K, const uint32_t* __restrict__ hist, int32_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[kRankMax + 2];
    __shared__ uint32_t s_wbase[kRowRegs * (kSelThreads / kWave)];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[kSelThreads / kWave + 3];
    const int q = blockIdx.x;
    const int nvis = q_nvis[q];
    const int n = min((nvis + (1 << bs_log2) - 1) >> bs_log2, nmax);
    int32_t* o = out + (size_t)q * K;
    if (n <= K) {
        for (int i = threadIdx.x; i < K; i += kSelThreads) o[i] = i < n ? i : -1;
        return;
    }
    const uint32_t* row = keys + (size_t)q * stride;
    uint4 v[kRowRegs];
    load_row_regs(row, n, v);
    uint32_t b1, nabove;
    find_digit_4096<kSelThreads>(hist + (size_t)q * kHistBins, (uint32_t)K, s_tmp, b1, nabove);
    if (select_row_regs(v, max(1u, b1 << kDigitShift), K, o, s_cand, s_wbase, s_hist, s_dig, s_tmp))
        return;
    select_global_row<kSelThreads>(row, n, K, o, s_hist, s_dig, s_tmp);
}

// -------------------------------------------------- prefill indexer

// A prefill chunk of Q queries of one sequence scores the same key rows for
// every query, so it is a dense contraction S = Qi K^T ([Q x RW] x [RW x N])
// on the bf16 matrix cores:
//   k_prefill_convert: one bf16 copy of the chunk's query rows (heads summed
//     when the key row is shared, Hk == 1) and of the sequence's key rows,
//     each value split x = hi + lo (lo = x - hi rounded to bf16), rows padded
//     to tiles with zeros, and one flag per 128-row tile: some lo part is
//     non-zero (only then are the tile's lo rows written);
//   k_prefill_gemm: 128 x 128 score tiles; hi*hi always, hi*lo when the key
//     tile is flagged, lo*hi when the query tile is (lo*lo is dropped: about
//     2^-16 of each product, and exactly zero when either side is integer).
// The Top-K never materialises the [Q x N] scores: a GEMM over 16 sampled
// key tiles gives each query a threshold (k_sample_thr), the full GEMM
// appends only the scores at or above it to the query's candidate list, and
// k_cand_select selects exactly over the list.  A list that cannot hold the
// answer (too short above the threshold, or overflowing) sends its query
// tile through the full score rows and k_row_select instead; the result is
// the exact Top-K either way.
// Integer-valued inputs of magnitude <= 256 are exact in bf16 (no lo part)
// and, while every partial sum stays below 2^24 in magnitude, the fp32
// accumulation is exact in any order: the scores equal the definition bit
// for bit.  Other fp32 inputs get about 16 significand bits.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGM = 128, kGN = 128, kGK = 64;   // score tile and K chunk
constexpr int kGStr = kGK + 8;                  // LDS row stride (bf16): 144 B
constexpr int kGVec = kGM * kGK / 8 / 256;      // 16-byte pieces per thread and operand
constexpr int kCvtRows = 128;                   // rows per conversion workgroup and flag (a tile)
constexpr int kCvtThreads = 1024;               // threads per conversion workgroup
static_assert(kCvtRows == kGM && kCvtRows == kGN, "one lo flag per score tile side");

__device__ __forceinline__ float4 load_qrow4(const float* __restrict__ qI, int q, int Hi, int Hk,
                                             int Di, int c) {
    if (Hk == Hi) return *reinterpret_cast<const float4*>(qI + (size_t)q * Hi * Di + c);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int h = 0; h < Hi; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(qI + ((size_t)q * Hi + h) * Di + c);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    return s;
}

// Four fp32 -> packed bf16 hi and lo parts (round to nearest even); returns
// whether a lo part is non-zero.
__device__ __forceinline__ bool split4_bf16(float4 x, uint2& hi, uint2& lo) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    uint32_t h[4], l[4];
    bool any = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 hb = (__bf16)v[i];
        const __bf16 lb = (__bf16)(v[i] - (float)hb);
        h[i] = __builtin_bit_cast(uint16_t, hb);
        l[i] = __builtin_bit_cast(uint16_t, lb);
        any |= (l[i] & 0x7FFFu) != 0;
    }
    hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
    return any;
}

// Four consecutive key values as fp32: an fp32 key row is read as is, E4M3
// key bytes are decoded exactly (gfx950 OCP FP8 conversion).
__device__ __forceinline__ float4 load_key4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load_key4(const uint8_t* p) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    const float2 lo = fp8x2_to_f32<false>(w), hi = fp8x2_to_f32<true>(w);
    return make_float4(lo.x, lo.y, hi.x, hi.y);
}

// Workgroups [0, Qp/64) convert query rows, the rest key rows (64 each).
// A thread converts NG groups of 8 consecutive values (16-byte stores),
// four groups' loads issued together.  The first pass writes the hi parts
// and finds whether some lo part of the block is non-zero; only then does a
// second pass re-read the rows (from the caches) and write the lo parts,
// since the score GEMM reads lo rows only for flagged blocks.
template <typename KT, int NG>
__global__ __launch_bounds__(kCvtThreads) void k_prefill_convert(
    const float* __restrict__ qI, const KT* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, int Q, int Qp, int Hi, int Hk,
    int Di, int N, uint16_t* __restrict__ qh, uint16_t* __restrict__ ql,
    uint16_t* __restrict__ kh, uint16_t* __restrict__ kl, uint32_t* __restrict__ qflag,
    uint32_t* __restrict__ kflag) {
    constexpr int kU = 4;
    const int RW = Hk * Di, f8 = RW / 8;   // RW = 64 NG (kCvtRows rows, kCvtThreads threads)
    const KT* kb = kI + seq_row_off[0] * (int64_t)RW;
    const int nqb = Qp / kCvtRows;
    const bool isq = (int)blockIdx.x < nqb;
    const int blk = isq ? blockIdx.x : blockIdx.x - nqb;
    const int r0 = blk * kCvtRows, nrow = isq ? Q : N;
    uint16_t* dh = isq ? qh : kh;
    uint16_t* dl = isq ? ql : kl;
    int any = 0;
    // groups g0 .. g0 + kU - 1; pass 0 writes hi (and finds any), pass 1 lo
    auto groups = [&](int g0, int pass) {
        float4 x[kU][2];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int f = threadIdx.x + kCvtThreads * (g0 + u), r = r0 + f / f8, c = 8 * (f % f8);
            x[u][0] = x[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < nrow) {
                if (isq) {
                    x[u][0] = load_qrow4(qI, r, Hi, Hk, Di, c);
                    x[u][1] = load_qrow4(qI, r, Hi, Hk, Di, c + 4);
                } else {
                    x[u][0] = load_key4(kb + (size_t)r * RW + c);
                    x[u][1] = load_key4(kb + (size_t)r * RW + c + 4);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int f = threadIdx.x + kCvtThreads * (g0 + u), r = r0 + f / f8, c = 8 * (f % f8);
            uint2 h0, l0, h1, l1;
            any |= split4_bf16(x[u][0], h0, l0) ? 1 : 0;
            any |= split4_bf16(x[u][1], h1, l1) ? 1 : 0;
            uint16_t* d = (pass == 0 ? dh : dl) + (size_t)r * RW + c;
            *reinterpret_cast<uint4*>(d) = pass == 0 ? make_uint4(h0.x, h0.y, h1.x, h1.y)
                                                     : make_uint4(l0.x, l0.y, l1.x, l1.y);
        }
    };
#pragma unroll 1
    for (int g0 = 0; g0 < NG; g0 += kU) groups(g0, 0);
    any = __syncthreads_or(any);
    if (any) {
#pragma unroll 1
        for (int g0 = 0; g0 < NG; g0 += kU) groups(g0, 1);
    }
    if (threadIdx.x == 0) (isq ? qflag : kflag)[blk] = any ? 1u : 0u;
}

// A thread's share of one K chunk: kGVec x 16 B of the query tile and of the
// key tile (row f / (kGK/8), 8 bf16 at column 8 (f % (kGK/8)), f = thread + 256 j).
// Chunk c of the (pass, K chunk) sequence: the passes are hi*hi, then
// hi*lo when the key tile has lo parts, then lo*hi when the query tile has
// them (p1: the second pass).  (Native vector types keep the staging in
// registers.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define CSA2_GEMM_LOAD(RA, RB, c)                                                          \
    do {                                                                                   \
        const int seq_ = (c) / nch, kc_ = ((c) - seq_ * nch) * kGK;                        \
        const int pass_ = seq_ == 0 ? 0 : seq_ == 1 ? p1 : 2;                              \
        const uint16_t* A_ = pass_ == 2 ? ql : qh;                                         \
        const uint16_t* B_ = pass_ == 1 ? kl : kh;                                         \
        _Pragma("unroll") for (int j_ = 0; j_ < kGVec; ++j_) {                             \
            const int f_ = threadIdx.x + 256 * j_, r_ = f_ / (kGK / 8), c8_ = f_ % (kGK / 8); \
            RA[j_] = *reinterpret_cast<const u32x4*>(A_ + (size_t)(m0 + r_) * RW + kc_ + 8 * c8_); \
            RB[j_] = *reinterpret_cast<const u32x4*>(B_ + (size_t)(n0 + r_) * RW + kc_ + 8 * c8_); \
        }                                                                                  \
    } while (0)
#define CSA2_GEMM_STORE(RA, RB)                                                            \
    do {                                                                                   \
        _Pragma("unroll") for (int j_ = 0; j_ < kGVec; ++j_) {                             \
            const int f_ = threadIdx.x + 256 * j_, r_ = f_ / (kGK / 8), c8_ = f_ % (kGK / 8); \
            *reinterpret_cast<u32x4*>(sA + r_ * kGStr + 8 * c8_) = RA[j_];                 \
            *reinterpret_cast<u32x4*>(sB + r_ * kGStr + 8 * c8_) = RB[j_];                 \
        }                                                                                  \
    } while (0)

// The products of the chunk in LDS for this wave's 64 x 64 sub-tile.
__device__ __forceinline__ void gemm_mma(const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                                         int l32, int hh, f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 16) {
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            av[i] = *reinterpret_cast<const bf16x8*>(sA + (wm + 32 * i + l32) * kGStr + ks + 8 * hh);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bv[j] = *reinterpret_cast<const bf16x8*>(sB + (wn + 32 * j + l32) * kGStr + ks + 8 * hh);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
}

// Modes of the score GEMM's epilogue (what a tile of scores turns into).
constexpr int kGemmKeys = 0;        // every visible score's key into its row
constexpr int kGemmSample = 1;      // sampled key tiles: keys (0 if invisible) into a sample row
constexpr int kGemmCand = 2;        // keys at or above the query's threshold, appended to its list
constexpr int kSampleTiles = 16;    // key tiles sampled per query (2,048 keys)
constexpr int kCandCapPre = 4096;   // candidates a prefill query keeps
constexpr int kFbGrid = 1024;       // workgroups of the exact-path score GEMM

// The min(K, #non-empty) largest of the register-resident composite keys
// of a workgroup of NT threads (score word | ~index word; 0 = empty;
// non-empty keys distinct), written to o as their indices in ascending
// order, -1 padded.
template <int NT, int IPT>
__device__ void select_top_ckeys(const uint64_t (&it)[IPT], int K, int32_t* __restrict__ o) {
    __shared__ __attribute__((aligned(16))) int32_t s_out[CSA2_MAX_TOPK + 4];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[NT / kWave + 3];
    __shared__ uint32_t s_count;
    uint32_t nv = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) nv += it[j] != 0;
    uint32_t total;
    (void)block_exclusive_sum<NT>(nv, s_tmp, total);
    const int k = min((int)total, K);
    if (k == 0) {
        for (int i = threadIdx.x; i < K; i += NT) o[i] = -1;
        return;
    }
    const uint64_t T = block_select_kth<NT, IPT>(it, (uint32_t)k, s_hist, s_dig, 56);
    if (threadIdx.x == 0) s_count = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        if (it[j] != 0 && it[j] >= T) {
            const uint32_t pos = atomicAdd(&s_count, 1u);
            if (pos < (uint32_t)K) s_out[pos] = (int32_t)comp_idx(it[j]);
        }
    }
    __syncthreads();
    rank_and_write<NT>(s_out, min((int)s_count, K), K, o);
}

constexpr int kXcdsIdx = 8;   // XCDs of an MI355X (L2 domains)

// Score tile (key tile kt, query tile qt) of workgroup g in a grid of ntk x
// nqt tiles.  Workgroups are dealt to the XCDs round-robin by linear id.
// When the key tiles split evenly over the XCDs, XCD x takes key tiles
// [x ntk/8, (x+1) ntk/8) for every query tile and walks them in groups of
// up to 8 query tiles, query tile fastest: its L2 keeps the group's query
// rows while its share of the key rows streams past them, and no other XCD
// reads those key rows.  (A key-tile-fastest order over the whole grid
// makes every XCD stream every key row once per query tile.)
__device__ __forceinline__ void gemm_tile(int g, int ntk, int nqt, int& kt, int& qt) {
    if (ntk % kXcdsIdx == 0) {
        const int gq = nqt % 8 == 0 ? 8 : nqt % 4 == 0 ? 4 : nqt % 2 == 0 ? 2 : 1;
        const int x = g % kXcdsIdx, local = g / kXcdsIdx, kr = ntk / kXcdsIdx;
        const int qi = local % gq, rest = local / gq;
        kt = x * kr + rest % kr;
        qt = (rest / kr) * gq + qi;
    } else {
        kt = g % ntk;
        qt = g / ntk;
    }
}

// Tile g of the score GEMM: 128 x 128 scores (4 waves of 64 x 64 on the
// 32x32x16 bf16 MFMA), ntk x nqt tiles in a 1-D grid (order: gemm_tile).
// The chunk sequence is (pass, K chunk) with pass 0 = hi*hi, 1 = hi*lo,
// 2 = lo*hi; a chunk is loaded into registers during the previous chunk's
// products and stored to LDS right before its own, so one 36 KB LDS buffer
// serves.  Four workgroups per CU (the register budget is capped to fit
// them) hide the operand loads' latency better than deeper staging in fewer
// workgroups: 128-wide chunks with two workgroups per CU took 25 % longer.
//   MODE kGemmKeys: keys[q * kstride + t] for every visible t; with
//     tile_fail set (word 0: any tile flagged, word 1 + t: query tile t),
//     only query tiles whose flag is set run (the exact
//     path of the queries whose candidate list missed).
//   MODE kGemmSample: grid key tile kt is key tile kt * tile_step; its keys
//     go to keys[q * kstride + 128 kt + col] (0 for an invisible key).
//   MODE kGemmCand: the composite keys (score, index) of the visible scores
//     whose key is >= thr[q] are appended to cand[q * kCandCapPre ..]; cnt[q]
//     counts them all (also those past the list's capacity).  A workgroup
//     counts its candidates per query first and reserves their slots with
//     one atomic per query, then writes them.
#define CSA2_GEMM_PARAMS                                                                   \
    const uint16_t* __restrict__ qh, const uint16_t* __restrict__ ql,                      \
        const uint16_t* __restrict__ kh, const uint16_t* __restrict__ kl,                  \
        const uint32_t* __restrict__ qflag, const uint32_t* __restrict__ kflag, int RW, int Q, \
        const int32_t* __restrict__ q_nvis, int max_nvis, uint32_t* __restrict__ keys,     \
        int64_t kstride, int ntk, int nqt, int tile_step,                                  \
        const uint32_t* __restrict__ tile_fail, const uint32_t* __restrict__ thr,          \
        uint64_t* __restrict__ cand, uint32_t* __restrict__ cnt
#define CSA2_GEMM_ARGS                                                                     \
    qh, ql, kh, kl, qflag, kflag, RW, Q, q_nvis, max_nvis, keys, kstride, ntk, nqt,        \
        tile_step, tile_fail, thr, cand, cnt

template <int MODE>
__device__ __forceinline__ void prefill_gemm_tile(int g, CSA2_GEMM_PARAMS) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[kGM * kGStr];
    __shared__ __attribute__((aligned(16))) uint16_t sB[kGN * kGStr];
    __shared__ int s_nv[kGM];
    __shared__ uint32_t s_thr[kGM];
    int kt, qt;
    gemm_tile(g, ntk, nqt, kt, qt);
    if (MODE == kGemmKeys && tile_fail && tile_fail[1 + qt] == 0u) return;
    const int n0 = kt * tile_step * kGN, m0 = qt * kGM;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = lane >> 5, l32 = lane & 31;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
    if (threadIdx.x < kGM) {
        const int q = m0 + threadIdx.x;
        s_nv[threadIdx.x] = q < Q ? min(q_nvis[q], max_nvis) : 0;
        if (MODE == kGemmCand) s_thr[threadIdx.x] = q < Q ? thr[q] : 0u;
    }
    // lo rows exist (are written) only for flagged tiles
    const bool lo_q = qflag[m0 / kCvtRows] != 0u, lo_k = kflag[n0 / kCvtRows] != 0u;
    const int p1 = lo_k ? 1 : 2;
    const int nch = RW / kGK, total = (1 + (int)lo_q + (int)lo_k) * nch;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    u32x4 ra[kGVec], rb[kGVec];
    CSA2_GEMM_LOAD(ra, rb, 0);
    for (int c = 0; c < total; ++c) {
        __syncthreads();   // the previous chunk's operand reads are done
        CSA2_GEMM_STORE(ra, rb);
        __syncthreads();
        CSA2_GEMM_LOAD(ra, rb, min(c + 1, total - 1));   // next chunk, during these products
        gemm_mma(sA, sB, wm, wn, l32, hh, acc);
    }
#undef CSA2_GEMM_LOAD
#undef CSA2_GEMM_STORE
    __syncthreads();   // s_nv / s_thr
    // lane (hh, l32) of tile (i, j), register r holds S[query m0 + lr]
    // [key n0 + wn + 32j + l32], lr = wm + 32i + 8(r/4) + 4hh + r%4
    if constexpr (MODE == kGemmCand) {
        // the 32 lanes of a half-wave share one query row; per row, the wave
        // with wn = 0 takes the first slots of the workgroup's run
        __shared__ uint32_t s_cnt[2][kGM];
        __shared__ uint32_t s_base[kGM];
        const uint32_t below = (1u << l32) - 1u;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
                const int nv = s_nv[lr];
                const uint32_t T = s_thr[lr];
                const int t0 = n0 + wn + l32;
                const bool v0 = t0 < nv && ord_key(acc[i][0][r]) >= T;
                const bool v1 = t0 + 32 < nv && ord_key(acc[i][1][r]) >= T;
                const uint32_t b0 = (uint32_t)(__ballot(v0) >> (32 * hh));
                const uint32_t b1 = (uint32_t)(__ballot(v1) >> (32 * hh));
                if (l32 == 0) s_cnt[wn >> 6][lr] = __popc(b0) + __popc(b1);
            }
        __syncthreads();
        if (threadIdx.x < kGM) {
            const uint32_t n = s_cnt[0][threadIdx.x] + s_cnt[1][threadIdx.x];
            s_base[threadIdx.x] = n ? atomicAdd(&cnt[m0 + threadIdx.x], n) : 0u;   // n > 0: q < Q
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
                const int nv = s_nv[lr];
                const uint32_t T = s_thr[lr];
                const int t0 = n0 + wn + l32;
                const uint32_t k0 = ord_key(acc[i][0][r]), k1 = ord_key(acc[i][1][r]);
                const bool v0 = t0 < nv && k0 >= T;
                const bool v1 = t0 + 32 < nv && k1 >= T;
                const uint32_t b0 = (uint32_t)(__ballot(v0) >> (32 * hh));
                const uint32_t b1 = (uint32_t)(__ballot(v1) >> (32 * hh));
                const uint32_t base = s_base[lr] + (wn ? s_cnt[0][lr] : 0u);
                uint64_t* crow = cand + (size_t)(m0 + lr) * kCandCapPre;   // used only if q < Q
                if (v0) {
                    const uint32_t pos = base + __popc(b0 & below);
                    if (pos < (uint32_t)kCandCapPre) crow[pos] = comp_key(k0, (uint32_t)t0);
                }
                if (v1) {
                    const uint32_t pos = base + __popc(b0) + __popc(b1 & below);
                    if (pos < (uint32_t)kCandCapPre) crow[pos] = comp_key(k1, (uint32_t)(t0 + 32));
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
                const int q = m0 + lr;
                if (q >= Q) continue;
                const int nv = s_nv[lr];
                uint32_t* krow = keys + (size_t)q * kstride;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int t = n0 + wn + 32 * j + l32;
                    if (MODE == kGemmSample)
                        krow[kt * kGN + wn + 32 * j + l32] = t < nv ? ord_key(acc[i][j][r]) : 0u;
                    else if (t < nv)
                        krow[t] = ord_key(acc[i][j][r]);
                }
            }
    }
    __syncthreads();   // before a next tile's s_nv / s_thr
}

// The score GEMM: one tile per workgroup; kGemmKeysFb is kGemmKeys with
// tile_fail over a small grid that takes tiles g, g + grid, ... in turn.
constexpr int kGemmKeysFb = 3;
template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_prefill_gemm(
    CSA2_GEMM_PARAMS) {
    if constexpr (MODE == kGemmKeysFb) {
        if (tile_fail[0] == 0u) return;   // no query tile was flagged
        for (int g = blockIdx.x; g < ntk * nqt; g += gridDim.x)
            prefill_gemm_tile<kGemmKeys>(g, CSA2_GEMM_ARGS);
    } else {
        prefill_gemm_tile<MODE>(blockIdx.x, CSA2_GEMM_ARGS);
    }
}
#undef CSA2_GEMM_PARAMS
#undef CSA2_GEMM_ARGS

// Threshold of each prefill query from its sampled keys (one workgroup per
// query): a query with at most kCandCapPre visible entries takes every entry
// (threshold 0); otherwise the threshold is the j-th largest visible sampled
// key cut to its top 24 bits, j chosen so that about 3 K entries are
// expected at or above it.  The
// candidate list then holds every entry whose key is >= the threshold; a
// list with fewer than K of them, or more than it can hold, sends the query
// to the exact path (the threshold only decides how much work is skipped).
__global__ __launch_bounds__(256) void k_sample_thr(const uint32_t* __restrict__ samp, int ns,
                                                    const int32_t* __restrict__ q_nvis,
                                                    int max_nvis, int K,
                                                    uint32_t* __restrict__ thr) {
    constexpr int NT = 256, IPT = kSampleTiles * kGN / NT;
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[NT / kWave + 3];
    const int q = blockIdx.x;
    const int nv = min(q_nvis[q], max_nvis);
    if (nv <= kCandCapPre) {
        if (threadIdx.x == 0) thr[q] = 0u;
        return;
    }
    uint32_t it[IPT];   // 0 = invisible (no visible score has key 0)
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int i = threadIdx.x + NT * j;
        it[j] = i < ns ? samp[(size_t)q * ns + i] : 0u;
        c += it[j] != 0u;
    }
    uint32_t total;
    (void)block_exclusive_sum<NT>(c, s_tmp, total);
    if (total == 0u) {   // no visible sample: every entry is a candidate
        if (threadIdx.x == 0) thr[q] = 0u;
        return;
    }
    const uint64_t want = ((uint64_t)3 * K * total + nv - 1) / (uint64_t)nv;
    const uint32_t j = (uint32_t)max<uint64_t>(1, min<uint64_t>(want, total));
    // the top 24 bits of the j-th largest sample: its value to about 2^-15
    // relative (exactly, for integer scores below 2^15 in magnitude)
    uint32_t need;
    const int64_t t = block_kth_u32<NT, IPT>(it, j, s_hist, s_dig, need, 8);
    // the j largest samples are >= t when need > 0, else > t
    if (threadIdx.x == 0) thr[q] = (uint32_t)(need ? t : t + 1);
}

// Exact Top-K of each prefill query over its candidate list; a query whose
// list cannot hold the answer (fewer than K entries above a non-zero
// threshold, or more entries than the list holds) flags its query tile for
// the exact path instead (tile_fail word 1 + tile, and word 0: any tile).
constexpr int kCandThreads = 256;
__global__ __launch_bounds__(kCandThreads) void k_cand_select(const uint64_t* __restrict__ cand,
                                                             const uint32_t* __restrict__ cnt,
                                                             const uint32_t* __restrict__ thr,
                                                             int K, int32_t* __restrict__ out,
                                                             uint32_t* __restrict__ tile_fail) {
    constexpr int IPT = kCandCapPre / kCandThreads;
    const int q = blockIdx.x;
    const uint32_t n = cnt[q];
    if (n > (uint32_t)kCandCapPre || (thr[q] != 0u && n < (uint32_t)K)) {
        if (threadIdx.x == 0) {
            atomicOr(&tile_fail[1 + q / kGM], 1u);
            atomicOr(&tile_fail[0], 1u);
        }
        return;
    }
    uint64_t it[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int i = threadIdx.x + j * kCandThreads;
        it[j] = i < (int)n ? cand[(size_t)q * kCandCapPre + i] : 0ull;
    }
    select_top_ckeys<kCandThreads, IPT>(it, K, out + (size_t)q * K);
}

// Exact Top-K of one row of score keys (prefill: one workgroup per query).
// Rows of up to kSmallRow keys are read once, into registers: the keys at
// 1024 spread-out positions give a threshold T (a few times more sampled keys
// lie above T than the K-th key is expected to leave); when the row then
// holds between K and kRankMax keys >= T, those are the candidates, written
// to LDS in index order; a radix select finds the K-th key value among them
// and one ordered pass writes the winners.  Otherwise (and for longer rows): a
// 4096-bin LDS histogram of the top 12 bits finds the bin b1 of the K-th
// key; a second pass over the row keeps the keys above b1 and collects the
// keys in b1, of which the best are picked in LDS.  More than kRankMax keys
// in b1 falls back to the exact whole-row select.

__global__ __launch_bounds__(kSelThreads) void k_row_select(const uint32_t* __restrict__ keys,
                                                            int64_t stride,
                                                            const int32_t* __restrict__ q_nvis,
                                                            int nmax, int K,
                                                            int32_t* __restrict__ out,
                                                            const uint32_t* __restrict__ tile_fail) {
    __shared__ __attribute__((aligned(16))) uint32_t s_h[kHistBins];
    __shared__ __attribute__((aligned(16))) int32_t s_out[CSA2_MAX_TOPK + 4];
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[kRankMax + 2];
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[kSelThreads / kWave + 3];
    __shared__ uint32_t s_na, s_nc, s_count;
    __shared__ __attribute__((aligned(16))) uint32_t s_rtop[kWave];      // 4 per wave
    __shared__ uint32_t s_wbase[kRowRegs * (kSelThreads / kWave)];       // per (slot, wave)
    const int q = blockIdx.x;
    if (tile_fail && tile_fail[1 + q / kGM] == 0u) return;   // its candidate list held the answer
    const int n = min(q_nvis[q], nmax);
    int32_t* o = out + (size_t)q * K;
    if (n <= K) {
        for (int i = threadIdx.x; i < K; i += kSelThreads) o[i] = i < n ? i : -1;
        return;
    }
    const uint32_t* row = keys + (size_t)q * stride;   // 16-byte aligned (stride % 64 == 0)
    if (n <= kSmallRow) {
        uint4 v[kRowRegs];
        load_row_regs(row, n, v);
        const int wv = threadIdx.x / kWave, ln = lane_id();
        uint32_t tord = 1u;   // every key is a candidate for rows of up to kRankMax keys
        if (n > kRankMax) {
            // threshold T: each wave publishes its 4 largest samples (the key
            // in slot t % kRowRegs of each thread); T is the m-th largest of
            // those 64, m about twice the number of samples expected above the
            // K-th key (at most the m-th largest sample, so a too-low T only
            // costs candidates)
            uint32_t smp = 0;
#pragma unroll
            for (int j = 0; j < kRowRegs; ++j)
                if (j == (int)threadIdx.x % kRowRegs) smp = v[j].x;
            uint32_t rest = smp;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t mx = rest;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
                const uint64_t hv = __ballot(rest == mx);
                if (ln == __builtin_ctzll(hv)) rest = 0u;
                if (ln == 0) s_rtop[wv * 4 + r] = mx;
            }
            const uint32_t ns = __syncthreads_count(smp != 0u);
            const uint32_t expect = (uint32_t)(((int64_t)K * ns + n - 1) / n);
            const uint32_t m = min(64u, 2u * expect + 4u);
            if (wv == 0) {   // rank among the 64: larger ones, and equal ones at lower lanes
                const uint32_t x = s_rtop[ln];
                uint32_t rank = 0;
                for (int i = 0; i < kWave; ++i) {
                    const uint32_t y = (uint32_t)__shfl((int)x, i);
                    rank += (y > x || (y == x && i < ln)) ? 1u : 0u;
                }
                if (rank == m - 1) s_dig[0] = x;
            }
            __syncthreads();
            tord = max(1u, s_dig[0]);
        }
        if (select_row_regs(v, tord, K, o, s_cand, s_wbase, s_hist, s_dig, s_tmp)) return;
    }
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) s_h[i] = 0u;
    if (threadIdx.x == 0) { s_na = 0; s_nc = 0; }
    __syncthreads();
    // both passes read 32 keys per thread per round (8 uint4 loads in flight)
    constexpr int kVec = 8;
    for (int base = 0; base < n; base += 4 * kVec * kSelThreads) {
        uint4 v[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int e = base + 4 * (threadIdx.x + kSelThreads * j);
            v[j] = e < n ? *reinterpret_cast<const uint4*>(row + e) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int e = base + 4 * (threadIdx.x + kSelThreads * j);
            const uint32_t kk[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (e + x < n) atomicAdd(&s_h[kk[x] >> kDigitShift], 1u);
        }
    }
    __syncthreads();
    uint32_t b1, nabove;
    find_digit_4096<kSelThreads>(s_h, (uint32_t)K, s_tmp, b1, nabove);
    for (int base = 0; base < n; base += 4 * kVec * kSelThreads) {
        uint4 v[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int e = base + 4 * (threadIdx.x + kSelThreads * j);
            v[j] = e < n ? *reinterpret_cast<const uint4*>(row + e) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int e = base + 4 * (threadIdx.x + kSelThreads * j);
            const uint32_t kk[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t d = kk[x] >> kDigitShift;
                if (e + x < n && d > b1) {
                    const uint32_t p = atomicAdd(&s_na, 1u);
                    if (p < (uint32_t)K) s_out[p] = e + x;
                } else if (e + x < n && d == b1) {
                    const uint32_t p = atomicAdd(&s_nc, 1u);
                    if (p < (uint32_t)kRankMax) s_cand[p] = comp_key(kk[x], (uint32_t)(e + x));
                }
            }
        }
    }
    __syncthreads();
    const uint32_t NA = min(s_na, (uint32_t)K - 1u), NC = s_nc;
    if (NC > (uint32_t)kRankMax) {
        select_global_row<kSelThreads>(row, n, K, o, s_hist, s_dig, s_tmp);
        return;
    }
    pick_lds_candidates(s_cand, NC, (uint32_t)K - NA, NA, s_out, s_hist, s_dig, &s_count);
    rank_and_write(s_out, K, K, o);
}

// Candidate pool of a prefill chunk (the encoder-side form of the
// hierarchical indexer): each query's row of score keys becomes a row of
// block keys, blocks of 2^bs_log2 entries clipped to the query's visible
// entries, scored by their largest key (= the key of the largest score) or by
// the key of the sum of their scores; nblk[q] receives the query's block
// count.  One thread per block; the rows then go through k_row_select.
__global__ __launch_bounds__(256) void k_block_keys(const uint32_t* __restrict__ keys,
                                                    int64_t stride,
                                                    const int32_t* __restrict__ q_nvis,
                                                    int max_nvis, int bs_log2, int block_sum,
                                                    uint32_t* __restrict__ bkeys, int64_t bstride,
                                                    int32_t* __restrict__ nblk) {
    const int q = blockIdx.y;
    const int n = min(q_nvis[q], max_nvis);
    const int nb = (n + (1 << bs_log2) - 1) >> bs_log2;
    if (blockIdx.x == 0 && threadIdx.x == 0) nblk[q] = nb;
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= nb) return;
    const uint32_t* row = keys + (size_t)q * stride;
    const int i0 = b << bs_log2, i1 = min(n, i0 + (1 << bs_log2));
    uint32_t bk = 0u;
    if (block_sum) {
        float sum = 0.f;
        for (int i = i0; i < i1; ++i) sum += ord_key_to_f32(row[i]);
        bk = ord_key(sum);
    } else {
        for (int i = i0; i < i1; ++i) bk = max(bk, row[i]);
    }
    bkeys[(size_t)q * bstride + b] = bk;
}

// ------------------------------------------------------------- reindex

template <int VPR>
__global__ __launch_bounds__(kReindexThreads) void k_reindex_score(
    const float* __restrict__ qI, const float* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_nvis, int Hi, int Hk, int Di, const int32_t* __restrict__ pool,
    int P, int bs, uint32_t* __restrict__ ckeys) {
    constexpr int RW = 256 * VPR;
    const int q = blockIdx.y;
    const int ncand = P * bs;
    const int c0 = blockIdx.x * kReindexPerWG;
    if (c0 >= ncand) return;
    const int c1 = min(ncand, c0 + kReindexPerWG);
    float4 qv[VPR];
    load_qvec<VPR>(qI, q, Hi, Hk, Di, qv);
    const int nvis = q_nvis[q];
    const int64_t row0 = seq_row_off[q_seq ? q_seq[q] : 0];
    const float* kb = kI + row0 * RW;
    const int32_t* prow = pool + (size_t)q * P;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int myrow = (lane >> 3) & 7;
    // wave w scores candidates c0 + 64 w .. +63: lane l first resolves
    // candidate c0 + 64 w + l to its entry row (-1: none), so that every row
    // address of the gathers below is a lane read away, not a load away
    constexpr int kRows = VPR >= 4 ? 8 : 16;   // rows per gather round
    const int cw = c0 + kWave * wave;
    int64_t tl = -1;
    {
        const int c = cw + lane;
        if (c < c1) {
            const int b = prow[c / bs];
            tl = b >= 0 ? (int64_t)b * bs + c % bs : -1;
            if (tl >= nvis) tl = -1;
        }
    }
    const uint32_t tlo = (uint32_t)tl, thi = (uint32_t)(tl >> 32);
#pragma unroll
    for (int it = 0; it < kWave / kRows; ++it) {
        if (cw + kRows * it >= c1) break;   // wave-uniform
        const float* rows[kRows];
        bool ok[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            const int src = kRows * it + i;
            const int64_t t = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(thi, src) << 32) |
                                        __builtin_amdgcn_readlane(tlo, src));
            ok[i] = t >= 0;
            rows[i] = kb + (ok[i] ? t : 0) * RW;
        }
        float sv[kRows / 8];
        dot_rows<VPR, kRows>(rows, ok, qv, sv);
#pragma unroll
        for (int hh = 0; hh < kRows / 8; ++hh) {
            const int r = kRows * it + 8 * hh + myrow;   // this lane's candidate within the wave
            const int64_t t = (int64_t)(((uint64_t)(uint32_t)__shfl((int)thi, r) << 32) |
                                        (uint32_t)__shfl((int)tlo, r));
            const int c = cw + r;
            // the score key only (0: no candidate; no score maps to 0): the
            // select rebuilds the entry from the pool.  Nontemporal: written
            // once, read once by the select kernel, and kept out of the way
            // of this kernel's row stream (with plain stores the gather ran
            // about 4 % slower)
            if ((lane & 7) == 0 && c < c1)
                __builtin_nontemporal_store(t >= 0 ? ord_key(sv[hh]) : 0u,
                                            ckeys + (size_t)q * ncand + c);
        }
    }
}

// Reindex scorer over E4M3 key rows (RB = 256 * VPR bytes), in the 16-lanes-
// per-row layout of dot_rows16: wave w scores candidates c0 + 64 w .. +63 in
// rounds of G groups of four rows (16 KB; issuing all 64 rows at once needs
// registers that cost more occupancy than the deeper gather gains); each lane
// first resolves one candidate to its entry (-1: none),
// and the rows of a round are read with entries taken from those lanes.  A
// lane whose candidate is empty reads its 16-byte columns of this query's
// indexer row instead (always valid memory, at least RB bytes) and the result
// is discarded.
template <int VPR>
__global__ __launch_bounds__(kReindexThreads) void k_reindex_score_e4m3(
    const float* __restrict__ qI, const uint8_t* __restrict__ kI,
    const int64_t* __restrict__ seq_row_off, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_nvis, int Hi, int Hk, int Di, const int32_t* __restrict__ pool,
    int P, int bs, uint32_t* __restrict__ ckeys) {
    constexpr int RB = 256 * VPR;
    constexpr int G = 16 / VPR;
    constexpr int RPB = 4 * G;                        // rows per sub-block
    constexpr int NB = 1;                             // sub-blocks per round
    constexpr int RPI = NB * RPB;                     // rows per round
    constexpr int GSH = 4 - log2_groups<G>();
    const int q = blockIdx.y;
    const int ncand = P * bs;
    const int c0 = blockIdx.x * kReindexPerWG;
    if (c0 >= ncand) return;
    const int c1 = min(ncand, c0 + kReindexPerWG);
    float4 qv[VPR][4];
    load_qvec16<VPR>(qI, q, Hi, Hk, Di, qv);
    const int nvis = q_nvis[q];
    const int64_t row0 = seq_row_off[q_seq ? q_seq[q] : 0];
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int u16 = 16 * (lane & 15), rq = lane >> 4;
    const int myrow = 4 * ((lane & 15) >> GSH) + rq;
    const bool writer = (lane & ((1 << GSH) - 1)) == 0;
    const uint8_t* kl = kI + row0 * RB + u16;
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(qI + (size_t)q * Hi * Di) + u16;
    const int32_t* prow = pool + (size_t)q * P;
    const int cw = c0 + kWave * wave;
    int tl = -1;
    {
        const int c = cw + lane;
        if (c < c1) {
            const int b = prow[c / bs];
            tl = b >= 0 ? b * bs + c % bs : -1;
            if (tl >= nvis) tl = -1;
        }
    }
#pragma unroll
    for (int it = 0; it < kWave / RPI; ++it) {
        if (cw + RPI * it >= c1) break;   // wave-uniform
        const uint8_t* grow[NB][G];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int t = __shfl(tl, RPI * it + RPB * b + 4 * g + rq);
                grow[b][g] = t >= 0 ? kl + (int64_t)t * RB : dummy;
            }
        float sv[NB];
        dot_rows16<VPR, G, NB>(grow, qv, sv);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = RPI * it + RPB * b + myrow;   // this lane's candidate within the wave
            const int t = __shfl(tl, r);
            const int c = cw + r;
            if (writer && c < c1)
                __builtin_nontemporal_store(t >= 0 ? ord_key(sv[b]) : 0u,
                                            ckeys + (size_t)q * ncand + c);
        }
    }
}

// Top-K of one query's Reindex candidates by one workgroup.  The gather
// leaves a 4-byte score key per candidate (0: none); the histogram and the
// placement work on those, and the entry of a candidate (from the pool row
// staged in LDS) is looked up only for the keys that need it, the winners
// and the composite keys (score, then the lower entry) of the K-th key's
// bin.  A 4096-bin histogram of the keys' top 12 bits (the score's)
// places the K-th largest key in bin b1; the keys above b1 win outright and
// the best of b1's keys are picked in LDS (direct ranking, or a radix select
// from bit 48 when there are many).  More than kRankMax keys in b1
// (degenerate score distributions) falls back to the radix select over all
// candidates.  The K indices are written in ascending order.
template <bool POW2>
__global__ __launch_bounds__(kSelThreads) void k_reindex_select(
    const uint32_t* __restrict__ skeys, int ncand, int K, int32_t* __restrict__ out,
    const int32_t* __restrict__ pool, int P, int bs) {
    __shared__ __attribute__((aligned(16))) int32_t s_out[CSA2_MAX_TOPK + 4];
    __shared__ int32_t s_pool[CSA2_MAX_TOPK];
    __shared__ __attribute__((aligned(16))) uint64_t s_cand[kRankMax + 2];
    __shared__ uint32_t s_h[4][kHistBins];   // four sub-histograms, then their sum in s_h[0]
    __shared__ uint32_t s_hist[256];
    __shared__ uint32_t s_dig[2];
    __shared__ uint32_t s_tmp[kSelThreads / kWave + 3];
    __shared__ uint32_t s_count;
    const int q = blockIdx.x;
    int32_t* o = out + (size_t)q * K;
    uint32_t sk[kSelItems];
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        const int i = threadIdx.x + j * kSelThreads;
        sk[j] = i < ncand ? skeys[(size_t)q * ncand + i] : 0u;
    }
    for (int i = threadIdx.x; i < P; i += kSelThreads) s_pool[i] = pool[(size_t)q * P + i];
    for (int i = threadIdx.x; i < 4 * kHistBins; i += kSelThreads) (&s_h[0][0])[i] = 0u;
    __syncthreads();
    // entry of candidate c: position c % bs of pool block s_pool[c / bs]
    // (taken only for the keys that need it; POW2: bs a power of two)
    const int lbs = __ffs(bs) - 1;
    auto entry = [&](int c) __attribute__((always_inline)) -> uint32_t {
        if constexpr (POW2)
            return (uint32_t)(s_pool[min(c >> lbs, CSA2_MAX_TOPK - 1)] * bs + (c & (bs - 1)));
        else
            return (uint32_t)(s_pool[min(c / bs, CSA2_MAX_TOPK - 1)] * bs + c % bs);
    };
    // lane l counts into sub-histogram l % 4: lanes of one instruction that
    // hit the same bin (scores cluster in a few bins) serialise a quarter as
    // often
    uint32_t* const hsub = s_h[lane_id() & 3];
    uint32_t nv = 0;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        if (sk[j] == 0u) continue;
        ++nv;
        atomicAdd(&hsub[sk[j] >> kDigitShift], 1u);
    }
    uint32_t total;
    (void)block_exclusive_sum<kSelThreads>(nv, s_tmp, total);   // ends with a barrier
    for (int i = threadIdx.x; i < kHistBins; i += kSelThreads)
        s_h[0][i] = (s_h[0][i] + s_h[1][i]) + (s_h[2][i] + s_h[3][i]);
    __syncthreads();
    const uint32_t k = min(total, (uint32_t)K);
    if (k == 0u) {
        for (int i = threadIdx.x; i < K; i += kSelThreads) o[i] = -1;
        return;
    }
    uint32_t b1, nabove;
    find_digit_4096<kSelThreads>(s_h[0], k, s_tmp, b1, nabove);
    const uint32_t nb = s_h[0][b1];
    if (nb > (uint32_t)kRankMax) {
        uint64_t it[kSelItems];
#pragma unroll
        for (int j = 0; j < kSelItems; ++j)
            it[j] = sk[j] ? comp_key(sk[j], entry(threadIdx.x + j * kSelThreads)) : 0ull;
        select_top_ckeys<kSelThreads, kSelItems>(it, K, o);
        return;
    }
    // winners to s_out, b1's keys to s_cand (composite), at offsets from one
    // block scan of the per-thread counts (packed: fewer than 2^16 of either)
    uint32_t na = 0, nc = 0;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        const uint32_t d = sk[j] >> kDigitShift;
        na += sk[j] != 0u && d > b1;
        nc += sk[j] != 0u && d == b1;
    }
    uint32_t tot2;
    const uint32_t ex = block_exclusive_sum<kSelThreads>((na << 16) | nc, s_tmp, tot2);
    uint32_t pa = ex >> 16, pc = ex & 0xFFFFu;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        const uint32_t d = sk[j] >> kDigitShift;
        const int c = threadIdx.x + j * kSelThreads;
        if (sk[j] != 0u && d > b1) s_out[pa++] = (int32_t)entry(c);
        else if (sk[j] != 0u && d == b1) s_cand[pc++] = comp_key(sk[j], entry(c));
    }
    __syncthreads();
    // nabove keys above b1 (fewer than k) and nb >= k - nabove keys in b1
    pick_lds_candidates(s_cand, nb, k - nabove, nabove, s_out, s_hist, s_dig, &s_count, 48);
    rank_and_write<kSelThreads>(s_out, (int)k, K, o);
}

// ------------------------------------------------------ host helpers

struct IndexWs {
    uint32_t *keys_e, *keys_b, *hist_e, *hist_b, *cnt_e, *cnt_b;
    int32_t *above_e, *above_b;
    uint64_t *cand_e, *cand_b;
    int32_t* nblk;   // prefill pool: blocks per query
    int64_t se, sb;
    size_t zero_words;
    size_t bytes;
};

inline int ilog2(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

IndexWs carve_index(void* ws, int Q, int max_nvis, int topk, int pool_blocks, int block_size) {
    IndexWs w{};
    Carver c(ws);
    const int bs = pool_blocks > 0 ? block_size : 1;
    w.se = ((int64_t)max_nvis + 63) / 64 * 64;
    w.sb = pool_blocks > 0 ? (((int64_t)max_nvis + bs - 1) / bs + 63) / 64 * 64 : 0;
    // zeroed region first: histograms and counters
    w.hist_e = c.take<uint32_t>((size_t)Q * kHistBins);
    w.hist_b = c.take<uint32_t>(pool_blocks > 0 ? (size_t)Q * kHistBins : 0);
    w.cnt_e = c.take<uint32_t>((size_t)Q * 2);
    w.cnt_b = c.take<uint32_t>((size_t)Q * 2);
    w.zero_words = c.bytes() / 4;
    w.keys_e = c.take<uint32_t>((size_t)Q * w.se);
    w.keys_b = c.take<uint32_t>((size_t)Q * w.sb);
    w.above_e = c.take<int32_t>((size_t)Q * topk);
    w.above_b = c.take<int32_t>((size_t)Q * pool_blocks);
    w.cand_e = c.take<uint64_t>(topk > 0 ? (size_t)Q * kCandCap : 0);
    w.cand_b = c.take<uint64_t>(pool_blocks > 0 ? (size_t)Q * kCandCap : 0);
    w.nblk = c.take<int32_t>(pool_blocks > 0 ? (size_t)Q : 0);
    w.bytes = c.bytes();
    return w;
}

// Shared argument checks of the indexer entry points.
int check_indexer_shape(int Q, int Hi, int Hk, int Di, int* vpr) {
    if (Q < 0 || Hi <= 0 || Hk <= 0 || Di <= 0) return CSA2_ERR_SHAPE;
    if (Hk != Hi && Hk != 1) return CSA2_ERR_UNSUPPORTED;
    const long rw = (long)Hk * Di;
    if (rw == 256) *vpr = 1;
    else if (rw == 512) *vpr = 2;
    else if (rw == 1024) *vpr = 4;
    else return CSA2_ERR_UNSUPPORTED;
    if (Q > 65535) return CSA2_ERR_UNSUPPORTED;
    return CSA2_OK;
}

}  // namespace
}  // namespace csa2

using namespace csa2;

// The prefill form's bf16 copies, carved after the index region (at `at`,
// a multiple of 256) of the same workspace; returns the total bytes.
struct PrefillWs {
    uint16_t *qh, *ql, *kh, *kl;
    uint32_t *qflag, *kflag;
    int Qp, Np;   // rows padded to whole score tiles
    // candidate path of the Top-K: sampled keys, thresholds, candidate
    // lists, their counts and the flags of query tiles sent to the exact path
    uint32_t *samp, *thr, *cnt, *tfail;
    uint64_t* cand;
    int ns;       // sampled keys per query
    size_t zero_words;   // cnt and tfail, cleared together
};

size_t carve_prefill(void* ws, size_t at, int Q, int max_nvis, int RW, PrefillWs* p) {
    Carver c(ws);
    (void)c.take<uint8_t>(at);
    p->Qp = (Q + kGM - 1) / kGM * kGM;
    p->Np = (max_nvis + kGN - 1) / kGN * kGN;
    p->qh = c.take<uint16_t>((size_t)p->Qp * RW);
    p->ql = c.take<uint16_t>((size_t)p->Qp * RW);
    p->kh = c.take<uint16_t>((size_t)p->Np * RW);
    p->kl = c.take<uint16_t>((size_t)p->Np * RW);
    p->qflag = c.take<uint32_t>(p->Qp / kCvtRows);
    p->kflag = c.take<uint32_t>(p->Np / kCvtRows);
    const int ntiles = p->Np / kGN;
    p->ns = kGN * std::min(ntiles, kSampleTiles);
    p->samp = c.take<uint32_t>((size_t)Q * p->ns);
    p->thr = c.take<uint32_t>((size_t)Q);
    p->cand = c.take<uint64_t>((size_t)Q * kCandCapPre);
    // counts, then the any-tile flag and the tile flags
    p->cnt = c.take<uint32_t>((size_t)Q + 1 + p->Qp / kGM);
    p->tfail = p->cnt ? p->cnt + Q : nullptr;
    p->zero_words = (size_t)Q + 1 + p->Qp / kGM;
    return c.bytes();
}

extern "C" size_t csa2_index_prefill_workspace_bytes_ex(int32_t Q, int32_t max_nvis,
                                                        int32_t topk, int32_t pool_blocks,
                                                        int32_t block_size, int32_t Hk,
                                                        int32_t Di) {
    if (Q < 0 || max_nvis < 0 || topk < 0 || pool_blocks < 0 || Hk <= 0 || Di <= 0) return 0;
    if (pool_blocks > 0 && block_size <= 0) return 0;
    PrefillWs p;
    const size_t at = carve_index(nullptr, Q, max_nvis, topk, pool_blocks, block_size).bytes;
    return carve_prefill(nullptr, at, Q, max_nvis, Hk * Di, &p);
}

extern "C" size_t csa2_index_prefill_workspace_bytes(int32_t Q, int32_t max_nvis, int32_t topk,
                                                     int32_t Hk, int32_t Di) {
    return csa2_index_prefill_workspace_bytes_ex(Q, max_nvis, topk, 0, 1, Hk, Di);
}

extern "C" size_t csa2_index_full_workspace_bytes(int32_t Q, int32_t max_nvis, int32_t topk,
                                                  int32_t pool_blocks, int32_t block_size) {
    if (Q < 0 || max_nvis < 0 || topk < 0 || pool_blocks < 0) return 0;
    if (pool_blocks > 0 && block_size <= 0) return 0;
    return carve_index(nullptr, Q, max_nvis, topk, pool_blocks, block_size).bytes;
}

// Full-mode indexer over a key cache of KT values (float or E4M3 bytes).
template <typename KT>
static int index_full_impl(const float* qI, const KT* kI, const int64_t* seq_row_off,
                    const int32_t* q_seq, const int32_t* q_nvis, int32_t Q, int32_t Hi,
                    int32_t Hk, int32_t Di, int32_t max_nvis, int32_t topk, int32_t* topk_idx,
                    int32_t pool_blocks, int32_t block_size, int32_t* pool_block_idx,
                    int32_t block_rule, void* ws, size_t ws_bytes, void* stream_) {
    int vpr = 0;
    int st = check_indexer_shape(Q, Hi, Hk, Di, &vpr);
    if (st != CSA2_OK) return st;
    if (max_nvis < 0 || topk < 0 || pool_blocks < 0) return CSA2_ERR_SHAPE;
    if (topk > CSA2_MAX_TOPK || pool_blocks > CSA2_MAX_TOPK) return CSA2_ERR_UNSUPPORTED;
    if (pool_blocks > 0 && block_size != 1 && block_size != 2 && block_size != 4 && block_size != 8)
        return block_size <= 0 ? CSA2_ERR_SHAPE : CSA2_ERR_UNSUPPORTED;
    if (block_rule != CSA2_BLOCK_MAX && block_rule != CSA2_BLOCK_SUM) return CSA2_ERR_UNSUPPORTED;
    if (Q == 0 || (topk == 0 && pool_blocks == 0)) return CSA2_OK;
    if (!qI || !kI || !seq_row_off || !q_nvis || !ws) return CSA2_ERR_NULL;
    if ((topk > 0 && !topk_idx) || (pool_blocks > 0 && !pool_block_idx)) return CSA2_ERR_NULL;
    if (((uintptr_t)qI | (uintptr_t)kI) & 15) return CSA2_ERR_UNSUPPORTED;
    IndexWs w = carve_index(ws, Q, max_nvis, topk, pool_blocks, block_size);
    if (ws_bytes < w.bytes) return CSA2_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream_;
    const int bs_log2 = pool_blocks > 0 ? ilog2(block_size) : 0;

    if (!q_seq) {
        // prefill chunk of one sequence: bf16 copies of the query and key
        // rows, bf16-MFMA score tiles, then one selecting workgroup per query
        // (and per query's row of block keys for a pool)
        PrefillWs pw;
        if (ws_bytes < carve_prefill(ws, w.bytes, Q, max_nvis, Hk * Di, &pw))
            return CSA2_ERR_WORKSPACE;
        if (max_nvis > 0) {
            const int RW = Hk * Di;
            auto cvt = RW == 256 ? k_prefill_convert<KT, 4>
                     : RW == 512 ? k_prefill_convert<KT, 8> : k_prefill_convert<KT, 16>;
            st = CSA2_LAUNCH("prefill_convert", cvt,
                             dim3((pw.Qp + pw.Np) / kCvtRows), dim3(kCvtThreads), s, qI, kI,
                             seq_row_off,
                             Q, pw.Qp, Hi, Hk, Di, max_nvis, pw.qh, pw.ql, pw.kh, pw.kl,
                             pw.qflag, pw.kflag);
            if (st) return st;
        }
        const int ntiles = pw.Np / kGN, nqt = pw.Qp / kGM;
        if (topk > 0 && pool_blocks == 0 && max_nvis > 0) {
            // Top-K without the full score rows: thresholds from sampled key
            // tiles, candidate lists from the score tiles, exact selection over
            // the lists, and the full rows only for query tiles whose lists
            // could not hold the answer
            const int step = (ntiles + kSampleTiles - 1) / kSampleTiles;
            const int nst = (ntiles + step - 1) / step;
            st = CSA2_LAUNCH("zero", k_zero_u32, dim3(64), dim3(256), s, pw.cnt, pw.zero_words);
            if (st) return st;
            st = CSA2_LAUNCH("prefill_sample", k_prefill_gemm<kGemmSample>,
                             dim3(nst * nqt), dim3(256), s, pw.qh, pw.ql, pw.kh, pw.kl,
                             pw.qflag, pw.kflag, Hk * Di, Q, q_nvis, max_nvis, pw.samp,
                             (int64_t)nst * kGN, nst, nqt, step, (const uint32_t*)nullptr,
                             (const uint32_t*)nullptr, (uint64_t*)nullptr, (uint32_t*)nullptr);
            if (st) return st;
            st = CSA2_LAUNCH("sample_thr", k_sample_thr, dim3(Q), dim3(256), s, pw.samp, nst * kGN,
                             q_nvis, max_nvis, topk, pw.thr);
            if (st) return st;
            st = CSA2_LAUNCH("prefill_scores", k_prefill_gemm<kGemmCand>,
                             dim3(ntiles * nqt), dim3(256), s, pw.qh, pw.ql, pw.kh, pw.kl,
                             pw.qflag, pw.kflag, Hk * Di, Q, q_nvis, max_nvis, (uint32_t*)nullptr,
                             (int64_t)0, ntiles, nqt, 1, (const uint32_t*)nullptr, pw.thr, pw.cand,
                             pw.cnt);
            if (st) return st;
            st = CSA2_LAUNCH("cand_select", k_cand_select, dim3(Q), dim3(kCandThreads), s, pw.cand,
                             pw.cnt, pw.thr, topk, topk_idx, pw.tfail);
            if (st) return st;
            // exact path, flagged query tiles only (a small grid that skips
            // the other tiles: the launch costs little when nothing failed)
            st = CSA2_LAUNCH("prefill_scores_fb", k_prefill_gemm<kGemmKeysFb>,
                             dim3(std::min(ntiles * nqt, kFbGrid)), dim3(256), s, pw.qh, pw.ql, pw.kh, pw.kl,
                             pw.qflag, pw.kflag, Hk * Di, Q, q_nvis, max_nvis, w.keys_e, w.se,
                             ntiles, nqt, 1,
                             (const uint32_t*)pw.tfail, (const uint32_t*)nullptr,
                             (uint64_t*)nullptr, (uint32_t*)nullptr);
            if (st) return st;
            st = CSA2_LAUNCH("row_select_fb", k_row_select, dim3(Q), dim3(kSelThreads), s,
                             w.keys_e, w.se, q_nvis, max_nvis, topk, topk_idx,
                             (const uint32_t*)pw.tfail);
            if (st) return st;
            return CSA2_OK;
        }
        if (max_nvis > 0) {
            st = CSA2_LAUNCH("prefill_scores", k_prefill_gemm<kGemmKeys>,
                             dim3(ntiles * nqt), dim3(256), s, pw.qh, pw.ql, pw.kh, pw.kl,
                             pw.qflag, pw.kflag, Hk * Di, Q, q_nvis, max_nvis, w.keys_e, w.se,
                             ntiles, nqt, 1,
                             (const uint32_t*)nullptr, (const uint32_t*)nullptr,
                             (uint64_t*)nullptr, (uint32_t*)nullptr);
            if (st) return st;
        }
        if (topk > 0) {
            st = CSA2_LAUNCH("row_select", k_row_select, dim3(Q), dim3(kSelThreads), s, w.keys_e,
                             w.se, q_nvis, max_nvis, topk, topk_idx, (const uint32_t*)nullptr);
            if (st) return st;
        }
        if (pool_blocks > 0) {
            const int nbmax = (max_nvis + block_size - 1) / block_size;
            st = CSA2_LAUNCH("block_keys", k_block_keys, dim3((nbmax + 255) / 256 + (nbmax == 0), Q),
                             dim3(256), s, w.keys_e, w.se, q_nvis, max_nvis, bs_log2,
                             (int)(block_rule == CSA2_BLOCK_SUM), w.keys_b, w.sb, w.nblk);
            if (st) return st;
            st = CSA2_LAUNCH("row_select_b", k_row_select, dim3(Q), dim3(kSelThreads), s,
                             w.keys_b, w.sb, w.nblk, nbmax, pool_blocks, pool_block_idx,
                             (const uint32_t*)nullptr);
            if (st) return st;
        }
        return CSA2_OK;
    }
    st = CSA2_LAUNCH("zero", k_zero_u32, dim3(256), dim3(256), s, w.hist_e, w.zero_words);
    if (st) return st;
    if (max_nvis == 0) {
        // no visible entries anywhere: the finalize kernels write -1 rows
    } else {
        uint32_t* bk = pool_blocks > 0 ? w.keys_b : nullptr;
        st = launch_score_stream(vpr, sizeof(KT) == 1, max_nvis, Q, s, qI, kI, seq_row_off,
                                 q_seq, q_nvis, Hi, Hk, Di, w.keys_e, w.se, w.hist_e, bk, w.sb,
                                 bs_log2, block_rule == CSA2_BLOCK_SUM, w.hist_b);
        if (st) return st;
    }
    // selection of one row per query: a single workgroup for short rows,
    // filter + finalize otherwise
    auto select = [&](bool blocks, uint32_t* keys, int64_t stride, int bsl, int nmax, int K,
                      uint32_t* hist, uint32_t* cnt, int32_t* above, uint64_t* cand,
                      int32_t* out) -> int {
        if (nmax <= kSmallRow)
            return CSA2_LAUNCH(blocks ? "select_small_b" : "select_small", k_select_small,
                               dim3(Q), dim3(kSelThreads), s, keys, stride, q_nvis, nmax, bsl,
                               K, hist, out);
        dim3 g((nmax + kSelElems - 1) / kSelElems, Q);
        int r = CSA2_LAUNCH(blocks ? "filter_b" : "filter", k_filter, g, dim3(256), s, keys,
                            stride, q_nvis, nmax, bsl, K, hist, cnt, above, cand);
        if (r) return r;
        return CSA2_LAUNCH(blocks ? "finalize_b" : "finalize", k_finalize, dim3(Q),
                           dim3(kSelThreads), s, keys, stride, q_nvis, nmax, bsl, K, cnt, above,
                           cand, out);
    };
    if (topk > 0) {
        st = select(false, w.keys_e, w.se, 0, max_nvis, topk, w.hist_e, w.cnt_e, w.above_e, w.cand_e,
                    topk_idx);
        if (st) return st;
    }
    if (pool_blocks > 0) {
        const int nb = (max_nvis + block_size - 1) / block_size;
        st = select(true, w.keys_b, w.sb, bs_log2, nb, pool_blocks, w.hist_b, w.cnt_b, w.above_b,
                    w.cand_b, pool_block_idx);
        if (st) return st;
    }
    return CSA2_OK;
}

extern "C" int csa2_index_full(const float* qI, const float* kI, const int64_t* seq_row_off,
                               const int32_t* q_seq, const int32_t* q_nvis, int32_t Q, int32_t Hi,
                               int32_t Hk, int32_t Di, int32_t max_nvis, int32_t topk,
                               int32_t* topk_idx, int32_t pool_blocks, int32_t block_size,
                               int32_t* pool_block_idx, void* ws, size_t ws_bytes,
                               void* stream) {
    return index_full_impl<float>(qI, kI, seq_row_off, q_seq, q_nvis, Q, Hi, Hk, Di, max_nvis,
                                  topk, topk_idx, pool_blocks, block_size, pool_block_idx,
                                  CSA2_BLOCK_MAX, ws, ws_bytes, stream);
}

extern "C" int csa2_index_full_e4m3(const float* qI, const uint8_t* kI,
                                    const int64_t* seq_row_off, const int32_t* q_seq,
                                    const int32_t* q_nvis, int32_t Q, int32_t Hi, int32_t Hk,
                                    int32_t Di, int32_t max_nvis, int32_t topk,
                                    int32_t* topk_idx, int32_t pool_blocks, int32_t block_size,
                                    int32_t* pool_block_idx, void* ws, size_t ws_bytes,
                                    void* stream) {
    return index_full_impl<uint8_t>(qI, kI, seq_row_off, q_seq, q_nvis, Q, Hi, Hk, Di, max_nvis,
                                    topk, topk_idx, pool_blocks, block_size, pool_block_idx,
                                    CSA2_BLOCK_MAX, ws, ws_bytes, stream);
}

extern "C" int csa2_index_full_ex(const float* qI, const void* kI, int32_t key_format,
                                  const int64_t* seq_row_off, const int32_t* q_seq,
                                  const int32_t* q_nvis, int32_t Q, int32_t Hi, int32_t Hk,
                                  int32_t Di, int32_t max_nvis, int32_t topk, int32_t* topk_idx,
                                  int32_t pool_blocks, int32_t block_size,
                                  int32_t* pool_block_idx, int32_t block_rule, void* ws,
                                  size_t ws_bytes, void* stream) {
    if (key_format == CSA2_KEYS_F32)
        return index_full_impl<float>(qI, static_cast<const float*>(kI), seq_row_off, q_seq,
                                      q_nvis, Q, Hi, Hk, Di, max_nvis, topk, topk_idx,
                                      pool_blocks, block_size, pool_block_idx, block_rule, ws,
                                      ws_bytes, stream);
    if (key_format == CSA2_KEYS_E4M3)
        return index_full_impl<uint8_t>(qI, static_cast<const uint8_t*>(kI), seq_row_off, q_seq,
                                        q_nvis, Q, Hi, Hk, Di, max_nvis, topk, topk_idx,
                                        pool_blocks, block_size, pool_block_idx, block_rule, ws,
                                        ws_bytes, stream);
    return CSA2_ERR_UNSUPPORTED;
}

extern "C" size_t csa2_reindex_workspace_bytes(int32_t Q, int32_t pool_blocks, int32_t block_size) {
    if (Q < 0 || pool_blocks < 0 || block_size <= 0) return 0;
    Carver c(nullptr);
    c.take<uint32_t>((size_t)Q * pool_blocks * block_size);
    return c.bytes();
}

// Reindex over a key cache of KT values (float or E4M3 bytes).
template <typename KT>
static int reindex_impl(const float* qI, const KT* kI, const int64_t* seq_row_off,
                 const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_block_idx,
                 int32_t pool_blocks, int32_t block_size, int32_t Q, int32_t Hi, int32_t Hk,
                 int32_t Di, int32_t topk, int32_t* topk_idx, void* ws, size_t ws_bytes,
                 void* stream_) {
    int vpr = 0;
    int st = check_indexer_shape(Q, Hi, Hk, Di, &vpr);
    if (st != CSA2_OK) return st;
    if (pool_blocks < 0 || block_size <= 0 || topk < 0) return CSA2_ERR_SHAPE;
    if (topk > CSA2_MAX_TOPK || (int64_t)pool_blocks * block_size > CSA2_MAX_POOL_CAND)
        return CSA2_ERR_UNSUPPORTED;
    if (Q == 0 || topk == 0) return CSA2_OK;
    if (!qI || !kI || !seq_row_off || !q_nvis || !topk_idx || !ws) return CSA2_ERR_NULL;
    if (pool_blocks > 0 && !pool_block_idx) return CSA2_ERR_NULL;
    if (((uintptr_t)qI | (uintptr_t)kI) & 15) return CSA2_ERR_UNSUPPORTED;
    if (ws_bytes < csa2_reindex_workspace_bytes(Q, pool_blocks, block_size))
        return CSA2_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream_;
    uint32_t* ck = static_cast<uint32_t*>(ws);
    const int ncand = pool_blocks * block_size;
    if (ncand > 0) {
        dim3 g((ncand + kReindexPerWG - 1) / kReindexPerWG, Q);
#define CSA2_RS(K, NAME)                                                                      \
    CSA2_LAUNCH(NAME, K, g, dim3(kReindexThreads), s, qI, kI, seq_row_off, q_seq, q_nvis, Hi,  \
                Hk, Di, pool_block_idx, pool_blocks, block_size, ck)
        if constexpr (sizeof(KT) == 1)
            st = vpr == 1   ? CSA2_RS(k_reindex_score_e4m3<1>, "reindex_score_e4m3")
                 : vpr == 2 ? CSA2_RS(k_reindex_score_e4m3<2>, "reindex_score_e4m3")
                            : CSA2_RS(k_reindex_score_e4m3<4>, "reindex_score_e4m3");
        else
            st = vpr == 1   ? CSA2_RS(k_reindex_score<1>, "reindex_score")
                 : vpr == 2 ? CSA2_RS(k_reindex_score<2>, "reindex_score")
                            : CSA2_RS(k_reindex_score<4>, "reindex_score");
#undef CSA2_RS
        if (st) return st;
    }
    if ((block_size & (block_size - 1)) == 0)
        return CSA2_LAUNCH("reindex_select", k_reindex_select<true>, dim3(Q), dim3(kSelThreads),
                           s, ck, ncand, topk, topk_idx, pool_block_idx, pool_blocks, block_size);
    return CSA2_LAUNCH("reindex_select", k_reindex_select<false>, dim3(Q), dim3(kSelThreads), s,
                       ck, ncand, topk, topk_idx, pool_block_idx, pool_blocks, block_size);
}

extern "C" int csa2_reindex(const float* qI, const float* kI, const int64_t* seq_row_off,
                            const int32_t* q_seq, const int32_t* q_nvis,
                            const int32_t* pool_block_idx, int32_t pool_blocks, int32_t block_size,
                            int32_t Q, int32_t Hi, int32_t Hk, int32_t Di, int32_t topk,
                            int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
    return reindex_impl<float>(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, pool_blocks,
                               block_size, Q, Hi, Hk, Di, topk, topk_idx, ws, ws_bytes, stream);
}

extern "C" int csa2_reindex_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                                 const int32_t* q_seq, const int32_t* q_nvis,
                                 const int32_t* pool_block_idx, int32_t pool_blocks,
                                 int32_t block_size, int32_t Q, int32_t Hi, int32_t Hk,
                                 int32_t Di, int32_t topk, int32_t* topk_idx, void* ws,
                                 size_t ws_bytes, void* stream) {
    return reindex_impl<uint8_t>(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, pool_blocks,
                                 block_size, Q, Hi, Hk, Di, topk, topk_idx, ws, ws_bytes, stream);
}

// ------------------------------------------------ allocation-free Reindex

// Scratch of csa2_reindex_noalloc: the candidates' score keys (4 bytes per
// candidate) that k_reindex_score writes and k_reindex_select reads, in a
// static array that each GPU the library runs on holds until the process
// ends.  Host code never passes this name to a kernel: on the host it stands
// for no device address; the address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint32_t scratch[CSA2_NOALLOC_MAX_CAND];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device
}  // namespace

// The device address of the current device's scratch; looked up once per
// device (with that device current) and kept.
static int current_device_scratch(uint32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return CSA2_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_last_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return CSA2_ERR_HIP;
        }
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return CSA2_OK;
}

extern "C" int csa2_reindex_noalloc(const float* qI, const float* kI,
                                    const int64_t* seq_row_off, const int32_t* q_seq,
                                    const int32_t* q_nvis, const int32_t* pool_block_idx,
                                    int32_t pool_blocks, int32_t block_size, int32_t Q,
                                    int32_t Hi, int32_t Hk, int32_t Di, int32_t topk,
                                    int32_t* topk_idx, void* stream) {
    if (Q < 0 || pool_blocks < 0 || block_size <= 0 || topk < 0) return CSA2_ERR_SHAPE;
    if ((int64_t)Q * pool_blocks * block_size > CSA2_NOALLOC_MAX_CAND) return CSA2_ERR_UNSUPPORTED;
    uint32_t* ws = nullptr;
    if (Q > 0 && topk > 0) {
        const int st = current_device_scratch(&ws);
        if (st != CSA2_OK) return st;
    }
    return reindex_impl<float>(qI, kI, seq_row_off, q_seq, q_nvis, pool_block_idx, pool_blocks,
                               block_size, Q, Hi, Hk, Di, topk, topk_idx, ws,
                               sizeof(uint32_t) * (size_t)CSA2_NOALLOC_MAX_CAND, stream);
}
