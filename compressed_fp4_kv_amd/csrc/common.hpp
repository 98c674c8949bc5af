// Device helpers shared by the CSA2 kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kWave = 64;

// Order-preserving map of an fp32 score onto uint32: larger score -> larger
// key.  -0.0 is folded onto +0.0 so that equal scores tie exactly.
__device__ __forceinline__ uint32_t ord_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ord_key (a key of an fp32 score back to the score).
__device__ __forceinline__ float ord_key_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Composite selection key: score first, then the LOWER index.  Distinct
// indices make every key distinct, so "the k largest keys" is a unique set.
// 0 is reserved for "no candidate" (no real key is 0: ord_key >= 0x007FFFFF).
__device__ __forceinline__ uint64_t comp_key(uint32_t ord, uint32_t idx) {
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t comp_idx(uint64_t key) {
    return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set lanes of `mask` strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-aggregated append: every lane with `pred` gets a distinct slot of
// `counter`; returns the slot (valid only where pred).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
    uint64_t m = __ballot(pred);
    uint32_t base = 0;
    if (m) {
        int leader = __builtin_ctzll(m);
        if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
        base = __shfl(base, leader);
    }
    return base + (uint32_t)lanes_below(m);
}

// E4M3FN byte -> fp32, from the OCP definition: bias 7, subnormals at
// exponent 0, S.1111.111 = NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
    float mag;
    if (e == 0) mag = (float)m * 0x1p-9f;
    else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 15 && m == 7) mag = __uint_as_float(0x7FC00000u);
    return __uint_as_float(__float_as_uint(mag) | s);
}

// ------------------------------------------------------------ block scans

// Exclusive prefix sum over the block (NT threads, NT % 64 == 0); `total`
// receives the block sum.  `s_tmp` needs NT/64 + 1 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* s_tmp,
                                                        uint32_t& total) {
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) s_tmp[wid] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (int w = 0; w < NT / kWave; ++w) {
            uint32_t t = s_tmp[w];
            s_tmp[w] = run;
            run += t;
        }
        s_tmp[NT / kWave] = run;
    }
    __syncthreads();
    uint32_t res = s_tmp[wid] + incl - v;
    total = s_tmp[NT / kWave];
    __syncthreads();
    return res;
}

// Given a 256-bin histogram in LDS (counts of keys whose current digit is d),
// find the digit holding the `want`-th largest key (want >= 1): returns d and
// sets `above` to the number of keys with a larger digit.  Executed by the
// first wave; results broadcast through s_out[0..1].
__device__ __forceinline__ void find_digit_256(const uint32_t* s_hist, uint32_t want,
                                               uint32_t* s_out) {
    if (threadIdx.x < kWave) {
        const int l = threadIdx.x;
        uint32_t c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = s_hist[4 * l + j]; tot += c[j]; }
        // inclusive suffix sum of lane totals (lanes above and this one)
        uint32_t suf = tot;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            uint32_t y = __shfl_down(suf, off);
            if (l + off < kWave) suf += y;
        }
        uint32_t run = suf - tot;  // keys in digits above this lane's 4
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (run < want && run + c[j] >= want) { s_out[0] = 4 * l + j; s_out[1] = run; }
            run += c[j];
        }
    }
    __syncthreads();
}

// Same search over a 4096-bin histogram in global memory (first-level digit
// of the score stream), by a whole block of NT threads.  Returns the digit
// of the `want`-th largest key and the count strictly above it.  s_tmp needs
// NT/64 + 3 words; 1 <= want <= total count is required.
template <int NT>
__device__ __forceinline__ void find_digit_4096(const uint32_t* hist, uint32_t want,
                                                uint32_t* s_tmp, uint32_t& digit,
                                                uint32_t& above) {
    constexpr int PER = 4096 / NT;
    // thread t owns bins [4096 - PER*(t+1), 4096 - PER*t): thread 0 the top ones
    const int hi = 4096 - PER * threadIdx.x;
    uint32_t c[PER], tot = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) { c[j] = hist[hi - 1 - j]; tot += c[j]; }
    uint32_t total;
    uint32_t run = block_exclusive_sum<NT>(tot, s_tmp, total);
    // s_tmp reused as the broadcast slot
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (run < want && run + c[j] >= want) { s_tmp[NT / kWave + 1] = hi - 1 - j; s_tmp[NT / kWave + 2] = run; }
        run += c[j];
    }
    __syncthreads();
    digit = s_tmp[NT / kWave + 1];
    above = s_tmp[NT / kWave + 2];
    __syncthreads();
}

// Bitonic sort (ascending) of n32 = power-of-two int32 values in LDS.
template <int NT>
__device__ __forceinline__ void block_bitonic_sort(int32_t* s, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
                int ixj = i ^ j;
                if (ixj > i) {
                    int32_t a = s[i], b = s[ixj];
                    bool up = (i & k) == 0;
                    if ((a > b) == up) { s[i] = b; s[ixj] = a; }
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace csa2

namespace csa2 {

// E2M1 pair -> fp32: byte `SEL` of `w` holds channel 2k in its low nibble and
// channel 2k+1 in its high nibble.  Uses the gfx950 FP4 conversion with a
// unit scale (the E4M3 group scale is applied separately, so any scale value
// stays exact: a 2-bit by 4-bit significand product fits fp32).
template <int SEL>
__device__ __forceinline__ float2 fp4x2_to_f32(uint32_t w) {
    auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    return make_float2(v[0], v[1]);
}

// Same decode from the E2M1 definition (sign, 2-bit exponent with bias 1,
// 1-bit mantissa, subnormal 0.5 at exponent 0), without the hardware path.
__device__ __forceinline__ float e2m1_to_f32(uint32_t n) {
    const uint32_t m = n & 7u;
    const uint32_t bits = m >= 2 ? (m + 252u) << 22 : (m == 1 ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((n & 8u) << 28));
}

// Two E4M3FN bytes (bytes 0,1 of w when !HI, bytes 2,3 when HI) -> fp32 with
// the gfx950 OCP FP8 conversion.
template <bool HI>
__device__ __forceinline__ float2 fp8x2_to_f32(uint32_t w) {
    auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    return make_float2(v[0], v[1]);
}

}  // namespace csa2
