// FP4 main-KV writer (gfx950): fp32 rows -> E2M1 codes with one E4M3 scale
// per 16 channels, the format the attention kernels gather.
//
// Method (jaehun.me review, section "3) FP4 main KV + SWA Bounded Replay";
// ainewsway.com article): main KV is stored as E2M1 values with one E4M3
// scale per 16 channels.  The pages fix the format, not the rounding; this
// writer takes the smallest E4M3 scale s with 6 s >= the group's largest
// magnitude (448, and saturation at 6, beyond 6 x 448; byte 0 for an all-zero
// group) and rounds |x| / s to the nearest E2M1 magnitude, ties to the even
// code, with the sign of x and no negative zero.  The result is the
// definition's, bit for bit: the scale comes from exact compares against
// 6 x e4m3(b), and each code from the hardware's rounding of x / s bracketed
// tightly from both sides, or, where the bracket straddles a midpoint between
// E2M1 values, from exact compares of |x| against midpoint x s (products of
// at most 7 significant bits, exact in fp32).
#include <limits.h>

#include "common.hpp"
#include "internal.hpp"

namespace csa2 {
namespace {

// Scale byte (and its value) of a group whose largest magnitude is am: the
// smallest E4M3 byte b in [1, 126] with 6 e4m3(b) >= am, 126 when there is
// none, 0 when am == 0.
//   t is am / 6 rounded up by more than its rounding error (1/6 rounded up,
//   then two ulps), and below am / 6 (1 + 2^-21); E4M3 values lie at least
//   1/16 apart relatively, so the E4M3 ceiling of t, read off its bits, is
//   the wanted byte or the one above it, and one exact compare decides.
//   For am == 0 that compare picks byte 0.
__device__ __forceinline__ uint32_t fp4_scale(float am, float& s) {
    const float t = __uint_as_float(__float_as_uint(am * (1.f / 6.f)) + 2u);
    const uint32_t u = (__float_as_uint(t) + 0xFFFFFu) & ~0xFFFFFu;   // ceil to 3 bits
    const uint32_t e = min(u >> 23, 136u);                           // >= 2^16: saturates
    const uint32_t bn = ((e - 120u) << 3) | ((u >> 20) & 7u);        // normal scales
    const uint32_t bs = (uint32_t)ceilf(t * 512.f);                  // m 2^-9 (8 -> 2^-6)
    const uint32_t b = min(max(t < 0x1p-6f ? bs : bn, 1u), 126u);
    // values of bytes b - 1 and b (gfx950 OCP E4M3 conversion, exact)
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)((b - 1u) | (b << 8)), false);
    const bool lower = 6.f * d[0] >= am;
    s = lower ? d[0] : d[1];
    return lower ? b - 1u : b;
}

// The float just below p > 0 ("a >= p" is "a > below(p)"); NaN for p == 0.
__device__ __forceinline__ float below(float p) { return __uint_as_float(__float_as_uint(p) - 1u); }

// max over the four lanes of a quad (DPP quad permutes)
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
}

// E2M1 codes of four values by counting the midpoints between E2M1 values
// that |x| / s lies above; at a midpoint a value goes to the even code (the
// boundaries below 1, 2 and 4 are taken inclusively).  All products are exact
// in fp32.  For s = 0 every bound is 0 or NaN and every code 0.  x < -t0 is
// "negative with a non-zero magnitude", so no code is a negative zero.
__device__ __forceinline__ uint32_t fp4_codes_exact(float x0, float x1, float x2,
                                                    float x3, float s) {
    const float t0 = 0.25f * s, t1 = below(0.75f * s), t2 = 1.25f * s, t3 = below(1.75f * s),
                t4 = 2.5f * s, t5 = below(3.5f * s), t6 = 5.f * s;
    auto enc = [&](float xv) -> uint32_t {
        const float a = fabsf(xv);
        const uint32_t mag = (uint32_t)(a > t0) + (uint32_t)(a > t1) + (uint32_t)(a > t2) +
                             (uint32_t)(a > t3) + (uint32_t)(a > t4) + (uint32_t)(a > t5) +
                             (uint32_t)(a > t6);
        return mag | (xv < -t0 ? 8u : 0u);
    };
    return enc(x0) | (enc(x1) << 4) | (enc(x2) << 8) | (enc(x3) << 12);
}

// gfx950 conversion of two fp32 values to E2M1 (round to nearest, ties to
// even, saturating at 6; unit scale), first value in the low nibble
__device__ __forceinline__ uint32_t cvt_fp4x2(float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Codes and scale byte of the four channels of float4 i (one lane of the
// quad that holds its 16-channel group).
//   x / s lies between x * ilo and x * ihi, with ilo and ihi the reciprocal of
//   s moved down and up by 2^-20, far more than the rounding of the
//   reciprocal and of the products (a few 2^-24).  Rounding to nearest is
//   monotone, so when both bounds round to the same code that is the code of
//   x / s; when they differ x / s is within 2^-19 of a midpoint, possibly on
//   it, and the lane takes the exact count instead.
__device__ __forceinline__ void quantize_quad(f32x4 v, int64_t i, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales) {
    const float am = quad_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    float s;
    const uint32_t sb = fp4_scale(am, s);
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
    const float ilo = inv * (1.f - 0x1p-20f), ihi = inv * (1.f + 0x1p-20f);
    const uint32_t lo = cvt_fp4x2(v.x * ilo, v.y * ilo) | (cvt_fp4x2(v.z * ilo, v.w * ilo) << 8);
    const uint32_t hi = cvt_fp4x2(v.x * ihi, v.y * ihi) | (cvt_fp4x2(v.z * ihi, v.w * ihi) << 8);
    uint32_t packed = lo == hi ? lo : fp4_codes_exact(v.x, v.y, v.z, v.w, s);
    // a zero magnitude keeps no sign
    const uint32_t mag = packed & 0x7777u;
    packed = mag | (packed & (mag + 0x7777u) & 0x8888u);
    reinterpret_cast<uint16_t*>(codes)[i] = (uint16_t)packed;
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)sb;
}

// Four lanes (one quad) per 16-channel group, one float4 per lane and load,
// so that a wave reads 1 KB of consecutive channels per load and writes 128 B
// of codes.  Rows are contiguous, so float4 i of the whole array holds
// channels 4i .. 4i+3 of its row, their codes are bytes 2i, 2i+1 and their
// group is i / 4.  A block takes 2 x 256 consecutive float4s, both loads
// issued before either is converted (one load per lane left HBM idle).
constexpr int kQuantThreads = 256;
constexpr int kQuantPerLane = 2;

__global__ __launch_bounds__(kQuantThreads) void k_fp4_quantize(const float* __restrict__ x,
                                                                int64_t n4,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
    const int64_t base = (int64_t)blockIdx.x * (kQuantThreads * kQuantPerLane) + threadIdx.x;
    f32x4 v[kQuantPerLane];
    // n4 and every offset are multiples of 4: a quad is all in range or all out
#pragma unroll
    for (int p = 0; p < kQuantPerLane; ++p) {
        const int64_t i = base + (int64_t)p * kQuantThreads;
        // streamed once: read non-temporally
        if (i < n4) v[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + i);
    }
#pragma unroll
    for (int p = 0; p < kQuantPerLane; ++p) {
        const int64_t i = base + (int64_t)p * kQuantThreads;
        if (i < n4) quantize_quad(v[p], i, codes, scales);
    }
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" int csa2_kv_quantize_fp4(const float* x, int64_t rows, int32_t D, uint8_t* codes,
                                    uint8_t* scales, void* stream) {
    if (rows < 0 || D <= 0) return CSA2_ERR_SHAPE;
    if (D % 16 != 0) return CSA2_ERR_UNSUPPORTED;
    if (rows == 0) return CSA2_OK;
    if (!x || !codes || !scales) return CSA2_ERR_NULL;
    if (((uintptr_t)x & 15) || ((uintptr_t)codes & 1)) return CSA2_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / D) return CSA2_ERR_SHAPE;
    const int64_t n4 = rows * (int64_t)D / 4;
    const int64_t per_block = kQuantThreads * kQuantPerLane;
    const int64_t blocks = (n4 + per_block - 1) / per_block;
    if (blocks > INT_MAX) return CSA2_ERR_UNSUPPORTED;
    return CSA2_LAUNCH("kv_quantize_fp4", k_fp4_quantize, dim3((unsigned)blocks), dim3(kQuantThreads),
                       (hipStream_t)stream, x, n4, codes, scales);
}
