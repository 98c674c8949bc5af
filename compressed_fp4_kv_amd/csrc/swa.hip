// FP8 window ring append (gfx950): a decode step's K and V rows, fp32 ->
// E4M3FN, into each sequence's W-slot ring, the window the attention kernels
// read.
//
// Method (jaehun.me review, section "3) FP4 main KV + SWA Bounded Replay";
// ainewsway.com article): the last 128 tokens are kept in FP8 beside the
// sparse main KV.  The pages give no rounding rule; this writer rounds to the
// nearest E4M3FN value (ties to even), keeps the sign of zero and saturates
// magnitudes beyond 448 instead of producing NaN.
#include <limits.h>

#include "common.hpp"
#include "internal.hpp"

namespace csa2 {
namespace {

// Token b's K and V rows, fp32 -> E4M3FN (round to nearest even, magnitudes
// beyond 448 saturated to 448, sign of zero kept), into slot pos[b] mod W of
// sequence b's ring.  One lane per 8 channels of both rows: two float4 loads
// per row, one 8-byte store per ring.  A negative position writes nothing.
__device__ __forceinline__ uint32_t cvt_fp8x4(float4 v) {
    const auto sat = [](float f) { return fminf(fmaxf(f, -448.f), 448.f); };
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v.x), sat(v.y), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(sat(v.z), sat(v.w), w, true);
}

__global__ __launch_bounds__(256) void k_swa_append(const float* __restrict__ k_new,
                                                    const float* __restrict__ v_new,
                                                    const int64_t* __restrict__ pos, int B, int D8,
                                                    int W, uint8_t* __restrict__ swa_k,
                                                    uint8_t* __restrict__ swa_v) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)B * D8) return;
    const int b = (int)(t / D8), c8 = (int)(t % D8);
    const int64_t p = pos[b];
    if (p < 0) return;
    const int64_t src = (int64_t)b * D8 * 2 + 2 * c8;                  // float4 index
    const int64_t dst = ((int64_t)b * W + p % W) * D8 + c8;            // 8-byte index
    const float4* k4 = reinterpret_cast<const float4*>(k_new);
    const float4* v4 = reinterpret_cast<const float4*>(v_new);
    const float4 k0 = k4[src], k1 = k4[src + 1], v0 = v4[src], v1 = v4[src + 1];
    reinterpret_cast<uint2*>(swa_k)[dst] = make_uint2(cvt_fp8x4(k0), cvt_fp8x4(k1));
    reinterpret_cast<uint2*>(swa_v)[dst] = make_uint2(cvt_fp8x4(v0), cvt_fp8x4(v1));
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" int csa2_swa_append(const float* k_new, const float* v_new, const int64_t* pos,
                               int32_t B, int32_t D, int32_t W, uint8_t* swa_k, uint8_t* swa_v,
                               void* stream) {
    if (B < 0 || D <= 0 || W <= 0) return CSA2_ERR_SHAPE;
    if (D % 8 != 0) return CSA2_ERR_UNSUPPORTED;
    if (B == 0) return CSA2_OK;
    if (!k_new || !v_new || !pos || !swa_k || !swa_v) return CSA2_ERR_NULL;
    if (((uintptr_t)k_new & 15) || ((uintptr_t)v_new & 15) || ((uintptr_t)swa_k & 7) ||
        ((uintptr_t)swa_v & 7))
        return CSA2_ERR_UNSUPPORTED;
    const int64_t n = (int64_t)B * (D / 8);
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT_MAX) return CSA2_ERR_UNSUPPORTED;
    return CSA2_LAUNCH("swa_append", k_swa_append, dim3((unsigned)blocks), dim3(256),
                       (hipStream_t)stream, k_new, v_new, pos, B, D / 8, W, swa_k, swa_v);
}
