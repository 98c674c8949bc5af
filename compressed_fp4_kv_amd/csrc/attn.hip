// Sparse attention of CSA2 over the selected FP4 main-KV entries plus the
// FP8 sliding window, for decode and for prefill chunks (gfx950).
//
// Method (jaehun.me review of arXiv 2609.19969, sections "2) CSA2" and
// "3) FP4 main KV + SWA Bounded Replay"; ainewsway.com article): each layer
// attends with its own query over the Top-K main-KV entries (key = value =
// the E2M1 row times its E4M3 per-16-channel scales) and the last 128 tokens
// of its own FP8 window; one softmax covers both sets.
//
// Structure on the GPU.  With 64 heads sharing one 512-channel KV set per
// query, the two contractions (S = Q K^T over channels, O = P V over keys)
// are dense, so they run on the fp32 matrix cores
// (V_MFMA_F32_16X16X4_F32: exact fp32 products, fp32 accumulation).
//   - a workgroup owns one query (token), up to 64 heads (16 per wave) and a
//     range of 16-key tiles; splits of the key range across workgroups are
//     merged by k_attn_combine (log-sum-exp weights).
//   - per tile the workgroup dequantises 16 keys x 512 channels into LDS
//     twice: row-major K (A operand of S^T = K Q^T, one ds_read_b128 feeds 4
//     MFMAs) and transposed V (A operand of O^T = V^T P^T, likewise).
//   - each wave keeps its 16 heads' query slice (128 fp32 per lane) and the
//     16 x 512 output accumulator (128 fp32 per lane) in registers.  S^T comes
//     out of the MFMA with lane (g, h) holding keys 4g..4g+3 of head h, which
//     is exactly the B-operand layout the P V MFMA needs: P never leaves
//     registers.  Online softmax in base 2, one max/sum per head.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 512;
constexpr int kTK = 16;             // keys per tile
constexpr int kKStr = kD + 4;       // LDS row stride of the K tile (floats)
constexpr int kVStr = kTK + 4;      // LDS row stride of the transposed V tile
constexpr float kLn2 = 0.69314718055994530942f;

struct AttnArgs {
    const float* q;              // [rows_q, H, D]
    const uint8_t* kv_codes;     // [rows, D/2]
    const uint8_t* kv_scales;    // [rows, D/16]
    const int64_t* seq_row_off;  // decode: [B]; prefill: nullptr
    const int32_t* topk_idx;     // [rows_q, topk]
    const uint8_t* swa_k;        // decode: [B, W, D]; prefill: [Qn + W - 1, D]
    const uint8_t* swa_v;
    const int32_t* swa_len;      // decode: [B]; prefill: nullptr
    int topk, W, H;
    float scale_log2;            // softmax_scale * log2(e)
    int64_t p0;                  // prefill: position of query 0
    int prefill;
    int ntiles_main, ntiles, tiles_per_split, nsplit;
    float* out;                  // [rows_q, H, D]
    float* lse;                  // [rows_q, H] or nullptr
    float* part_o;               // [nsplit, rows_q, H, D] (nsplit > 1)
    float* part_ml;              // [nsplit, rows_q, H, 2]
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Raw bytes of one tile for one thread: ITEMS items of 4 keys x 8 channels.
// Main keys: k.x = 4 code bytes (8 channels), k.y = scale byte.  Window
// keys: k = 8 K bytes, v = 8 V bytes.
template <int ITEMS>
struct TileRaw {
    uint2 k[ITEMS][4];
    uint2 v[ITEMS][4];
    uint32_t ok[ITEMS];   // bit j: key 4*kq + j is real
};

// Global loads of tile t (issued early; consumed by store_tile).
template <int NT, int ITEMS>
__device__ __forceinline__ void fetch_tile(const AttnArgs& a, const int32_t* s_idx, int t0,
                                           int64_t row0, int wlo, int whi, int t,
                                           TileRaw<ITEMS>& r) {
    const bool main = t < a.ntiles_main;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = threadIdx.x + it * NT;
        const int c8 = item >> 2, kq = item & 3;
        r.ok[it] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = 4 * kq + j;
            r.k[it][j] = make_uint2(0, 0);
            r.v[it][j] = make_uint2(0, 0);
            if (main) {
                const int32_t idx = s_idx[kTK * (t - t0) + key];
                if (idx >= 0) {
                    const int64_t row = row0 + idx;
                    r.k[it][j].x = *reinterpret_cast<const uint32_t*>(a.kv_codes + row * (kD / 2) + 4 * c8);
                    r.k[it][j].y = a.kv_scales[row * (kD / 16) + (c8 >> 1)];
                    r.ok[it] |= 1u << j;
                }
            } else {
                const int w_ = kTK * (t - a.ntiles_main) + key;
                if (w_ >= wlo && w_ < whi) {
                    const size_t off = (size_t)w_ * kD + 8 * c8;
                    r.k[it][j] = *reinterpret_cast<const uint2*>(a.swa_k + off);
                    r.v[it][j] = *reinterpret_cast<const uint2*>(a.swa_v + off);
                    r.ok[it] |= 1u << j;
                }
            }
        }
    }
}

// Dequantises the fetched tile into sK (row-major K) and sVt (transposed V);
// sValid[k] = 1 for a real key, 0 for padding.
template <int NT, int ITEMS>
__device__ __forceinline__ void store_tile(bool main, const TileRaw<ITEMS>& r, float* sK,
                                           float* sVt, int* sValid) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int item = threadIdx.x + it * NT;
        const int c8 = item >> 2, kq = item & 3;
        float v[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float kk[8];
            if (main) {
                const uint32_t w = r.k[it][j].x;
                const float sc = e4m3_to_f32(r.k[it][j].y);
                const float2 p0 = fp4x2_to_f32<0>(w), p1 = fp4x2_to_f32<1>(w);
                const float2 p2 = fp4x2_to_f32<2>(w), p3 = fp4x2_to_f32<3>(w);
                v[j][0] = p0.x * sc; v[j][1] = p0.y * sc; v[j][2] = p1.x * sc; v[j][3] = p1.y * sc;
                v[j][4] = p2.x * sc; v[j][5] = p2.y * sc; v[j][6] = p3.x * sc; v[j][7] = p3.y * sc;
#pragma unroll
                for (int x = 0; x < 8; ++x) kk[x] = v[j][x];
            } else {
                const uint2 kb = r.k[it][j], vb = r.v[it][j];
                const float2 k0 = fp8x2_to_f32<false>(kb.x), k1 = fp8x2_to_f32<true>(kb.x);
                const float2 k2 = fp8x2_to_f32<false>(kb.y), k3 = fp8x2_to_f32<true>(kb.y);
                const float2 v0 = fp8x2_to_f32<false>(vb.x), v1 = fp8x2_to_f32<true>(vb.x);
                const float2 v2 = fp8x2_to_f32<false>(vb.y), v3 = fp8x2_to_f32<true>(vb.y);
                kk[0] = k0.x; kk[1] = k0.y; kk[2] = k1.x; kk[3] = k1.y;
                kk[4] = k2.x; kk[5] = k2.y; kk[6] = k3.x; kk[7] = k3.y;
                v[j][0] = v0.x; v[j][1] = v0.y; v[j][2] = v1.x; v[j][3] = v1.y;
                v[j][4] = v2.x; v[j][5] = v2.y; v[j][6] = v3.x; v[j][7] = v3.y;
            }
            float4* dk = reinterpret_cast<float4*>(sK + (4 * kq + j) * kKStr + 8 * c8);
            dk[0] = make_float4(kk[0], kk[1], kk[2], kk[3]);
            dk[1] = make_float4(kk[4], kk[5], kk[6], kk[7]);
        }
#pragma unroll
        for (int x = 0; x < 8; ++x)
            *reinterpret_cast<float4*>(sVt + (8 * c8 + x) * kVStr + 4 * kq) =
                make_float4(v[0][x], v[1][x], v[2][x], v[3][x]);
        if (c8 == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sValid[4 * kq + j] = (r.ok[it] >> j) & 1u;
        }
    }
}

// Rescale threshold (log2 units): the running maximum used for the
// exponentials is only moved when a new logit exceeds it by more than this,
// so p <= 2^8 and most tiles skip the rescale of the accumulators.
constexpr float kRescale = 8.f;

// One workgroup = 4 waves = up to 64 heads of one query; with fewer heads
// (H not a multiple of 64) the surplus waves only help load the tiles.
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
    constexpr int NT = 256;
    constexpr int ITEMS = 1;
    __shared__ __attribute__((aligned(16))) float sK[kTK * kKStr];
    __shared__ __attribute__((aligned(16))) float sVt[kD * kVStr];
    __shared__ int sValid[kTK];
    __shared__ int32_t s_idx[CSA2_MAX_TOPK];

    const int split = blockIdx.x;
    const int qi = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, hl = lane & 15;
    const int h0 = (blockIdx.y * 4 + wave) * 16;
    const bool active = h0 < a.H;          // wave-uniform
    const int h = active ? h0 + hl : hl;   // idle waves read head hl, write nothing

    int64_t row0 = 0;
    int wlo = 0, whi = 0;
    if (a.prefill) {
        const int64_t p = a.p0 + qi;
        wlo = (int)max((int64_t)0, (int64_t)(a.W - 1) - p);
        whi = a.W;
    } else {
        row0 = a.seq_row_off[qi];
        whi = min(a.swa_len[qi], a.W);
    }
    AttnArgs aa = a;
    if (a.prefill) {
        aa.swa_k = a.swa_k + (size_t)qi * kD;
        aa.swa_v = a.swa_v + (size_t)qi * kD;
    } else {
        aa.swa_k = a.swa_k + (size_t)qi * a.W * kD;
        aa.swa_v = a.swa_v + (size_t)qi * a.W * kD;
    }
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(a.ntiles, t0 + a.tiles_per_split);
    // this split's main-KV indices, staged once
    {
        const int nslot = kTK * (min(t1, a.ntiles_main) - t0);
        for (int i = threadIdx.x; i < nslot; i += NT) {
            const int slot = kTK * t0 + i;
            s_idx[i] = slot < a.topk ? a.topk_idx[(size_t)qi * a.topk + slot] : -1;
        }
    }

    // query slice: qreg[4u + i] = q[h][16u + 4g + i]
    float qreg[128];
    {
        const float4* qp = reinterpret_cast<const float4*>(a.q + ((size_t)qi * a.H + h) * kD);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            const float4 v = qp[4 * u + g];
            qreg[4 * u + 0] = v.x; qreg[4 * u + 1] = v.y; qreg[4 * u + 2] = v.z; qreg[4 * u + 3] = v.w;
        }
    }
    f32x4 o[32];
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    __syncthreads();
    TileRaw<ITEMS> raw;
    if (t0 < t1) fetch_tile<NT, ITEMS>(aa, s_idx, t0, row0, wlo, whi, t0, raw);
    for (int t = t0; t < t1; ++t) {
        __syncthreads();   // previous tile's LDS reads are done
        store_tile<NT, ITEMS>(t < a.ntiles_main, raw, sK, sVt, sValid);
        __syncthreads();
        // next tile's global loads overlap this tile's matrix work
        if (t + 1 < t1) fetch_tile<NT, ITEMS>(aa, s_idx, t0, row0, wlo, whi, t + 1, raw);

        if (!active) continue;
        // S^T[key 4g+i][head hl] over all channels.  Eight independent
        // accumulation chains (channel block u mod 8) summed as a tree keep
        // the fp32 rounding error of the 512-term dot well below the error
        // budget of the outputs (one sequential chain does not).
        f32x4 sc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) sc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float* kr = sK + hl * kKStr + 4 * g;
        for (int uo = 0; uo < 32; uo += 8) {
#pragma unroll
            for (int ui = 0; ui < 8; ++ui) {
                const int u = uo + ui;
                const float4 kv = *reinterpret_cast<const float4*>(kr + 16 * u);
                sc[ui] = mfma4(kv.x, qreg[4 * u + 0], sc[ui]);
                sc[ui] = mfma4(kv.y, qreg[4 * u + 1], sc[ui]);
                sc[ui] = mfma4(kv.z, qreg[4 * u + 2], sc[ui]);
                sc[ui] = mfma4(kv.w, qreg[4 * u + 3], sc[ui]);
            }
        }
        const f32x4 s = ((sc[0] + sc[1]) + (sc[2] + sc[3])) + ((sc[4] + sc[5]) + (sc[6] + sc[7]));
        float z[4], p[4];
        float tm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = sValid[4 * g + i] ? s[i] * a.scale_log2 : -INFINITY;
            tm = fmaxf(tm, z[i]);
        }
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        const bool bump = tm > m + kRescale;   // true for any finite tm while m = -inf
        if (__ballot(bump)) {
            const float mn = bump ? tm : m;
            const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int cb = 0; cb < 32; ++cb) o[cb] = o[cb] * alpha;
            m = mn;
        }
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m);
            ps += p[i];
        }
        l += ps;
        // O^T[channel 16cb + 4g + r][head hl] += sum_keys V^T P^T
        const float* vr = sVt + hl * kVStr + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) {
            f32x4 acc = o[cb];
            const float4 vv = *reinterpret_cast<const float4*>(vr + 16 * cb * kVStr);
            acc = mfma4(vv.x, p[0], acc);
            acc = mfma4(vv.y, p[1], acc);
            acc = mfma4(vv.z, p[2], acc);
            acc = mfma4(vv.w, p[3], acc);
            o[cb] = acc;
        }
    }
    if (!active) return;
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const size_t orow = ((size_t)qi * a.H + h) * kD;
    if (a.nsplit == 1) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) {
            const f32x4 v = o[cb] * inv;
            *reinterpret_cast<float4*>(a.out + orow + 16 * cb + 4 * g) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
        if (a.lse && g == 0)
            a.lse[(size_t)qi * a.H + h] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    } else {
        const size_t rows_q = gridDim.z;
        float* po = a.part_o + ((size_t)split * rows_q * a.H) * kD + orow;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb)
            *reinterpret_cast<float4*>(po + 16 * cb + 4 * g) =
                make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
        if (g == 0) {
            float* pm = a.part_ml + (((size_t)split * rows_q + qi) * a.H + h) * 2;
            pm[0] = m;
            pm[1] = lt;
        }
    }
}

// Merges the key-range splits of one (query, head): weights 2^(m_s - M).
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int nsplit, int rows_q, int H,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse) {
    const int qh = blockIdx.x;  // qi * H + h
    const size_t stride_o = (size_t)rows_q * H * kD;
    const size_t stride_ml = (size_t)rows_q * H * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[s * stride_ml + (size_t)qh * 2]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nsplit; ++s) {
        const float ms = part_ml[s * stride_ml + (size_t)qh * 2];
        const float ls = part_ml[s * stride_ml + (size_t)qh * 2 + 1];
        if (ms == -INFINITY || ls == 0.f) continue;
        const float w = exp2f(ms - M);
        L += w * ls;
        const float4 v = reinterpret_cast<const float4*>(part_o + s * stride_o + (size_t)qh * kD)[threadIdx.x];
        acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    reinterpret_cast<float4*>(out + (size_t)qh * kD)[threadIdx.x] =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (lse && threadIdx.x == 0) lse[qh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// Test hook: decodes every FP4 byte and FP8 byte with the helpers above.
__global__ void k_decode_tables(float* fp4_hw, float* fp4_ref, float* fp8_hw, float* fp8_ref) {
    const uint32_t b = threadIdx.x;  // 0..255
    const uint32_t w = b | (b << 8) | (b << 16) | (b << 24);
    const float2 p = fp4x2_to_f32<2>(w);
    fp4_hw[2 * b] = p.x;
    fp4_hw[2 * b + 1] = p.y;
    fp4_ref[2 * b] = e2m1_to_f32(b & 15u);
    fp4_ref[2 * b + 1] = e2m1_to_f32(b >> 4);
    const float2 f = fp8x2_to_f32<true>(w);
    fp8_hw[b] = f.y;
    fp8_ref[b] = e4m3_to_f32(b);
}

struct AttnPlan {
    int hgroups, ntiles_main, ntiles, nsplit, tps;
    size_t ws_bytes;
};

int plan_attn(int rows_q, int H, int D, int topk, int W, bool allow_split, AttnPlan* p) {
    if (rows_q < 0 || H <= 0 || D <= 0 || topk < 0 || W < 0) return CSA2_ERR_SHAPE;
    if (D != kD || H % 16 != 0 || topk > CSA2_MAX_TOPK || W > 1024 || rows_q > 65535)
        return CSA2_ERR_UNSUPPORTED;
    p->hgroups = (H + 63) / 64;
    p->ntiles_main = (topk + kTK - 1) / kTK;
    p->ntiles = p->ntiles_main + (W + kTK - 1) / kTK;
    int nsplit = 1;
    if (allow_split && p->ntiles > 1) {
        const long wgs = (long)rows_q * p->hgroups;
        const long target = 256;
        if (wgs < target) nsplit = (int)((target + wgs - 1) / wgs);
        if (nsplit > p->ntiles) nsplit = p->ntiles;
    }
    p->tps = p->ntiles > 0 ? (p->ntiles + nsplit - 1) / nsplit : 0;
    if (p->tps > 0) nsplit = (p->ntiles + p->tps - 1) / p->tps;
    p->nsplit = nsplit;
    Carver c(nullptr);
    if (nsplit > 1) {
        c.take<float>((size_t)nsplit * rows_q * H * kD);
        c.take<float>((size_t)nsplit * rows_q * H * 2);
    }
    p->ws_bytes = c.bytes();
    return CSA2_OK;
}

int launch_attn(AttnArgs a, const AttnPlan& pl, int rows_q, void* ws, hipStream_t s) {
    a.ntiles_main = pl.ntiles_main;
    a.ntiles = pl.ntiles;
    a.tiles_per_split = pl.tps;
    a.nsplit = pl.nsplit;
    if (pl.nsplit > 1) {
        Carver c(ws);
        a.part_o = c.take<float>((size_t)pl.nsplit * rows_q * a.H * kD);
        a.part_ml = c.take<float>((size_t)pl.nsplit * rows_q * a.H * 2);
    }
    dim3 grid(pl.nsplit, pl.hgroups, rows_q);
    int st = CSA2_LAUNCH("attn", k_attn, grid, dim3(256), s, a);
    if (st || pl.nsplit == 1) return st;
    return CSA2_LAUNCH("attn_combine", k_attn_combine, dim3(rows_q * a.H), dim3(128), s,
                       a.part_o, a.part_ml, pl.nsplit, rows_q, a.H, a.out, a.lse);
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_decode_workspace_bytes(int32_t B, int32_t H, int32_t D, int32_t topk,
                                              int32_t W) {
    AttnPlan p;
    if (plan_attn(B, H, D, topk, W, true, &p) != CSA2_OK) return 0;
    return p.ws_bytes;
}

extern "C" int csa2_sparse_attn_decode(const float* q, const uint8_t* kv_codes,
                                       const uint8_t* kv_scales, const int64_t* seq_row_off,
                                       const int32_t* topk_idx, int32_t topk,
                                       const uint8_t* swa_k, const uint8_t* swa_v,
                                       const int32_t* swa_len, int32_t W, int32_t B, int32_t H,
                                       int32_t D, float softmax_scale, float* out, float* lse,
                                       void* ws, size_t ws_bytes, void* stream) {
    AttnPlan pl;
    int st = plan_attn(B, H, D, topk, W, true, &pl);
    if (st) return st;
    if (B == 0) return CSA2_OK;
    if (!q || !out || !swa_len) return CSA2_ERR_NULL;
    if (topk > 0 && (!kv_codes || !kv_scales || !seq_row_off || !topk_idx)) return CSA2_ERR_NULL;
    if (W > 0 && (!swa_k || !swa_v)) return CSA2_ERR_NULL;
    if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)swa_k | (uintptr_t)swa_v) & 15)
        return CSA2_ERR_UNSUPPORTED;
    if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) return CSA2_ERR_WORKSPACE;
    AttnArgs a{};
    a.q = q; a.kv_codes = kv_codes; a.kv_scales = kv_scales; a.seq_row_off = seq_row_off;
    a.topk_idx = topk_idx; a.swa_k = swa_k; a.swa_v = swa_v; a.swa_len = swa_len;
    a.topk = topk; a.W = W; a.H = H;
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    a.prefill = 0;
    a.out = out; a.lse = lse;
    return launch_attn(a, pl, B, ws, (hipStream_t)stream);
}

extern "C" size_t csa2_prefill_workspace_bytes(int32_t Qn, int32_t H, int32_t D, int32_t topk,
                                               int32_t W) {
    AttnPlan p;
    if (plan_attn(Qn, H, D, topk, W, true, &p) != CSA2_OK) return 0;
    return p.ws_bytes;
}

extern "C" int csa2_sparse_attn_prefill_chunk(const float* q, int64_t p0, const uint8_t* kv_codes,
                                              const uint8_t* kv_scales, const int32_t* topk_idx,
                                              int32_t topk, const uint8_t* swa_k,
                                              const uint8_t* swa_v, int32_t W, int32_t Qn,
                                              int32_t H, int32_t D, float softmax_scale,
                                              float* out, float* lse, void* ws, size_t ws_bytes,
                                              void* stream) {
    AttnPlan pl;
    int st = plan_attn(Qn, H, D, topk, W, true, &pl);
    if (st) return st;
    if (p0 < 0) return CSA2_ERR_SHAPE;
    if (Qn == 0) return CSA2_OK;
    if (!q || !out) return CSA2_ERR_NULL;
    if (topk > 0 && (!kv_codes || !kv_scales || !topk_idx)) return CSA2_ERR_NULL;
    if (W > 0 && (!swa_k || !swa_v)) return CSA2_ERR_NULL;
    if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)swa_k | (uintptr_t)swa_v) & 15)
        return CSA2_ERR_UNSUPPORTED;
    if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) return CSA2_ERR_WORKSPACE;
    AttnArgs a{};
    a.q = q; a.kv_codes = kv_codes; a.kv_scales = kv_scales; a.seq_row_off = nullptr;
    a.topk_idx = topk_idx; a.swa_k = swa_k; a.swa_v = swa_v; a.swa_len = nullptr;
    a.topk = topk; a.W = W; a.H = H;
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    a.p0 = p0;
    a.prefill = 1;
    a.out = out; a.lse = lse;
    return launch_attn(a, pl, Qn, ws, (hipStream_t)stream);
}

extern "C" int csa2_debug_decode_tables(float* fp4_hw, float* fp4_ref, float* fp8_hw,
                                        float* fp8_ref, void* stream) {
    if (!fp4_hw || !fp4_ref || !fp8_hw || !fp8_ref) return CSA2_ERR_NULL;
    return CSA2_LAUNCH("decode_tables", k_decode_tables, dim3(1), dim3(256),
                       (hipStream_t)stream, fp4_hw, fp4_ref, fp8_hw, fp8_ref);
}
