// Sparse attention of CSA2 over the selected FP4 main-KV entries plus the
// FP8 sliding window, for decode and for prefill chunks (gfx950).
//
// Method (jaehun.me review of arXiv 2609.19969, sections "2) CSA2" and
// "3) FP4 main KV + SWA Bounded Replay"; ainewsway.com article): each layer
// attends with its own query over the Top-K main-KV entries (key = value =
// the E2M1 row times its E4M3 per-16-channel scales) and the last 128 tokens
// of its own FP8 window; one softmax covers both sets.
//
// Structure on the GPU.  64 heads share one 512-channel key set per query,
// so S = Q K^T (over channels) and O = P V (over keys) are dense
// contractions; they run on the fp16 matrix cores (V_MFMA_F32_32X32X16_F16)
// at close to fp32 accuracy:
//   - dequantised K and V are exact in fp16 (an E2M1 value times an E4M3
//     scale has at most 6 significant bits and lies in [2^-10, 2688]; E4M3
//     itself has 4 bits and lies in [2^-9, 448]);
//   - the fp32 query and the fp32 probabilities are split into two fp16
//     parts (x = x1 + x2, relative residual about 2^-22), each multiplied
//     exactly and accumulated in fp32.  The query of each head is first
//     scaled by a power of two that puts its largest element in
//     [2^13, 2^14), so both parts stay in fp16's normal range; the logits
//     are scaled back exactly, together with the softmax scale.
// Work split: a workgroup (4 waves, one per SIMD) owns one query token, 32
// heads and a range of 32-key tiles; wave w handles channels 128*w.. of the
// 32 heads.  Each wave gathers and dequantises only its own channel quarter
// of a tile (lane = key of the tile and a 64-channel half of the quarter):
// the fp16 key fragments feed S^T = K Q^T straight from registers as its A
// operand, and are also written to the wave's private quarter tile in LDS,
// row-major [key][channel], from which the gfx950 transposed LDS read
// (ds_read_b64_tr_b16) forms the A operand of O^T = V^T P^T.  The four
// channel quarters add their partial logits through LDS in a fixed order,
// each wave runs the softmax of 8 of the 32 keys, and every wave
// accumulates its quarter of the output from all 32 probabilities: three
// block barriers per tile.  The next tile's bytes are gathered into
// registers while the current one is processed.  A wave needs 256 registers
// per lane (accumulators, the two-part query slice, a tile's gathered bytes
// and key fragments), so a CU holds two such workgroups; each runs its tile
// loop on its own, and one's matrix-core chains overlap the other's softmax,
// dequantisation and barriers.  Key-range splits across workgroups are
// merged by k_attn_combine.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kD = 512;
constexpr int kTK = 32;             // keys per tile

// A quarter tile's rows (256 B, 16 chunks of 8 fp16) are not padded;
// instead chunk ch of row `row` is stored at chunk ch ^ tile_swz(row) of
// that row.  The swizzle keeps both of the tile's LDS access patterns free
// of bank conflicts whether the LDS serves 128 or 256 bytes a cycle: the
// fragment writes (8 or 16 consecutive rows, one chunk each) and the
// transposed V reads (4 consecutive rows, 2 or 4 chunks each).  Its high
// part is row & 3 and its low part swz_lo(row).
__device__ __forceinline__ int swz_lo(int row) {
    return (row & 3) ^ ((row >> 2) & 1) ^ (((row >> 3) & 1) << 1);
}
__device__ __forceinline__ int tile_swz(int row) { return 4 * (row & 3) + swz_lo(row); }
constexpr float kLn2 = 0.69314718055994530942f;

constexpr int kMaxLayers = 8;   // layers of one decode call (a layer group)

struct AttnArgs {
    const float* q[kMaxLayers];  // per layer: [rows_q, H, D]
    const uint8_t* kv_codes;     // [rows, D/2]
    const uint8_t* kv_scales;    // [rows, D/16]
    const int64_t* seq_row_off;  // decode: [B]; prefill: nullptr
    const int32_t* topk_idx;     // [rows_q, topk]
    const uint8_t* swa_k[kMaxLayers];   // per layer; decode: [B, W, D]; prefill: [Qn + W - 1, D]
    const uint8_t* swa_v[kMaxLayers];
    const int32_t* swa_len;      // decode: [B]; prefill: nullptr
    int topk, W, H;
    float scale_log2;            // softmax_scale * log2(e)
    int64_t p0;                  // prefill: position of query 0
    int prefill;
    int ntiles_main, ntiles, tiles_per_split, nsplit;   // split s: tiles [s tps, (s+1) tps)
    float* out[kMaxLayers];      // per layer: [rows_q, H, D]
    float* lse[kMaxLayers];      // per layer: [rows_q, H] or nullptr
    int rows_q, nlayers;         // the grid's z covers rows_q x nlayers (layer-major)
    float* part_o;               // [nsplit, nlayers * rows_q, H, D] (nsplit > 1)
    float* part_ml;              // [nsplit, nlayers * rows_q, H, 2]
};

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// Two fp32 values -> one dword of two fp16 (element a in the low half).
__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b) {
    const f16x2v r = __builtin_convertvector((f32x2v){a, b}, f16x2v);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float2 f16pk_to_f32(uint32_t p) {
    const f32x2v r = __builtin_convertvector(__builtin_bit_cast(f16x2v, p), f32x2v);
    return make_float2(r[0], r[1]);
}

// Pair (a, b) -> two packed fp16 pairs with a == p0.lo + p1.lo and
// b == p0.hi + p1.hi up to the rounding of the (exact) residual to fp16.
__device__ __forceinline__ void split2_pk(float a, float b, uint32_t& p0, uint32_t& p1) {
    p0 = cvt_pk_f16(a, b);
    const float2 h = f16pk_to_f32(p0);
    p1 = cvt_pk_f16(a - h.x, b - h.y);
}

__device__ __forceinline__ f16x8 as_f16x8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const uint32_t w[4] = {w0, w1, w2, w3};
    return __builtin_bit_cast(f16x8, w);
}

constexpr int kAttnThreads = 256;   // 4 waves
constexpr int kHeadsWG = 32;        // heads per workgroup
constexpr int kXcds = 8;            // XCDs of an MI355X (L2 domains)

constexpr int kQStr = 128;   // row stride (fp16 elements) of a wave's quarter tile: 256 B

// Main-KV bytes of one lane for a tile: its key (l32 of the tile) and its
// 64 channels 128 wave + 64 hh .. +64: 32 bytes of E2M1 codes (two 16-byte
// loads) and the 4 E4M3 scales of those channels (one 4-byte load).
struct RawQ {
    uint4 code[2];    // byte b holds channels 2b, 2b+1 of the 64
    uint32_t scale;   // byte g: scale of channels 16 g .. 16 g + 15 of the 64
};
// Window bytes of one lane for a tile: 64 E4M3 bytes of K (or of V) of its
// key row, the same 64 channels.
struct RawWQ {
    uint4 b[4];
};

// Byte range of the main-KV buffer resources: a sequence's rows are read at
// offsets below 2^31 (fewer than 2^23 entries per sequence); a larger offset
// is outside the resource and reads 0 without touching memory.
constexpr uint32_t kKvRange = 0x80000000u;
constexpr int kBufFlags = 0x00020000;   // raw 32-bit buffer (gfx9 family)

// Gather of a lane's main-KV bytes (issued early; consumed by dequant_q)
// through buffer resources based at the sequence's first row, with no
// branch and no select: the byte offset of a padding key (index -1, or any
// index in [-2^23, 0)) wraps to 2^32 minus at most 2^31 and is outside the
// range, so its loads read 0; a more negative index reads some row of the
// sequence and is masked like any padding key.
__device__ __forceinline__ void fetch_q(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                        int32_t idx, int wave, int hh, RawQ& r) {
    const uint32_t oc = (uint32_t)idx * (kD / 2) + 64 * wave + 32 * hh;
    r.code[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 0));
    r.code[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc + 16, 0, 0));
    r.scale = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)idx * (kD / 16) + 8 * wave + 4 * hh,
                                                   0, 0);
}

// Gather of a lane's window bytes of tile tw (row 32 tw + l32) from sw; a
// row past the window reads its last row instead (and is masked).
__device__ __forceinline__ void fetch_wq(const uint8_t* sw, int W, int tw, int wave, int hh,
                                         RawWQ& r) {
    const int row = min(kTK * tw + (int)(threadIdx.x & 31), W - 1);
    const uint8_t* p = sw + (size_t)row * kD + 128 * wave + 64 * hh;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.b[i] = *reinterpret_cast<const uint4*>(p + 16 * i);
}

// Writes fragment s of a lane's key (channels 8 s .. +8 of its 64) into its
// row of a wave's quarter tile: chunk 8 hh + s of row l32, swizzled.
__device__ __forceinline__ void put_q1(const f16x8& f, int s, uint16_t* vt) {
    const int l32 = threadIdx.x & 31, hh = (threadIdx.x >> 5) & 1;
    *reinterpret_cast<f16x8*>(vt + l32 * kQStr + 8 * ((8 * hh + s) ^ tile_swz(l32))) = f;
}
__device__ __forceinline__ void put_q(const f16x8 (&kf)[8], uint16_t* vt) {
#pragma unroll
    for (int s = 0; s < 8; ++s) put_q1(kf[s], s, vt);
}

// Eight E4M3 bytes as four fp16 pairs (exact), ANDed with `keep` (all ones
// or zero).
__device__ __forceinline__ void dequant_fp8x8(uint2 w, uint32_t keep, uint32_t (&o)[4]) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false)) & keep;
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true)) & keep;
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false)) & keep;
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true)) & keep;
}

// A lane's main-KV bytes as its 8 key fragments (fp16; K = V): fragment s
// is code word s (byte x holds channels 2x, 2x+1, low nibble first) times
// the E4M3 scale of its 16-channel group (scale byte s / 2).  Exact: the
// gfx950 FP4 -> fp16 conversion is exact, the four scale bytes become fp16
// in two packed conversions, exactly (4 significant bits, |s| in
// [2^-9, 448]), and so is each product (at most 6 significant bits,
// magnitude in [2^-10, 2688]).  A padding key's bytes were read as 0
// (outside the buffer range), so its fragments are 0.
__device__ __forceinline__ void dequant_q(const RawQ& r, f16x8 (&kf)[8]) {
    const uint32_t w[8] = {r.code[0].x, r.code[0].y, r.code[0].z, r.code[0].w,
                           r.code[1].x, r.code[1].y, r.code[1].z, r.code[1].w};
    const f16x2v sc01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.scale, 1.0f, false);
    const f16x2v sc23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.scale, 1.0f, true);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int g = s >> 1;   // scale group of fragment s
        const _Float16 sg = g == 0 ? sc01[0] : g == 1 ? sc01[1] : g == 2 ? sc23[0] : sc23[1];
        const f16x2v sc = {sg, sg};
        const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 0) * sc);
        const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 1) * sc);
        const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 2) * sc);
        const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[s], 1.0f, 3) * sc);
        kf[s] = as_f16x8(o0, o1, o2, o3);
    }
}

// Fragment s (channels 8 s .. +8 of the lane's 64) of a lane's window bytes
// (E4M3) in fp16; a row outside the window becomes 0 (it is real memory
// that may hold anything): keep is all ones or zero.
__device__ __forceinline__ f16x8 dequant_wq(const RawWQ& r, uint32_t keep, int s) {
    const uint4 b = r.b[s >> 1];
    const uint2 w = (s & 1) ? make_uint2(b.z, b.w) : make_uint2(b.x, b.y);
    uint32_t o[4];
    dequant_fp8x8(w, keep, o);
    return as_f16x8(o[0], o[1], o[2], o[3]);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// gfx950 transposed LDS read: within each 16-lane group, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 of the group.
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16 __attribute__((address_space(3)))*)(p));
}

// Matrix-core chains (the S^T and the P V products of a tile) run at raised
// wave priority: the two workgroups of a CU share each SIMD, and while one
// wave's products issue, the other wave's softmax and dequantisation fill
// the gaps (measured: prefill attention 959-965 -> 943-945 us per layer,
// decode group 90-91 -> 88.5 us).
// Rescale threshold (log2 units): the running maximum used for the
// exponentials is only moved when a new logit exceeds it by more than this,
// so p <= 2^8 and most tiles skip the rescale of the accumulators.
constexpr float kRescale = 8.f;

__global__ __launch_bounds__(kAttnThreads, 2) void k_attn(AttnArgs a) {
    // each wave's own quarter of a tile (32 keys x its 128 channels, fp16,
    // row-major [key][channel], rows of 256 B): the V^T operand of its P V
    // products through the transposed LDS read
    __shared__ __attribute__((aligned(16))) uint16_t sV[4][kTK * kQStr];
    __shared__ __attribute__((aligned(16))) float4 sS[4][4][64];   // partial logits per wave
    __shared__ uint4 sP[2][2][64];        // probabilities: [16-key half][fp16 part][lane]
    __shared__ float s_tmax[4][kHeadsWG];   // per wave: maximum logit of its keys per head

    // Work item (unit = query-layer row x 32-head group, split).  Workgroups
    // are dealt to the XCDs round-robin by linear id; when the items divide
    // evenly among them, each XCD takes a contiguous run of items in (unit,
    // split) order, so that the layers, head groups and key-range splits of
    // a query share its L2 (they gather the same FP4 rows) and so do
    // neighbouring prefill queries (whose windows overlap in all but one row).  Any other
    // count keeps the plain order; the mapping is a bijection either way.
    const int nsp = gridDim.x, nhg = gridDim.y;
    const long items = (long)nsp * nhg * gridDim.z;
    const int L = blockIdx.x + nsp * (blockIdx.y + nhg * blockIdx.z);
    const int item = items % kXcds == 0 ? (int)((L % kXcds) * (items / kXcds) + L / kXcds) : L;
    const int split = item % nsp, unit = item / nsp;
    // units run query-major (query, layer, head group), so that the layers of
    // a decode query, which gather the same FP4 rows, share an XCD's L2
    const int hgrp = unit % nhg, qq = unit / nhg;   // qq = query * nlayers + layer
    const int qi = qq / a.nlayers, layer = qq - qi * a.nlayers;
    const int qz = layer * a.rows_q + qi;           // row of the split partials (layer-major)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = lane >> 5, l32 = lane & 31;      // lane half, lane in half
    const int h = hgrp * kHeadsWG + l32;             // this lane's head
    const bool hvalid = h < a.H;
    const int cbase = 128 * wave;                    // this wave's channel quarter

    int64_t row0 = 0;   // first main-KV row of this query's sequence
    int wlo = 0, whi = 0;
    const uint8_t *swk, *swv;
    if (a.prefill) {
        const int64_t p = a.p0 + qi;
        wlo = (int)max((int64_t)0, (int64_t)(a.W - 1) - p);
        whi = a.W;
        swk = a.swa_k[layer] + (size_t)qi * kD;
        swv = a.swa_v[layer] + (size_t)qi * kD;
    } else {
        row0 = a.seq_row_off[qi];
        whi = min(a.swa_len[qi], a.W);
        swk = a.swa_k[layer] + (size_t)qi * a.W * kD;
        swv = a.swa_v[layer] + (size_t)qi * a.W * kD;
    }
    // tile range of this split: tiles are numbered main-KV first, then
    // window, and a split's range may hold both (run in that order)
    const int t0 = a.nsplit == 1 ? 0 : split * a.tiles_per_split;
    const int t1 = a.nsplit == 1 ? a.ntiles : min(a.ntiles, t0 + a.tiles_per_split);
    const int tm = min(t1, a.ntiles_main);           // main tiles are [t0, tm)
    const int32_t* qidx = a.topk_idx + (size_t)qi * a.topk;
    const __amdgpu_buffer_rsrc_t rcode = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kv_codes + row0 * (kD / 2)), (short)0, (int)kKvRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rscale = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.kv_scales + row0 * (kD / 16)), (short)0, (int)kKvRange, kBufFlags);
    // the query's Top-K row as a buffer resource: slots past topk read 0 and
    // are masked to -1
    const __amdgpu_buffer_rsrc_t ridx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)qidx, (short)0, a.topk * 4, kBufFlags);
    // The entry of this lane's key (key l32) of main tile t is loaded as
    // key_raw(t) and masked by key_sel(t, raw) (-1 for padding) only when it
    // is used, a tile later: a select next to the load would make the wave
    // wait for it at once, and with it for every gather issued before it.
    auto key_raw = [&](int t) __attribute__((always_inline)) -> int32_t {
        return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ridx, (kTK * t + l32) * 4, 0, 0);
    };
    auto key_sel = [&](int t, int32_t raw) __attribute__((always_inline)) -> int32_t {
        return (t < tm && kTK * t + l32 < a.topk) ? raw : -1;
    };
    // Prologue, in issue order: the first two tiles' key entries, the query
    // slice (16 loads per lane), then the first gather once its entry is in.
    int32_t idx_t = key_raw(t0), raw_n = key_raw(t0 + 1);
    idx_t = key_sel(t0, idx_t);
    RawQ rq;   // bytes of the next main-KV tile (this lane's key and channels)
    // query slice in two fp16 parts after a power-of-two scaling: MFMA step
    // s of this lane is channels cbase + 64 hh + 8 s .. +8 of head h (the
    // key fragments take the same channels)
    f16x8 q0[8], q1[8];
    float zscale;     // softmax scale (log2 units) times the exact inverse of the scaling
    {
        const float* qp = a.q[layer] + ((size_t)qi * a.H + (hvalid ? h : 0)) * kD + cbase + 64 * hh;
        // head 0 stands in for a padding head (zeroed below)
        float4 xq[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) xq[i] = *reinterpret_cast<const float4*>(qp + 4 * i);
        // the first tile's gather (a window-only split's keys are all
        // padding: nothing is read)
        fetch_q(rcode, rscale, idx_t, wave, hh, rq);

        // largest magnitude of this head's 128 channels (both lane halves),
        // then of all its 512
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xq[i].x), fabsf(xq[i].y)),
                                 fmaxf(fabsf(xq[i].z), fabsf(xq[i].w))));
        if (!hvalid) mx = 0.f;
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // one scale per head for its four channel quarters (the waves), so
        // that their partial logits add as they are and the inverse scaling
        // joins the softmax scale
        if (hh == 0) s_tmax[wave][l32] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(s_tmax[0][l32], s_tmax[1][l32]), fmaxf(s_tmax[2][l32], s_tmax[3][l32]));
        int e = 0;
        (void)frexpf(mx, &e);                          // mx in [2^(e-1), 2^e)
        const int sh = mx > 0.f ? 14 - e : 0;          // mx * 2^sh in [2^13, 2^14)
        const float qscale = ldexpf(1.f, sh);
        zscale = a.scale_log2 * ldexpf(1.f, -sh);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            float4 x0 = xq[2 * st], x1 = xq[2 * st + 1];
            if (!hvalid) x0 = x1 = make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t a0[4], a1[4];
            split2_pk(x0.x * qscale, x0.y * qscale, a0[0], a1[0]);
            split2_pk(x0.z * qscale, x0.w * qscale, a0[1], a1[1]);
            split2_pk(x1.x * qscale, x1.y * qscale, a0[2], a1[2]);
            split2_pk(x1.z * qscale, x1.w * qscale, a0[3], a1[3]);
            q0[st] = as_f16x8(a0[0], a0[1], a0[2], a0[3]);
            q1[st] = as_f16x8(a1[0], a1[1], a1[2], a1[3]);
        }
    }
    f32x16 o[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
    float m = -INFINITY, l = 0.f;
    uint16_t* const vt = sV[wave];   // this wave's quarter tile

    // S^T of a tile over this wave's 128 channels from its key fragments in
    // registers, published in sS (by the caller's barrier) in the query's
    // scaled units.
    auto s_chain = [&](auto&& frag) __attribute__((always_inline)) {
        f32x16 s0 = f32x16{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const f16x8 f = frag(st);
            s0 = mfma32(f, q0[st], s0);
            s0 = mfma32(f, q1[st], s0);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            sS[wave][r4][lane] = make_float4(s0[4 * r4], s0[4 * r4 + 1], s0[4 * r4 + 2], s0[4 * r4 + 3]);
    };

    // Lane part of the transposed reads of V: lane l = 16 g + 4 b + c points
    // at key row 4 (g >> 1) + b, channels 16 (g & 1) + 4 c .. +3 of a
    // 32-channel block of the quarter, so that lane l receives channel
    // (l & 31) of the block for 4 consecutive keys.  In quarter-tile terms:
    // row 16 u + 8 hi + trrow, chunk 4 ct + tsub; since tile_swz(row) = 4
    // (row & 3) + swz_lo(row), the chunk's swizzle splits into tsub ^
    // swz_lo(row), fixed per lane and hi (u adds 16 rows, which swz_lo does
    // not see), and ct ^ (row & 3), fixed per lane.
    const int trrow = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int tsub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int trhi = (lane >> 2) & 3;   // row & 3
    const int trb0 = trrow * kQStr + 8 * (tsub ^ swz_lo(trrow)) + 4 * (lane & 1);
    const int trb1 = (trrow + 8) * kQStr + 8 * (tsub ^ swz_lo(trrow + 8)) + 4 * (lane & 1);

    // Softmax of a tile, split over the four waves: wave w takes keys
    // 8w .. 8w+7 (its registers' rows 4w .. 4w+3 of S^T), so it reads one
    // quarter of the partial logits.  tile_max: the full logits of those keys
    // (the four channel quarters added in a fixed order; a padding key's
    // logit is -inf by the tile's key mask) and their maximum per head,
    // published in s_tmax.  probs (after a barrier): the tile's maximum per
    // head from the four waves (the same in every wave, so every wave moves m
    // alike), the lazy rescale, and this wave's probabilities, split into two
    // fp16 parts and written to sP in the B-operand layout of the P V
    // products; after another barrier every wave reads all of them (read_p).
    auto tile_max = [&](uint64_t vmask, float (&z)[4]) __attribute__((always_inline)) {
        const float4 c0 = sS[0][wave][lane], c1 = sS[1][wave][lane];
        const float4 c2 = sS[2][wave][lane], c3 = sS[3][wave][lane];
        const float v0[4] = {c0.x, c0.y, c0.z, c0.w}, v1[4] = {c1.x, c1.y, c1.z, c1.w};
        const float v2[4] = {c2.x, c2.y, c2.z, c2.w}, v3[4] = {c3.x, c3.y, c3.z, c3.w};
        const uint32_t kbits = (uint32_t)(vmask >> (8 * wave + 4 * hh));   // keys 8 wave + 4 hh + i
        float tw = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float zz = ((v0[i] + v1[i]) + (v2[i] + v3[i])) * zscale;   // lane l32: head h
            z[i] = (kbits >> i) & 1u ? zz : -INFINITY;
            tw = fmaxf(tw, z[i]);
        }
        tw = fmaxf(tw, __shfl_xor(tw, 32));
        if (hh == 0) s_tmax[wave][l32] = tw;
    };
    auto probs = [&](const float (&z)[4]) __attribute__((always_inline)) {
        const float tm_ = fmaxf(fmaxf(s_tmax[0][l32], s_tmax[1][l32]),
                                fmaxf(s_tmax[2][l32], s_tmax[3][l32]));
        const bool bump = tm_ > m + kRescale;   // true for any finite tm_ while m = -inf
        if (__ballot(bump)) {
            const float mn = bump ? tm_ : m;   // finite where bump
            const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 from m = -inf
            l *= alpha;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) o[ct] = o[ct] * alpha;
            m = mn;
        }
        // each probability (<= 2^8) in two fp16 parts.  m = -inf only while
        // every logit so far is -inf: those give exp2(-inf) = 0.
        const float ms = m == -INFINITY ? 0.f : m;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // raw v_exp_f32: results below 2^-126 flush to 0 (negligible next
            // to the running maximum's 1)
            pv[i] = __builtin_amdgcn_exp2f(z[i] - ms);
        }
        l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        uint32_t x0[2], x1[2];
        split2_pk(pv[0], pv[1], x0[0], x1[0]);
        split2_pk(pv[2], pv[3], x0[1], x1[1]);
        // MFMA u's B operand, element j: key 16u + 8(j/4) + 4hh + j%4; this
        // wave's keys are u = wave/2, j/4 = wave%2: dwords 2(wave%2) .. +1
        uint32_t* d0 = reinterpret_cast<uint32_t*>(&sP[wave >> 1][0][lane]) + 2 * (wave & 1);
        uint32_t* d1 = reinterpret_cast<uint32_t*>(&sP[wave >> 1][1][lane]) + 2 * (wave & 1);
        *reinterpret_cast<uint2*>(d0) = make_uint2(x0[0], x0[1]);
        *reinterpret_cast<uint2*>(d1) = make_uint2(x1[0], x1[1]);
    };
    auto read_p = [&](f16x8 (&pp)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int part = 0; part < 2; ++part)
                pp[u][part] = __builtin_bit_cast(f16x8, sP[u][part][lane]);
    };
    // O^T += V^T P^T with V this wave's row-major quarter tile in `vb`.
    auto pv_mma = [&](const uint16_t* vb, const f16x8 (&pp)[2][2]) __attribute__((always_inline)) {
        // O^T[channel cbase + 32 ct + m][head] += V^T P^T over the 32 keys;
        // the A operand's 8 keys are 16u + 4hh + 0..3 and 16u + 8 + 4hh + 0..3.
        // The V^T fragments of one 16-key half are requested before its
        // products; consecutive products go to different accumulators.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f16x8 vv[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int cto = 32 * (ct ^ trhi);
                const v4i16 lo = lds_read_tr16(vb + trb0 + 16 * u * kQStr + cto);
                const v4i16 hi = lds_read_tr16(vb + trb1 + 16 * u * kQStr + cto);
                vv[ct] = __builtin_bit_cast(
                    f16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                                        hi[0], hi[1], hi[2], hi[3]});
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) o[ct] = mfma32(vv[ct], pp[u][part], o[ct]);
            }
        }
    };
    // Main-KV tiles: three block barriers per tile (the partial logits, the
    // tile maxima and the probabilities are exchanged; each wave's tile data
    // is its own).  Tile t's bytes are in rq when its step starts; they
    // become the key fragments, the gather of tile t+1 goes out, and the
    // fragments are written to the wave's quarter tile for the P V products
    // (the wave's earlier reads of it precede these writes in its own LDS
    // order).
    for (int t = t0; t < tm; ++t) {
        f16x8 kf[8];
        dequant_q(rq, kf);
        const uint64_t vm = __ballot(idx_t >= 0);
        // unconditional: past the last tile the entry is -1 and nothing is read
        idx_t = key_sel(t + 1, raw_n);
        fetch_q(rcode, rscale, idx_t, wave, hh, rq);
        raw_n = key_raw(t + 2);
        put_q(kf, vt);
        __builtin_amdgcn_s_setprio(1);   // raised priority: see above k_attn
        s_chain([&](int st) __attribute__((always_inline)) { return kf[st]; });
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();   // logits of t published
        float z[4];
        tile_max(vm, z);
        __syncthreads();   // the waves' maxima published
        probs(z);
        __syncthreads();   // probabilities published
        f16x8 pp[2][2];
        read_p(pp);
        __builtin_amdgcn_s_setprio(1);
        pv_mma(vt, pp);
        __builtin_amdgcn_s_setprio(0);
    }
    // Window tiles: the same steps with the key fragments from the window's
    // K rows and the quarter tile from its V rows (rows outside the window
    // are zeroed and masked), converted one fragment at a time; each of the
    // next tile's row sets is gathered as soon as this tile's is consumed
    // (unconditionally: past the last tile every lane reads the window's
    // last row, which is unused).
    const int w0 = max(t0, a.ntiles_main);
    if (w0 < t1) {
        RawWQ rk, rv;
        fetch_wq(swk, a.W, w0 - a.ntiles_main, wave, hh, rk);
        fetch_wq(swv, a.W, w0 - a.ntiles_main, wave, hh, rv);
        for (int t = w0; t < t1; ++t) {
            const int tw = t - a.ntiles_main;
            const int w_ = kTK * tw + l32;   // this lane's window row
            const bool valid = w_ >= wlo && w_ < whi;
            const uint64_t vm = __ballot(valid);
            const uint32_t keep = valid ? ~0u : 0u;
#pragma unroll
            for (int st = 0; st < 8; ++st) put_q1(dequant_wq(rv, keep, st), st, vt);
            fetch_wq(swv, a.W, tw + 1, wave, hh, rv);
            __builtin_amdgcn_s_setprio(1);
            s_chain([&](int st) __attribute__((always_inline)) { return dequant_wq(rk, keep, st); });
            __builtin_amdgcn_s_setprio(0);
            fetch_wq(swk, a.W, tw + 1, wave, hh, rk);
            __syncthreads();   // logits of t published
            float z[4];
            tile_max(vm, z);
            __syncthreads();   // the waves' maxima published
            probs(z);
            __syncthreads();   // probabilities published
            f16x8 pp[2][2];
            read_p(pp);
            __builtin_amdgcn_s_setprio(1);
            pv_mma(vt, pp);
            __builtin_amdgcn_s_setprio(0);
        }
    }
    // l holds this lane's keys' share: add the two lane halves, then the
    // four waves (s_tmax is free: every read of it is behind a barrier)
    {
        const float lw = l + __shfl_xor(l, 32);
        __syncthreads();
        if (hh == 0) s_tmax[wave][l32] = lw;
        __syncthreads();
    }
    const float lt = (s_tmax[0][l32] + s_tmax[1][l32]) + (s_tmax[2][l32] + s_tmax[3][l32]);
    if (!hvalid) return;
    // lane (hh, head) holds channels cbase + 32 ct + 8 q + 4 hh + 0..3, q = 0..3
    const size_t orow = ((size_t)qi * a.H + h) * kD + cbase + 4 * hh;
    if (a.nsplit == 1) {
        float* const out = a.out[layer];
        float* const lse = a.lse[layer];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4*>(out + orow + 32 * ct + 8 * q4) =
                    make_float4(o[ct][4 * q4] * inv, o[ct][4 * q4 + 1] * inv,
                                o[ct][4 * q4 + 2] * inv, o[ct][4 * q4 + 3] * inv);
        if (lse && hh == 0 && wave == 0)
            lse[(size_t)qi * a.H + h] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
    } else {
        // partial rows: every layer's rows, layer-major (qz)
        const size_t rows_all = gridDim.z;
        float* po = a.part_o + ((size_t)split * rows_all * a.H) * kD +
                    ((size_t)qz * a.H + h) * kD + cbase + 4 * hh;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4*>(po + 32 * ct + 8 * q4) =
                    make_float4(o[ct][4 * q4], o[ct][4 * q4 + 1], o[ct][4 * q4 + 2], o[ct][4 * q4 + 3]);
        if (hh == 0 && wave == 0) {
            float* pm = a.part_ml + (((size_t)split * rows_all + qz) * a.H + h) * 2;
            pm[0] = m;
            pm[1] = lt;
        }
    }
}

// Merges the key-range splits of one (query, head): weights 2^(m_s - M).
// All partials are requested in one round (up to kMaxSplitRegs in
// registers), then weighted.
constexpr int kMaxSplitRegs = 24;

// Output rows of a combine: layer l's rows are partial rows
// [l * rows_q, (l + 1) * rows_q).
struct CombineOut {
    float* out[kMaxLayers];
    float* lse[kMaxLayers];
    int rows_q, nlayers;
};

// One workgroup merges HPW heads of one row (HPW x 512 channels, a float4
// per thread and head); every partial of the HPW heads is requested before
// the first is weighted (MAXS >= nsplit).
template <int HPW, int MAXS>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int nsplit, int rows_all, int H,
                                                      CombineOut co) {
    // (row, head group) of this workgroup: the attention kernel gives each
    // XCD a contiguous run of its query-major (query, layer, 32-head group)
    // units when they divide evenly; the merges take the same contiguous
    // runs, so that a unit's partials are merged on the XCD whose L2 holds them
    const int n = gridDim.x, L = blockIdx.x;
    const int item = n % kXcds == 0 ? (L % kXcds) * (n / kXcds) + L / kXcds : L;
    const int qq = item * HPW / H, h0 = item * HPW - qq * H;   // qq = query * nlayers + layer
    const int qi = qq / co.nlayers, lyr = qq - qi * co.nlayers;
    const int qh0 = (lyr * co.rows_q + qi) * H + h0;   // qz * H + h, qz = layer * rows_q + query
    const size_t stride_o = (size_t)rows_all * H * kD;
    const size_t stride_ml = (size_t)rows_all * H * 2;
    float2 ml[HPW][MAXS];
    float4 po[HPW][MAXS];
#pragma unroll
    for (int j = 0; j < HPW; ++j)
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s < nsplit) {
                const size_t qh = (size_t)qh0 + j;
                ml[j][s] = *reinterpret_cast<const float2*>(part_ml + s * stride_ml + qh * 2);
                po[j][s] = reinterpret_cast<const float4*>(part_o + s * stride_o + qh * kD)[threadIdx.x];
            }
        }
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
        const int qh = qh0 + j;
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
            if (s < nsplit) M = fmaxf(M, ml[j][s].x);
        float L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int s = 0; s < MAXS; ++s) {
            if (s < nsplit && ml[j][s].x != -INFINITY && ml[j][s].y != 0.f) {
                const float w = exp2f(ml[j][s].x - M);
                L += w * ml[j][s].y;
                acc.x += w * po[j][s].x; acc.y += w * po[j][s].y;
                acc.z += w * po[j][s].z; acc.w += w * po[j][s].w;
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const int layer = qh / (co.rows_q * H), r = qh - layer * co.rows_q * H;
        reinterpret_cast<float4*>(co.out[layer] + (size_t)r * kD)[threadIdx.x] =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        float* const lse = co.lse[layer];
        if (lse && threadIdx.x == 0) lse[r] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
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

// Test hook: the attention's own dequantisation, converted back to fp32, of
// every (E2M1 code, E4M3 scale byte) pair at each of the 8 nibble positions
// of a code dword, and of every E4M3 byte at each of the 8 byte positions of
// a window chunk (the other positions hold other values).
// main_out [256 scale bytes][16 codes][8 positions], win_out [256][8].
__global__ void k_dequant_tables(float* main_out, float* win_out) {
    const uint32_t sb = blockIdx.x, c = threadIdx.x & 15u, pos = threadIdx.x >> 4;
    uint32_t w = 0;
    for (uint32_t x = 0; x < 8; ++x) w |= (x == pos ? c : (c + 3 * x + 1) & 15u) << (4 * x);
    // through the attention's own path: every code word is w and every
    // group scale byte is sb, and fragment pos (scale byte pos / 2) is read
    RawQ r;
    r.code[0] = r.code[1] = make_uint4(w, w, w, w);
    r.scale = sb * 0x01010101u;
    f16x8 kf[8];
    dequant_q(r, kf);
    float v = 0.f;
#pragma unroll
    for (uint32_t f = 0; f < 8; ++f)
        if (f == pos) v = (float)kf[f][pos];
    main_out[(sb * 16 + c) * 8 + pos] = v;
    if (threadIdx.x < 8) {
        uint32_t wb[2] = {0u, 0u};
        for (uint32_t x = 0; x < 8; ++x)
            wb[x >> 2] |= (x == threadIdx.x ? sb : (sb + 37 * x + 11) & 255u) << (8 * (x & 3));
        uint32_t o8[4];
        dequant_fp8x8(make_uint2(wb[0], wb[1]), ~0u, o8);
        win_out[sb * 8 + threadIdx.x] =
            (float)__builtin_bit_cast(f16x2v, o8[threadIdx.x >> 1])[threadIdx.x & 1];
    }
}

struct AttnPlan {
    int hgroups, ntiles_main, ntiles, nsplit, tps;
    size_t ws_bytes;
};

// Key-range splits.  Two workgroups fit a CU (registers: 256 per lane at
// four waves); a lone workgroup costs about kPrologueTiles tiles of fixed
// latency (index, query and first gathers in flight) plus its tiles, and a CU
// runs two together in kPairTenths / 10 of that.  Splitting adds the combine
// launch (about kCombineTiles).  The plan takes the tiles per split with the
// lowest modelled cost; a split takes consecutive tiles, main-KV then window
// ones as a single workgroup runs them.
constexpr int kCUs = 256;
constexpr int kPrologueTiles = 3;
constexpr int kCombineTiles = 2;
constexpr long kPairTenths = 14;

// Modelled time, in tenths of a lone tile, of `wgs` workgroups of `tiles` tiles.
long attn_cost(long wgs, int tiles) {
    const long per_cu = (wgs + kCUs - 1) / kCUs;
    return ((per_cu / 2) * kPairTenths + (per_cu % 2) * 10) * (kPrologueTiles + tiles);
}

int plan_attn(int rows_q, int H, int D, int topk, int W, bool allow_split, AttnPlan* p) {
    if (rows_q < 0 || H <= 0 || D <= 0 || topk < 0 || W < 0) return CSA2_ERR_SHAPE;
    if (D != kD || H % 16 != 0 || topk > CSA2_MAX_TOPK || W > 1024 || rows_q > 65535)
        return CSA2_ERR_UNSUPPORTED;
    p->hgroups = (H + kHeadsWG - 1) / kHeadsWG;
    p->ntiles_main = (topk + kTK - 1) / kTK;
    p->ntiles = p->ntiles_main + (W + kTK - 1) / kTK;
    const long units = (long)rows_q * p->hgroups;
    int nsplit = 1;
    p->tps = p->ntiles;
    if (allow_split && p->ntiles > 1) {
        long best = attn_cost(units, p->ntiles);   // no split
        for (int tps = 1; tps < p->ntiles; ++tps) {
            const int ns = (p->ntiles + tps - 1) / tps;
            if (ns < 2 || ns > kMaxSplitRegs) continue;
            const long cost = attn_cost(units * ns, tps) + 10 * kCombineTiles;
            if (cost < best) {
                best = cost;
                nsplit = ns;
                p->tps = tps;
            }
        }
    }
    p->nsplit = nsplit;
    Carver c(nullptr);
    if (nsplit > 1) {
        c.take<float>((size_t)nsplit * rows_q * H * kD);
        c.take<float>((size_t)nsplit * rows_q * H * 2);
    }
    p->ws_bytes = c.bytes();
    return CSA2_OK;
}

// rows_all = rows_q x nlayers (the plan was made for that many rows)
int launch_attn(AttnArgs a, const AttnPlan& pl, int rows_all, void* ws, hipStream_t s) {
    const int rows_q = rows_all;
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
    int st = CSA2_LAUNCH("attn", k_attn, grid, dim3(kAttnThreads), s, a);
    if (st || pl.nsplit == 1) return st;
    CombineOut co{};
    for (int l = 0; l < a.nlayers; ++l) {
        co.out[l] = a.out[l];
        co.lse[l] = a.lse[l];
    }
    co.rows_q = a.rows_q;
    co.nlayers = a.nlayers;
    // four heads per workgroup when every partial of four fits the registers
    if (pl.nsplit <= 4 && a.H % 4 == 0)
        return CSA2_LAUNCH("attn_combine", (k_attn_combine<4, 4>), dim3(rows_q * a.H / 4),
                           dim3(128), s, a.part_o, a.part_ml, pl.nsplit, rows_q, a.H, co);
    return CSA2_LAUNCH("attn_combine", (k_attn_combine<1, kMaxSplitRegs>), dim3(rows_q * a.H),
                       dim3(128), s, a.part_o, a.part_ml, pl.nsplit, rows_q, a.H, co);
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_decode_layers_workspace_bytes(int32_t L, int32_t B, int32_t H, int32_t D,
                                                     int32_t topk, int32_t W) {
    if (L < 1 || L > kMaxLayers || B < 0 || (int64_t)B * L > 65535) return 0;
    AttnPlan p;
    if (plan_attn(B * L, H, D, topk, W, true, &p) != CSA2_OK) return 0;
    return p.ws_bytes;
}

extern "C" size_t csa2_decode_workspace_bytes(int32_t B, int32_t H, int32_t D, int32_t topk,
                                              int32_t W) {
    return csa2_decode_layers_workspace_bytes(1, B, H, D, topk, W);
}

extern "C" int csa2_sparse_attn_decode_layers(
    int32_t L, const float* const* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
    const int64_t* seq_row_off, const int32_t* topk_idx, int32_t topk,
    const uint8_t* const* swa_k, const uint8_t* const* swa_v, const int32_t* swa_len, int32_t W,
    int32_t B, int32_t H, int32_t D, float softmax_scale, float* const* out, float* const* lse,
    void* ws, size_t ws_bytes, void* stream) {
    if (L < 1 || B < 0) return CSA2_ERR_SHAPE;
    if (L > kMaxLayers || (int64_t)B * L > 65535) return CSA2_ERR_UNSUPPORTED;
    AttnPlan pl;
    int st = plan_attn(B * L, H, D, topk, W, true, &pl);
    if (st) return st;
    if (B == 0) return CSA2_OK;
    if (!q || !out || !swa_len || (W > 0 && (!swa_k || !swa_v))) return CSA2_ERR_NULL;
    if (topk > 0 && (!kv_codes || !kv_scales || !seq_row_off || !topk_idx)) return CSA2_ERR_NULL;
    AttnArgs a{};
    for (int l = 0; l < L; ++l) {
        if (!q[l] || !out[l] || (W > 0 && (!swa_k[l] || !swa_v[l]))) return CSA2_ERR_NULL;
        const uintptr_t al = (uintptr_t)q[l] | (uintptr_t)out[l] |
                             (W > 0 ? ((uintptr_t)swa_k[l] | (uintptr_t)swa_v[l]) : 0);
        if (al & 15) return CSA2_ERR_UNSUPPORTED;
        a.q[l] = q[l];
        a.out[l] = out[l];
        a.lse[l] = lse ? lse[l] : nullptr;
        a.swa_k[l] = W > 0 ? swa_k[l] : nullptr;
        a.swa_v[l] = W > 0 ? swa_v[l] : nullptr;
    }
    if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) return CSA2_ERR_WORKSPACE;
    a.kv_codes = kv_codes; a.kv_scales = kv_scales; a.seq_row_off = seq_row_off;
    a.topk_idx = topk_idx; a.swa_len = swa_len;
    a.topk = topk; a.W = W; a.H = H;
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    a.prefill = 0;
    a.rows_q = B;
    a.nlayers = L;
    return launch_attn(a, pl, B * L, ws, (hipStream_t)stream);
}

extern "C" int csa2_sparse_attn_decode(const float* q, const uint8_t* kv_codes,
                                       const uint8_t* kv_scales, const int64_t* seq_row_off,
                                       const int32_t* topk_idx, int32_t topk,
                                       const uint8_t* swa_k, const uint8_t* swa_v,
                                       const int32_t* swa_len, int32_t W, int32_t B, int32_t H,
                                       int32_t D, float softmax_scale, float* out, float* lse,
                                       void* ws, size_t ws_bytes, void* stream) {
    const float* qs[1] = {q};
    const uint8_t* ks[1] = {swa_k};
    const uint8_t* vs[1] = {swa_v};
    float* os[1] = {out};
    float* ls[1] = {lse};
    return csa2_sparse_attn_decode_layers(1, qs, kv_codes, kv_scales, seq_row_off, topk_idx, topk,
                                          ks, vs, swa_len, W, B, H, D, softmax_scale, os, ls, ws,
                                          ws_bytes, stream);
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
    a.q[0] = q; a.kv_codes = kv_codes; a.kv_scales = kv_scales; a.seq_row_off = nullptr;
    a.topk_idx = topk_idx; a.swa_k[0] = swa_k; a.swa_v[0] = swa_v; a.swa_len = nullptr;
    a.topk = topk; a.W = W; a.H = H;
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    a.p0 = p0;
    a.prefill = 1;
    a.out[0] = out; a.lse[0] = lse;
    a.rows_q = Qn;
    a.nlayers = 1;
    return launch_attn(a, pl, Qn, ws, (hipStream_t)stream);
}

extern "C" int csa2_debug_decode_tables(float* fp4_hw, float* fp4_ref, float* fp8_hw,
                                        float* fp8_ref, void* stream) {
    if (!fp4_hw || !fp4_ref || !fp8_hw || !fp8_ref) return CSA2_ERR_NULL;
    return CSA2_LAUNCH("decode_tables", k_decode_tables, dim3(1), dim3(256),
                       (hipStream_t)stream, fp4_hw, fp4_ref, fp8_hw, fp8_ref);
}

extern "C" int csa2_debug_dequant_tables(float* main_out, float* win_out, void* stream) {
    if (!main_out || !win_out) return CSA2_ERR_NULL;
    return CSA2_LAUNCH("dequant_tables", k_dequant_tables, dim3(256), dim3(128),
                       (hipStream_t)stream, main_out, win_out);
}
