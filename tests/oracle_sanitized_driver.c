/*
 * Host driver that runs every oracle function on small seeded inputs held in
 * exact-size heap buffers, including the edge cases (empty and short
 * sequences, K above the context, padded pools, empty windows, a window that
 * starts before position 0).  Built with AddressSanitizer and UBSan by
 * tests/test_oracle_sanitized.py; any out-of-bounds access, leak or undefined
 * operation ends the run with a report.  Prints "ok" at the end.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1(int code);
double oracle_e4m3(int byte);
void oracle_dequant_row(const uint8_t* codes, const uint8_t* scales, int D, double* out);
void oracle_fp4_quantize_row(const float* x, int D, uint8_t* codes, uint8_t* scales);
uint8_t oracle_e4m3_encode(float x);
void oracle_swa_append(const float* k_new, const float* v_new, const int64_t* pos, int B, int D,
                       int W, uint8_t* swa_k, uint8_t* swa_v);
int oracle_index_full_ex(const float* qI, const void* kI, int key_format,
                         const int64_t* seq_row_off, const int32_t* q_seq, const int32_t* q_nvis,
                         int Q, int Hi, int Hk, int Di, int topk, int32_t* topk_idx,
                         int pool_blocks, int block_size, int32_t* pool_idx, int block_rule);
int oracle_reindex(const float* qI, const float* kI, const int64_t* seq_row_off,
                   const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_idx,
                   int pool_blocks, int block_size, int Q, int Hi, int Hk, int Di, int topk,
                   int32_t* topk_idx);
int oracle_reindex_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                        const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_idx,
                        int pool_blocks, int block_size, int Q, int Hi, int Hk, int Di, int topk,
                        int32_t* topk_idx);
int oracle_attn_decode(const float* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                       const int64_t* seq_row_off, const int32_t* topk_idx, int topk,
                       const uint8_t* swa_k, const uint8_t* swa_v, const int32_t* swa_len, int W,
                       int B, int H, int D, float softmax_scale, float* out, float* lse);
int oracle_attn_prefill(const float* q, int64_t p0, const uint8_t* kv_codes,
                        const uint8_t* kv_scales, const int32_t* topk_idx, int topk,
                        const uint8_t* swa_k, const uint8_t* swa_v, int W, int Qn, int H, int D,
                        float softmax_scale, float* out, float* lse);
int oracle_scores_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                       const int32_t* q_seq, const int32_t* q_nvis, int q, int Hi, int Hk, int Di,
                       double* out);

static uint64_t g_state = 88172645463325252ull;
static uint32_t rnd(void) {   /* xorshift64 */
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (uint32_t)(g_state >> 32);
}
static int ri(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
#define CHECK(x) do { if (!(x)) { fprintf(stderr, "check failed: %s (line %d)\n", #x, __LINE__); exit(1); } } while (0)

int main(void) {
    /* codecs */
    for (int c = 0; c < 16; ++c) (void)oracle_e2m1(c);
    for (int b = 0; b < 256; ++b) (void)oracle_e4m3(b);
    for (int i = 0; i < 4096; ++i) (void)oracle_e4m3_encode(((float)ri(-100000, 100000)) / 97.0f);
    {
        const int D = 64;
        float* x = xmalloc(sizeof(float) * D);
        uint8_t* codes = xmalloc(D / 2);
        uint8_t* scales = xmalloc(D / 16);
        double* row = xmalloc(sizeof(double) * D);
        for (int r = 0; r < 64; ++r) {
            for (int c = 0; c < D; ++c) x[c] = (r % 5 == 0) ? 0.f : ((float)ri(-3000, 3000)) / 7.0f;
            oracle_fp4_quantize_row(x, D, codes, scales);
            oracle_dequant_row(codes, scales, D, row);
        }
        free(x); free(codes); free(scales); free(row);
    }
    {   /* window ring: 2 sequences, W = 5, positions including negative */
        const int B = 2, D = 16, W = 5;
        float* k = xmalloc(sizeof(float) * B * D);
        float* v = xmalloc(sizeof(float) * B * D);
        int64_t* pos = xmalloc(sizeof(int64_t) * B);
        uint8_t* rk = xmalloc((size_t)B * W * D);
        uint8_t* rv = xmalloc((size_t)B * W * D);
        memset(rk, 0, (size_t)B * W * D);
        memset(rv, 0, (size_t)B * W * D);
        for (int step = 0; step < 13; ++step) {
            for (int i = 0; i < B * D; ++i) { k[i] = (float)ri(-50, 50); v[i] = (float)ri(-50, 50); }
            pos[0] = step - 2;
            pos[1] = step + 3;
            oracle_swa_append(k, v, pos, B, D, W, rk, rv);
        }
        free(k); free(v); free(pos); free(rk); free(rv);
    }
    /* indexer over packed sequences: an empty one, a short one, K above the
     * context, both key formats, both block rules */
    for (int trial = 0; trial < 6; ++trial) {
        const int Hi = 2, Hk = (trial & 1) ? 1 : 2, Di = 16, RW = Hk * Di;
        const int S = 4;
        int ctx[4] = {ri(100, 400), 0, ri(1, 9), ri(30, 80)};
        int64_t off[4];
        int64_t rows = 0;
        for (int s = 0; s < S; ++s) { off[s] = rows; rows += ctx[s]; }
        float* kI = xmalloc(sizeof(float) * rows * RW);
        uint8_t* k8 = xmalloc((size_t)rows * RW);
        for (int64_t i = 0; i < rows * RW; ++i) {
            const int v = ri(-8, 8);
            kI[i] = (float)v;
            k8[i] = oracle_e4m3_encode((float)v);
        }
        const int Q = S;
        float* qI = xmalloc(sizeof(float) * Q * Hi * Di);
        for (int i = 0; i < Q * Hi * Di; ++i) qI[i] = (float)ri(-8, 8);
        int32_t qs[4] = {0, 1, 2, 3}, nv[4];
        for (int s = 0; s < S; ++s) nv[s] = ctx[s] - (s == 0 ? 7 : 0);
        const int topk = ri(1, 40), P = ri(1, 30), bs = 1 << ri(0, 3);
        int32_t* idx = xmalloc(sizeof(int32_t) * Q * topk);
        int32_t* pool = xmalloc(sizeof(int32_t) * Q * P);
        int32_t* re = xmalloc(sizeof(int32_t) * Q * topk);
        for (int fmt = 0; fmt < 2; ++fmt) {
            CHECK(oracle_index_full_ex(qI, fmt ? (const void*)k8 : (const void*)kI, fmt, off, qs, nv,
                                       Q, Hi, Hk, Di, topk, idx, P, bs, pool, trial % 2) == 0);
            CHECK((fmt ? oracle_reindex_e4m3(qI, k8, off, qs, nv, pool, P, bs, Q, Hi, Hk, Di,
                                             topk, re)
                       : oracle_reindex(qI, kI, off, qs, nv, pool, P, bs, Q, Hi, Hk, Di, topk,
                                        re)) == 0);
        }
        double* sc = xmalloc(sizeof(double) * (nv[0] > 0 ? nv[0] : 1));
        CHECK(oracle_scores_e4m3(qI, k8, off, qs, nv, 0, Hi, Hk, Di, sc) == 0);
        CHECK(oracle_index_full_ex(qI, kI, 0, off, qs, nv, Q, Hi, Hk, Di, topk, idx, P, bs, pool,
                                   5) == -1);   /* unknown block rule */
        free(sc); free(kI); free(k8); free(qI); free(idx); free(pool); free(re);
    }
    /* decode attention: -1 padding, an empty window, no main keys */
    {
        const int B = 3, H = 2, D = 32, W = 4, topk = 6, rows = 20;
        float* q = xmalloc(sizeof(float) * B * H * D);
        for (int i = 0; i < B * H * D; ++i) q[i] = (float)ri(-100, 100) / 50.0f;
        uint8_t* codes = xmalloc((size_t)rows * D / 2);
        uint8_t* scales = xmalloc((size_t)rows * D / 16);
        for (int i = 0; i < rows * D / 2; ++i) codes[i] = (uint8_t)ri(0, 255);
        for (int i = 0; i < rows * D / 16; ++i) scales[i] = (uint8_t)((ri(-4, 4) + 7) << 3);
        int64_t off[3] = {0, 8, 8};
        int32_t idx[3 * 6] = {0, 3, 7, -1, -1, -1, 1, 2, 3, 4, 5, 11, -1, -1, -1, -1, -1, -1};
        uint8_t* sk = xmalloc((size_t)B * W * D);
        uint8_t* sv = xmalloc((size_t)B * W * D);
        for (int i = 0; i < B * W * D; ++i) { sk[i] = oracle_e4m3_encode((float)ri(-9, 9) / 4.f); sv[i] = sk[i] ^ 0x08; }
        int32_t sl[3] = {4, 0, 0};   /* the last query has no key at all */
        float* out = xmalloc(sizeof(float) * B * H * D);
        float* lse = xmalloc(sizeof(float) * B * H);
        CHECK(oracle_attn_decode(q, codes, scales, off, idx, topk, sk, sv, sl, W, B, H, D, 0.17f,
                                 out, lse) == 0);
        CHECK(oracle_attn_decode(q, codes, scales, off, idx, topk, sk, sv, sl, W, B, H, D, 0.17f,
                                 out, NULL) == 0);
        /* prefill: a window that starts before position 0 */
        const int Qn = 3;
        uint8_t* pk = xmalloc((size_t)(Qn + W - 1) * D);
        uint8_t* pv = xmalloc((size_t)(Qn + W - 1) * D);
        for (int i = 0; i < (Qn + W - 1) * D; ++i) { pk[i] = sk[i % (B * W * D)]; pv[i] = sv[i % (B * W * D)]; }
        CHECK(oracle_attn_prefill(q, 1, codes, scales, idx, topk, pk, pv, W, Qn, H, D, 0.17f, out,
                                  lse) == 0);
        free(q); free(codes); free(scales); free(sk); free(sv); free(out); free(lse);
        free(pk); free(pv);
    }
    printf("ok\n");
    return 0;
}
