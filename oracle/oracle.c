/*
 * CPU oracle for the CSA2 sparse-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library and never calls it.
 *
 * Sources (web pages on arXiv 2609.19969, "DeepSeek-V4.1-Flash: Pushing the
 * Limits of KV Cache Compression"); citations below use these tags:
 *   [J-CSA2]  jaehun.me review, section "2) CSA2" (paper 2.3, 2.3.1, 2.3.2,
 *             Fig. 4, Fig. 5): three static per-layer modes Full / Reindex /
 *             Reuse; every mode has its own query and SWA KV; the Full layer
 *             builds a 2,048-block x 8-position candidate pool that later
 *             Reindex layers pick 512 entries from.
 *   [J-FP4]   jaehun.me review, section "3) FP4 main KV + SWA Bounded Replay"
 *             (paper 2.4.4): main KV stored as E2M1 with one E4M3 scale per 16
 *             channels; SWA KV kept in FP8; window n_win = 128.
 *   [J-EX]    jaehun.me review, worked example "작동 원리" (paper 2.3.1,
 *             4.2.1): Full scores all entries and keeps the Top-K (512 in the
 *             model); Reuse attends over the Full layer's KV and indices as
 *             they are; Reindex rescores with its own indexer query.
 *   [A-NEWS]  ainewsway.com article, section on why the KV cache became the
 *             bottleneck: E2M1 FP4 with a scaling factor per 16 channels; a
 *             128-token sliding window combined with global sparse retrieval.
 *
 * Everything is computed in double and follows the plain definitions:
 * exact scores, a full sort for every selection, softmax over the union of
 * the selected main-KV entries and the window.  Readings of points the
 * pages leave open are marked READING.
 *
 * Parity status: every function here is pinned by the CPU tests (codec
 * tables against the OCP formulas and torch's FP8 decoder, integer
 * recomputation of scores over fp32 and over E4M3 key caches, a float64 sum
 * over every finite E4M3 key value, selection invariants and brute force, dense
 * attention special cases and a float64 textbook softmax attention; the
 * writers by round trips, brute-force nearest values, torch's FP8 cast within
 * its finite range and the ring's contents after many appends).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ codecs */

/* E2M1 (OCP Microscaling spec, FP4 element): sign bit, 2 exponent bits with
 * bias 1, 1 mantissa bit, no inf/NaN.  exponent 0 is subnormal: 0.5 * m.
 * [J-FP4], [A-NEWS] name the format; the bit layout is the OCP one. */
double oracle_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP 8-bit floating point spec): sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; S.1111.111 is NaN; no infinities; max 448.
 * READING: "E4M3" on the pages is taken as the OCP FN variant. */
double oracle_e4m3(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* One main-KV row, dequantised: channel c takes the low nibble of byte c/2
 * when c is even and the high nibble when odd, times the E4M3 scale of its
 * 16-channel group [J-FP4].  READING: even channel in the low nibble. */
void oracle_dequant_row(const uint8_t* codes, const uint8_t* scales, int D, double* out) {
    for (int c = 0; c < D; ++c) {
        int byte = codes[c / 2];
        int nib = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
        out[c] = oracle_e2m1(nib) * oracle_e4m3(scales[c / 16]);
    }
}

/* ------------------------------------------------------ FP4 main-KV writer */

/* Quantises one fp32 row of D channels (D % 16 == 0) into the main-KV
 * format [J-FP4], [A-NEWS]: E2M1 codes (channel c in the low nibble of byte
 * c/2 when even, the high nibble when odd) with one E4M3 scale per 16
 * channels.  READING (the pages fix the format, not the rounding): a group's
 * scale is the smallest positive finite E4M3 value s with 6 s >= amax, the
 * group's largest magnitude (so nothing clips; above 6 x 448 the scale stays
 * 448 and magnitudes saturate at 6); amax = 0 gives scale byte 0.  Each value
 * takes the E2M1 magnitude nearest to |x| / s, ties to the even code, the
 * sign of x, and no negative zero.  The comparisons |x| against a midpoint
 * times s are exact in double (and in fp32: the products have at most 7
 * significant bits). */
void oracle_fp4_quantize_row(const float* x, int D, uint8_t* codes, uint8_t* scales) {
    /* midpoints between E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 */
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    for (int g = 0; g < D / 16; ++g) {
        double amax = 0.0;
        for (int c = 16 * g; c < 16 * g + 16; ++c) amax = fmax(amax, fabs((double)x[c]));
        int sb = 0;
        if (amax > 0.0) {
            sb = 0x7E;   /* 448, the largest finite E4M3 value */
            for (int b = 1; b <= 0x7E; ++b)
                if (6.0 * oracle_e4m3(b) >= amax) { sb = b; break; }
        }
        scales[g] = (uint8_t)sb;
        const double sc = oracle_e4m3(sb);
        for (int c = 16 * g; c < 16 * g + 16; ++c) {
            const double a = fabs((double)x[c]);
            int mag = 0;
            if (sc > 0.0)
                for (int k = 0; k < 7; ++k) {
                    const double t = mid[k] * sc;   /* between magnitude codes k and k+1 */
                    if (a > t || (a == t && (k + 1) % 2 == 0)) mag = k + 1;
                }
            const int code = mag == 0 ? 0 : ((x[c] < 0.0f ? 8 : 0) | mag);
            if (c % 2 == 0) codes[c / 2] = (uint8_t)code;
            else codes[c / 2] = (uint8_t)(codes[c / 2] | (code << 4));
        }
    }
}

/* E4M3FN encoding of one fp32 value for the FP8 window (jaehun.me review,
 * section "3) FP4 main KV + SWA Bounded Replay": the 128-token window is kept
 * in FP8).  READING (the pages give no rounding rule): the nearest E4M3FN
 * value, ties to the code with an even mantissa (round to nearest even), the
 * sign of x kept (a negative value that rounds to zero gives 0x80), and
 * magnitudes beyond 448, the largest finite value, saturate to 448 instead of
 * becoming NaN.  Brute force over the 127 non-negative finite codes, in
 * double (every E4M3 value and every fp32 input are exact there). */
uint8_t oracle_e4m3_encode(float x) {
    const double a = fabs((double)x);
    const int sign = signbit(x) ? 0x80 : 0;
    if (a >= 448.0) return (uint8_t)(0x7E | sign);   /* 448 is the nearest finite value */
    int best = 0;
    double bd = a;                           /* distance to code 0 */
    /* below 448 the distances to the two neighbours of a are exact in double,
     * and every other value is farther by at least an E4M3 step */
    for (int b = 1; b <= 0x7E; ++b) {
        const double d = fabs(a - oracle_e4m3(b));
        if (d < bd || (d == bd && (b & 1) == 0 && (best & 1) == 1)) { best = b; bd = d; }
    }
    return (uint8_t)(best | sign);
}

/* Window ring update (same section: the window holds the W most recent
 * tokens).  READING: sequence b keeps W slots [W, D]; the token at position
 * pos[b] goes to slot pos[b] mod W, so after position p the ring holds
 * exactly the tokens max(0, p - W + 1) .. p, in slot order rather than
 * position order (attention over the window does not depend on the order).
 * A negative position (no token) appends nothing.
 * k_new, v_new [B, D] fp32; swa_k, swa_v [B, W, D] E4M3 bytes. */
void oracle_swa_append(const float* k_new, const float* v_new, const int64_t* pos, int B, int D,
                       int W, uint8_t* swa_k, uint8_t* swa_v) {
    for (int b = 0; b < B; ++b) {
        if (pos[b] < 0) continue;
        const size_t row = ((size_t)b * W + (size_t)(pos[b] % W)) * D;
        for (int c = 0; c < D; ++c) {
            swa_k[row + c] = oracle_e4m3_encode(k_new[(size_t)b * D + c]);
            swa_v[row + c] = oracle_e4m3_encode(v_new[(size_t)b * D + c]);
        }
    }
}

/* ----------------------------------------------------------------- scores */

/* Indexer score of one query against one key row.
 * READING (the pages give no formula): the plain sum over the Hi indexer
 * heads of the per-head dot products; no weights, activation or scale.  Key
 * rows hold Hk heads; query head h uses key head h mod Hk (Hk = 1 is a key
 * shared by all heads). */
double oracle_score(const float* qI, const float* krow, int Hi, int Hk, int Di) {
    double s = 0.0;
    for (int h = 0; h < Hi; ++h) {
        const float* k = krow + (size_t)(h % Hk) * Di;
        const float* q = qI + (size_t)h * Di;
        for (int d = 0; d < Di; ++d) s += (double)q[d] * (double)k[d];
    }
    return s;
}

/* -------------------------------------------------------------- selection */

typedef struct {
    double s;
    int64_t id;
} cand_t;

/* Rank order of every selection: higher score first; among equal scores the
 * lower index first.  READING: the pages state no tie rule; the lower index
 * wins, which makes the selected set unique. */
static int by_rank(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int by_value_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Keep the first min(k, n) candidates of the rank order and write their ids
 * in ascending order, padding the k slots with -1.  READING: the pages do not
 * say in which order indices are handed on; ascending is used. */
static void select_topk(cand_t* c, int64_t n, int k, int32_t* out) {
    qsort(c, (size_t)n, sizeof(cand_t), by_rank);
    int take = (n < k) ? (int)n : k;
    for (int i = 0; i < take; ++i) out[i] = (int32_t)c[i].id;
    qsort(out, (size_t)take, sizeof(int32_t), by_value_i32);
    for (int i = take; i < k; ++i) out[i] = -1;
}

/* An indexer-key cache: rows of Hk*Di values, stored either as fp32 or, in
 * the compact form, as one E4M3FN byte per value; exactly one of the two
 * pointers is set.  READING: the pages give no storage format for indexer
 * keys; a compact cache holds plain E4M3FN values with no scale (integers of
 * magnitude up to 16 are exact in it). */
typedef struct {
    const float* f32;
    const uint8_t* e4m3;
    float dec[256];   /* oracle_e4m3 of every byte, filled by keys_e4m3() */
} keys_t;

static keys_t keys_f32(const float* kI) {
    keys_t k;
    k.f32 = kI;
    k.e4m3 = NULL;
    return k;
}

static keys_t keys_e4m3(const uint8_t* kI) {
    keys_t k;
    k.f32 = NULL;
    k.e4m3 = kI;
    for (int b = 0; b < 256; ++b) k.dec[b] = (float)oracle_e4m3(b);
    return k;
}

/* Key row r (absolute row number) as fp32 values: the fp32 cache is read in
 * place, E4M3 bytes are decoded into buf (every E4M3FN value is exact in
 * fp32). */
static const float* key_row(const keys_t* k, int64_t r, int RW, float* buf) {
    if (k->f32) return k->f32 + (size_t)r * RW;
    for (int i = 0; i < RW; ++i) buf[i] = k->dec[k->e4m3[(size_t)r * RW + i]];
    return buf;
}

/* Full mode [J-CSA2], [J-EX]: score every visible entry t < q_nvis[q] of the
 * query's sequence and keep the Top-K.  With pool_blocks > 0 it also builds
 * the candidate pool [J-CSA2]: entries are grouped into aligned blocks
 * [b*bs, b*bs + bs); READING: a block scores the maximum of its visible
 * entries' scores (block_rule 0; block_rule 1, a variant: their sum), and the
 * top pool_blocks blocks (ties to the lower block id) form the pool, written
 * ascending and padded with -1.
 * Index arrays are local to the sequence.  Returns 0, or -1 on a bad
 * argument. */
static int index_full(const float* qI, const keys_t* kI, const int64_t* seq_row_off,
                      const int32_t* q_seq, const int32_t* q_nvis, int Q, int Hi, int Hk, int Di,
                      int topk, int32_t* topk_idx, int pool_blocks, int block_size,
                      int32_t* pool_idx, int block_rule) {
    if (Q < 0 || Hi <= 0 || Hk <= 0 || Di <= 0 || topk < 0 || pool_blocks < 0) return -1;
    if (pool_blocks > 0 && block_size <= 0) return -1;
    if (block_rule != 0 && block_rule != 1) return -1;
    const int RW = Hk * Di;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int q = 0; q < Q; ++q) {
        int64_t n = q_nvis[q];
        const int64_t row0 = seq_row_off[q_seq[q]];
        cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
        float* buf = (float*)malloc(sizeof(float) * (size_t)RW);
        if (!c || !buf) { free(c); free(buf); bad = 1; continue; }
        for (int64_t t = 0; t < n; ++t) {
            c[t].s = oracle_score(qI + (size_t)q * Hi * Di, key_row(kI, row0 + t, RW, buf), Hi, Hk,
                                  Di);
            c[t].id = t;
        }
        free(buf);
        if (pool_blocks > 0) {
            int64_t nb = (n + block_size - 1) / block_size;
            cand_t* b = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nb > 0 ? nb : 1));
            if (!b) { free(c); bad = 1; continue; }
            for (int64_t j = 0; j < nb; ++j) {
                double m = block_rule == 0 ? -INFINITY : 0.0;
                for (int64_t t = j * block_size; t < (j + 1) * block_size && t < n; ++t) {
                    if (block_rule == 0) {
                        if (c[t].s > m) m = c[t].s;
                    } else {
                        m += c[t].s;
                    }
                }
                b[j].s = m;
                b[j].id = j;
            }
            select_topk(b, nb, pool_blocks, pool_idx + (size_t)q * pool_blocks);
            free(b);
        }
        if (topk > 0) select_topk(c, n, topk, topk_idx + (size_t)q * topk);
        free(c);
    }
    return bad ? -1 : 0;
}

int oracle_index_full(const float* qI, const float* kI, const int64_t* seq_row_off,
                      const int32_t* q_seq, const int32_t* q_nvis, int Q, int Hi, int Hk, int Di,
                      int topk, int32_t* topk_idx, int pool_blocks, int block_size,
                      int32_t* pool_idx) {
    keys_t k = keys_f32(kI);
    return index_full(qI, &k, seq_row_off, q_seq, q_nvis, Q, Hi, Hk, Di, topk, topk_idx,
                      pool_blocks, block_size, pool_idx, 0);
}

/* The Full mode with a choice of key cache (key_format 0: fp32 rows at kI,
 * 1: E4M3FN bytes) and of block score (block_rule 0: maximum, 1: sum of the
 * block's visible entries' scores). */
int oracle_index_full_ex(const float* qI, const void* kI, int key_format,
                         const int64_t* seq_row_off, const int32_t* q_seq, const int32_t* q_nvis,
                         int Q, int Hi, int Hk, int Di, int topk, int32_t* topk_idx,
                         int pool_blocks, int block_size, int32_t* pool_idx, int block_rule) {
    if (key_format != 0 && key_format != 1) return -1;
    keys_t k = key_format == 0 ? keys_f32((const float*)kI) : keys_e4m3((const uint8_t*)kI);
    return index_full(qI, &k, seq_row_off, q_seq, q_nvis, Q, Hi, Hk, Di, topk, topk_idx,
                      pool_blocks, block_size, pool_idx, block_rule);
}

/* Reindex mode [J-CSA2], [J-EX]: the candidates are the visible positions of
 * the pool's blocks, {b*bs + j : b in the pool row (b >= 0), j < bs,
 * b*bs + j < q_nvis[q]}; they are rescored with this layer's own indexer
 * query against the shared key cache and the Top-K taken, ties to the lower
 * entry index.  READING: the keys are the Full layer's indexer-key cache. */
static int reindex(const float* qI, const keys_t* kI, const int64_t* seq_row_off, const int32_t* q_seq,
                   const int32_t* q_nvis, const int32_t* pool_idx, int pool_blocks,
                   int block_size, int Q, int Hi, int Hk, int Di, int topk, int32_t* topk_idx) {
    if (Q < 0 || Hi <= 0 || Hk <= 0 || Di <= 0 || topk < 0 || pool_blocks < 0 || block_size <= 0)
        return -1;
    const int RW = Hk * Di;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int q = 0; q < Q; ++q) {
        int64_t n = q_nvis[q];
        const int64_t row0 = seq_row_off[q_seq[q]];
        cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)pool_blocks * block_size + 1);
        float* buf = (float*)malloc(sizeof(float) * (size_t)RW);
        if (!c || !buf) { free(c); free(buf); bad = 1; continue; }
        int64_t m = 0;
        for (int j = 0; j < pool_blocks; ++j) {
            int64_t b = pool_idx[(size_t)q * pool_blocks + j];
            if (b < 0) continue;
            for (int i = 0; i < block_size; ++i) {
                int64_t t = b * block_size + i;
                if (t >= n) break;
                c[m].s = oracle_score(qI + (size_t)q * Hi * Di, key_row(kI, row0 + t, RW, buf), Hi,
                                      Hk, Di);
                c[m].id = t;
                ++m;
            }
        }
        free(buf);
        if (topk > 0) select_topk(c, m, topk, topk_idx + (size_t)q * topk);
        free(c);
    }
    return bad ? -1 : 0;
}

int oracle_reindex(const float* qI, const float* kI, const int64_t* seq_row_off,
                   const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_idx,
                   int pool_blocks, int block_size, int Q, int Hi, int Hk, int Di, int topk,
                   int32_t* topk_idx) {
    keys_t k = keys_f32(kI);
    return reindex(qI, &k, seq_row_off, q_seq, q_nvis, pool_idx, pool_blocks, block_size, Q, Hi,
                   Hk, Di, topk, topk_idx);
}

/* The same Reindex mode over a compact key cache of E4M3FN bytes. */
int oracle_reindex_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                        const int32_t* q_seq, const int32_t* q_nvis, const int32_t* pool_idx,
                        int pool_blocks, int block_size, int Q, int Hi, int Hk, int Di, int topk,
                        int32_t* topk_idx) {
    keys_t k = keys_e4m3(kI);
    return reindex(qI, &k, seq_row_off, q_seq, q_nvis, pool_idx, pool_blocks, block_size, Q, Hi,
                   Hk, Di, topk, topk_idx);
}

/* -------------------------------------------------------------- attention */

/* Softmax attention of one query head over nk keys/values (rows of length D,
 * already decoded to double): z_j = scale * q.k_j, o = sum_j e^{z_j} v_j /
 * sum_j e^{z_j}, evaluated with the maximum subtracted.  lse = log sum e^{z_j}.
 * No key at all gives o = 0 and lse = -inf. */
static void attend(const float* q, const double* keys, const double* vals, int nk, int D,
                   double scale, float* out, float* lse, double* z) {
    if (nk == 0) {
        for (int c = 0; c < D; ++c) out[c] = 0.0f;
        if (lse) *lse = -INFINITY;
        return;
    }
    double zmax = -INFINITY;
    for (int j = 0; j < nk; ++j) {
        double s = 0.0;
        for (int c = 0; c < D; ++c) s += (double)q[c] * keys[(size_t)j * D + c];
        z[j] = scale * s;
        if (z[j] > zmax) zmax = z[j];
    }
    double l = 0.0;
    for (int j = 0; j < nk; ++j) {
        z[j] = exp(z[j] - zmax);
        l += z[j];
    }
    for (int c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int j = 0; j < nk; ++j) acc += z[j] * vals[(size_t)j * D + c];
        out[c] = (float)(acc / l);
    }
    if (lse) *lse = (float)(zmax + log(l));
}

/* Gathers the key set of one query: the selected main-KV rows (key = value =
 * the dequantised row, [J-FP4], [J-EX]) followed by the window tokens (their
 * own FP8 K and V, [J-FP4]).  READING: one softmax over the union of both
 * sets ([A-NEWS]: the window and the global sparse retrieval form one
 * attention); an entry present in both sets is counted twice. */
static int gather_keys(const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t row0,
                       const int32_t* idx, int topk, const uint8_t* wk, const uint8_t* wv,
                       int nwin, int D, double* keys, double* vals) {
    int nk = 0;
    for (int i = 0; i < topk; ++i) {
        if (idx[i] < 0) continue;
        int64_t r = row0 + idx[i];
        oracle_dequant_row(kv_codes + (size_t)r * (D / 2), kv_scales + (size_t)r * (D / 16), D,
                           keys + (size_t)nk * D);
        memcpy(vals + (size_t)nk * D, keys + (size_t)nk * D, sizeof(double) * D);
        ++nk;
    }
    for (int w = 0; w < nwin; ++w) {
        for (int c = 0; c < D; ++c) {
            keys[(size_t)nk * D + c] = oracle_e4m3(wk[(size_t)w * D + c]);
            vals[(size_t)nk * D + c] = oracle_e4m3(wv[(size_t)w * D + c]);
        }
        ++nk;
    }
    return nk;
}

/* Decode attention of one CSA2 layer (Full, Reindex or Reuse alike: the mode
 * only decides where topk_idx comes from [J-CSA2], [J-EX]).  Sequence b has
 * query heads q[b][H][D], main-KV rows seq_row_off[b] + topk_idx[b][i]
 * (-1 entries skipped) and window rows swa_k/swa_v[b][w][D] for
 * w < swa_len[b] (order inside the window is irrelevant to softmax).
 * out[b][H][D]; lse[b][H] when not NULL. Returns 0, or -1 on a bad argument. */
int oracle_attn_decode(const float* q, const uint8_t* kv_codes, const uint8_t* kv_scales,
                       const int64_t* seq_row_off, const int32_t* topk_idx, int topk,
                       const uint8_t* swa_k, const uint8_t* swa_v, const int32_t* swa_len, int W,
                       int B, int H, int D, float softmax_scale, float* out, float* lse) {
    if (B < 0 || H <= 0 || D <= 0 || D % 16 != 0 || topk < 0 || W < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        int nwin = swa_len[b] < W ? swa_len[b] : W;
        if (nwin < 0) nwin = 0;
        size_t cap = (size_t)topk + (size_t)nwin;
        double* keys = (double*)malloc(sizeof(double) * (cap + 1) * D);
        double* vals = (double*)malloc(sizeof(double) * (cap + 1) * D);
        double* z = (double*)malloc(sizeof(double) * (cap + 1));
        if (!keys || !vals || !z) { free(keys); free(vals); free(z); bad = 1; continue; }
        int nk = gather_keys(kv_codes, kv_scales, seq_row_off[b], topk_idx + (size_t)b * topk, topk,
                             swa_k + (size_t)b * W * D, swa_v + (size_t)b * W * D, nwin, D, keys,
                             vals);
        for (int h = 0; h < H; ++h)
            attend(q + ((size_t)b * H + h) * D, keys, vals, nk, D, (double)softmax_scale,
                   out + ((size_t)b * H + h) * D, lse ? lse + (size_t)b * H + h : NULL, z);
        free(keys); free(vals); free(z);
    }
    return bad ? -1 : 0;
}

/* Prefill chunk of one sequence: query i sits at position p = p0 + i and is
 * exactly a decode query with idx row i and the window of the W tokens ending
 * at p ([J-FP4]: n_win = 128) that have position >= 0.  swa_k/swa_v hold
 * rows for positions p0 - W + 1 ... p0 + Qn - 1, so query i uses rows
 * i ... i + W - 1.  kv rows are this sequence's rows. */
int oracle_attn_prefill(const float* q, int64_t p0, const uint8_t* kv_codes,
                        const uint8_t* kv_scales, const int32_t* topk_idx, int topk,
                        const uint8_t* swa_k, const uint8_t* swa_v, int W, int Qn, int H, int D,
                        float softmax_scale, float* out, float* lse) {
    if (Qn < 0 || H <= 0 || D <= 0 || D % 16 != 0 || topk < 0 || W <= 0 || p0 < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < Qn; ++i) {
        int64_t p = p0 + i;
        /* first window row with position >= 0: position of row r is p0-W+1+r */
        int64_t r0 = i, r1 = (int64_t)i + W; /* rows [r0, r1) */
        int64_t first_valid = (W - 1) - p0; /* row of position 0 */
        if (r0 < first_valid) r0 = first_valid;
        int nwin = (int)(r1 - r0);
        (void)p;
        size_t cap = (size_t)topk + (size_t)W;
        double* keys = (double*)malloc(sizeof(double) * (cap + 1) * D);
        double* vals = (double*)malloc(sizeof(double) * (cap + 1) * D);
        double* z = (double*)malloc(sizeof(double) * (cap + 1));
        if (!keys || !vals || !z) { free(keys); free(vals); free(z); bad = 1; continue; }
        int nk = gather_keys(kv_codes, kv_scales, 0, topk_idx + (size_t)i * topk, topk,
                             swa_k + (size_t)r0 * D, swa_v + (size_t)r0 * D, nwin, D, keys, vals);
        for (int h = 0; h < H; ++h)
            attend(q + ((size_t)i * H + h) * D, keys, vals, nk, D, (double)softmax_scale,
                   out + ((size_t)i * H + h) * D, lse ? lse + (size_t)i * H + h : NULL, z);
        free(keys); free(vals); free(z);
    }
    return bad ? -1 : 0;
}

/* Scores of query q against all of its visible entries (double), for tests. */
int oracle_scores(const float* qI, const float* kI, const int64_t* seq_row_off,
                  const int32_t* q_seq, const int32_t* q_nvis, int q, int Hi, int Hk, int Di,
                  double* out) {
    const float* base = kI + (size_t)seq_row_off[q_seq[q]] * Hk * Di;
    for (int64_t t = 0; t < q_nvis[q]; ++t)
        out[t] = oracle_score(qI + (size_t)q * Hi * Di, base + (size_t)t * Hk * Di, Hi, Hk, Di);
    return 0;
}

int oracle_scores_e4m3(const float* qI, const uint8_t* kI, const int64_t* seq_row_off,
                       const int32_t* q_seq, const int32_t* q_nvis, int q, int Hi, int Hk, int Di,
                       double* out) {
    keys_t k = keys_e4m3(kI);
    const int RW = Hk * Di;
    float* buf = (float*)malloc(sizeof(float) * (size_t)RW);
    if (!buf) return -1;
    for (int64_t t = 0; t < q_nvis[q]; ++t)
        out[t] = oracle_score(qI + (size_t)q * Hi * Di,
                              key_row(&k, seq_row_off[q_seq[q]] + t, RW, buf), Hi, Hk, Di);
    free(buf);
    return 0;
}

#ifdef _OPENMP
#include <omp.h>
#endif

/* Thread control for timing runs (queries are independent, so the number of
 * threads never changes a result). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
