/* Host half of the seeded input generator (definitions in gen.h). */
#include "gen.h"

uint64_t gen_hash(uint64_t seed, uint64_t tensor, uint64_t i) {
    uint64_t z = (seed << 56) | ((tensor & 0xFFull) << 48) | (i & 0xFFFFFFFFFFFFull);
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint32_t draw(uint64_t h, uint32_t n) {
    return (uint32_t)(((h >> 32) * (uint64_t)n) >> 32);
}

void gen_host_ints(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                   int32_t lo, int32_t hi, float* out) {
    uint32_t n = (uint32_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j)
        out[j] = (float)(lo + (int32_t)draw(gen_hash(seed, tensor, start + (uint64_t)j), n));
}

static inline uint8_t fp4_code(uint64_t h) {
    uint32_t r = draw(h, 15);
    return (uint8_t)(r <= 7 ? r : r + 1);
}

void gen_host_fp4(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j) {
        uint64_t k = 2 * (start + (uint64_t)j);
        out[j] = (uint8_t)(fp4_code(gen_hash(seed, tensor, k)) |
                           (fp4_code(gen_hash(seed, tensor, k + 1)) << 4));
    }
}

void gen_host_pow2_scales(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                          int32_t kmin, int32_t kmax, uint8_t* out) {
    uint32_t n = (uint32_t)(kmax - kmin + 1);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j) {
        int32_t k = kmin + (int32_t)draw(gen_hash(seed, tensor, start + (uint64_t)j), n);
        out[j] = (uint8_t)((k + 7) << 3);
    }
}

void gen_host_ints_runs(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nruns,
                        int64_t run, int32_t lo, int32_t hi, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nruns; ++r)
        gen_host_ints(seed, tensor, (uint64_t)starts[r], (uint64_t)run, lo, hi, out + r * run);
}

void gen_host_fp4_runs(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nruns,
                       int64_t run, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nruns; ++r)
        gen_host_fp4(seed, tensor, (uint64_t)starts[r], (uint64_t)run, out + r * run);
}

void gen_host_pow2_scales_runs(uint64_t seed, uint64_t tensor, const int64_t* starts,
                               int64_t nruns, int64_t run, int32_t kmin, int32_t kmax,
                               uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nruns; ++r)
        gen_host_pow2_scales(seed, tensor, (uint64_t)starts[r], (uint64_t)run, kmin, kmax,
                             out + r * run);
}
