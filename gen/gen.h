/*
 * Seeded synthetic-input generator, shared by the CPU oracle side and the
 * GPU side of the tests and the benchmark.  It holds none of the method's
 * arithmetic: it only turns (seed, tensor id, element index) into integers,
 * FP4 code bytes and power-of-two E4M3 scale bytes.
 *
 * Hash: the SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to the counter
 *     z = (seed << 56) | (tensor << 48) | i          (i < 2^48)
 * Range reduction: r = ((h >> 32) * n) >> 32, uniform on [0, n) (Lemire's
 * multiply-shift).
 *
 *   ints     : value = lo + r,  n = hi - lo + 1, stored as fp32
 *   fp4 bytes: nibble k (k = 2*byte + {0 low, 1 high}) draws r on [0,15);
 *              code = r (r <= 7) else r + 1, i.e. every 4-bit code except
 *              0x8 (negative zero), uniformly
 *   scales   : k = kmin + r, n = kmax - kmin + 1; byte = (k + 7) << 3, the
 *              E4M3FN encoding of 2^k (exponent bias 7, zero mantissa)
 *
 * The host functions below are plain C (OpenMP over elements); the device
 * functions (gen_dev_*) fill device memory with the same values.
 */
#ifndef CSA2_GEN_H
#define CSA2_GEN_H
#include <stdint.h>
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

uint64_t gen_hash(uint64_t seed, uint64_t tensor, uint64_t i);

/* out[j] = integer drawn for element start+j, as float */
void gen_host_ints(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                   int32_t lo, int32_t hi, float* out);
/* out[j] = two FP4 codes for nibbles 2(start+j), 2(start+j)+1 */
void gen_host_fp4(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint8_t* out);
/* out[j] = E4M3FN byte of 2^k, k drawn for element start+j */
void gen_host_pow2_scales(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                          int32_t kmin, int32_t kmax, uint8_t* out);

/* The same values for `nruns` runs of `run` elements each, run r starting at
 * element starts[r]; out holds the runs back to back (nruns * run values).
 * Regenerates scattered slices (a query's pool blocks, its selected rows). */
void gen_host_ints_runs(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nruns,
                        int64_t run, int32_t lo, int32_t hi, float* out);
void gen_host_fp4_runs(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nruns,
                       int64_t run, uint8_t* out);
void gen_host_pow2_scales_runs(uint64_t seed, uint64_t tensor, const int64_t* starts,
                               int64_t nruns, int64_t run, int32_t kmin, int32_t kmax,
                               uint8_t* out);

/* Device fills: same values, written asynchronously on `stream`.  Return 0 on
 * success, otherwise the hipError_t of the launch. */
int gen_dev_ints(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                 int32_t lo, int32_t hi, float* out, void* stream);
int gen_dev_fp4(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint8_t* out,
                void* stream);
int gen_dev_pow2_scales(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                        int32_t kmin, int32_t kmax, uint8_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif
