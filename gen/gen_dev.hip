// Device half of the seeded input generator (definitions in gen.h): fills
// device buffers with exactly the values the host half produces.
#include <hip/hip_runtime.h>
#include "gen.h"

namespace {

__device__ __forceinline__ uint64_t hash_dev(uint64_t seed, uint64_t tensor, uint64_t i) {
    uint64_t z = (seed << 56) | ((tensor & 0xFFull) << 48) | (i & 0xFFFFFFFFFFFFull);
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t draw_dev(uint64_t h, uint32_t n) {
    return (uint32_t)(((h >> 32) * (uint64_t)n) >> 32);
}

__device__ __forceinline__ uint8_t fp4_code_dev(uint64_t h) {
    uint32_t r = draw_dev(h, 15);
    return (uint8_t)(r <= 7 ? r : r + 1);
}

__global__ void k_ints(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                       int32_t lo, uint32_t n, float* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride)
        out[j] = (float)(lo + (int32_t)draw_dev(hash_dev(seed, tensor, start + j), n));
}

__global__ void k_fp4(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count, uint8_t* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride) {
        uint64_t k = 2 * (start + j);
        out[j] = (uint8_t)(fp4_code_dev(hash_dev(seed, tensor, k)) |
                           (fp4_code_dev(hash_dev(seed, tensor, k + 1)) << 4));
    }
}

__global__ void k_scales(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                         int32_t kmin, uint32_t n, uint8_t* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride) {
        int32_t k = kmin + (int32_t)draw_dev(hash_dev(seed, tensor, start + j), n);
        out[j] = (uint8_t)((k + 7) << 3);
    }
}

inline unsigned grid_for(uint64_t count) {
    uint64_t g = (count + 255) / 256;
    if (g > 65536) g = 65536;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" int gen_dev_ints(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                            int32_t lo, int32_t hi, float* out, void* stream) {
    if (count == 0) return 0;
    hipLaunchKernelGGL(k_ints, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, seed,
                       tensor, start, count, lo, (uint32_t)(hi - lo + 1), out);
    return (int)hipGetLastError();
}

extern "C" int gen_dev_fp4(uint64_t seed, uint64_t tensor, uint64_t start, uint64_t count,
                           uint8_t* out, void* stream) {
    if (count == 0) return 0;
    hipLaunchKernelGGL(k_fp4, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, seed,
                       tensor, start, count, out);
    return (int)hipGetLastError();
}

extern "C" int gen_dev_pow2_scales(uint64_t seed, uint64_t tensor, uint64_t start,
                                   uint64_t count, int32_t kmin, int32_t kmax, uint8_t* out,
                                   void* stream) {
    if (count == 0) return 0;
    hipLaunchKernelGGL(k_scales, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, seed,
                       tensor, start, count, kmin, (uint32_t)(kmax - kmin + 1), out);
    return (int)hipGetLastError();
}
