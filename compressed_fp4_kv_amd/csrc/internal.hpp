// Host-side helpers shared by the CSA2 entry points: status plumbing,
// workspace carving and optional per-kernel event timing.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

// Records the HIP error of a failed launch for csa2_last_hip_error().
void set_last_hip_error(hipError_t e);

// Returns CSA2_OK or CSA2_ERR_HIP for the last launch on this thread.
int check_launch();

// Kernel timing hooks (no-ops unless csa2_profile_enable(1)).
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// Linear bump allocator over a caller-provided workspace; every piece is
// 256-byte aligned.  With base == nullptr it only measures.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
    size_t bytes() const { return (off + 255) & ~size_t(255); }
};

// Score stream launcher (stream.hip): key rows of 256 * vpr values (vpr = 1,
// 2 or 4), fp32 (kI a const float*) or E4M3FN bytes (e4m3, kI a const
// uint8_t*); one grid row per query, enough workgroups for max_nvis rows.
// With bkeys set, blocks of 2^bs_log2 rows are scored by the maximum of their
// rows' scores, or by their sum when block_sum is non-zero.
int launch_score_stream(int vpr, bool e4m3, int max_nvis, int Q, hipStream_t s,
                        const float* qI, const void* kI, const int64_t* seq_row_off,
                        const int32_t* q_seq, const int32_t* q_nvis, int Hi, int Hk, int Di,
                        uint32_t* keys, int64_t kstride, uint32_t* hist_e, uint32_t* bkeys,
                        int64_t bstride, int bs_log2, int block_sum, uint32_t* hist_b);

}  // namespace csa2

// Launch helper: kernel<<<grid, block, 0, stream>>>(args...) bracketed by the
// timing hooks; evaluates to the launch status.
#define CSA2_LAUNCH(name, kernel, grid, block, stream, ...)                \
    ([&]() -> int {                                                        \
        ::csa2::prof_begin(name, stream);                                  \
        kernel<<<grid, block, 0, stream>>>(__VA_ARGS__);                   \
        ::csa2::prof_end(stream);                                          \
        return ::csa2::check_launch();                                     \
    }())
