#pragma once
// Host/device declarations of the backward of the chunked forward: argument
// block, workspace layout and launcher. Kept apart from the forward's
// declarations so that the forward kernels do not depend on it.

#include "kda_internal.h"

namespace kda {

// Backward of the chunked forward (fp32 arithmetic, kBwdChunk-token chunks).
constexpr int kBwdChunk = 32;
struct BwdArgs {
    const void* q; const void* k; const void* v; const void* z; const void* beta_raw;
    const float* A_log; const float* S0; const void* dout; const float* dS_T;
    void* dq; void* dk; void* dv; void* dz; void* dbeta_raw; float* dA_log; float* dS0;
    float* ops; float* states; float* adj; float* dA_part;  // workspace regions
    int B, T, H, Dv, NC;
    float g_min;
    unsigned flags;
    // grouped value heads: H value heads read q/k head h / G of H / G; a gate
    // bias [H, DK] on the logit; per-value-head q/k gradients (fp32, [2][B,T,H,DK])
    // summed per group afterwards, and per-chunk bias gradient parts [B NC][H][DK]
    int G = 1;
    const float* dt_bias = nullptr;
    float* ddt_bias = nullptr;
    float* dqk_part = nullptr;
    float* dbias_part = nullptr;
};
// fp32 elements of the per-chunk operator block for a key dimension DK: the
// state pass's region, the adjoint pass's region (operand tiles of 16 rows x
// 32 contraction slots, 512 floats each, plus gamma and beta; each region a
// whole number of KiB) and the row-major At.
__host__ __device__ constexpr size_t bwd_tiles(size_t rows, size_t kext) {
    return rows / 16 * ((kext + 31) / 32) * 512;
}
__host__ __device__ constexpr size_t bwd_op_region_s(int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_tiles(C, DK) + bwd_tiles(DK, C) + bwd_tiles(C, C) + DK + C, 256);
}
__host__ __device__ constexpr size_t bwd_op_region_a(int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_tiles(C, DK) + 2 * bwd_tiles(DK, C) + 2 * bwd_tiles(C, C) + DK + C, 256);
}
__host__ __device__ constexpr size_t bwd_op_floats(int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_op_region_s(DK) + bwd_op_region_a(DK) + C * C, 256);
}
hipError_t launch_chunk_bwd(int dt, int DK, const BwdArgs& a, hipStream_t s);

}  // namespace kda
