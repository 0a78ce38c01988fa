#pragma once
// Host/device declarations of the backward of the chunked forward: argument
// block, workspace layout and launcher. Kept apart from the forward's
// declarations so that the forward kernels do not depend on it.

#include "kda_internal.h"

namespace kda {

// Backward of the chunked forward (kBwdChunk-token chunks; fp32 states and
// accumulation, matrix-core operands in the input precision).
constexpr int kBwdChunk = 32;
struct BwdArgs {
    const void* q; const void* k; const void* v; const void* z; const void* beta_raw;
    const float* A_log; const float* S0; const void* dout; const float* dS_T;
    void* dq; void* dk; void* dv; void* dz; void* dbeta_raw; float* dA_log; float* dS0;
    unsigned char* ops; float* states; float* adj; float* dA_part;  // workspace regions
    // per chunk-head, from the serial passes to the gradient kernel: E = V - Kd S and
    // U (eu, two [C x Dv] matrices), W = T^T dU (w, one), in fragment order:
    // element ((strip * 2 + tb) * 64 + lane) * 4 + i is row 16 tb + 4 (lane / 16) + i,
    // column 16 strip + lane % 16
    float* eu; float* w;
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
// Bytes of the per-chunk operator block for operand elements of eb bytes (4
// for fp32 inputs, 2 for bf16) and key dimension DK: the state pass's region,
// the adjoint pass's region (operand tiles of 16 rows x 32 contraction slots,
// 512 elements each, plus gamma and beta in fp32; each region a whole number
// of KiB) and the row-major fp32 At.
__host__ __device__ constexpr size_t bwd_tile_bytes(size_t rows, size_t kext, size_t eb) {
    return rows / 16 * ((kext + 31) / 32) * 512 * eb;
}
__host__ __device__ constexpr size_t bwd_region_s_bytes(size_t eb, int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_tile_bytes(C, DK, eb) + bwd_tile_bytes(DK, C, eb) + bwd_tile_bytes(C, C, eb) + (DK + C) * 4,
                    1024);
}
__host__ __device__ constexpr size_t bwd_region_a_bytes(size_t eb, int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_tile_bytes(C, DK, eb) + 2 * bwd_tile_bytes(DK, C, eb) + 2 * bwd_tile_bytes(C, C, eb) +
                    (DK + C) * 4, 1024);
}
__host__ __device__ constexpr size_t bwd_op_bytes(size_t eb, int DK) {
    const size_t C = kBwdChunk;
    return round_up(bwd_region_s_bytes(eb, DK) + bwd_region_a_bytes(eb, DK) + C * C * 4, 1024);
}
hipError_t launch_chunk_bwd(int dt, int DK, const BwdArgs& a, hipStream_t s);

}  // namespace kda
