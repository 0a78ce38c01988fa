// kda_internal.h - host/device shared sizes and the internal launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum : unsigned { kQkL2 = 1u, kBetaSig = 2u, kGateIn = 4u, kGateSoftplus = 8u };

// Per chunk-head block of intermediates written by the intra kernel and read
// by the inter kernel.  All matrices are stored as fragment-major tiles of
// 64 lanes x 8 elements (see kda_device.h), in the operand element type:
//   Kd  = K_hat * exp(G)           [C x Dk]   tiles (token block, channel step)
//   Qp  = Q_hat * exp(G)           [C x Dk]   tiles (token block, channel step)
//   KpT = (K_hat * exp(G_C - G))^T [Dk x C]   tiles (channel block, token step)
//   Tb  = (I + A_kk)^-1 Diag(beta) [C x C]    tiles (token block, token step)
//   Aqk = tril(Q K^T with decay)   [C x C]    tiles (token block, token step)
// followed by gamma = exp(G_C) [Dk] in fp32.  No tile that is zero by
// construction is stored: of Tb and Aqk only the steps s with 2 s <= Ib, and
// the step 2 s == Ib (whose second 16 tokens lie above the diagonal) as a
// half tile of 64 lanes x 4 elements (the fragment's slots 0..3); of KpT a
// step whose second 16 tokens lie past the chunk (C = 16) as a half tile.
__host__ __device__ constexpr bool tri_half(int Ib, int s) { return 2 * s == Ib; }
// element offset of stored tile (Ib, s), 2 s <= Ib, of a Tb / Aqk area
__host__ __device__ constexpr size_t tri_offset(int Ib, int s, int ksc) {
    size_t off = 0;
    for (int i = 0; i < Ib; ++i)
        for (int t = 0; t < ksc; ++t)
            if (2 * t <= i) off += (2 * t == i) ? 256 : 512;
    for (int t = 0; t < s; ++t)
        if (2 * t <= Ib) off += (2 * t == Ib) ? 256 : 512;
    return off;
}
__host__ __device__ constexpr bool kpt_half(int s, int nbk) { return 2 * s + 1 >= nbk; }
// element offset of KpT tile (R, s)
__host__ __device__ constexpr size_t kpt_offset(int R, int s, int ksc, int nbk) {
    size_t row = 0;
    for (int t = 0; t < ksc; ++t) row += kpt_half(t, nbk) ? 256 : 512;
    size_t off = (size_t)R * row;
    for (int t = 0; t < s; ++t) off += kpt_half(t, nbk) ? 256 : 512;
    return off;
}

struct BlockLayout {
    int nbk, ksd, nbd, ksc;
    size_t kd, qp, kpt, tb, aqk, end;   // element offsets
    size_t gamma_byte, bytes;
};

__host__ __device__ constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ constexpr BlockLayout block_layout(int elem_bytes, int DK, int C) {
    BlockLayout L{};
    L.nbk = C / 16;
    L.ksd = (DK + 31) / 32;
    L.nbd = DK / 16;
    L.ksc = (C + 31) / 32;
    const size_t tile = 512;
    L.kd = 0;
    L.qp = L.kd + (size_t)L.nbk * L.ksd * tile;
    L.kpt = L.qp + (size_t)L.nbk * L.ksd * tile;
    L.tb = L.kpt + kpt_offset(L.nbd, 0, L.ksc, L.nbk);
    L.aqk = L.tb + tri_offset(L.nbk, 0, L.ksc);
    L.end = L.aqk + tri_offset(L.nbk, 0, L.ksc);
    L.gamma_byte = L.end * (size_t)elem_bytes;
    L.bytes = round_up(L.gamma_byte + (size_t)DK * 4, 256);
    return L;
}

// Chunks per slice of the sequence: intra and inter kernels alternate over
// slices whose chunk blocks take at most kSliceBytes.  Measured on MI355X,
// smaller slices (64-128 MB) lose more to partial grids and per-launch
// prologues than they gain, so the layer-sized workloads run as one slice.
constexpr size_t kSliceBytes = 1ull << 30;

inline int slice_chunks(int BH, int NC, size_t block_bytes, size_t budget = kSliceBytes) {
    if (NC <= 0) return 0;
    size_t per = budget / ((size_t)(BH > 0 ? BH : 1) * (block_bytes > 0 ? block_bytes : 1));
    if (per < 1) per = 1;
    const int nsl = (int)((NC + per - 1) / per);
    return (NC + nsl - 1) / nsl;
}

// Workspace: nbuf buffers of `per` chunk blocks for every (b, h), then the
// running state carried between slices (S [BH, Dk, Dv] and M [BH, Dk, Dk]).
__host__ __device__ constexpr size_t chunk_workspace_bytes(int elem_bytes, int DK, int Dv, int C, size_t BH,
                                                           size_t per, size_t nbuf) {
    return nbuf * BH * per * block_layout(elem_bytes, DK, C).bytes + round_up(BH * (size_t)DK * (DK + Dv) * 4, 256);
}

// Workgroups that can share a head's value columns in the fused output side
// (one per 16 value columns or more, Dv <= 128).
constexpr int kGateGroups = 8;
// Workspace of the layer body: that of the chunk call, then the output side's
// exchange area, kGateGroups x C floats per chunk-head of a slice.
__host__ __device__ constexpr size_t layer_gss_offset(int elem_bytes, int DK, int Dv, int C, size_t BH, size_t per) {
    return chunk_workspace_bytes(elem_bytes, DK, Dv, C, BH, per, 1);
}
__host__ __device__ constexpr size_t layer_workspace_bytes(int elem_bytes, int DK, int Dv, int C, size_t BH,
                                                           size_t per) {
    return layer_gss_offset(elem_bytes, DK, Dv, C, BH, per) + round_up(BH * per * (size_t)kGateGroups * C * 4, 256);
}

struct StepArgs {
    const void* q; const void* k; const void* v; const void* z; const void* beta_raw;
    const float* A_log; float* S; void* o;
    int B, H; float g_min; unsigned flags;   // H: value heads
    int G = 1;                        // value heads per q/k head
    const float* dt_bias = nullptr;   // [H, Dk] gate bias
};

struct ChunkArgs {
    const void* q; const void* k; const void* v; const void* z; const void* beta_raw;
    const float* A_log; const float* S0;
    void* o; float* S_out; float* M_out; void* P_out;
    void* ws; size_t ws_bytes;
    int B, T, H, Dv, NC;   // H: value heads
    float g_min; unsigned flags;
    int G = 1;                        // value heads per q/k head
    const float* dt_bias = nullptr;   // [H, Dk] gate bias
    bool wide_decay = false;          // decays may leave the factored range: the GENERAL intra kernel
    size_t slice_budget = kSliceBytes;  // bytes of chunk blocks per slice of the sequence
    // fused input-side convolution: q, k and v are the raw inputs of
    // SiLU(ShortConv_4(.)); taps [Hk Dk + Hk Dk + H Dv][4] fp32 in the order q,
    // k, v channels, biases of the same channels (nullable), carried window
    // [B][3][channels] in the input type (nullable: zeros).  conv_w NULL: none.
    const float* conv_w = nullptr;
    const float* conv_b = nullptr;
    const void* conv_state = nullptr;
    // fused output side (launch_layer): o receives
    // sigmoid(gate) * o / sqrt(mean o^2 + 1e-6) * gate_w per head row; gate
    // [B,T,H,Dv] in the input type, gate_w [Dv] fp32 or NULL (ones); gss the
    // exchange area of its per-token partial sums (gss_n floats per
    // chunk-head of a slice), set by the launch
    const void* gate = nullptr;
    const float* gate_w = nullptr;
    float* gss = nullptr;
    int gss_n = 0;
};

// Built-in device scratch of the allocation-free chunk entry point (one copy
// per GPU, held until the process ends).
constexpr size_t kScratchBytes = 64ull << 20;
// Device address of the current device's scratch (looked up once per device).
hipError_t scratch_pointer(void** ptr);

struct ComposeArgs {
    const float* M; const float* S_tilde; const float* S_in; float* S_prefix;
    int n_seg, B, H, Dv;
};

struct FixupArgs {
    const void* P; const float* S_in; const float* S_prefix; void* o;
    int n_seg, B, T_seg, H, Dv;
};

// dt: 0 = fp32, 1 = bf16.  Return the launch status (hipSuccess on success).
hipError_t launch_step(int dt, int DK, int DV, const StepArgs& a, hipStream_t s);
// ev (nullable, n_ev events): ev[0] is recorded before the first kernel and
// ev[k + 1] after kernel k, on the same stream (kernels alternate intra,
// inter over the slices of the sequence; events past n_ev are skipped).
hipError_t launch_chunk(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s, hipEvent_t* ev, int n_ev);
// Kernels one kda_chunk_fwd call launches for these sizes.
int chunk_kernel_count(int elem_bytes, int DK, int C, int BH, int NC);
// The intra-chunk kernel alone, over chunks [c0, c0 + nc) into `buf` of `per`
// chunk blocks per (b, h) (with the exchange area marks of a.gss, if set).
hipError_t launch_chunk_intra(int dt, int DK, int C, const ChunkArgs& a, void* buf, int per, int c0, int nc,
                              hipStream_t s);
// The layer body: the chunk kernels with the output side applied to o (a.gate
// set; a.o receives y).  The workspace is layer_workspace_bytes.
hipError_t launch_layer(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s);
hipError_t launch_compose(int DK, const ComposeArgs& a, hipStream_t s);
hipError_t launch_fixup(int dt, int DK, const FixupArgs& a, hipStream_t s);

// Input side: causal short convolution (kernel 4) and SiLU over [B, T, C].
struct ShortConvArgs {
    const void* x; const float* w; const float* bias;
    const void* state_in; void* state_out; void* y;
    int B, T, C, silu;
};
int short_conv_tile();  // tokens per thread; an in-place window needs T <= this
hipError_t launch_short_conv(int dt, const ShortConvArgs& a, hipStream_t s);

// Output side: per-head RMS normalisation under a sigmoid gate, rows of DV.
struct GateArgs {
    const void* o; const void* gate; const float* weight; void* y;
    size_t rows;
};
hipError_t launch_output_gate(int dt, int DV, const GateArgs& a, hipStream_t s);

}  // namespace kda
