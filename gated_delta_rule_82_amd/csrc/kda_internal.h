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
// followed by gamma = exp(G_C) [Dk] in fp32.
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
    L.tb = L.kpt + (size_t)L.nbd * L.ksc * tile;
    L.aqk = L.tb + (size_t)L.nbk * L.ksc * tile;
    L.end = L.aqk + (size_t)L.nbk * L.ksc * tile;
    L.gamma_byte = L.end * (size_t)elem_bytes;
    L.bytes = round_up(L.gamma_byte + (size_t)DK * 4, 256);
    return L;
}

// Chunks per slice of the sequence: intra and inter kernels alternate over
// slices whose chunk blocks take at most kSliceBytes.  Measured on MI355X,
// smaller slices (64-128 MB) lose more to partial grids and per-launch
// prologues than they gain, so the layer-sized workloads run as one slice.
constexpr size_t kSliceBytes = 1ull << 30;

inline int slice_chunks(int BH, int NC, size_t block_bytes) {
    if (NC <= 0) return 0;
    size_t per = kSliceBytes / ((size_t)(BH > 0 ? BH : 1) * (block_bytes > 0 ? block_bytes : 1));
    if (per < 1) per = 1;
    const int nsl = (int)((NC + per - 1) / per);
    return (NC + nsl - 1) / nsl;
}

// Slices of the overlapped schedule (intra of slice s + 1 runs beside inter of
// slice s): two, of at least two chunks, within the slice budget.  Measured on
// MI355X (layer workload), two slices gain about 9 % over one stream while
// four or eight lose: every inter launch refills its LDS ring and reloads the
// state, and the intra kernel only gets the CUs the inter kernel leaves free.
inline int overlap_slice_chunks(int BH, int NC, size_t block_bytes) {
    if (NC <= 0) return 0;
    int per = (NC + 1) / 2;
    if (per < 2) per = 2;
    const int cap = slice_chunks(BH, NC, block_bytes);
    return per < cap ? per : cap;
}

// Workspace: nbuf buffers of `per` chunk blocks for every (b, h), then the
// running state carried between slices (S [BH, Dk, Dv] and M [BH, Dk, Dk]).
__host__ __device__ constexpr size_t chunk_workspace_bytes(int elem_bytes, int DK, int Dv, int C, size_t BH,
                                                           size_t per, size_t nbuf) {
    return nbuf * BH * per * block_layout(elem_bytes, DK, C).bytes + round_up(BH * (size_t)DK * (DK + Dv) * 4, 256);
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
};

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
// Overlapped schedule: intra kernels on `s`, inter kernels on `aux`; sync holds
// 5 events (see kda_chunk_fwd_overlap); tev (nullable, n_tev) gets a start and
// an end event per kernel k at 2k and 2k + 1, recorded on the kernel's stream.
hipError_t launch_chunk_overlap(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s, hipStream_t aux,
                                hipEvent_t* sync, hipEvent_t* tev, int n_tev);
int chunk_overlap_kernel_count(int elem_bytes, int DK, int C, int BH, int NC);
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
