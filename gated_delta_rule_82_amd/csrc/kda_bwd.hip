// kda_bwd.hip - backward of the chunked KDA forward on gfx950.
//
// Gradients of a loss L with dL/do = dout and dL/dS_T = dS_T with respect to
// q, k, v, the gate logit z, beta_raw, A_log and the initial state.  The pages
// do not derive a backward pass; this is the derivative of the chunk form of
// "KDA 模块交互式演示" §1.5 and "Implémenter KDA" 'La forme par blocs'
// (decay first, post-update readout), for chunks of C = 32 tokens with
// incoming state S, cumulative log-decay G, A_kk = Diag(beta) At,
// T = (I + A_kk)^-1:
//
//   E = V - Kd S,  U = T Diag(beta) E,  O = Qp S + Aqk U,
//   S' = Diag(gamma) S + Kp^T U.
//
// Given dO and dS' (the adjoint of S'):
//
//   dU  = Aqk^T dO + Kp dS'        W = T^T dU        dV = Diag(beta) W
//   dS  = Qp^T dO - Kd^T Diag(beta) W + Diag(gamma) dS'
//   dA_kk = -W U^T (strictly lower)     dAqk = dO U^T (lower)
//   dQp = dO S^T,  dKd = -Diag(beta) W S^T,  dKp = U dS'^T,
//   dgamma = rowsum(dS' * S),  dbeta = rowsum(W * E) + rowsum(dA_kk * At)
//
// and the decay-weighted entries of Aqk, At, Kd, Qp, Kp, gamma carry these
// to q_hat, k_hat and G (every exp(+G) factor gives x dx, every exp(-G) factor
// -x dx), G to the per-token log-decay by a reverse cumulative sum, and the
// switched activations (L2 norm, sigmoid beta, gate) to the raw inputs.
//
// Five kernels (matrix-core operands in the input precision, fp32 states and
// accumulation):
//  1. kda_bwd_ops:     per chunk-head, the chunk operators: Aqk and At as
//                      16 x 16 blocks with the decay factored per block, T by
//                      blocked substitution, Kd, Qp, Kp and the transposes as
//                      operand tiles.
//  2. kda_bwd_states:  per (b, h) and 32 value columns, serial over chunks:
//                      the state at each chunk start, and each chunk's E, U.
//  3. kda_bwd_adjoint: the same in reverse: the adjoint at each chunk end,
//                      each chunk's W, and dS0.
//  4. kda_bwd_grads:   per chunk-head: every input gradient of the chunk.
//  5. kda_bwd_dA:      the sum of the per-chunk dA_log parts.
//
// Workgroups share data through LDS only, so their barriers wait for LDS
// operations alone (lds_barrier): global stores drain, and global loads issued
// ahead stay in flight, across them.
#include <type_traits>

#include "kda_device.h"
#include "kda_bwd.h"

namespace kda {

namespace {

constexpr int C = kBwdChunk;

// A 16-token block whose decay on some channel exceeds 2^-kBwdWideLog2 (log2
// units) has its decay-weighted gradient sums taken element by element: the
// factored form's factors reach 2^(kBwdWideLog2 / 2), which leaves 2^48 of the
// fp32 (and bf16) range for the coefficients and the 32-term sums.  Bounded
// gates never reach it (a block spans 15 decay steps, 2^-108 at g_min = -5).
constexpr float kBwdWideLog2 = 160.f;

// Byte offsets of the operator block of one chunk-head, operand tiles in the
// input precision E (fp32 or bf16).  Matrices that serve as matrix-core A
// operands are stored as operand tiles: tile (row block rb, contraction step
// ks) holds 64 lanes x 8 slots, lane 16 gq + r supplying row 16 rb + r at
// contraction index 32 ks + slot_index(gq, j), so a lane reads its fragment as
// 8 contiguous elements (no LDS bank conflicts, whole global lines).
template <typename E, int DK> struct Ops {
    static constexpr size_t eb = sizeof(E);
    // region S (the state pass)
    static constexpr size_t Kd = 0;                                  // tiles [C x DK]   k_hat exp(G)
    static constexpr size_t KpT = Kd + bwd_tile_bytes(C, DK, eb);    // tiles [DK x C]   (k_hat exp(G_C - G))^T
    static constexpr size_t Tm = KpT + bwd_tile_bytes(DK, C, eb);    // tiles [C x C]    (I + Diag(beta) At)^-1
    static constexpr size_t gamS = Tm + bwd_tile_bytes(C, C, eb);    // fp32 [DK]  exp(G_C)
    static constexpr size_t betaS = gamS + DK * 4;                   // fp32 [C]
    static constexpr size_t sizeS = bwd_region_s_bytes(eb, DK);
    // region A (the adjoint pass), offsets from the block start
    static constexpr size_t A0 = sizeS;
    static constexpr size_t Kp = A0;                                 // tiles [C x DK]
    static constexpr size_t QpT = Kp + bwd_tile_bytes(C, DK, eb);    // tiles [DK x C]   (q_hat exp(G))^T
    static constexpr size_t KdT = QpT + bwd_tile_bytes(DK, C, eb);   // tiles [DK x C]
    static constexpr size_t AqkT = KdT + bwd_tile_bytes(DK, C, eb);  // tiles [C x C]    Aqk^T
    static constexpr size_t TT = AqkT + bwd_tile_bytes(C, C, eb);    // tiles [C x C]    T^T
    static constexpr size_t gamA = TT + bwd_tile_bytes(C, C, eb);    // fp32 [DK]
    static constexpr size_t betaA = gamA + DK * 4;                   // fp32 [C]
    static constexpr size_t sizeA = bwd_region_a_bytes(eb, DK);
    // row-major fp32 At (strictly lower, no beta)
    static constexpr size_t At = A0 + sizeA;
    static constexpr size_t bytes = bwd_op_bytes(eb, DK);
    static_assert(betaS + C * 4 <= sizeS && betaA + C * 4 <= A0 + sizeA && At + C * C * 4 <= bytes, "layout");
    static_assert(sizeS % 1024 == 0 && sizeA % 1024 == 0 && bytes % 1024 == 0, "whole KiB regions");
    static __device__ __forceinline__ const E* tiles(const unsigned char* base, size_t off) {
        return reinterpret_cast<const E*>(base + off);
    }
    static __device__ __forceinline__ const float* f32(const unsigned char* base, size_t off) {
        return reinterpret_cast<const float*>(base + off);
    }
};

// Position of element (row, k) in operand tiles with kext contraction indices.
__device__ __forceinline__ size_t tile_pos(int row, int k, int kext) {
    const int ks = k >> 5, kk = k & 31;
    const int grp = kk < 16 ? kk >> 2 : (kk - 16) >> 2;
    const int j = kk < 16 ? (kk & 3) : 4 + (kk & 3);
    const int KS = (kext + 31) / 32;
    return ((size_t)((row >> 4) * KS + ks) * 64 + 16 * grp + (row & 15)) * 8 + j;
}

// This lane's fragment of tile (rb, ks) of operand tiles with KS steps.
template <typename E>
__device__ __forceinline__ Frag<E> frag_tile(const E* M, int rb, int ks, int KS) {
    Frag<E> f;
    frag_load_row8(f, M + ((size_t)(rb * KS + ks) * 64 + (threadIdx.x & 63)) * 8);
    return f;
}

// A fragment in the operand precision E (identity for fp32).
template <typename E>
__device__ __forceinline__ Frag<E> cvt_frag(const Frag<float>& x) {
    Frag<E> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.set(j, x.v[j]);
    return f;
}

// Eight consecutive floats stored as E (32 or 16 bytes, aligned to it).
__device__ __forceinline__ void store_row8(float* p, const float* x) {
    reinterpret_cast<float4*>(p)[0] = *reinterpret_cast<const float4*>(x);
    reinterpret_cast<float4*>(p)[1] = *reinterpret_cast<const float4*>(x + 4);
}
__device__ __forceinline__ void store_row8(bf16_t* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16_t)x[j];
    *reinterpret_cast<bf16x8*>(p) = v;
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, size_t i) {
    return to_f<T>(reinterpret_cast<const T*>(p)[i]);
}
template <typename T>
__device__ __forceinline__ void stf(void* p, size_t i, float x) {
    reinterpret_cast<T*>(p)[i] = from_f<T>(x);
}

// A load kept as its raw bits (bf16 zero-extended) until `settle`, an empty
// asm that needs the register there: the compiler cannot move the conversion,
// and so the wait for the load, ahead of it.  Loads issued early stay in
// flight across the work before their use.
template <typename T> __device__ __forceinline__ uint32_t ldraw(const void* p, size_t i);
template <> __device__ __forceinline__ uint32_t ldraw<bf16_t>(const void* p, size_t i) {
    return reinterpret_cast<const uint16_t*>(p)[i];
}
template <> __device__ __forceinline__ uint32_t ldraw<float>(const void* p, size_t i) {
    return reinterpret_cast<const uint32_t*>(p)[i];
}
template <typename T> __device__ __forceinline__ float raw_value(uint32_t x) {
    return sizeof(T) == 2 ? __uint_as_float(x << 16) : __uint_as_float(x);
}
__device__ __forceinline__ void settle(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }

// Fragment of rows row0 .. row0 + 15 of a row-major fp32 matrix (leading
// dimension ld) at contraction indices k0 + slot_index(gq, j); indices past
// klen (16 or >= 32) are zero.
__device__ __forceinline__ Frag<float> frag_rows(const float* M, int ld, int row0, int k0, int klen) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, gq = lane >> 4;
    Frag<float> f;
    const float* p = M + (size_t)(row0 + r) * ld + k0 + 4 * gq;
    const float4 lo = *reinterpret_cast<const float4*>(p);
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    if (klen >= 32) {
        const float4 hi = *reinterpret_cast<const float4*>(p + 16);
        f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    } else {
        f.v[4] = f.v[5] = f.v[6] = f.v[7] = 0.f;
    }
    return f;
}

// B operand of a 16-row-block strip held as C-layout tiles X[0 .. NB-1] for
// contraction step s (rows 32 s .. 32 s + 31).
template <typename E, int NB>
__device__ __forceinline__ Frag<E> frag_strip(const floatx4 (&X)[NB], int s) {
    if (2 * s + 1 < NB) return frag_from_c<E>(X[2 * s], X[2 * s + 1]);
    return frag_from_c_lo<E>(X[2 * s]);
}

// Per-element log-decay of the switched gate (natural log units).
__device__ __forceinline__ float gate_of(float zv, float eA, float g_min, unsigned flags) {
    if (!(flags & kGateIn)) return zv;
    if (flags & kGateSoftplus) return -eA * (fmaxf(zv, 0.f) + log1pf(expf(-fabsf(zv))));
    return g_min * sigmoidf_(eA * zv);
}

// The raw inputs of one chunk for one thread: channel d = tid % DK at the NPT
// consecutive tokens of its thread group tid / DK.  Loaded before any other
// global operand of the chunk, so that the wait for them does not wait for
// loads issued later.  Loads of tokens past the end read the last token (a
// valid address, so no branch and no wait before use) and are replaced by
// zero afterwards.
template <int DK, int NTHR>
struct PrepIn {
    static constexpr int NG = NTHR / DK, NPT = C / NG;
    static_assert(NG * DK == NTHR && NG * NPT == C, "whole channel rows per thread group");
    float q[NPT], k[NPT], z[NPT], br;
};

template <typename T, int DK, int NTHR>
__device__ __forceinline__ void prep_load(const BwdArgs& a, int b, int h, int t0, PrepIn<DK, NTHR>& in) {
    constexpr int NPT = PrepIn<DK, NTHR>::NPT;
    const int tid = threadIdx.x, d = tid % DK, tg = (tid / DK) * NPT;
    const int Hk = a.H / a.G, hq = h / a.G;  // value head h reads q/k head h / G
    // the biased logit; without a bias, a valid address is read and the value dropped
    // (no branch around a load)
    const float zbl = *(a.dt_bias ? a.dt_bias + (size_t)h * DK + d : a.A_log + h);
    const float zb = a.dt_bias ? zbl : 0.f;
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        const int tok = min(t0 + tg + u, a.T - 1);
        const size_t idx_qk = (((size_t)b * a.T + tok) * Hk + hq) * DK + d;
        in.q[u] = ldf<T>(a.q, idx_qk);
        in.k[u] = ldf<T>(a.k, idx_qk);
        in.z[u] = ldf<T>(a.z, (((size_t)b * a.T + tok) * a.H + h) * DK + d) + zb;
    }
    in.br = ldf<T>(a.beta_raw, ((size_t)b * a.T + min(t0 + tid % C, a.T - 1)) * a.H + h);  // used by tid < C
}

// Sum over the RL lanes (16, 32 or 64, aligned) that share this lane's group,
// in every lane: row sums with DPP moves (xor 1, xor 2, half-row mirror, row
// mirror), then the rows' lane 0 read out and added.
template <int RL>
__device__ __forceinline__ float group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
    if constexpr (RL == 16) return x;
    const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    if constexpr (RL == 32) return (threadIdx.x & 32) ? a2 + a3 : a0 + a1;
    return (a0 + a1) + (a2 + a3);
}

// The switched activations of the chunk into LDS: q_hat, k_hat, cumulative
// log-decay G in log2 units (pitch P), beta and the inverse norms.  Tokens
// past the end are zero rows with g = 0 and beta = 0 (identity transitions).
// Everything a thread needs for its channel's tokens is computed in registers:
// G summed over its own tokens, then offset by the totals of the earlier
// thread groups; the squared norms reduced over the wave's lanes of the group
// for all of its tokens at once, then (DK = 128) with the other wave of the
// group.  sPart: NTHR floats; sNrm: 2 x (NTHR / 64) x NPT floats.  The
// barriers order LDS only: global loads issued before stay in flight.
template <int DK, int NTHR>
constexpr int prep_norm_floats() { return 2 * (NTHR / 64) * PrepIn<DK, NTHR>::NPT; }

template <typename T, int DK, int P, int NTHR>
__device__ void prep_finish(const BwdArgs& a, int h, int t0, const PrepIn<DK, NTHR>& in, float (*sQ)[P],
                            float (*sK)[P], float (*sG)[P], float* sB, float* sRq, float* sRk, float* sPart,
                            float* sNrm) {
    constexpr int NPT = PrepIn<DK, NTHR>::NPT;
    constexpr int NW = NTHR / 64;
    constexpr int RL = DK < 64 ? DK : 64;  // lanes of one thread group within a wave
    const int tid = threadIdx.x, d = tid % DK, grp = tid / DK, tg = grp * NPT;
    const int wave = tid >> 6;
    const float Al = a.A_log[h];
    const float eA = (a.flags & kGateIn) ? expf(Al) : 0.f;
    const bool l2 = (a.flags & kQkL2) != 0;
    float q[NPT], k[NPT], g[NPT], nq[NPT], nk[NPT];
    // the per-token log-decay (the gate chosen once, not per element), on a
    // valid logit even past the end
    if (!(a.flags & kGateIn)) {
#pragma unroll
        for (int u = 0; u < NPT; ++u) g[u] = in.z[u];
    } else if (a.flags & kGateSoftplus) {
#pragma unroll
        for (int u = 0; u < NPT; ++u) g[u] = -eA * (fmaxf(in.z[u], 0.f) + log1pf(expf(-fabsf(in.z[u]))));
    } else {
#pragma unroll
        for (int u = 0; u < NPT; ++u) g[u] = a.g_min * sigmoidf_(eA * in.z[u]);
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        const bool valid = t0 + tg + u < a.T;
        q[u] = valid ? in.q[u] : 0.f;
        k[u] = valid ? in.k[u] : 0.f;
        g[u] = (valid ? g[u] : 0.f) * kLog2e;  // log2 units: one exp2 per factor
        if (u > 0) g[u] += g[u - 1];
        nq[u] = q[u] * q[u];
        nk[u] = k[u] * k[u];
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        nq[u] = group_sum<RL>(nq[u]);
        nk[u] = group_sum<RL>(nk[u]);
    }
    sPart[tid] = g[NPT - 1];
    if (DK > 64 && (tid & 63) == 0) {
#pragma unroll
        for (int u = 0; u < NPT; ++u) {
            sNrm[wave * NPT + u] = nq[u];
            sNrm[(NW + wave) * NPT + u] = nk[u];
        }
    }
    if (tid < C) {
        const float bt = (a.flags & kBetaSig) ? sigmoidf_(in.br) : in.br;
        sB[tid] = (t0 + tid < a.T) ? bt : 0.f;
    }
    lds_barrier();
    float off = 0.f;
    for (int gg = 0; gg < grp; ++gg) off += sPart[gg * DK + d];
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
        if (DK > 64) {  // the group's other wave
            nq[u] += sNrm[(wave ^ 1) * NPT + u];
            nk[u] += sNrm[(NW + (wave ^ 1)) * NPT + u];
        }
        const float rq = l2 ? __builtin_amdgcn_rsqf(nq[u] + kL2Eps) : 1.f;  // hardware 1/sqrt (about 1 ulp)
        const float rk = l2 ? __builtin_amdgcn_rsqf(nk[u] + kL2Eps) : 1.f;
        sQ[tg + u][d] = q[u] * rq;
        sK[tg + u][d] = k[u] * rk;
        sG[tg + u][d] = g[u] + off;
        if (d == 0) {
            sRq[tg + u] = rq;
            sRk[tg + u] = rk;
        }
    }
    lds_barrier();
}

}  // namespace

// ------------------------------------------------------------------ 1. ops

// The operand tiles of K_d, K_p and the transposes are written fragment by
// fragment; Aqk^T, T and T^T are assembled in LDS in tile order first.
template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_bwd_ops_kernel(const BwdArgs a) {
    using O = Ops<T, DK>;
    constexpr int P = DK + 1;  // odd pitch: the pair loop reads columns across rows
    constexpr int KSD = (DK + 31) / 32;
    constexpr int kStage = 2 * C * C;  // Aqk^T, then T and T^T, in tile order
    __shared__ float sQ[C][P], sK[C][P], sG[C][P];
    __shared__ float sB[C], sRq[C], sRk[C];
    __shared__ float sAt[C][C + 1], sTT[C][C + 1];
    __shared__ __align__(16) float sSt[kStage];
    __shared__ float sPart[256], sNrm[prep_norm_floats<DK, 256>()];
    const int n = blockIdx.x % a.NC;
    const int bh = blockIdx.x / a.NC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    {
        PrepIn<DK, 256> pin;
        prep_load<T, DK, 256>(a, b, h, n * C, pin);
        prep_finish<T, DK, P, 256>(a, h, n * C, pin, sQ, sK, sG, sB, sRq, sRk, sPart, sNrm);
    }
    unsigned char* op = a.ops + ((size_t)bh * a.NC + n) * O::bytes;
    float* opf = reinterpret_cast<float*>(op);  // the fp32 parts, in floats
    auto flush = [&](size_t dst, int count) {   // sSt[0, count) -> elements [0, count) at byte dst, as T
        lds_barrier();
        T* out = reinterpret_cast<T*>(op + dst);
        for (int e = 8 * tid; e < count; e += 8 * 256) store_row8(out + e, sSt + e);
        lds_barrier();
    };
    // The operand tiles of K_d, K_p and the transposes, fragment by fragment:
    // item (tile, lane) is the lane's 8 slots of the tile, computed and stored
    // (16 or 32 bytes) by one thread, so a wave writes 64 consecutive items.
    auto put8 = [&](size_t off, int item, const float (&x)[8]) {
        store_row8(reinterpret_cast<T*>(op + off) + (size_t)item * 8, x);
    };
    // [C x DK]: Kd = k_hat exp(G), Kp = k_hat exp(G_C - G); slots past DK are zero
    for (int it = tid; it < (C / 16) * KSD * 64; it += 256) {
        const int ln = it & 63, tile = it >> 6, rb = tile / KSD, ks = tile % KSD;
        const int t = 16 * rb + (ln & 15), g4 = ln >> 4;
        float xd[8], xp[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 32 * ks + slot_index(g4, j);
            const bool in = k < DK;
            const int kc = in ? k : 0;
            const float G = sG[t][kc], Kv = sK[t][kc];
            xd[j] = in ? Kv * exp2_fast(G) : 0.f;                   // exponent <= 0
            xp[j] = in ? Kv * exp2_fast(sG[C - 1][kc] - G) : 0.f;
        }
        put8(O::Kd, it, xd);
        put8(O::Kp, it, xp);
    }
    // [DK x C]: KpT, QpT = (q_hat exp(G))^T, KdT
    for (int it = tid; it < (DK / 16) * 64; it += 256) {
        const int ln = it & 63, rb = it >> 6;
        const int d = 16 * rb + (ln & 15), g4 = ln >> 4;
        const float GC = sG[C - 1][d];
        float xkp[8], xq[8], xkd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = slot_index(g4, j);
            const float G = sG[t][d], Kv = sK[t][d], e = exp2_fast(G);
            xkp[j] = Kv * exp2_fast(GC - G);
            xq[j] = sQ[t][d] * e;
            xkd[j] = Kv * e;
        }
        put8(O::KpT, it, xkp);
        put8(O::QpT, it, xq);
        put8(O::KdT, it, xkd);
    }
    for (int d = tid; d < DK; d += 256) opf[O::gamS / 4 + d] = opf[O::gamA / 4 + d] = exp2_fast(sG[C - 1][d]);
    for (int t = tid; t < C; t += 256) opf[O::betaS / 4 + t] = opf[O::betaA / 4 + t] = sB[t];
    // A_kk (strictly lower, no beta) and Aqk (lower) as 16 x 16 blocks on the
    // matrix cores: wave 0 block (0, 0), wave 1 (1, 1), wave 2 (1, 0), wave 3
    // the zero block (0, 1).  exp(G_i - G_j) = exp(G_i - rho) exp(rho - G_j)
    // with rho, per channel, the mean of the first and last G of a diagonal
    // block (both factors within 2^(+-span / 2)) or G at token 15 for the
    // off-diagonal block (both factors <= 1).  A diagonal block wider than
    // 2^kBwdWideLog2 on some channel is summed element by element (one
    // exponent <= 1 per term).  At goes out row-major, Aqk^T as tiles.
    const int w = tid >> 6, lane = tid & 63, r = lane & 15, gq = lane >> 4;
    if (w < 3) {
        const int bi = w == 0 ? 0 : 1, bj = w == 1 ? 1 : 0;
        const bool diag = bi == bj;
        bool wide_lane = false;
        if (diag)
            for (int d = lane; d < DK; d += 64) wide_lane |= sG[16 * bi][d] - sG[16 * bi + 15][d] > kBwdWideLog2;
        floatx4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = akk;
        if (__ballot(wide_lane) == 0) {
            const int i = 16 * bi + r, j = 16 * bj + r;  // this lane's A row and B column
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                Frag<float> fk, fq, fb;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int d = 32 * ks + slot_index(gq, jj);
                    const bool in = d < DK;
                    const int dc = in ? d : 0;
                    const float rho = diag ? 0.5f * (sG[16 * bi][dc] + sG[16 * bi + 15][dc]) : sG[15][dc];
                    const float up = exp2_fast(sG[i][dc] - rho), dn = exp2_fast(rho - sG[j][dc]);
                    fk.v[jj] = in ? sK[i][dc] * up : 0.f;
                    fq.v[jj] = in ? sQ[i][dc] * up : 0.f;
                    fb.v[jj] = in ? sK[j][dc] * dn : 0.f;
                }
                akk = mma(fk, fb, akk);
                aqk = mma(fq, fb, aqk);
            }
        } else {  // lane (r, gq) owns the block's entries (4 gq + ii, r)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * bi + 4 * gq + ii, j = 16 * bj + r;
                if (j > i) continue;
                for (int d = 0; d < DK; ++d) {
                    const float x = sK[j][d] * exp2_fast(sG[i][d] - sG[j][d]);
                    akk[ii] = fmaf(sK[i][d], x, akk[ii]);
                    aqk[ii] = fmaf(sQ[i][d], x, aqk[ii]);
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {  // C layout: row 16 bi + 4 gq + ii, column 16 bj + r
            const int i = 16 * bi + 4 * gq + ii, j = 16 * bj + r;
            const float vkk = j < i ? akk[ii] : 0.f, vqk = j <= i ? aqk[ii] : 0.f;
            sAt[i][j] = vkk;
            opf[O::At / 4 + i * C + j] = vkk;
            sSt[tile_pos(j, i, C)] = vqk;
        }
    } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 4 * gq + ii, j = 16 + r;
            sAt[i][j] = 0.f;
            opf[O::At / 4 + i * C + j] = 0.f;
            sSt[tile_pos(j, i, C)] = 0.f;
        }
    }
    flush(O::AqkT, C * C);
    // T = (I + L)^-1 with L = Diag(beta) At (unit lower triangular) by 16 x 16
    // blocks: the diagonal blocks by forward substitution (lane 16 blk + c:
    // column c of block blk), then T21 = -T22 (L21 T11) on the matrix cores.
    if (w == 0) {
        if (lane < 32) {
            const int blk = lane >> 4, c = lane & 15, o = 16 * blk;
            float col[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float sacc = (i == c) ? 1.f : 0.f;
                const float nb = -sB[o + i];
#pragma unroll
                for (int m = 0; m < i; ++m) sacc = fmaf(nb * sAt[o + i][o + m], col[m], sacc);
                col[i] = sacc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sTT[o + i][o + c] = col[i];
                sTT[i][16 + c] = 0.f;  // the zero block above the diagonal
            }
        }
        // R layout of L21 (lane: row r, columns 4 gq + i), C layout of T11 and
        // of the product (lane: rows 4 gq + i, column r)
        floatx4 l21, t11, t22;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            l21[i] = sB[16 + r] * sAt[16 + r][4 * gq + i];
            t11[i] = sTT[4 * gq + i][r];
            t22[i] = sTT[16 + r][16 + 4 * gq + i];
        }
        const floatx4 pm = mm16(l21, t11);  // L21 T11
        const floatx4 t21 = mm16(t22, pm);  // T22 (L21 T11)
#pragma unroll
        for (int i = 0; i < 4; ++i) sTT[16 + 4 * gq + i][r] = -t21[i];
    }
    lds_barrier();
    // T into sSt[0, C^2) and T^T into sSt[C^2, 2 C^2), as tiles
    for (int e = tid; e < C * C; e += 256) {
        const int i = e / C, j = e % C;
        const float x = sTT[i][j];
        sSt[tile_pos(i, j, C)] = x;
        sSt[C * C + tile_pos(j, i, C)] = x;
    }
    lds_barrier();
    for (int e = 8 * tid; e < C * C; e += 8 * 256) {
        store_row8(reinterpret_cast<T*>(op + O::Tm) + e, sSt + e);
        store_row8(reinterpret_cast<T*>(op + O::TT) + e, sSt + C * C + e);
    }
}

// ------------------------------------------------------- copies into LDS

// Copy `pieces` KiB from src (global) to dst (LDS) with the wave's lanes, as
// 16-byte direct-to-LDS loads; piece p goes out from wave p % nwaves.
__device__ __forceinline__ void stage_kib(const unsigned char* src, float* dst, int pieces, int wave, int nwaves) {
    const int lane = threadIdx.x & 63;
    for (int p = wave; p < pieces; p += nwaves)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + p * 1024 + lane * 16),
                                         (__attribute__((address_space(3))) void*)(dst + p * 256), 16, 0, 0);
}

// A serial pass's workgroup writes its NSW 16-column strips of a [DK x ld]
// row-major fp32 matrix through an LDS tile (pitch SW + 4, SW = 16 NSW): each
// compute wave puts its strip (C layout: lane (r, gq) holds rows 16 R + 4 gq + i
// at column 16 w + r), and after the next workgroup barrier each wave stores
// DK / NSW rows as whole SW * 4-byte pieces, 16 bytes a lane.  Row pieces of
// a full 128-byte line store fast; scattered four-byte or 64-byte pieces make
// the pass wait on its stores.
template <int NBD, int NSW>
__device__ __forceinline__ void put_strip(float* tile, int w, const floatx4 (&X)[NBD]) {
    constexpr int kP = 16 * NSW + 4;
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[(16 * R + 4 * gq + i) * kP + 16 * w + r] = X[R][i];
}
template <int NBD, int NSW>
__device__ __forceinline__ void flush_rows(float* dst, size_t ld, int c0, int w, const float* tile) {
    constexpr int SW = 16 * NSW, kP = SW + 4, LPR = SW / 4, RPI = 64 / LPR;
    constexpr int ROWS = 16 * NBD / NSW;  // rows per wave
    static_assert(ROWS % RPI == 0, "whole instructions");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < ROWS / RPI; ++p) {
        const int row = w * ROWS + p * RPI + lane / LPR, c = 4 * (lane % LPR);
        const float4 v = *reinterpret_cast<const float4*>(tile + row * kP + c);
        *reinterpret_cast<float4*>(dst + (size_t)row * ld + c0 + c) = v;
    }
}

// LDS ring of the serial passes: slots of one chunk's operator region each;
// the copy wave keeps up to kSlots - 1 chunks ahead.  bf16 regions are small
// enough for three slots; fp32 regions take two.
template <typename T> constexpr int bwd_ring_slots() { return sizeof(T) == 2 ? 3 : 2; }

// Wait until at most m chunks of P pieces each are in flight (m <= MAXM);
// loads complete in issue order.
template <int P, int MAXM>
__device__ __forceinline__ void wait_chunks(int m) {
    static_assert(MAXM * P < 64, "vmcnt range");
    if constexpr (MAXM >= 2) {
        if (m >= 2) { wait_vmcnt<2 * P>(); return; }
    }
    if constexpr (MAXM >= 1) {
        if (m >= 1) { wait_vmcnt<P>(); return; }
    }
    wait_vmcnt<0>();
}

// Value rows of one chunk for a serial pass's workgroup: token rows of its
// NSW * 16 columns (RB bytes each, from column c0 of the [B, T, H, Dv] tensor
// x), as whole KiB pieces of 16-byte lane copies into LDS.  Tokens past the
// end read the last token; the compute waves zero them.
template <typename T, int NSW>
struct ValueRows {
    static constexpr int RB = NSW * 16 * (int)sizeof(T);  // bytes of one token's row
    static constexpr int LPT = RB / 16;                    // lanes per token
    static constexpr int TPP = 64 / LPT;                   // tokens per piece
    static constexpr int PIECES = C / TPP;
    static_assert(LPT * 16 == RB && TPP * LPT == 64 && PIECES * TPP == C, "whole pieces");
    static __device__ __forceinline__ void stage(const void* x, const BwdArgs& a, int b, int h, int c0, int n,
                                                 float* dst) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int p = 0; p < PIECES; ++p) {
            const int tok = min(n * C + p * TPP + lane / LPT, a.T - 1);
            const unsigned char* src = reinterpret_cast<const unsigned char*>(x) +
                                       ((((size_t)b * a.T + tok) * a.H + h) * a.Dv + c0) * sizeof(T) + (lane % LPT) * 16;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)(dst + p * 256), 16, 0, 0);
        }
    }
};

// The copy wave of a serial pass: ring slot i % K receives chunk i's P pieces
// (stage(i, slot) issues them) for i = 0 .. NC - 1; one barrier before the
// first chunk and one after each (the compute waves' barriers).  The compute
// waves load nothing from global memory, so none of their waits counts a
// store.
template <int K, int P, int SLOT, typename F>
__device__ __forceinline__ void ring_copy(int NC, float (*ring)[SLOT], F stage) {
    const int pre = NC < K - 1 ? NC : K - 1;
    for (int i = 0; i < pre; ++i) stage(i, ring[i % K]);
    wait_chunks<P, K - 2>(pre - 1);  // chunk 0 has landed
    lds_barrier();
    for (int i = 0; i < NC; ++i) {
        // the slot of chunk i - 1 is free: every compute wave passed the barrier after it
        if (i + K - 1 < NC) stage(i + K - 1, ring[(i + K - 1) % K]);
        const int later = (NC - 1) - (i + 1);  // chunks issued after chunk i + 1, at most K - 2
        wait_chunks<P, K - 2>(later < 0 ? 0 : (later > K - 2 ? K - 2 : later));
        lds_barrier();
    }
}

// --------------------------------------------------------------- 2. states

// One workgroup per (b, h) and group of NSW value strips; wave w holds the
// fp32 strip of value columns 16 st .. 16 st + 15 of S in C layout (rows
// 16 R + 4 gq + i, column r).  Each chunk's state-pass operators and value
// rows are copied into an LDS ring ahead of use by a copy wave.
template <typename T, int DK, int NSW>
__global__ __launch_bounds__(64 * (NSW + 1)) void kda_bwd_states_kernel(const BwdArgs a) {
    using O = Ops<T, DK>;
    using VR = ValueRows<T, NSW>;
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    constexpr int kPieces = (int)(O::sizeS / 1024);
    constexpr int P = kPieces + VR::PIECES;  // KiB per ring slot: operators, then value rows
    constexpr int K = bwd_ring_slots<T>();
    __shared__ __align__(16) float sOp[K][P * 256];
    __shared__ __align__(16) float sTr[2][DK * (16 * NSW + 4)];  // the chunk-start state on its way out
    const int ngrp = (a.Dv / 16) / NSW;
    const int bh = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    const int b = bh / a.H, h = bh % a.H;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int c0 = 16 * grp * NSW;  // the workgroup's first value column
    const int col = c0 + 16 * w + r;
    const unsigned char* blk = a.ops + (size_t)bh * a.NC * O::bytes;
    // wave NSW only copies each chunk's operators and value rows into LDS (up to
    // K - 1 chunks ahead); the compute waves never load from global memory
    if (w == NSW) {
        ring_copy<K, P>(a.NC, sOp, [&](int i, float* slot) {
            stage_kib(blk + (size_t)i * O::bytes, slot, kPieces, 0, 1);
            VR::stage(a.v, a, b, h, c0, i, slot + kPieces * 256);
        });
        return;
    }
    floatx4 S[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[R][i] = a.S0 ? a.S0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    // the state at the start of chunk n, stored through the LDS tile
    auto flush_state = [&](int n) {
        flush_rows<NBD, NSW>(a.states + ((size_t)bh * a.NC + n) * DK * a.Dv, a.Dv, c0, w, sTr[n & 1]);
    };
    if (a.NC > 0) put_strip<NBD, NSW>(sTr[0], w, S);
    lds_barrier();
    if (a.NC > 0) flush_state(0);
    for (int n = 0; n < a.NC; ++n) {
        const float* slot = sOp[n % K];
        const unsigned char* op = reinterpret_cast<const unsigned char*>(slot);
        const T* vrow = reinterpret_cast<const T*>(slot + kPieces * 256);  // [C][16 NSW] value rows
        const float* betaS = O::f32(op, O::betaS);
        const float* gamS = O::f32(op, O::gamS);
        // E = V - Kd S, scaled by beta per token
        floatx4 E[2], Eb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSD; ++s) acc = mma(frag_tile(O::tiles(op, O::Kd), tb, s, KSD), frag_strip<T>(S, s), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                const float vv = n * C + t < a.T ? to_f<T>(vrow[t * (16 * NSW) + col - c0]) : 0.f;
                E[tb][i] = vv - acc[i];
                Eb[tb][i] = betaS[t] * E[tb][i];
            }
        }
        // the state at the start of this chunk, put into the LDS tile before the
        // last barrier, goes out here, behind the products just issued
        if (n > 0) flush_state(n);
        // U = T (beta E)
        floatx4 U[2];
        const Frag<T> Ebf = frag_from_c<T>(Eb[0], Eb[1]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            U[tb] = mma(frag_tile(O::tiles(op, O::Tm), tb, 0, 1), Ebf, z4);
        }
        // S <- Diag(gamma) S + Kp^T U
        const Frag<T> Uf = frag_from_c<T>(U[0], U[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gamS[16 * R + 4 * gq + i] * S[R][i];
            S[R] = mma(frag_tile(O::tiles(op, O::KpT), R, 0, 1), Uf, acc);
        }
        // this chunk's E and U for the gradient kernel, in fragment order
        float4* eu = reinterpret_cast<float4*>(a.eu + ((size_t)bh * a.NC + n) * 2 * C * a.Dv);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            eu[((col >> 4) * 2 + tb) * 64 + lane] = make_float4(E[tb][0], E[tb][1], E[tb][2], E[tb][3]);
            eu[(C * a.Dv) / 4 + ((col >> 4) * 2 + tb) * 64 + lane] = make_float4(U[tb][0], U[tb][1], U[tb][2], U[tb][3]);
        }
        if (n + 1 < a.NC) put_strip<NBD, NSW>(sTr[(n + 1) & 1], w, S);
        lds_barrier();   // the next chunk is in LDS, this chunk's slot no longer read
    }
}

// -------------------------------------------------------------- 3. adjoint

template <typename T, int DK, int NSW>
__global__ __launch_bounds__(64 * (NSW + 1)) void kda_bwd_adjoint_kernel(const BwdArgs a) {
    using O = Ops<T, DK>;
    using VR = ValueRows<T, NSW>;
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    constexpr int kPieces = (int)(O::sizeA / 1024);
    constexpr int P = kPieces + VR::PIECES;  // KiB per ring slot: operators, then dO rows
    constexpr size_t A0 = O::A0;
    constexpr int K = bwd_ring_slots<T>();
    __shared__ __align__(16) float sOp[K][P * 256];
    __shared__ __align__(16) float sTr[2][DK * (16 * NSW + 4)];  // the chunk-end adjoint on its way out
    const int ngrp = (a.Dv / 16) / NSW;
    const int bh = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    const int b = bh / a.H, h = bh % a.H;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int c0 = 16 * grp * NSW;  // the workgroup's first value column
    const int col = c0 + 16 * w + r;
    const unsigned char* blk = a.ops + (size_t)bh * a.NC * O::bytes + A0;
    if (w == NSW) {  // the copy wave: chunks in reverse order, operators then dO rows
        ring_copy<K, P>(a.NC, sOp, [&](int i, float* slot) {
            stage_kib(blk + (size_t)(a.NC - 1 - i) * O::bytes, slot, kPieces, 0, 1);
            VR::stage(a.dout, a, b, h, c0, a.NC - 1 - i, slot + kPieces * 256);
        });
        return;
    }
    floatx4 dS[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[R][i] = a.dS_T ? a.dS_T[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    // the adjoint at the end of chunk n, stored through the LDS tile
    auto flush_adj = [&](int n, int slot) {
        flush_rows<NBD, NSW>(a.adj + ((size_t)bh * a.NC + n) * DK * a.Dv, a.Dv, c0, w, sTr[slot]);
    };
    if (a.NC > 0) put_strip<NBD, NSW>(sTr[0], w, dS);
    lds_barrier();
    if (a.NC > 0) flush_adj(a.NC - 1, 0);
    for (int it = 0; it < a.NC; ++it) {
        const int n = a.NC - 1 - it;
        const float* slot = sOp[it % K];
        const unsigned char* op = reinterpret_cast<const unsigned char*>(slot);  // region A: offsets - A0
        const T* drow = reinterpret_cast<const T*>(slot + kPieces * 256);      // [C][16 NSW] dO rows
        const float* betaA = O::f32(op, O::betaA - A0);
        const float* gamA = O::f32(op, O::gamA - A0);
        // dO as the B operand of products over the chunk's tokens
        Frag<T> dOf;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = slot_index(gq, j);
            dOf.set(j, n * C + t < a.T ? to_f<T>(drow[t * (16 * NSW) + col - c0]) : 0.f);
        }
        // dU = Aqk^T dO + Kp dS'
        floatx4 dU[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            floatx4 acc = mma(frag_tile(O::tiles(op, O::AqkT - A0), tb, 0, 1), dOf, z4);
#pragma unroll
            for (int s = 0; s < KSD; ++s)
                acc = mma(frag_tile(O::tiles(op, O::Kp - A0), tb, s, KSD), frag_strip<T>(dS, s), acc);
            dU[tb] = acc;
        }
        // the adjoint at the end of this chunk, put into the LDS tile before the
        // last barrier, goes out here, behind the products just issued
        if (it > 0) flush_adj(n, it & 1);
        // -beta W with W = T^T dU
        floatx4 X[2];
        const Frag<T> dUf = frag_from_c<T>(dU[0], dU[1]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 wv = mma(frag_tile(O::tiles(op, O::TT - A0), tb, 0, 1), dUf, z4);
#pragma unroll
            for (int i = 0; i < 4; ++i) X[tb][i] = -betaA[16 * tb + 4 * gq + i] * wv[i];
            // this chunk's W for the gradient kernel, in fragment order
            reinterpret_cast<float4*>(a.w + ((size_t)bh * a.NC + n) * C * a.Dv)[((col >> 4) * 2 + tb) * 64 + lane] =
                make_float4(wv[0], wv[1], wv[2], wv[3]);
        }
        // dS = Diag(gamma) dS' + Qp^T dO - Kd^T (beta W)
        const Frag<T> Xf = frag_from_c<T>(X[0], X[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gamA[16 * R + 4 * gq + i] * dS[R][i];
            acc = mma(frag_tile(O::tiles(op, O::QpT - A0), R, 0, 1), dOf, acc);
            dS[R] = mma(frag_tile(O::tiles(op, O::KdT - A0), R, 0, 1), Xf, acc);
        }
        if (n > 0) put_strip<NBD, NSW>(sTr[(it + 1) & 1], w, dS);
        lds_barrier();
    }
    if (a.dS0) {
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] = dS[R][i];
    }
}

// ---------------------------------------------------------------- 4. grads

// Sum over the 16 lanes that share lane / 16 (DPP row moves).
__device__ __forceinline__ float row_sum16(float x) { return group_sum<16>(x); }

// One workgroup (eight waves) per chunk-head.  Wave w owns value columns
// 16 w .. 16 w + 15 for the per-token terms (E, U and W of the chunk, handed
// over by the serial passes in C layout), and channel block 16 w ..
// 16 w + 15 for the products over the value dimension (dQp, dKd, dKp, with
// the rows of dO, U and W read from LDS and the rows of S and dS' as
// contiguous global fragments), and for the decay-weighted sums and the
// outputs, where lane (r, gq) owns channel 16 w + r and the eight tokens
// 16 tb + 4 gq + i.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(512) void kda_bwd_grads_kernel(const BwdArgs a) {
    constexpr int NT = 512;
    constexpr int NBV = DV / 16, NBK = DK / 16;
    constexpr int KSV = (DV + 31) / 32;
    constexpr int PV = DV + 4;  // row pitch of the value rows (16-byte rows, spread banks)
    __shared__ float sQ[C][DK], sK[C][DK], sG[C][DK];
    __shared__ float sB[C], sRq[C], sRk[C];
    __shared__ float sdBp[2][NT / 64][C];  // dbeta parts per wave (E.W, then dA_kk.At), summed in a fixed order
    __shared__ float sPq[NBK][C], sPk[NBK][C], sPqT[C], sPkT[C];
    __shared__ __align__(16) float sBig[3 * C * PV];
    __shared__ float sdAqk[C][C + 1], sdAt[C][C + 1];
    __shared__ float sRed[NT / 64];
    __shared__ float sPart[NT], sNrm[prep_norm_floats<DK, NT>()];
    float* sdO = sBig;              // [C][PV]
    float* sU = sBig + C * PV;      // [C][PV]
    float* sW = sBig + 2 * C * PV;  // [C][PV]

    const int n = blockIdx.x % a.NC;
    const int bh = blockIdx.x / a.NC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, r = lane & 15, gq = lane >> 4;
    const int t0 = n * C;
    using O = Ops<T, DK>;
    const unsigned char* op = a.ops + ((size_t)bh * a.NC + n) * O::bytes;
    const float* S0 = a.states + ((size_t)bh * a.NC + n) * DK * DV;
    const float* dSC = a.adj + ((size_t)bh * a.NC + n) * DK * DV;
    auto row_of = [&](int t) { return ((size_t)b * a.T + t0 + t) * a.H + h; };
    auto in_row = [&](int t) { return ((size_t)b * a.T + min(t0 + t, a.T - 1)) * a.H + h; };  // clamped

    // Every global operand of the chunk is requested up front, the activations'
    // inputs first: dO rows, then for the products over tokens this wave's
    // value column of S, dS' and V.  They arrive while the activations are
    // prepared in LDS.
    PrepIn<DK, NT> pin;
    prep_load<T, DK, NT>(a, b, h, t0, pin);
    constexpr int NDO = C * DV / NT;
    static_assert(NDO * NT == C * DV, "whole dO rows per pass");
    uint32_t dOr[NDO];
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
        const int e = tid + u * NT, t = e / DV, j = e % DV;
        dOr[u] = ldraw<T>(a.dout, in_row(t) * DV + j);
    }
    const int col = 16 * (w % NBV) + r;
    floatx4 Ef[2], Uf[2], Wf[2];  // this wave's strip of E, U and W, settled where used
    if (w < NBV) {
        const floatx4* eu = reinterpret_cast<const floatx4*>(a.eu + ((size_t)bh * a.NC + n) * 2 * C * DV);
        const floatx4* wf = reinterpret_cast<const floatx4*>(a.w + ((size_t)bh * a.NC + n) * C * DV);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            Ef[tb] = eu[(w * 2 + tb) * 64 + lane];
            Uf[tb] = eu[(C * DV) / 4 + (w * 2 + tb) * 64 + lane];
            Wf[tb] = wf[(w * 2 + tb) * 64 + lane];
        }
    }
    prep_finish<T, DK, DK, NT>(a, h, t0, pin, sQ, sK, sG, sB, sRq, sRk, sPart, sNrm);
#pragma unroll
    for (int u = 0; u < NDO; ++u) {
        const int e = tid + u * NT, t = e / DV, j = e % DV;
        settle(dOr[u]);
        sdO[t * PV + j] = (t0 + t < a.T) ? raw_value<T>(dOr[u]) : 0.f;
    }
    for (int e = tid; e < (NT / 64) * C; e += NT) sdBp[1][e / C][e % C] = 0.f;  // dA_kk waves fill half their rows
    lds_barrier();

    // ---- per token, value column block w: dV = Diag(beta) W, the E.W part of
    // dbeta, and the rows of U and W for the products over the value dimension
    if (w < NBV) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float E = Ef[tb][i], U = Uf[tb][i], W = Wf[tb][i];
                settle(E);
                settle(U);
                settle(W);
                const int t = 16 * tb + 4 * gq + i;
                if (t0 + t < a.T) stf<T>(a.dv, row_of(t) * DV + col, sB[t] * W);
                const float p = row_sum16(W * E);
                if (r == 0) sdBp[0][w][t] = p;
                sU[t * PV + col] = U;
                sW[t * PV + col] = W;
            }
    }
    lds_barrier();

    // ---- products over the value dimension
    {   // dA_kk = -W U^T (strictly lower) and dAqk = dO U^T (lower): eight 16x16 tiles
        const int kind = w >> 2, tb = (w >> 1) & 1, sb = w & 1;
        const float* X = kind == 0 ? sW : sdO;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSV; ++s)
            acc = mma(cvt_frag<T>(frag_rows(X, PV, 16 * tb, 32 * s, DV)), cvt_frag<T>(frag_rows(sU, PV, 16 * sb, 32 * s, DV)),
                      acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * tb + 4 * gq + i, s = 16 * sb + r;
            if (kind == 0) {
                const float dakk = (s < t) ? -acc[i] : 0.f;
                sdAt[t][s] = sB[t] * dakk;  // dAt = Diag(beta) dA_kk
                const float p = row_sum16(dakk * O::f32(op, O::At)[t * C + s]);
                if (r == 0) sdBp[1][w][t] = p;
            } else {
                sdAqk[t][s] = (s <= t) ? acc[i] : 0.f;
            }
        }
    }
    floatx4 dQp[2], dKd[2], dKp[2];
    float dgam = 0.f;
    if (w < NBK) {  // channel block w: dQp = dO S^T, dKd = -Diag(beta) W S^T, dKp = U dS'^T
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) dQp[tb] = dKd[tb] = dKp[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSV; ++s) {
            const Frag<float> S0f = frag_rows(S0, DV, 16 * w, 32 * s, DV);
            const Frag<float> dSf = frag_rows(dSC, DV, 16 * w, 32 * s, DV);
#pragma unroll
            for (int j = 0; j < 8; ++j) dgam = fmaf(S0f.v[j], dSf.v[j], dgam);
            const Frag<T> S0o = cvt_frag<T>(S0f), dSo = cvt_frag<T>(dSf);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                dQp[tb] = mma(cvt_frag<T>(frag_rows(sdO, PV, 16 * tb, 32 * s, DV)), S0o, dQp[tb]);
                dKd[tb] = mma(cvt_frag<T>(frag_rows(sW, PV, 16 * tb, 32 * s, DV)), S0o, dKd[tb]);
                dKp[tb] = mma(cvt_frag<T>(frag_rows(sU, PV, 16 * tb, 32 * s, DV)), dSo, dKp[tb]);
            }
        }
        dgam += __shfl_xor(dgam, 16, 64);
        dgam += __shfl_xor(dgam, 32, 64);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) dKd[tb][i] *= -sB[16 * tb + 4 * gq + i];
    }
    lds_barrier();

    // ---- decay-weighted sums: lane (r, gq) of wave w owns channel 16 w + r
    // at tokens 16 tb + 4 gq + i, here and for the outputs
    float dqh[2][4], dkh[2][4], dGv[2][4], Kt[2][4], Qt[2][4];
    uint32_t zr[2][4];  // gate logits, raw until dz (their wait then falls after the decay sums)
    float zb = 0.f;
    float gce = 0.f;  // the chunk-end terms of dg, entering at the last token
    if (w < NBK) {
        const int d = 16 * w + r;
        // the (biased) gate logits for dz: requested now, used at the end
        zb = a.dt_bias ? a.dt_bias[(size_t)h * DK + d] : 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = min(t0 + 16 * tb + 4 * gq + i, a.T - 1);
                zr[tb][i] = ldraw<T>(a.z, (((size_t)b * a.T + tok) * a.H + h) * DK + d);
            }
        const float GC = sG[C - 1][d];
        float gcpart = 0.f;
        float Gt[2][4], dkp[2][4], dkm[2][4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                Gt[tb][i] = sG[t][d];
                Kt[tb][i] = sK[t][d];
                Qt[tb][i] = sQ[t][d];
                const float et = exp2_fast(Gt[tb][i]), ect = exp2_fast(GC - Gt[tb][i]);
                dqh[tb][i] = dQp[tb][i] * et;
                dkp[tb][i] = dKd[tb][i] * et;
                dkm[tb][i] = dKp[tb][i] * ect;
                gcpart = fmaf(dKp[tb][i], Kt[tb][i] * ect, gcpart);
            }
        // The sums over partners s weigh each term by exp(G_t - G_s).  Factored
        // about rho, the mean of the first and last G of t's 16-token block, every
        // factor of a same-block pair lies within 2^(+-span / 2) (span: the
        // block's decay on this channel) and every cross-block factor is <= 1, so
        // the sums are products on the matrix cores:
        //   dqh += e^(G_t - rho) dAqk [K e^(rho - G)]            (s <= t)
        //   dkp += e^(G_t - rho) dAt  [K e^(rho - G)]            (s < t)
        //   dkm += e^(rho - G_t) (dAqk^T [Q e^(G - rho)] + dAt^T [K e^(G - rho)])   (s >= t)
        // A B operand's slot j is this lane's own token slot_index(gq, j); the
        // slots of the block on the masked side, whose factor could overflow,
        // are zero.  A wave with a block wider than 2^kBwdWideLog2 sums element
        // by element instead (one exponent <= 1 per term).
        float rho[2];
        bool wide_lane = false;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float first = __shfl(Gt[tb][0], r, 64), last = __shfl(Gt[tb][3], 48 + r, 64);
            rho[tb] = 0.5f * (first + last);
            wide_lane |= first - last > kBwdWideLog2;
        }
        if (__ballot(wide_lane) == 0) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                Frag<float> bK, bQe, bKe, aQK, aT, aQKt, aTt;  // fp32: dG takes differences of these sums
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int sb = j >> 2, si = j & 3;  // the slot's token: 16 sb + 4 gq + si
                    const float g = Gt[sb][si];
                    bK.set(j, sb <= tb ? Kt[sb][si] * exp2_fast(rho[tb] - g) : 0.f);
                    const float eh = sb >= tb ? exp2_fast(g - rho[tb]) : 0.f;
                    bQe.set(j, Qt[sb][si] * eh);
                    bKe.set(j, Kt[sb][si] * eh);
                    const int s = slot_index(gq, j), t = 16 * tb + r;
                    aQK.set(j, sdAqk[t][s]);
                    aT.set(j, sdAt[t][s]);
                    aQKt.set(j, sdAqk[s][t]);
                    aTt.set(j, sdAt[s][t]);
                }
                const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
                const floatx4 cq = mma(aQK, bK, z4);
                const floatx4 cp = mma(aT, bK, z4);
                const floatx4 cm = mma(aTt, bKe, mma(aQKt, bQe, z4));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float up = exp2_fast(Gt[tb][i] - rho[tb]), dn = exp2_fast(rho[tb] - Gt[tb][i]);
                    dqh[tb][i] = fmaf(up, cq[i], dqh[tb][i]);
                    dkp[tb][i] = fmaf(up, cp[i], dkp[tb][i]);
                    dkm[tb][i] = fmaf(dn, cm[i], dkm[tb][i]);
                }
            }
        } else {
            // partner s outermost: its G, k_hat, q_hat are read once for the eight
            // tokens.  The stored triangles are zero outside their masks (dAqk[t][s]
            // for s > t, dAt[t][s] for s >= t), so every term is taken, with the
            // one exponent exp(-|G_t - G_s|) <= 1 for both orders.
            for (int s = 0; s < C; ++s) {
                const float Gs = sG[s][d], Ks = sK[s][d], Qs = sQ[s][d];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * tb + 4 * gq + i;
                        const float e = exp2_fast(-fabsf(Gt[tb][i] - Gs));
                        dqh[tb][i] = fmaf(sdAqk[t][s] * Ks, e, dqh[tb][i]);
                        dkp[tb][i] = fmaf(sdAt[t][s] * Ks, e, dkp[tb][i]);
                        dkm[tb][i] = fmaf(sdAqk[s][t] * Qs + sdAt[s][t] * Ks, e, dkm[tb][i]);
                    }
            }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dkh[tb][i] = dkp[tb][i] + dkm[tb][i];
                dGv[tb][i] = Qt[tb][i] * dqh[tb][i] + Kt[tb][i] * (dkp[tb][i] - dkm[tb][i]);
            }
        gcpart += __shfl_xor(gcpart, 16, 64);
        gcpart += __shfl_xor(gcpart, 32, 64);
        gce = gcpart + dgam * exp2_fast(GC);
    }

    // ---- outputs: dg by a reverse cumulative sum of dG over the chunk (within
    // the lane, over the four lane groups, then from the second 16-token block
    // into the first), dz through the gate, and the per-token dot products of
    // the L2-norm backward (over the 16 lanes of a group, then over the waves)
    const float Al = a.A_log[h];
    const float eA = (a.flags & kGateIn) ? expf(Al) : 0.f;
    float dApart = 0.f;
    if (w < NBK) {
        const int d = 16 * w + r;
        float suf[2][4], base[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            suf[tb][3] = dGv[tb][3];
#pragma unroll
            for (int i = 2; i >= 0; --i) suf[tb][i] = suf[tb][i + 1] + dGv[tb][i];
        }
        float incl[2];  // suffix sums of the lane totals over the lane groups gq .. 3
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            float x = suf[tb][0];
            float y = __shfl_down(x, 16, 64);
            x += gq < 3 ? y : 0.f;
            y = __shfl_down(x, 32, 64);
            x += gq < 2 ? y : 0.f;
            incl[tb] = x;
        }
        const float block1 = __shfl(incl[1], r, 64);  // all of the second block
        base[0] = gce + block1 + (incl[0] - suf[0][0]);
        base[1] = gce + (incl[1] - suf[1][0]);
        float dbias = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                const bool valid = t0 + t < a.T;
                const float acc = base[tb] + suf[tb][i];
                float dz = acc, dA = 0.f;
                if (a.flags & kGateIn) {
                    settle(zr[tb][i]);
                    const float zv = raw_value<T>(zr[tb][i]) + zb;
                    if (a.flags & kGateSoftplus) {
                        const float sg = sigmoidf_(zv);
                        dz = acc * (-eA * sg);
                        dA = acc * gate_of(zv, eA, a.g_min, a.flags);
                    } else {
                        const float sg = sigmoidf_(eA * zv);
                        const float dx = acc * a.g_min * sg * (1.f - sg);  // d / d(e^A z)
                        dz = dx * eA;
                        dA = dx * eA * zv;
                    }
                }
                if (valid) stf<T>(a.dz, row_of(t) * DK + d, dz);
                dApart += valid ? dA : 0.f;
                dbias += valid ? dz : 0.f;
            }
        dbias += __shfl_xor(dbias, 16, 64);
        dbias += __shfl_xor(dbias, 32, 64);
        if (a.dbias_part && gq == 0) a.dbias_part[(((size_t)b * a.NC + n) * a.H + h) * DK + d] = dbias;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                const float pq = row_sum16(Qt[tb][i] * dqh[tb][i]);
                const float pk = row_sum16(Kt[tb][i] * dkh[tb][i]);
                if (r == 0) {
                    sPq[w][t] = pq;
                    sPk[w][t] = pk;
                }
            }
    }
    lds_barrier();
    if (tid < C) {  // the per-token dot products over all channels; dbeta
        const int t = tid;
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int ww = 0; ww < NBK; ++ww) {
            pq += sPq[ww][t];
            pk += sPk[ww][t];
        }
        sPqT[t] = pq;
        sPkT[t] = pk;
        if (t0 + t < a.T) {
            const float bt = sB[t];
            float dbs = 0.f;
#pragma unroll
            for (int ww = 0; ww < NBV; ++ww) dbs += sdBp[0][ww][t];
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) dbs += sdBp[1][ww][t];
            const float db = (a.flags & kBetaSig) ? dbs * bt * (1.f - bt) : dbs;
            stf<T>(a.dbeta_raw, row_of(t), db);
        }
    }
    lds_barrier();
    // dq, dk through the L2 norm: dx = r (dx_hat - x_hat (x_hat . dx_hat))
    if (w < NBK) {
        const int d = 16 * w + r;
        const bool l2 = (a.flags & kQkL2) != 0;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                if (t0 + t >= a.T) continue;
                const size_t idx = row_of(t) * DK + d;
                const float gq_ = l2 ? sRq[t] * (dqh[tb][i] - Qt[tb][i] * sPqT[t]) : dqh[tb][i];
                const float gk_ = l2 ? sRk[t] * (dkh[tb][i] - Kt[tb][i] * sPkT[t]) : dkh[tb][i];
                if (a.G == 1) {
                    stf<T>(a.dq, idx, gq_);
                    stf<T>(a.dk, idx, gk_);
                } else {  // this value head's share; the group is summed afterwards
                    a.dqk_part[idx] = gq_;
                    a.dqk_part[(size_t)a.B * a.T * a.H * DK + idx] = gk_;
                }
            }
    }
    // the chunk's share of dA_log
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dApart += __shfl_xor(dApart, off, 64);
    if (lane == 0) sRed[w] = dApart;
    lds_barrier();
    if (tid == 0) {
        float s = 0.f;
        for (int ww = 0; ww < NT / 64; ++ww) s += sRed[ww];
        a.dA_part[((size_t)b * a.NC + n) * a.H + h] = s;
    }
}

// ------------------------------------------------------------------- 5. dA

// One workgroup per head: the B * NC chunk parts of dA_log[h], summed in a
// fixed order (deterministic).
__global__ __launch_bounds__(256) void kda_bwd_dA_kernel(const BwdArgs a) {
    __shared__ float sRed[4];
    const int h = blockIdx.x;
    float s = 0.f;
    for (int bn = threadIdx.x; bn < a.B * a.NC; bn += 256) s += a.dA_part[(size_t)bn * a.H + h];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) sRed[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) a.dA_log[h] = (a.flags & kGateIn) ? (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]) : 0.f;
}

// ------------------------------------------------- grouped-head reductions

// dq, dk of q/k head hq: the sum of the G value heads hq G .. hq G + G - 1.
template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_bwd_qk_reduce_kernel(const BwdArgs a) {
    const int Hk = a.H / a.G;
    const size_t n = (size_t)a.B * a.T * Hk * DK;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int d = (int)(i % DK);
    const size_t row = i / DK;  // (b, t, hq)
    const int hq = (int)(row % Hk);
    const size_t bt = row / Hk;
    const size_t half = (size_t)a.B * a.T * a.H * DK;
    float sq = 0.f, sk = 0.f;
    for (int j = 0; j < a.G; ++j) {
        const size_t src = (bt * a.H + (size_t)hq * a.G + j) * DK + d;
        sq += a.dqk_part[src];
        sk += a.dqk_part[half + src];
    }
    stf<T>(a.dq, i, sq);
    stf<T>(a.dk, i, sk);
}

// ddt_bias[h][d]: the per-chunk parts summed over batch and chunks.
template <int DK>
__global__ __launch_bounds__(256) void kda_bwd_bias_reduce_kernel(const BwdArgs a) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.H * DK) return;
    float s = 0.f;
    for (int bn = 0; bn < a.B * a.NC; ++bn) s += a.dbias_part[(size_t)bn * a.H * DK + i];
    a.ddt_bias[i] = s;
}

// ---------------------------------------------------------------- launches

template <typename T, int DK, int DV>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
    const unsigned chunk_heads = (unsigned)(a.B * a.H * a.NC);
    const unsigned heads = (unsigned)(a.B * a.H);
    constexpr int NSW = DV >= 32 ? 2 : 1;  // value strips per workgroup of the serial passes
    const unsigned serial_groups = heads * (unsigned)(DV / 16 / NSW);
    if (chunk_heads > 0) {
        hipLaunchKernelGGL((kda_bwd_ops_kernel<T, DK>), dim3(chunk_heads), dim3(256), 0, s, a);
        hipLaunchKernelGGL((kda_bwd_states_kernel<T, DK, NSW>), dim3(serial_groups), dim3(64 * (NSW + 1)), 0, s, a);
    }
    if (heads > 0)  // with no chunk it passes dS_T (or zero) to dS0
        hipLaunchKernelGGL((kda_bwd_adjoint_kernel<T, DK, NSW>), dim3(serial_groups), dim3(64 * (NSW + 1)), 0, s, a);
    if (chunk_heads > 0)
        hipLaunchKernelGGL((kda_bwd_grads_kernel<T, DK, DV>), dim3(chunk_heads), dim3(512), 0, s, a);
    if (a.H > 0)
        hipLaunchKernelGGL(kda_bwd_dA_kernel, dim3((unsigned)a.H), dim3(256), 0, s, a);
    if (a.G > 1 && chunk_heads > 0) {
        const size_t nqk = (size_t)a.B * a.T * (a.H / a.G) * DK;
        hipLaunchKernelGGL((kda_bwd_qk_reduce_kernel<T, DK>), dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, s, a);
    }
    if (a.ddt_bias && a.H > 0)
        hipLaunchKernelGGL((kda_bwd_bias_reduce_kernel<DK>), dim3((unsigned)((a.H * DK + 255) / 256)), dim3(256), 0,
                           s, a);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_bwd_dv(const BwdArgs& a, hipStream_t s) {
    switch (a.Dv) {
        case 16: return launch_bwd_t<T, DK, 16>(a, s);
        case 32: return launch_bwd_t<T, DK, 32>(a, s);
        case 64: return launch_bwd_t<T, DK, 64>(a, s);
        case 128: return launch_bwd_t<T, DK, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_bwd_dk(int DK, const BwdArgs& a, hipStream_t s) {
    switch (DK) {
        case 16: return launch_bwd_dv<T, 16>(a, s);
        case 32: return launch_bwd_dv<T, 32>(a, s);
        case 64: return launch_bwd_dv<T, 64>(a, s);
        case 128: return launch_bwd_dv<T, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_bwd(int dt, int DK, const BwdArgs& a, hipStream_t s) {
    return dt == 1 ? launch_bwd_dk<bf16_t>(DK, a, s) : launch_bwd_dk<float>(DK, a, s);
}

}  // namespace kda
