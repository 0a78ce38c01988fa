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
// Five kernels:
//  1. kda_bwd_ops:     per chunk-head, the chunk operators in fp32 (Aqk and
//                      At element by element in log space, T by forward
//                      substitution; Kd, Qp, Kp and the transposes the
//                      matrix cores read).
//  2. kda_bwd_states:  per (b, h), serial over chunks: the state at each
//                      chunk start (fp32 MFMA, one wave per 16 value columns).
//  3. kda_bwd_adjoint: per (b, h), serial over chunks in reverse: the adjoint
//                      at each chunk end, and dS0.
//  4. kda_bwd_grads:   per chunk-head: every input gradient of the chunk.
//  5. kda_bwd_dA:      the sum of the per-chunk dA_log parts.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = kBwdChunk;

// Element offsets of the fp32 operator block of one chunk-head.  Matrices
// that serve as matrix-core A operands are stored as operand tiles: tile
// (row block rb, contraction step ks) holds 64 lanes x 8 slots, lane 16 gq + r
// supplying row 16 rb + r at contraction index 32 ks + slot_index(gq, j), so
// a lane reads its fragment as 32 contiguous bytes (no LDS bank conflicts,
// whole global lines).
template <int DK> struct Ops {
    // region S (the state pass)
    static constexpr size_t Kd = 0;                                  // tiles [C x DK]   k_hat exp(G)
    static constexpr size_t KpT = Kd + bwd_tiles(C, DK);             // tiles [DK x C]   (k_hat exp(G_C - G))^T
    static constexpr size_t Tm = KpT + bwd_tiles(DK, C);             // tiles [C x C]    (I + Diag(beta) At)^-1
    static constexpr size_t gamS = Tm + bwd_tiles(C, C);             // [DK]  exp(G_C)
    static constexpr size_t betaS = gamS + DK;                       // [C]
    static constexpr size_t sizeS = bwd_op_region_s(DK);
    // region A (the adjoint pass), offsets from the block start
    static constexpr size_t A0 = sizeS;
    static constexpr size_t Kp = A0;                                 // tiles [C x DK]
    static constexpr size_t QpT = Kp + bwd_tiles(C, DK);             // tiles [DK x C]   (q_hat exp(G))^T
    static constexpr size_t KdT = QpT + bwd_tiles(DK, C);            // tiles [DK x C]
    static constexpr size_t AqkT = KdT + bwd_tiles(DK, C);           // tiles [C x C]    Aqk^T
    static constexpr size_t TT = AqkT + bwd_tiles(C, C);             // tiles [C x C]    T^T
    static constexpr size_t gamA = TT + bwd_tiles(C, C);             // [DK]
    static constexpr size_t betaA = gamA + DK;                       // [C]
    static constexpr size_t sizeA = bwd_op_region_a(DK);
    // row-major At (strictly lower, no beta)
    static constexpr size_t At = A0 + sizeA;
    static_assert(betaS + C <= sizeS && betaA + C <= A0 + sizeA && At + C * C <= bwd_op_floats(DK), "layout");
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
__device__ __forceinline__ Frag<float> frag_tile(const float* M, int rb, int ks, int KS) {
    const float4* p = reinterpret_cast<const float4*>(M + ((size_t)(rb * KS + ks) * 64 + (threadIdx.x & 63)) * 8);
    const float4 lo = p[0], hi = p[1];
    Frag<float> f;
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, size_t i) {
    return to_f<T>(reinterpret_cast<const T*>(p)[i]);
}
template <typename T>
__device__ __forceinline__ void stf(void* p, size_t i, float x) {
    reinterpret_cast<T*>(p)[i] = from_f<T>(x);
}

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
template <int NB>
__device__ __forceinline__ Frag<float> frag_strip(const floatx4 (&X)[NB], int s) {
    if (2 * s + 1 < NB) return frag_from_c<float>(X[2 * s], X[2 * s + 1]);
    return frag_from_c_lo<float>(X[2 * s]);
}

// Per-element log-decay of the switched gate (natural log units).
__device__ __forceinline__ float gate_of(float zv, float eA, float g_min, unsigned flags) {
    if (!(flags & kGateIn)) return zv;
    if (flags & kGateSoftplus) return -eA * (fmaxf(zv, 0.f) + log1pf(expf(-fabsf(zv))));
    return g_min / (1.f + expf(-eA * zv));
}

// The switched activations of one chunk into LDS: q_hat, k_hat, cumulative
// log-decay G (pitch P), beta and the inverse norms.  Tokens past the end are
// zero rows with g = 0 and beta = 0 (identity transitions).
template <typename T, int DK, int P>
__device__ void prep_chunk(const BwdArgs& a, int b, int h, int t0, float (*sQ)[P], float (*sK)[P], float (*sG)[P],
                           float* sB, float* sRq, float* sRk, float (*sZ)[P] = nullptr) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
    const float eA = (a.flags & kGateIn) ? expf(a.A_log[h]) : 0.f;
    for (int e = tid; e < C * DK; e += nthr) {
        const int t = e / DK, d = e % DK;
        const int tok = t0 + t;
        float qv = 0.f, kv = 0.f, zv = 0.f, g = 0.f;
        if (tok < a.T) {
            const size_t idx = (((size_t)b * a.T + tok) * a.H + h) * DK + d;
            qv = ldf<T>(a.q, idx);
            kv = ldf<T>(a.k, idx);
            zv = ldf<T>(a.z, idx);
            g = gate_of(zv, eA, a.g_min, a.flags);
        }
        sQ[t][d] = qv;
        sK[t][d] = kv;
        sG[t][d] = g;
        if (sZ) sZ[t][d] = zv;
    }
    for (int t = tid; t < C; t += nthr) {
        const int tok = t0 + t;
        float bt = 0.f;
        if (tok < a.T) {
            const float br = ldf<T>(a.beta_raw, ((size_t)b * a.T + tok) * a.H + h);
            bt = (a.flags & kBetaSig) ? 1.f / (1.f + expf(-br)) : br;
        }
        sB[t] = bt;
    }
    __syncthreads();
    // inverse norms: one wave per token at a time
    for (int t = wave; t < C; t += nw) {
        float sq = 0.f, sk = 0.f;
        for (int d = lane; d < DK; d += 64) {
            sq += sQ[t][d] * sQ[t][d];
            sk += sK[t][d] * sK[t][d];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            sq += __shfl_xor(sq, off, 64);
            sk += __shfl_xor(sk, off, 64);
        }
        if (lane == 0) {
            sRq[t] = (a.flags & kQkL2) ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
            sRk[t] = (a.flags & kQkL2) ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * DK; e += nthr) {
        const int t = e / DK, d = e % DK;
        sQ[t][d] *= sRq[t];
        sK[t][d] *= sRk[t];
    }
    for (int d = tid; d < DK; d += nthr) {
        float acc = 0.f;
        for (int t = 0; t < C; ++t) {
            acc += sG[t][d];
            sG[t][d] = acc;
        }
    }
    __syncthreads();
}

}  // namespace

// ------------------------------------------------------------------ 1. ops

template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_bwd_ops_kernel(const BwdArgs a) {
    constexpr int P = DK + 1;  // odd pitch: the pair loop reads columns across rows
    __shared__ float sQ[C][P], sK[C][P], sG[C][P];
    __shared__ float sB[C], sRq[C], sRk[C];
    __shared__ float sAt[C][C + 1];
    const int n = blockIdx.x % a.NC;
    const int bh = blockIdx.x / a.NC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    prep_chunk<T, DK, P>(a, b, h, n * C, sQ, sK, sG, sB, sRq, sRk);

    float* op = a.ops + ((size_t)bh * a.NC + n) * bwd_op_floats(DK);
    for (int e = tid; e < C * DK; e += blockDim.x) {
        const int t = e / DK, d = e % DK;
        const float G = sG[t][d], GC = sG[C - 1][d];
        const float kd = sK[t][d] * expf(G);
        const float qp = sQ[t][d] * expf(G);
        const float kp = sK[t][d] * expf(GC - G);  // exponent <= 0
        op[Ops<DK>::Kd + tile_pos(t, d, DK)] = kd;
        op[Ops<DK>::Kp + tile_pos(t, d, DK)] = kp;
        op[Ops<DK>::KdT + tile_pos(d, t, C)] = kd;
        op[Ops<DK>::QpT + tile_pos(d, t, C)] = qp;
        op[Ops<DK>::KpT + tile_pos(d, t, C)] = kp;
    }
    if constexpr (DK < 32) {  // the unused contraction slots of the [C x DK] tiles
        for (int e = tid; e < C * (32 - DK); e += blockDim.x) {
            const int t = e / (32 - DK), k = DK + e % (32 - DK);
            op[Ops<DK>::Kd + tile_pos(t, k, DK)] = 0.f;
            op[Ops<DK>::Kp + tile_pos(t, k, DK)] = 0.f;
        }
    }
    for (int d = tid; d < DK; d += blockDim.x) op[Ops<DK>::gamS + d] = op[Ops<DK>::gamA + d] = expf(sG[C - 1][d]);
    for (int t = tid; t < C; t += blockDim.x) op[Ops<DK>::betaS + t] = op[Ops<DK>::betaA + t] = sB[t];
    // At (strictly lower) and Aqk (lower incl. diagonal), each decay factor in
    // one exponent exp(G_i - G_j) <= 1
    for (int e = tid; e < C * C; e += blockDim.x) {
        const int i = e / C, j = e % C;
        float akk = 0.f, aqk = 0.f;
        if (j <= i) {
            for (int d = 0; d < DK; ++d) {
                const float x = sK[j][d] * expf(sG[i][d] - sG[j][d]);
                akk = fmaf(sK[i][d], x, akk);
                aqk = fmaf(sQ[i][d], x, aqk);
            }
        }
        if (j >= i) akk = 0.f;
        sAt[i][j] = akk;
        op[Ops<DK>::At + i * C + j] = akk;
        op[Ops<DK>::AqkT + tile_pos(j, i, C)] = aqk;
    }
    __syncthreads();
    // T = (I + Diag(beta) At)^-1: unit lower triangular, column j by lane j
    if (tid < C) {
        const int j = tid;
        float col[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float s = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s = fmaf(-sB[i] * sAt[i][m], col[m], s);
            col[i] = s;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
            op[Ops<DK>::Tm + tile_pos(i, j, C)] = col[i];
            op[Ops<DK>::TT + tile_pos(j, i, C)] = col[i];
        }
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

// --------------------------------------------------------------- 2. states

// One workgroup per (b, h) and group of NSW value strips; wave w holds the
// fp32 strip of value columns 16 st .. 16 st + 15 of S in C layout (rows
// 16 R + 4 gq + i, column r).  Each chunk's state-pass operators are copied
// into LDS one chunk ahead.
template <typename T, int DK, int NSW>
__global__ __launch_bounds__(64 * NSW) void kda_bwd_states_kernel(const BwdArgs a) {
    using O = Ops<DK>;
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    constexpr int kPieces = (int)(O::sizeS / 256);
    __shared__ __align__(16) float sOp[2][O::sizeS];
    const int ngrp = (a.Dv / 16) / NSW;
    const int bh = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    const int b = bh / a.H, h = bh % a.H;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int col = 16 * (grp * NSW + w) + r;
    const unsigned char* blk = reinterpret_cast<const unsigned char*>(a.ops + (size_t)bh * a.NC * bwd_op_floats(DK));
    floatx4 S[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[R][i] = a.S0 ? a.S0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    stage_kib(blk, sOp[0], kPieces, w, NSW);
    wait_vmcnt<0>();
    __syncthreads();
    for (int n = 0; n < a.NC; ++n) {
        const int buf = n & 1;
        if (n + 1 < a.NC) stage_kib(blk + (size_t)(n + 1) * bwd_op_floats(DK) * 4, sOp[buf ^ 1], kPieces, w, NSW);
        float* Sn = a.states + ((size_t)bh * a.NC + n) * DK * a.Dv;
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sn[(size_t)(16 * R + 4 * gq + i) * a.Dv + col] = S[R][i];
        const float* op = sOp[buf];
        // E = V - Kd S, scaled by beta per token
        floatx4 Eb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSD; ++s) acc = mma(frag_tile(op + O::Kd, tb, s, KSD), frag_strip(S, s), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i, tok = n * C + t;
                const float v = tok < a.T ? ldf<T>(a.v, (((size_t)b * a.T + tok) * a.H + h) * a.Dv + col) : 0.f;
                Eb[tb][i] = op[O::betaS + t] * (v - acc[i]);
            }
        }
        // U = T (beta E)
        floatx4 U[2];
        const Frag<float> Ebf = frag_from_c<float>(Eb[0], Eb[1]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            U[tb] = mma(frag_tile(op + O::Tm, tb, 0, 1), Ebf, z4);
        }
        // S <- Diag(gamma) S + Kp^T U
        const Frag<float> Uf = frag_from_c<float>(U[0], U[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = op[O::gamS + 16 * R + 4 * gq + i] * S[R][i];
            S[R] = mma(frag_tile(op + O::KpT, R, 0, 1), Uf, acc);
        }
        wait_vmcnt<0>();   // the next chunk's operators are in LDS
        __syncthreads();   // ... for every wave, and this chunk's are no longer read
    }
}

// -------------------------------------------------------------- 3. adjoint

template <typename T, int DK, int NSW>
__global__ __launch_bounds__(64 * NSW) void kda_bwd_adjoint_kernel(const BwdArgs a) {
    using O = Ops<DK>;
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    constexpr int kPieces = (int)(O::sizeA / 256);
    constexpr size_t A0 = O::A0;
    __shared__ __align__(16) float sOp[2][O::sizeA];
    const int ngrp = (a.Dv / 16) / NSW;
    const int bh = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
    const int b = bh / a.H, h = bh % a.H;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int col = 16 * (grp * NSW + w) + r;
    const unsigned char* blk = reinterpret_cast<const unsigned char*>(a.ops + (size_t)bh * a.NC * bwd_op_floats(DK) + A0);
    floatx4 dS[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[R][i] = a.dS_T ? a.dS_T[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    if (a.NC > 0) stage_kib(blk + (size_t)(a.NC - 1) * bwd_op_floats(DK) * 4, sOp[0], kPieces, w, NSW);
    wait_vmcnt<0>();
    __syncthreads();
    for (int n = a.NC - 1, it = 0; n >= 0; --n, ++it) {
        const int buf = it & 1;
        if (n > 0) stage_kib(blk + (size_t)(n - 1) * bwd_op_floats(DK) * 4, sOp[buf ^ 1], kPieces, w, NSW);
        float* An = a.adj + ((size_t)bh * a.NC + n) * DK * a.Dv;
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) An[(size_t)(16 * R + 4 * gq + i) * a.Dv + col] = dS[R][i];
        const float* op = sOp[buf];
        // dO as the B operand of a product over the chunk's tokens
        Frag<float> dOf;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tok = n * C + slot_index(gq, j);
            dOf.v[j] = tok < a.T ? ldf<T>(a.dout, (((size_t)b * a.T + tok) * a.H + h) * a.Dv + col) : 0.f;
        }
        // dU = Aqk^T dO + Kp dS'
        floatx4 dU[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            floatx4 acc = mma(frag_tile(op + (O::AqkT - A0), tb, 0, 1), dOf, z4);
#pragma unroll
            for (int s = 0; s < KSD; ++s) acc = mma(frag_tile(op + (O::Kp - A0), tb, s, KSD), frag_strip(dS, s), acc);
            dU[tb] = acc;
        }
        // -beta W with W = T^T dU
        floatx4 X[2];
        const Frag<float> dUf = frag_from_c<float>(dU[0], dU[1]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 wv = mma(frag_tile(op + (O::TT - A0), tb, 0, 1), dUf, z4);
#pragma unroll
            for (int i = 0; i < 4; ++i) X[tb][i] = -op[O::betaA - A0 + 16 * tb + 4 * gq + i] * wv[i];
        }
        // dS = Diag(gamma) dS' + Qp^T dO - Kd^T (beta W)
        const Frag<float> Xf = frag_from_c<float>(X[0], X[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = op[O::gamA - A0 + 16 * R + 4 * gq + i] * dS[R][i];
            acc = mma(frag_tile(op + (O::QpT - A0), R, 0, 1), dOf, acc);
            dS[R] = mma(frag_tile(op + (O::KdT - A0), R, 0, 1), Xf, acc);
        }
        wait_vmcnt<0>();
        __syncthreads();
    }
    if (a.dS0) {
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] = dS[R][i];
    }
}

// ---------------------------------------------------------------- 4. grads

// B operand of a product over rows k0 .. k0 + 31 of a row-major fp32 matrix
// (leading dimension ld) at column col: lane (r, gq) supplies rows
// k0 + slot_index(gq, j); rows past klen are zero.
__device__ __forceinline__ Frag<float> frag_cols(const float* M, int ld, int k0, int col, int klen) {
    const int gq = (threadIdx.x & 63) >> 4;
    Frag<float> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k = k0 + slot_index(gq, j);
        f.v[j] = k < klen ? M[(size_t)k * ld + col] : 0.f;
    }
    return f;
}

// Sum over the 16 lanes that share lane / 16.
__device__ __forceinline__ float row_sum16(float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 16);
    return x;
}

// One workgroup (eight waves) per chunk-head.  Wave w owns value columns
// 16 w .. 16 w + 15 for the products over tokens (E, dU, U, W stay in C
// layout and feed the next product directly), and channel block 16 w ..
// 16 w + 15 for the products over the value dimension (dQp, dKd, dKp, with
// the rows of dO, U and W read from LDS and the rows of S and dS' as
// contiguous global fragments) and for the decay-weighted sums, where lane
// (r, gq) owns channel 16 w + r and the eight tokens 16 tb + 4 gq + i.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(512) void kda_bwd_grads_kernel(const BwdArgs a) {
    constexpr int NT = 512;
    constexpr int NBV = DV / 16, NBK = DK / 16;
    constexpr int KSD = (DK + 31) / 32, KSV = (DV + 31) / 32;
    constexpr int PV = DV + 4;  // row pitch of the value rows (16-byte rows, spread banks)
    constexpr int kBig = (3 * C * PV > 3 * C * DK) ? 3 * C * PV : 3 * C * DK;
    __shared__ float sQ[C][DK], sK[C][DK], sG[C][DK], sZ[C][DK];
    __shared__ float sB[C], sRq[C], sRk[C], sdB[C];
    __shared__ float sGC[DK];
    __shared__ __align__(16) float sBig[kBig];
    __shared__ float sdAqk[C][C + 1], sdAt[C][C + 1];
    __shared__ float sRed[NT / 64];
    float* sdO = sBig;              // [C][PV]
    float* sU = sBig + C * PV;      // [C][PV]
    float* sW = sBig + 2 * C * PV;  // [C][PV]

    const int n = blockIdx.x % a.NC;
    const int bh = blockIdx.x / a.NC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, r = lane & 15, gq = lane >> 4;
    const int t0 = n * C;
    prep_chunk<T, DK, DK>(a, b, h, t0, sQ, sK, sG, sB, sRq, sRk, sZ);
    const float* op = a.ops + ((size_t)bh * a.NC + n) * bwd_op_floats(DK);
    const float* S0 = a.states + ((size_t)bh * a.NC + n) * DK * DV;
    const float* dSC = a.adj + ((size_t)bh * a.NC + n) * DK * DV;
    auto row_of = [&](int t) { return ((size_t)b * a.T + t0 + t) * a.H + h; };

    for (int e = tid; e < C * DV; e += NT) {
        const int t = e / DV, j = e % DV;
        sdO[t * PV + j] = (t0 + t < a.T) ? ldf<T>(a.dout, row_of(t) * DV + j) : 0.f;
    }
    for (int t = tid; t < C; t += NT) sdB[t] = 0.f;
    __syncthreads();

    // ---- products over tokens, value column block w
    if (w < NBV) {
        const int col = 16 * w + r;
        floatx4 E[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, dU[2] = {E[0], E[0]};
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            const Frag<float> Sf = frag_cols(S0, DV, 32 * s, col, DK);
            const Frag<float> Df = frag_cols(dSC, DV, 32 * s, col, DK);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                E[tb] = mma(frag_tile(op + Ops<DK>::Kd, tb, s, KSD), Sf, E[tb]);
                dU[tb] = mma(frag_tile(op + Ops<DK>::Kp, tb, s, KSD), Df, dU[tb]);
            }
        }
        floatx4 dO[2], Eb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                const float vv = (t0 + t < a.T) ? ldf<T>(a.v, row_of(t) * DV + col) : 0.f;
                E[tb][i] = vv - E[tb][i];           // E = V - Kd S
                Eb[tb][i] = sB[t] * E[tb][i];
                dO[tb][i] = sdO[t * PV + col];
            }
        const Frag<float> dOf = frag_from_c<float>(dO[0], dO[1]);
        const Frag<float> Ebf = frag_from_c<float>(Eb[0], Eb[1]);
        const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
        floatx4 U[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            dU[tb] = mma(frag_tile(op + Ops<DK>::AqkT, tb, 0, 1), dOf, dU[tb]);  // + Aqk^T dO
            U[tb] = mma(frag_tile(op + Ops<DK>::Tm, tb, 0, 1), Ebf, z4);         // T (beta E)
        }
        const Frag<float> dUf = frag_from_c<float>(dU[0], dU[1]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 W = mma(frag_tile(op + Ops<DK>::TT, tb, 0, 1), dUf, z4);  // T^T dU
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                if (t0 + t < a.T) stf<T>(a.dv, row_of(t) * DV + col, sB[t] * W[i]);
                const float p = row_sum16(W[i] * E[tb][i]);
                if (r == 0) atomicAdd(&sdB[t], p);
                sU[t * PV + col] = U[tb][i];
                sW[t * PV + col] = W[i];
            }
        }
    }
    __syncthreads();

    // ---- products over the value dimension
    {   // dA_kk = -W U^T (strictly lower) and dAqk = dO U^T (lower): eight 16x16 tiles
        const int kind = w >> 2, tb = (w >> 1) & 1, sb = w & 1;
        const float* X = kind == 0 ? sW : sdO;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSV; ++s) acc = mma(frag_rows(X, PV, 16 * tb, 32 * s, DV), frag_rows(sU, PV, 16 * sb, 32 * s, DV), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * tb + 4 * gq + i, s = 16 * sb + r;
            if (kind == 0) {
                const float dakk = (s < t) ? -acc[i] : 0.f;
                sdAt[t][s] = sB[t] * dakk;  // dAt = Diag(beta) dA_kk
                const float p = row_sum16(dakk * op[Ops<DK>::At + t * C + s]);
                if (r == 0) atomicAdd(&sdB[t], p);
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
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                dQp[tb] = mma(frag_rows(sdO, PV, 16 * tb, 32 * s, DV), S0f, dQp[tb]);
                dKd[tb] = mma(frag_rows(sW, PV, 16 * tb, 32 * s, DV), S0f, dKd[tb]);
                dKp[tb] = mma(frag_rows(sU, PV, 16 * tb, 32 * s, DV), dSf, dKp[tb]);
            }
        }
        dgam += __shfl_xor(dgam, 16, 64);
        dgam += __shfl_xor(dgam, 32, 64);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) dKd[tb][i] *= -sB[16 * tb + 4 * gq + i];
    }
    __syncthreads();

    // ---- decay-weighted sums: lane (r, gq) of wave w owns channel 16 w + r
    float dqh[2][4], dkh[2][4], dGv[2][4];
    if (w < NBK) {
        const int d = 16 * w + r;
        const float GC = sG[C - 1][d];
        float gcpart = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                const float Gt = sG[t][d];
                const float et = expf(Gt), ect = expf(GC - Gt);
                float dq = dQp[tb][i] * et;
                float dkp = dKd[tb][i] * et;
                float dkm = dKp[tb][i] * ect;
                gcpart = fmaf(dKp[tb][i], sK[t][d] * ect, gcpart);
#pragma unroll 2
                for (int s = 0; s < C; ++s) {
                    const float Gs = sG[s][d];
                    const float e = expf(-fabsf(Gt - Gs));  // exp(G_t - G_s) for s <= t, exp(G_s - G_t) for s >= t
                    if (s <= t) {
                        dq = fmaf(sdAqk[t][s] * sK[s][d], e, dq);
                        dkp = fmaf(sdAt[t][s] * sK[s][d], e, dkp);
                    }
                    if (s >= t) dkm = fmaf(sdAqk[s][t] * sQ[s][d] + sdAt[s][t] * sK[s][d], e, dkm);
                }
                dqh[tb][i] = dq;
                dkh[tb][i] = dkp + dkm;
                dGv[tb][i] = sQ[t][d] * dq + sK[t][d] * (dkp - dkm);
            }
        gcpart += __shfl_xor(gcpart, 16, 64);
        gcpart += __shfl_xor(gcpart, 32, 64);
        if (gq == 0) sGC[d] = gcpart + dgam * expf(GC);
    }
    __syncthreads();  // every read of the value rows is done: reuse their space
    float* fdq = sBig;
    float* fdk = sBig + C * DK;
    float* fdG = sBig + 2 * C * DK;
    if (w < NBK) {
        const int d = 16 * w + r;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i;
                fdq[t * DK + d] = dqh[tb][i];
                fdk[t * DK + d] = dkh[tb][i];
                fdG[t * DK + d] = dGv[tb][i];
            }
    }
    __syncthreads();

    // ---- outputs: dg by a reverse cumulative sum, then the activations
    float dApart = 0.f;
    const float eA = (a.flags & kGateIn) ? expf(a.A_log[h]) : 0.f;
    for (int dd = tid; dd < DK; dd += NT) {
        float acc = sGC[dd];  // the chunk-end terms enter at the last token
        for (int t = C - 1; t >= 0; --t) {
            acc += fdG[t * DK + dd];
            if (t0 + t < a.T) {
                const size_t idx = row_of(t) * DK + dd;
                float dz = acc;
                if (a.flags & kGateIn) {
                    const float zv = sZ[t][dd];
                    if (a.flags & kGateSoftplus) {
                        const float sg = 1.f / (1.f + expf(-zv));
                        dz = acc * (-eA * sg);
                        dApart += acc * gate_of(zv, eA, a.g_min, a.flags);
                    } else {
                        const float sg = 1.f / (1.f + expf(-eA * zv));
                        const float dx = acc * a.g_min * sg * (1.f - sg);  // d / d(e^A z)
                        dz = dx * eA;
                        dApart += dx * eA * zv;
                    }
                }
                stf<T>(a.dz, idx, dz);
            }
        }
    }
    // dq, dk through the L2 norm: dx = r (dx_hat - x_hat (x_hat . dx_hat)); one wave per token
    for (int t = w; t < C; t += NT / 64) {
        if (t0 + t >= a.T) continue;  // wave-uniform
        float pq = 0.f, pk = 0.f;
        for (int dd = lane; dd < DK; dd += 64) {
            pq += sQ[t][dd] * fdq[t * DK + dd];
            pk += sK[t][dd] * fdk[t * DK + dd];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            pq += __shfl_xor(pq, off, 64);
            pk += __shfl_xor(pk, off, 64);
        }
        const bool l2 = (a.flags & kQkL2) != 0;
        for (int dd = lane; dd < DK; dd += 64) {
            const size_t idx = row_of(t) * DK + dd;
            const float gq_ = l2 ? sRq[t] * (fdq[t * DK + dd] - sQ[t][dd] * pq) : fdq[t * DK + dd];
            const float gk_ = l2 ? sRk[t] * (fdk[t * DK + dd] - sK[t][dd] * pk) : fdk[t * DK + dd];
            stf<T>(a.dq, idx, gq_);
            stf<T>(a.dk, idx, gk_);
        }
        if (lane == 0) {
            const float bt = sB[t];
            const float db = (a.flags & kBetaSig) ? sdB[t] * bt * (1.f - bt) : sdB[t];
            stf<T>(a.dbeta_raw, row_of(t), db);
        }
    }
    // the chunk's share of dA_log
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dApart += __shfl_xor(dApart, off, 64);
    if (lane == 0) sRed[w] = dApart;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int ww = 0; ww < NT / 64; ++ww) s += sRed[ww];
        a.dA_part[((size_t)b * a.NC + n) * a.H + h] = s;
    }
}

// ------------------------------------------------------------------- 5. dA

__global__ __launch_bounds__(256) void kda_bwd_dA_kernel(const BwdArgs a) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= a.H) return;
    float s = 0.f;
    for (int bn = 0; bn < a.B * a.NC; ++bn) s += a.dA_part[(size_t)bn * a.H + h];
    a.dA_log[h] = (a.flags & kGateIn) ? s : 0.f;
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
        hipLaunchKernelGGL((kda_bwd_states_kernel<T, DK, NSW>), dim3(serial_groups), dim3(64 * NSW), 0, s, a);
    }
    if (heads > 0)  // with no chunk it passes dS_T (or zero) to dS0
        hipLaunchKernelGGL((kda_bwd_adjoint_kernel<T, DK, NSW>), dim3(serial_groups), dim3(64 * NSW), 0, s, a);
    if (chunk_heads > 0)
        hipLaunchKernelGGL((kda_bwd_grads_kernel<T, DK, DV>), dim3(chunk_heads), dim3(512), 0, s, a);
    if (a.H > 0)
        hipLaunchKernelGGL(kda_bwd_dA_kernel, dim3((unsigned)((a.H + 255) / 256)), dim3(256), 0, s, a);
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
