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

// Element offsets of the fp32 operator block of one chunk-head.
template <int DK> struct Ops {
    static constexpr size_t Kd = 0;                        // [C][DK]  k_hat exp(G)
    static constexpr size_t KdT = Kd + C * DK;             // [DK][C]
    static constexpr size_t QpT = KdT + DK * C;            // [DK][C]  (q_hat exp(G))^T
    static constexpr size_t Kp = QpT + DK * C;             // [C][DK]  k_hat exp(G_C - G)
    static constexpr size_t KpT = Kp + C * DK;             // [DK][C]
    static constexpr size_t Tm = KpT + DK * C;             // [C][C]   (I + Diag(beta) At)^-1
    static constexpr size_t TT = Tm + C * C;               // [C][C]   its transpose
    static constexpr size_t Aqk = TT + C * C;              // [C][C]   lower incl. diagonal
    static constexpr size_t AqkT = Aqk + C * C;            // [C][C]
    static constexpr size_t At = AqkT + C * C;             // [C][C]   strictly lower, no beta
    static constexpr size_t gam = At + C * C;              // [DK]     exp(G_C)
    static constexpr size_t beta = gam + DK;               // [C]
};

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
                           float* sB, float* sRq, float* sRk) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = nthr >> 6;
    const float eA = (a.flags & kGateIn) ? expf(a.A_log[h]) : 0.f;
    for (int e = tid; e < C * DK; e += nthr) {
        const int t = e / DK, d = e % DK;
        const int tok = t0 + t;
        float qv = 0.f, kv = 0.f, g = 0.f;
        if (tok < a.T) {
            const size_t idx = (((size_t)b * a.T + tok) * a.H + h) * DK + d;
            qv = ldf<T>(a.q, idx);
            kv = ldf<T>(a.k, idx);
            g = gate_of(ldf<T>(a.z, idx), eA, a.g_min, a.flags);
        }
        sQ[t][d] = qv;
        sK[t][d] = kv;
        sG[t][d] = g;
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
        op[Ops<DK>::Kd + t * DK + d] = kd;
        op[Ops<DK>::KdT + d * C + t] = kd;
        op[Ops<DK>::QpT + d * C + t] = qp;
        op[Ops<DK>::Kp + t * DK + d] = kp;
        op[Ops<DK>::KpT + d * C + t] = kp;
    }
    for (int d = tid; d < DK; d += blockDim.x) op[Ops<DK>::gam + d] = expf(sG[C - 1][d]);
    for (int t = tid; t < C; t += blockDim.x) op[Ops<DK>::beta + t] = sB[t];
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
        op[Ops<DK>::Aqk + i * C + j] = aqk;
        op[Ops<DK>::AqkT + j * C + i] = aqk;
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
            op[Ops<DK>::Tm + i * C + j] = col[i];
            op[Ops<DK>::TT + j * C + i] = col[i];
        }
    }
}

// --------------------------------------------------------------- 2. states

// One workgroup per (b, h); wave st holds the fp32 strip of value columns
// 16 st .. 16 st + 15 of S in C layout (rows 16 R + 4 gq + i, column r).
template <typename T, int DK>
__global__ __launch_bounds__(512) void kda_bwd_states_kernel(const BwdArgs a) {
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int st = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int col = 16 * st + r;
    floatx4 S[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[R][i] = a.S0 ? a.S0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    for (int n = 0; n < a.NC; ++n) {
        float* Sn = a.states + ((size_t)bh * a.NC + n) * DK * a.Dv;
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sn[(size_t)(16 * R + 4 * gq + i) * a.Dv + col] = S[R][i];
        const float* op = a.ops + ((size_t)bh * a.NC + n) * bwd_op_floats(DK);
        // E = V - Kd S, scaled by beta per token
        floatx4 Eb[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSD; ++s) acc = mma(frag_rows(op + Ops<DK>::Kd, DK, 16 * tb, 32 * s, DK), frag_strip(S, s), acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tb + 4 * gq + i, tok = n * C + t;
                const float v = tok < a.T ? ldf<T>(a.v, (((size_t)b * a.T + tok) * a.H + h) * a.Dv + col) : 0.f;
                Eb[tb][i] = op[Ops<DK>::beta + t] * (v - acc[i]);
            }
        }
        // U = T (beta E)
        floatx4 U[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            U[tb] = mma(frag_rows(op + Ops<DK>::Tm, C, 16 * tb, 0, C), frag_from_c<float>(Eb[0], Eb[1]), z4);
        }
        // S <- Diag(gamma) S + Kp^T U
        const Frag<float> Uf = frag_from_c<float>(U[0], U[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = op[Ops<DK>::gam + 16 * R + 4 * gq + i] * S[R][i];
            S[R] = mma(frag_rows(op + Ops<DK>::KpT, C, 16 * R, 0, C), Uf, acc);
        }
    }
}

// -------------------------------------------------------------- 3. adjoint

template <typename T, int DK>
__global__ __launch_bounds__(512) void kda_bwd_adjoint_kernel(const BwdArgs a) {
    constexpr int NBD = DK / 16, KSD = (DK + 31) / 32;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H;
    const int st = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
    const int col = 16 * st + r;
    floatx4 dS[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[R][i] = a.dS_T ? a.dS_T[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;
    for (int n = a.NC - 1; n >= 0; --n) {
        float* An = a.adj + ((size_t)bh * a.NC + n) * DK * a.Dv;
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) An[(size_t)(16 * R + 4 * gq + i) * a.Dv + col] = dS[R][i];
        const float* op = a.ops + ((size_t)bh * a.NC + n) * bwd_op_floats(DK);
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
            floatx4 acc = mma(frag_rows(op + Ops<DK>::AqkT, C, 16 * tb, 0, C), dOf, z4);
#pragma unroll
            for (int s = 0; s < KSD; ++s) acc = mma(frag_rows(op + Ops<DK>::Kp, DK, 16 * tb, 32 * s, DK), frag_strip(dS, s), acc);
            dU[tb] = acc;
        }
        // -beta W with W = T^T dU
        floatx4 X[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const floatx4 z4 = {0.f, 0.f, 0.f, 0.f};
            const floatx4 w = mma(frag_rows(op + Ops<DK>::TT, C, 16 * tb, 0, C), frag_from_c<float>(dU[0], dU[1]), z4);
#pragma unroll
            for (int i = 0; i < 4; ++i) X[tb][i] = -op[Ops<DK>::beta + 16 * tb + 4 * gq + i] * w[i];
        }
        // dS = Diag(gamma) dS' + Qp^T dO - Kd^T (beta W)
        const Frag<float> Xf = frag_from_c<float>(X[0], X[1]);
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = op[Ops<DK>::gam + 16 * R + 4 * gq + i] * dS[R][i];
            acc = mma(frag_rows(op + Ops<DK>::QpT, C, 16 * R, 0, C), dOf, acc);
            dS[R] = mma(frag_rows(op + Ops<DK>::KdT, C, 16 * R, 0, C), Xf, acc);
        }
    }
    if (a.dS0) {
#pragma unroll
        for (int R = 0; R < NBD; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] = dS[R][i];
    }
}

// ---------------------------------------------------------------- 4. grads

// One workgroup of 512 threads per chunk-head.  Column phases: thread
// (j = tid % DV, token group tid / DV); channel phases: (d = tid % DK, token
// group tid / DK).
template <typename T, int DK, int DV>
__global__ __launch_bounds__(512) void kda_bwd_grads_kernel(const BwdArgs a) {
    constexpr int NT = 512;
    constexpr int TPJ = C * DV / NT;   // tokens per thread, column phases
    constexpr int TPD = C * DK / NT;   // tokens per thread, channel phases
    static_assert(TPJ >= 1 && TPD >= 1, "C * D >= 512");
    constexpr int PV = DV + 1;  // odd pitch: the pair phase reads U across rows
    // value-row arrays E, dO, U, W, later reused for the channel rows dq_hat,
    // dk_hat, dG
    constexpr int kBig = (4 * C * PV > 3 * C * DK) ? 4 * C * PV : 3 * C * DK;
    __shared__ float sQ[C][DK], sK[C][DK], sG[C][DK];
    __shared__ float sB[C], sRq[C], sRk[C], sdB[C];
    __shared__ __align__(16) float sBig[kBig];
    float (*sE)[PV] = reinterpret_cast<float (*)[PV]>(sBig);
    float (*sdO)[PV] = sE + C;
    float (*sU)[PV] = sE + 2 * C;
    float (*sW)[PV] = sE + 3 * C;
    __shared__ float sdAqk[C][C + 1], sdAt[C][C + 1];
    __shared__ float sGC[DK];
    __shared__ float sRed[NT / 64];

    const int n = blockIdx.x % a.NC;
    const int bh = blockIdx.x / a.NC;
    const int b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x;
    const int t0 = n * C;
    prep_chunk<T, DK, DK>(a, b, h, t0, sQ, sK, sG, sB, sRq, sRk);
    const float* op = a.ops + ((size_t)bh * a.NC + n) * bwd_op_floats(DK);
    const float* S0 = a.states + ((size_t)bh * a.NC + n) * DK * DV;
    const float* dSC = a.adj + ((size_t)bh * a.NC + n) * DK * DV;
    auto row_of = [&](int t) { return ((size_t)b * a.T + t0 + t) * a.H + h; };

    for (int e = tid; e < C * DV; e += NT) {
        const int t = e / DV, j = e % DV;
        sdO[t][j] = (t0 + t < a.T) ? ldf<T>(a.dout, row_of(t) * DV + j) : 0.f;
    }
    for (int t = tid; t < C; t += NT) sdB[t] = 0.f;
    for (int d = tid; d < DK; d += NT) sGC[d] = 0.f;

    // ---- column phase 1: E = V - Kd S and Kp dS' for column j
    const int j = tid % DV, tgj = tid / DV;
    float kpds[TPJ];
    {
        float e0[TPJ];
#pragma unroll
        for (int u = 0; u < TPJ; ++u) e0[u] = kpds[u] = 0.f;
        for (int d = 0; d < DK; ++d) {
            const float s0 = S0[(size_t)d * DV + j], ds = dSC[(size_t)d * DV + j];
#pragma unroll
            for (int u = 0; u < TPJ; ++u) {
                const int t = tgj * TPJ + u;
                e0[u] = fmaf(op[Ops<DK>::KdT + d * C + t], s0, e0[u]);
                kpds[u] = fmaf(op[Ops<DK>::KpT + d * C + t], ds, kpds[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < TPJ; ++u) {
            const int t = tgj * TPJ + u;
            const float vv = (t0 + t < a.T) ? ldf<T>(a.v, row_of(t) * DV + j) : 0.f;
            sE[t][j] = vv - e0[u];
        }
    }
    __syncthreads();
    // ---- column phase 2: U = T (beta E), dU = Aqk^T dO + Kp dS'
    {
        float uu[TPJ], du[TPJ];
#pragma unroll
        for (int u = 0; u < TPJ; ++u) {
            const int t = tgj * TPJ + u;
            float x = 0.f, y = kpds[u];
            for (int s = 0; s < C; ++s) {
                x = fmaf(op[Ops<DK>::Tm + t * C + s], sB[s] * sE[s][j], x);
                y = fmaf(op[Ops<DK>::AqkT + t * C + s], sdO[s][j], y);
            }
            uu[u] = x;
            du[u] = y;
        }
#pragma unroll
        for (int u = 0; u < TPJ; ++u) {
            const int t = tgj * TPJ + u;
            sU[t][j] = uu[u];
            sW[t][j] = du[u];  // dU for now
        }
    }
    __syncthreads();
    // ---- column phase 3: W = T^T dU, dV = beta W, dbeta += W . E
    {
        float ww[TPJ];
#pragma unroll
        for (int u = 0; u < TPJ; ++u) {
            const int t = tgj * TPJ + u;
            float x = 0.f;
            for (int s = 0; s < C; ++s) x = fmaf(op[Ops<DK>::TT + t * C + s], sW[s][j], x);
            ww[u] = x;
        }
        __syncthreads();  // every dU read before W replaces it
#pragma unroll
        for (int u = 0; u < TPJ; ++u) {
            const int t = tgj * TPJ + u;
            sW[t][j] = ww[u];
            if (t0 + t < a.T) stf<T>(a.dv, row_of(t) * DV + j, sB[t] * ww[u]);
            atomicAdd(&sdB[t], ww[u] * sE[t][j]);
        }
    }
    __syncthreads();
    // ---- pair phase: dA_kk = -W U^T (strictly lower), dAqk = dO U^T (lower)
    for (int e = tid; e < C * C; e += NT) {
        const int t = e / C, s = e % C;
        float x = 0.f, y = 0.f;
        if (s <= t) {
            for (int jj = 0; jj < DV; ++jj) {
                x = fmaf(sW[t][jj], sU[s][jj], x);
                y = fmaf(sdO[t][jj], sU[s][jj], y);
            }
        }
        const float dakk = (s < t) ? -x : 0.f;
        sdAt[t][s] = sB[t] * dakk;                 // dAt = Diag(beta) dA_kk
        sdAqk[t][s] = (s <= t) ? y : 0.f;
        if (s < t) atomicAdd(&sdB[t], dakk * op[Ops<DK>::At + t * C + s]);
    }
    __syncthreads();
    // ---- channel phase: dQp, dKd, dKp, dgamma, then the decay-weighted sums
    const int d = tid % DK, tgd = tid / DK;
    float dQp[TPD], dKd[TPD], dKp[TPD];
    float dgam = 0.f;
#pragma unroll
    for (int u = 0; u < TPD; ++u) dQp[u] = dKd[u] = dKp[u] = 0.f;
    for (int jj = 0; jj < DV; ++jj) {
        const float s0 = S0[(size_t)d * DV + jj], ds = dSC[(size_t)d * DV + jj];
#pragma unroll
        for (int u = 0; u < TPD; ++u) {
            const int t = tgd * TPD + u;
            dQp[u] = fmaf(sdO[t][jj], s0, dQp[u]);
            dKd[u] = fmaf(-sB[t] * sW[t][jj], s0, dKd[u]);
            dKp[u] = fmaf(sU[t][jj], ds, dKp[u]);
        }
        dgam = fmaf(ds, s0, dgam);
    }
    const float GC = sG[C - 1][d];
    float gcpart = 0.f;
    float dqh[TPD], dkh[TPD], dG[TPD];
#pragma unroll
    for (int u = 0; u < TPD; ++u) {
        const int t = tgd * TPD + u;
        const float Gt = sG[t][d];
        const float et = expf(Gt);
        const float ect = expf(GC - Gt);
        float dq = dQp[u] * et;
        float dkp = dKd[u] * et;
        float dkm = dKp[u] * ect;
        gcpart = fmaf(dKp[u], sK[t][d] * ect, gcpart);
        for (int s = 0; s < C; ++s) {
            const float Gs = sG[s][d];
            if (s <= t) {
                const float e = expf(Gt - Gs);  // exp(G_t - G_s) <= 1
                dq = fmaf(sdAqk[t][s] * sK[s][d], e, dq);
                dkp = fmaf(sdAt[t][s] * sK[s][d], e, dkp);
            }
            if (s >= t) {
                const float e = expf(Gs - Gt);  // exp(G_s - G_t) <= 1
                dkm = fmaf(sdAqk[s][t] * sQ[s][d] + sdAt[s][t] * sK[s][d], e, dkm);
            }
        }
        dqh[u] = dq;
        dkh[u] = dkp + dkm;
        dG[u] = sQ[t][d] * dq + sK[t][d] * (dkp - dkm);
    }
    atomicAdd(&sGC[d], gcpart + (tgd == 0 ? dgam * expf(GC) : 0.f));
    __syncthreads();  // every read of the value rows is done: reuse their space
    float* fdq = sBig;
    float* fdk = sBig + C * DK;
    float* fdG = sBig + 2 * C * DK;
#pragma unroll
    for (int u = 0; u < TPD; ++u) {
        const int t = tgd * TPD + u;
        fdq[t * DK + d] = dqh[u];
        fdk[t * DK + d] = dkh[u];
        fdG[t * DK + d] = dG[u];
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
                    const float zv = ldf<T>(a.z, idx);
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
    const int lane = tid & 63, wave = tid >> 6;
    for (int t = wave; t < C; t += NT / 64) {
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
    if (lane == 0) sRed[wave] = dApart;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int w = 0; w < NT / 64; ++w) s += sRed[w];
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
    if (chunk_heads > 0) {
        hipLaunchKernelGGL((kda_bwd_ops_kernel<T, DK>), dim3(chunk_heads), dim3(256), 0, s, a);
        hipLaunchKernelGGL((kda_bwd_states_kernel<T, DK>), dim3(heads), dim3(64 * (DV / 16)), 0, s, a);
    }
    if (heads > 0)  // with no chunk it passes dS_T (or zero) to dS0
        hipLaunchKernelGGL((kda_bwd_adjoint_kernel<T, DK>), dim3(heads), dim3(64 * (DV / 16)), 0, s, a);
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
