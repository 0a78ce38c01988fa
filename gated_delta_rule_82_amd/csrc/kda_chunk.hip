// kda_chunk.hip - chunkwise KDA forward on gfx950.
//
// Two kernels per call:
//
//  1. kda_intra: one workgroup per (b, h, chunk), fully parallel.  Each wave
//     owns one 16-token block.  It applies the switched activations (L2 norm,
//     sigmoid beta, bounded gate), forms the in-chunk cumulative log-decay,
//     evaluates A_kk and A_qk on the matrix cores with the decay factored
//     around each block's entry point, inverts (I + A_kk) blockwise and writes
//     the chunk's operands to the workspace.
//
//  2. kda_inter: one wave per (b, h, 16-column strip of the state), serial over
//     chunks.  The strip of S stays in fp32 accumulators for the whole
//     sequence; per chunk it computes U = Tb (V - Kd S), O = Qp S + Aqk U and
//     S <- Diag(gamma) S + KpT U on the matrix cores.
//
// Equations ("KDA 模块交互式演示" §1.5 Eqs. 3-4, "Implémenter KDA" 'La forme par
// blocs'), for a chunk with incoming state S and cumulative log-decay G:
//   A_kk[i,j] = beta_i sum_d k_id k_jd exp(G_id - G_jd)  (j < i)
//   A_qk[i,j] =        sum_d q_id k_jd exp(G_id - G_jd)  (j <= i)
//   U = (I + A_kk)^-1 Diag(beta) (V - (K * exp(G)) S)
//   O = (Q * exp(G)) S + A_qk U
//   S <- Diag(exp(G_C)) S + (K * exp(G_C - G))^T U
//
// Overflow-free factoring: the inverse retention of a factored product
// exp(-G) overflows past ~17 tokens at g_min = -5 ("KDA 模块交互式演示" Tab 9;
// "Implémenter KDA" 'La décroissance bornée': a 16-token tile is the safe
// size).  Within a 16-token block with block-local cumulative L (from the
// block's entry), exp(G_i - G_j) = exp(L_i) * exp(-L_j) with both factors in
// [e^-80, e^80].  Across blocks J < I the column factor is taken from the end
// of block J and the gap between blocks is a per-channel scale <= 1.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

struct IntraArgs {
    const void* q; const void* k; const void* z; const void* beta_raw;
    const float* A_log; void* ws;
    int T, H, NC;
    float g_min;
    unsigned flags;
};

__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <typename T, int DK, int C>
__global__ __launch_bounds__(256) void kda_intra_kernel(const IntraArgs a) {
    constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    constexpr int NBK = C / 16;
    constexpr int KSD = (DK + 31) / 32;
    constexpr int NBD = DK / 16;
    constexpr int KSC = (C + 31) / 32;
    constexpr int NV = KSD * 8;
    constexpr int NOFF = NBK > 1 ? NBK - 1 : 1;
    constexpr int NPAIR = NBK > 1 ? NBK * (NBK - 1) / 2 : 1;
    constexpr int KPS = DK + 4;  // padded row stride of the K' staging tile

    __shared__ float s_tot[NBK][DK];     // block totals of the log2 decay
    __shared__ float s_eE[NBK][DK];      // exp2(E_I): decay from chunk start to block entry
    __shared__ float s_eLl[NBK][DK];     // exp2(Ll_I): decay over block I
    __shared__ float s_eK[NBK][DK];      // exp2(G_C - E_I - Ll_I): block end to chunk end
    __shared__ float s_pair[NPAIR][DK];  // exp2(E_I - E_{J+1}) <= 1 for J < I - 1
    __shared__ float s_beta[C];
    __shared__ __align__(16) float s_offb[NOFF][KSD][512];
    __shared__ __align__(16) float s_kp[C][KPS];
    __shared__ __align__(16) float s_akk[NPAIR][256];
    __shared__ __align__(16) float s_tdiag[NBK][256];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 15;
    const int gq = lane >> 4;

    const int cid = blockIdx.x;
    const int n = cid % a.NC;
    const int bh = cid / a.NC;
    const int h = bh % a.H;
    const int b = bh / a.H;

    const bool active = w < NBK;
    const int I = w;
    const int t = n * C + 16 * I + r;
    const bool valid = active && t < a.T;
    const size_t row = ((size_t)b * a.T + t) * a.H + h;

    T* ws = reinterpret_cast<T*>(a.ws) + (size_t)cid * (L.bytes / sizeof(T));
    float* ws_gamma = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) + L.gamma_byte);

    // ------------------------------------------------------------ phase A
    float qv[NV], kv[NV], gv[NV];
    float beta = 0.f;
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int c = 32 * s + 16 * hf + 4 * gq;
            float* dq = &qv[8 * s + 4 * hf];
            float* dk = &kv[8 * s + 4 * hf];
            float* dz = &gv[8 * s + 4 * hf];
            if (valid && c < DK) {
                load4(reinterpret_cast<const T*>(a.q) + row * DK + c, dq);
                load4(reinterpret_cast<const T*>(a.k) + row * DK + c, dk);
                load4(reinterpret_cast<const T*>(a.z) + row * DK + c, dz);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) { dq[i] = 0.f; dk[i] = 0.f; dz[i] = 0.f; }
            }
        }
    }
    if (valid) {
        const float braw = to_f<T>(reinterpret_cast<const T*>(a.beta_raw)[row]);
        beta = (a.flags & kBetaSig) ? sigmoidf_(braw) : braw;
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) { sq += qv[v] * qv[v]; sk += kv[v] * kv[v]; }
    sq = group_sum4(sq);
    sk = group_sum4(sk);
    const float rq = (a.flags & kQkL2) ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;
    const float rk = (a.flags & kQkL2) ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
    const bool gate = (a.flags & kGateIn) != 0;
    const float hscale = gate ? expf(a.A_log[h]) : 0.f;
    const float gm2 = a.g_min * kLog2e;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float g2 = 0.f;  // padding tokens are identity transitions (g = 0, beta = 0)
        if (valid) g2 = gate ? gm2 * sigmoidf_(hscale * gv[v]) : gv[v] * kLog2e;
        gv[v] = row_scan16(g2);  // block-local inclusive cumulative log2-decay L
    }
    if (active) {
        if (r == 15) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int c = 32 * (v / 8) + slot_index(gq, v % 8);
                if (c < DK) s_tot[I][c] = gv[v];
            }
        }
        if (gq == 0) s_beta[16 * I + r] = beta;
    }
    __syncthreads();

    // ------------------------------------------------------------ phase B
    for (int e = threadIdx.x; e < NBK * DK; e += 256) {
        const int Ib = e / DK, c = e % DK;
        float E = 0.f, GC = 0.f;
#pragma unroll
        for (int J = 0; J < NBK; ++J) {
            const float x = s_tot[J][c];
            if (J < Ib) E += x;
            GC += x;
        }
        const float Ll = s_tot[Ib][c];
        s_eE[Ib][c] = exp2f(E);
        s_eLl[Ib][c] = exp2f(Ll);
        s_eK[Ib][c] = exp2f(GC - E - Ll);
#pragma unroll
        for (int J = 0; J + 1 < NBK; ++J) {
            if (J + 1 < Ib) {
                float gap = 0.f;
#pragma unroll
                for (int K = 0; K < NBK; ++K)
                    if (K > J && K < Ib) gap += s_tot[K][c];
                s_pair[pair_index(Ib, J)][c] = exp2f(gap);  // gap <= 0: decay between the blocks
            }
        }
        if (Ib == 0) ws_gamma[c] = exp2f(GC);
    }
    __syncthreads();

    // ------------------------------------------------------------ phase C
    Frag<T> rkf[KSD], rqf[KSD], cdf[KSD];
    if (active) {
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            Frag<T> kd, qp;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int v = 8 * s + j;
                const int c = 32 * s + slot_index(gq, j);
                float rsq = 0.f, rsk = 0.f, cdg = 0.f, kdv = 0.f, qpv = 0.f, offv = 0.f, kpv = 0.f;
                if (c < DK) {
                    const float Lv = gv[v];
                    const float e1 = exp2_fast(Lv);
                    const float einv = exp2_fast(-Lv);
                    const float qh = qv[v] * rq;
                    const float kh = kv[v] * rk;
                    rsq = qh * e1;
                    rsk = kh * e1;
                    cdg = kh * einv;
                    const float eE = s_eE[I][c];
                    kdv = rsk * eE;
                    qpv = rsq * eE;
                    offv = cdg * s_eLl[I][c];
                    kpv = offv * s_eK[I][c];
                    s_kp[16 * I + r][c] = kpv;
                }
                rqf[s].set(j, rsq);
                rkf[s].set(j, rsk);
                cdf[s].set(j, cdg);
                kd.set(j, kdv);
                qp.set(j, qpv);
                if (NBK > 1 && I < NBK - 1) s_offb[I < NOFF ? I : 0][s][lane * 8 + j] = offv;
            }
            frag_store(kd, ws + L.kd + (size_t)(I * KSD + s) * 512, lane);
            frag_store(qp, ws + L.qp + (size_t)(I * KSD + s) * 512, lane);
        }
    }
    __syncthreads();

    // ------------------------------------------------------------ phase D
    floatx4 TdC = {0.f, 0.f, 0.f, 0.f}, TdR = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        floatx4 akkR = {0.f, 0.f, 0.f, 0.f}, aqkR = akkR, akkC = akkR;
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            akkR = mma(cdf[s], rkf[s], akkR);   // R layout: row r, col 4gq+i
            aqkR = mma(cdf[s], rqf[s], aqkR);
            akkC = mma(rkf[s], cdf[s], akkC);   // C layout: row 4gq+i, col r
        }
        float aq[4];
        floatx4 I4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 4 * gq + i;
            akkR[i] = (cc < r) ? akkR[i] * beta : 0.f;
            aq[i] = (cc <= r) ? aqkR[i] : 0.f;
            akkC[i] = (r < cc) ? akkC[i] * s_beta[16 * I + cc] : 0.f;
            I4[i] = (cc == r) ? 1.f : 0.f;
        }
        T* aqk_tile = ws + L.aqk + (size_t)(I * KSC + I / 2) * 512;
        half_store(aqk_tile, lane, I % 2, aq);
        if (I % 2 == 0) {
            const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
            half_store(aqk_tile, lane, 1, zero4);
        }
        // off-diagonal blocks J < I
#pragma unroll
        for (int J = 0; J < NBK - 1; ++J) {
            if (J < I) {
                floatx4 ak = {0.f, 0.f, 0.f, 0.f}, aqo = ak;
#pragma unroll
                for (int s = 0; s < KSD; ++s) {
                    Frag<T> cof;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int c = 32 * s + slot_index(gq, j);
                        float x = 0.f;
                        if (c < DK) {
                            x = s_offb[J][s][lane * 8 + j];
                            if (J + 1 < I) x *= s_pair[pair_index(I, J)][c];
                        }
                        cof.set(j, x);
                    }
                    ak = mma(cof, rkf[s], ak);
                    aqo = mma(cof, rqf[s], aqo);
                }
                float aqv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    aqv[i] = aqo[i];
                    s_akk[pair_index(I, J)][lane * 4 + i] = ak[i] * beta;
                }
                half_store(ws + L.aqk + (size_t)(I * KSC + J / 2) * 512, lane, J % 2, aqv);
            }
        }
        // (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for the strictly lower 16x16 N
        const floatx4 NR = akkR, NC = akkC;
        const floatx4 N2C = mm16(NR, NC), N2R = mm16(NC, NR);
        const floatx4 N3C = mm16(NR, N2C), N3R = mm16(N2C, NR);
        const floatx4 N4C = mm16(N2R, N2C), N4R = mm16(N2C, N2R);
        const floatx4 N8R = mm16(N4C, N4R);
        const floatx4 P1C = I4 - NC + N2C - N3C;
        const floatx4 P1R = I4 - NR + N2R - N3R;
        const floatx4 P2C = P1C + mm16(N4R, P1C);
        const floatx4 P2R = P1R + mm16(P1C, N4R);
        TdC = P2C + mm16(N8R, P2C);
        TdR = P2R + mm16(P2C, N8R);
#pragma unroll
        for (int i = 0; i < 4; ++i) s_tdiag[I][lane * 4 + i] = TdR[i];
    }
    // K'^T tiles (rows = channels, contraction = tokens) from the staged K'
    for (int tile = w; tile < NBD * KSC; tile += 4) {
        const int R = tile / KSC, s = tile % KSC;
        const int c = 16 * R + r;
        Frag<T> f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tok = 32 * s + slot_index(gq, j);
            f.set(j, tok < C ? s_kp[tok][c] : 0.f);
        }
        frag_store(f, ws + L.kpt + (size_t)tile * 512, lane);
    }
    __syncthreads();

    // ------------------------------------------------------------ phase E
    // Wave J builds block column J of T = (I + A_kk)^-1:
    //   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,  then writes R(T_IJ) Diag(beta).
    if (active) {
        const int J = w;
        floatx4 TcolC[NBK];
#pragma unroll
        for (int K = 0; K < NBK; ++K) TcolC[K] = TdC;
        auto write_tb = [&](int Ir, const floatx4& TR) {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = TR[i] * s_beta[16 * J + 4 * gq + i];
            half_store(ws + L.tb + (size_t)(Ir * KSC + J / 2) * 512, lane, J % 2, x);
        };
        write_tb(J, TdR);
        if (J % 2 == 0) {
            const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
            half_store(ws + L.tb + (size_t)(J * KSC + J / 2) * 512, lane, 1, zero4);
        }
#pragma unroll
        for (int Ir = 1; Ir < NBK; ++Ir) {
            if (Ir > J) {
                floatx4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = 0; K < NBK - 1; ++K) {
                    if (K >= J && K < Ir) {
                        floatx4 aR;
#pragma unroll
                        for (int i = 0; i < 4; ++i) aR[i] = s_akk[pair_index(Ir, K)][lane * 4 + i];
                        X += mm16(aR, TcolC[K]);
                    }
                }
                floatx4 TiiR;
#pragma unroll
                for (int i = 0; i < 4; ++i) TiiR[i] = s_tdiag[Ir][lane * 4 + i];
                TcolC[Ir] = -mm16(TiiR, X);
                const floatx4 TR = -mm16(X, TiiR);
                write_tb(Ir, TR);
            }
        }
    }
}

struct InterArgs {
    const void* v; const float* S0;
    void* o; float* S_out; float* M_out; void* P_out;
    const void* ws;
    int T, H, Dv, NC;
    int n_m, n_strips, n_groups;
};

template <typename T, int DK, int C, int NW>
__global__ __launch_bounds__(64 * NW) void kda_inter_kernel(const InterArgs a) {
    constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    constexpr int NBK = C / 16;
    constexpr int KSD = (DK + 31) / 32;
    constexpr int NBD = DK / 16;
    constexpr int KSC = (C + 31) / 32;
    extern __shared__ __align__(16) unsigned char s_raw[];
    const T* s_blk = reinterpret_cast<const T*>(s_raw);
    const float* s_gam = reinterpret_cast<const float*>(s_raw + L.gamma_byte);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 15;
    const int gq = lane >> 4;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = bid % a.n_groups;
    const int bh = bid / a.n_groups;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int strip = grp * NW + w;
    const bool live = strip < a.n_strips;
    const bool mstrip = strip < a.n_m;
    const int col = (mstrip ? strip : strip - a.n_m) * 16 + r;

    floatx4 S[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rw = 16 * R + 4 * gq + i;
            float x = 0.f;
            if (live) {
                if (mstrip) x = (rw == col) ? 1.f : 0.f;
                else if (a.S0) x = a.S0[((size_t)bh * DK + rw) * a.Dv + col];
            }
            S[R][i] = x;
        }
    }

    const size_t blk_elems = L.bytes / sizeof(T);
    const unsigned char* gblk = reinterpret_cast<const unsigned char*>(a.ws) +
                                (size_t)bh * a.NC * L.bytes;
    const T* vsrc = reinterpret_cast<const T*>(a.v);
    T* out = mstrip ? reinterpret_cast<T*>(a.P_out) : reinterpret_cast<T*>(a.o);
    const int out_w = mstrip ? DK : a.Dv;
    const bool store_o = live && out != nullptr;
    (void)blk_elems;

    for (int n = 0; n < a.NC; ++n) {
        floatx4 V[NBK];
#pragma unroll
        for (int J = 0; J < NBK; ++J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = n * C + 16 * J + 4 * gq + i;
                float x = 0.f;
                if (live && !mstrip && tok < a.T)
                    x = to_f<T>(vsrc[(((size_t)b * a.T + tok) * a.H + h) * a.Dv + col]);
                V[J][i] = x;
            }
        }
        __syncthreads();
        {
            const uint4* src = reinterpret_cast<const uint4*>(gblk + (size_t)n * L.bytes);
            uint4* dst = reinterpret_cast<uint4*>(s_raw);
            for (int i = threadIdx.x; i < (int)(L.bytes / 16); i += 64 * NW) dst[i] = src[i];
        }
        __syncthreads();
        if (!live) continue;

        Frag<T> Sf[KSD];
#pragma unroll
        for (int s = 0; s < KSD; ++s)
            Sf[s] = (2 * s + 1 < NBD) ? frag_from_c<T>(S[2 * s], S[2 * s + 1]) : frag_from_c_lo<T>(S[2 * s]);

        // R = V - Kd S
        floatx4 Rr[NBK];
#pragma unroll
        for (int J = 0; J < NBK; ++J) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                Frag<T> A;
                frag_load(A, s_blk + L.kd + (size_t)(J * KSD + s) * 512, lane);
                acc = mma(A, Sf[s], acc);
            }
            Rr[J] = V[J] - acc;
        }
        Frag<T> Rf[KSC];
#pragma unroll
        for (int s = 0; s < KSC; ++s)
            Rf[s] = (2 * s + 1 < NBK) ? frag_from_c<T>(Rr[2 * s], Rr[2 * s + 1]) : frag_from_c_lo<T>(Rr[2 * s]);
        // U = Tb R   (Tb is block lower triangular)
        floatx4 U[NBK];
#pragma unroll
        for (int Ib = 0; Ib < NBK; ++Ib) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSC; ++s) {
                if (2 * s <= Ib) {
                    Frag<T> A;
                    frag_load(A, s_blk + L.tb + (size_t)(Ib * KSC + s) * 512, lane);
                    acc = mma(A, Rf[s], acc);
                }
            }
            U[Ib] = acc;
        }
        Frag<T> Uf[KSC];
#pragma unroll
        for (int s = 0; s < KSC; ++s)
            Uf[s] = (2 * s + 1 < NBK) ? frag_from_c<T>(U[2 * s], U[2 * s + 1]) : frag_from_c_lo<T>(U[2 * s]);
        // O = Qp S + Aqk U
#pragma unroll
        for (int Ib = 0; Ib < NBK; ++Ib) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                Frag<T> A;
                frag_load(A, s_blk + L.qp + (size_t)(Ib * KSD + s) * 512, lane);
                acc = mma(A, Sf[s], acc);
            }
#pragma unroll
            for (int s = 0; s < KSC; ++s) {
                if (2 * s <= Ib) {
                    Frag<T> A;
                    frag_load(A, s_blk + L.aqk + (size_t)(Ib * KSC + s) * 512, lane);
                    acc = mma(A, Uf[s], acc);
                }
            }
            if (store_o) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = n * C + 16 * Ib + 4 * gq + i;
                    if (tok < a.T)
                        out[(((size_t)b * a.T + tok) * a.H + h) * out_w + col] = from_f<T>(acc[i]);
                }
            }
        }
        // S <- Diag(gamma) S + KpT U
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc = S[R];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= s_gam[16 * R + 4 * gq + i];
#pragma unroll
            for (int s = 0; s < KSC; ++s) {
                Frag<T> A;
                frag_load(A, s_blk + L.kpt + (size_t)(R * KSC + s) * 512, lane);
                acc = mma(A, Uf[s], acc);
            }
            S[R] = acc;
        }
    }

    if (live) {
        float* dst = mstrip ? a.M_out : a.S_out;
        const int dw = mstrip ? DK : a.Dv;
        if (dst) {
#pragma unroll
            for (int R = 0; R < NBD; ++R) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rw = 16 * R + 4 * gq + i;
                    dst[((size_t)bh * DK + rw) * dw + col] = S[R][i];
                }
            }
        }
    }
}

template <typename T, int DK, int C>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t stream) {
    constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    constexpr int NW = 4;
    const int BH = a.B * a.H;
    if (a.NC > 0) {
        IntraArgs ia{a.q, a.k, a.z, a.beta_raw, a.A_log, a.ws, a.T, a.H, a.NC, a.g_min, a.flags};
        hipLaunchKernelGGL((kda_intra_kernel<T, DK, C>), dim3((unsigned)BH * a.NC), dim3(256), 0,
                           stream, ia);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    InterArgs ea{};
    ea.v = a.v; ea.S0 = a.S0; ea.o = a.o; ea.S_out = a.S_out; ea.M_out = a.M_out; ea.P_out = a.P_out;
    ea.ws = a.ws; ea.T = a.T; ea.H = a.H; ea.Dv = a.Dv; ea.NC = a.NC;
    ea.n_m = (a.M_out || a.P_out) ? DK / 16 : 0;
    ea.n_strips = ea.n_m + a.Dv / 16;
    ea.n_groups = (ea.n_strips + NW - 1) / NW;
    auto kern = kda_inter_kernel<T, DK, C, NW>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.bytes);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3((unsigned)BH * ea.n_groups), dim3(64 * NW), L.bytes, stream, ea);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_chunk_c(int C, const ChunkArgs& a, hipStream_t s) {
    switch (C) {
        case 16: return launch_chunk_t<T, DK, 16>(a, s);
        case 32: return launch_chunk_t<T, DK, 32>(a, s);
        case 64: return launch_chunk_t<T, DK, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_chunk_d(int DK, int C, const ChunkArgs& a, hipStream_t s) {
    switch (DK) {
        case 16: return launch_chunk_c<T, 16>(C, a, s);
        case 32: return launch_chunk_c<T, 32>(C, a, s);
        case 64: return launch_chunk_c<T, 64>(C, a, s);
        case 128: return launch_chunk_c<T, 128>(C, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s) {
    return dt == 1 ? launch_chunk_d<bf16_t>(DK, C, a, s) : launch_chunk_d<float>(DK, C, a, s);
}

}  // namespace kda
