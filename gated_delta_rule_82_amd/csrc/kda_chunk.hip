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
#include <algorithm>
#include <atomic>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// cache policy of copies whose data is read once: non-temporal (the nt bit of
// the gfx950 cache-policy operand)
constexpr int kCopyNT = 2;

// Largest block-local decay (in log2 units) the factored diagonal product
// takes: its column factor 2^-L then stays 2^10 below the float maximum, the
// headroom kda_safe_chunk_size allows, so a bounded gate the library accepts
// (at most 16 |g_min| / ln 2 = 115.4 over a block at g_min = -5) never
// exceeds it.
constexpr float kWideLog2 = 118.f;

struct IntraArgs {
    const void* q; const void* k; const void* z; const void* beta_raw;
    const float* A_log; void* ws;
    int T, H;            // H: value heads; q and k have H / G heads
    int G;               // value heads per q/k head
    const float* dt_bias;  // [H, DK] gate bias or NULL
    int wsNC;            // chunk blocks per (b, h) in the workspace buffer, chunk c0 first
    int c0, nc;          // chunks [c0, c0 + nc) of every (b, h) in this launch
    float g_min;
    unsigned flags;
};

__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// GENERAL: the kernel for the unbounded v1 gate and for caller-supplied
// log-decays (any g <= 0); the bounded in-kernel gate, which the library only
// accepts when the factored products stay in range, takes the plain kernel.
template <typename T, int DK, int C, bool GENERAL>
__global__ __launch_bounds__(256) void kda_intra_kernel(const IntraArgs a) {
    constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    constexpr int NBK = C / 16;
    constexpr int KSD = (DK + 31) / 32;
    constexpr int NBD = DK / 16;
    constexpr int KSC = (C + 31) / 32;
    constexpr int NV = KSD * 8;
    constexpr int NOFF = NBK > 1 ? NBK - 1 : 1;
    constexpr int NPAIR = NBK > 1 ? NBK * (NBK - 1) / 2 : 1;
    constexpr int KSO = NBK > 1 ? KSD : 1;
    constexpr int NCH = 64 / C;  // chunks per workgroup: four waves of 16-token blocks

    // bf16 inputs are staged through LDS: each wave copies its 16 token rows
    // of q, k and z with whole-row requests (four 256-byte rows per
    // instruction for DK = 128) instead of reading 32-byte pieces of every row
    // from each of several register loads
    constexpr bool kStage = sizeof(T) == 2;
    constexpr int RB = DK * (int)sizeof(T);          // bytes of one token row of one tensor
    constexpr int LPR = RB / 16;                     // 16-byte granules (DMA lanes) per row
    constexpr int kStageWave = 3 * 16 * RB;          // q, k, z rows of one wave
    constexpr int kStagePieces = (16 * RB + 1023) / 1024;  // 1 KiB copies per tensor and wave

    // per chunk of the workgroup:
    __shared__ __align__(16) float s_tot_all[NCH][NBK][DK];     // block totals of the log2 decay
    __shared__ float s_beta_all[NCH][C];
    // phases B to E; the input staging of phase A shares their space (it is
    // dead once phase A's barrier is passed)
    struct PhaseArrays {
        float eE[NCH][NBK][DK];      // exp2(E_I): chunk start to block entry
        float eLl[NCH][NBK][DK];     // exp2(Ll_I): decay over block I
        float eK[NCH][NBK][DK];      // exp2(G_C - E_I - Ll_I): block end to chunk end
        float pair[NCH][NPAIR][DK];  // exp2(E_I - E_{J+1}) <= 1 for J < I - 1
        T offb[NCH][NOFF][KSO][512]; // column operands of off-diagonal blocks
        float akk[NCH][NPAIR][256];  // R layout of A_kk[I][J], J < I
        float tdiag[NCH][NBK][256];  // R layout of (I + A_kk[I][I])^-1
    };
    union SharedPhases {
        PhaseArrays ph;
        unsigned char stage[kStage ? 4 * kStageWave : 16];
    };
    __shared__ __align__(16) SharedPhases sh;
    auto& s_eE_all = sh.ph.eE;
    auto& s_eLl_all = sh.ph.eLl;
    auto& s_eK_all = sh.ph.eK;
    auto& s_pair_all = sh.ph.pair;
    auto& s_offb_all = sh.ph.offb;
    auto& s_akk_all = sh.ph.akk;
    auto& s_tdiag_all = sh.ph.tdiag;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int gq = lane >> 4;

    // workgroup: chunks [c0 + NCH g, c0 + NCH g + nsub) of (b, h); wave w owns
    // 16-token block I of chunk sub
    const int ncg = (a.nc + NCH - 1) / NCH;
    // head index fastest: the workgroups that run together read whole token
    // rows of q, k and z (all heads of the same tokens)
    const int hh = (int)blockIdx.x % a.H;
    const int rest = (int)blockIdx.x / a.H;
    const int g = rest % ncg;
    const int bh = (rest / ncg) * a.H + hh;
    const int nsub = min(NCH, a.nc - g * NCH);
    const int sub = w / NBK;
    const int I = w % NBK;
    const int n = a.c0 + g * NCH + sub;
    const int cid = bh * a.wsNC + (n - a.c0);  // workspace block of (b, h, chunk n)
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int Hk = a.H / a.G;   // q/k heads; value head h reads q/k head h / G
    const int hq = h / a.G;

    float (&s_tot)[NBK][DK] = s_tot_all[sub];
    float (&s_eE)[NBK][DK] = s_eE_all[sub];
    float (&s_eLl)[NBK][DK] = s_eLl_all[sub];
    float (&s_eK)[NBK][DK] = s_eK_all[sub];
    float (&s_pair)[NPAIR][DK] = s_pair_all[sub];
    float (&s_beta)[C] = s_beta_all[sub];
    T (&s_offb)[NOFF][KSO][512] = s_offb_all[sub];
    float (&s_akk)[NPAIR][256] = s_akk_all[sub];
    float (&s_tdiag)[NBK][256] = s_tdiag_all[sub];

    const bool active = sub < nsub;  // wave-uniform
    const int t = n * C + 16 * I + r;
    const bool valid = active && t < a.T;
    // tokens past the end read the last token (finite values); they are made
    // identity transitions below (g = 0, beta = 0), so what they hold never
    // reaches an output
    const size_t row = ((size_t)b * a.T + (t < a.T ? t : a.T - 1)) * a.H + h;
    const size_t row_qk = ((size_t)b * a.T + (t < a.T ? t : a.T - 1)) * Hk + hq;

    T* ws = reinterpret_cast<T*>(a.ws) + (size_t)(active ? cid : 0) * (L.bytes / sizeof(T));

    // ------------------------------------------------------------ phase A
    // Lane (r, gq) of wave I owns token 16 I + r and the channels of its
    // fragment slots; loads, norms, gate and the block-local scan are all
    // wave-local.
    Raw4<T> qr[2 * KSD], kr[2 * KSD];  // q, k as loaded; slot j of step s is element j % 4 of [2 s + j / 4]
    float gv[NV];
    float beta = 0.f;
    // staging of this wave: [tensor q, k, z][row rho][granule position], where
    // position j of row rho holds granule j ^ (rho % LPR) of the token row (a
    // swizzle that spreads the 16 rows read by one instruction over the banks)
    unsigned char* stage = sh.stage + (kStage ? w * kStageWave : 0);
    if constexpr (kStage) {
        if (active) {
            const unsigned char* srcs[3] = {reinterpret_cast<const unsigned char*>(a.q),
                                            reinterpret_cast<const unsigned char*>(a.k),
                                            reinterpret_cast<const unsigned char*>(a.z)};
            const int rho = lane / LPR;       // row within a piece
            const int jpos = lane % LPR;      // granule position written by this lane
#pragma unroll
            for (int p = 0; p < kStagePieces; ++p) {
                const int rw = p * (1024 / RB) + rho;  // token row within the wave's 16
                const int tr = n * C + 16 * I + (rw < 16 ? rw : 15);
                const size_t tok = (size_t)b * a.T + (tr < a.T ? tr : a.T - 1);
                const size_t grow_qk = tok * Hk + hq, grow_z = tok * a.H + h;
                const uint32_t goff = (uint32_t)((jpos ^ (rw % LPR)) * 16);
#pragma unroll
                for (int tn = 0; tn < 3; ++tn) {
                    if (rw < 16)
                        __builtin_amdgcn_global_load_lds(
                            (const __attribute__((address_space(1))) void*)(srcs[tn] + (tn < 2 ? grow_qk : grow_z) * RB + goff),
                            (__attribute__((address_space(3))) void*)(stage + tn * 16 * RB + p * 1024), 16, 0, kCopyNT);
                }
            }
            wait_vmcnt<0>();  // this wave's copies are in LDS (it reads only its own rows)
            asm volatile("" ::: "memory");
        }
    }
#pragma unroll
    for (int s = 0; s < KSD; ++s) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int c = 32 * s + 16 * hf + 4 * gq;
            float* dz = &gv[8 * s + 4 * hf];
            if (active && (DK >= 32 || hf == 0)) {
                if constexpr (kStage) {
                    // granule c / 8 of row r, 8 bytes at (c % 8) * 2 within it
                    const int off = r * RB + (((c / 8) ^ (r % LPR)) * 16) + (c % 8) * 2;
                    qr[2 * s + hf].v = *reinterpret_cast<const uint2*>(stage + off);
                    kr[2 * s + hf].v = *reinterpret_cast<const uint2*>(stage + 16 * RB + off);
                    const uint2 zz = *reinterpret_cast<const uint2*>(stage + 2 * 16 * RB + off);
                    dz[0] = bf16_bits_to_float(zz.x & 0xffffu);
                    dz[1] = bf16_bits_to_float(zz.x >> 16);
                    dz[2] = bf16_bits_to_float(zz.y & 0xffffu);
                    dz[3] = bf16_bits_to_float(zz.y >> 16);
                } else {
                    qr[2 * s + hf].load(reinterpret_cast<const T*>(a.q) + row_qk * DK + c);
                    kr[2 * s + hf].load(reinterpret_cast<const T*>(a.k) + row_qk * DK + c);
                    load4(reinterpret_cast<const T*>(a.z) + row * DK + c, dz);
                }
            } else {
                qr[2 * s + hf].zero();
                kr[2 * s + hf].zero();
#pragma unroll
                for (int i = 0; i < 4; ++i) dz[i] = 0.f;
            }
        }
    }
    {
        const float braw = to_f<T>(reinterpret_cast<const T*>(a.beta_raw)[row]);
        beta = (a.flags & kBetaSig) ? sigmoidf_(braw) : braw;
        beta = valid ? beta : 0.f;
    }
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float x = qr[v / 4].get(v % 4), y = kr[v / 4].get(v % 4);
        sq += x * x;
        sk += y * y;
    }
    sq = group_sum4(sq);
    sk = group_sum4(sk);
    const float rq = (a.flags & kQkL2) ? __builtin_amdgcn_rsqf(sq + kL2Eps) : 1.0f;
    const float rk = (a.flags & kQkL2) ? __builtin_amdgcn_rsqf(sk + kL2Eps) : 1.0f;
    // log2-decay per element; padding tokens are identity transitions (g = 0, beta = 0)
    if (a.flags & kGateIn) {
        if (a.dt_bias) {  // per-dimension gate bias on the logit
            const float* db = a.dt_bias + (size_t)h * DK;
#pragma unroll
            for (int s = 0; s < KSD; ++s)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    if (DK >= 32 || hf == 0) {
                        const float4 d = *reinterpret_cast<const float4*>(db + 32 * s + 16 * hf + 4 * gq);
                        gv[8 * s + 4 * hf] += d.x; gv[8 * s + 4 * hf + 1] += d.y;
                        gv[8 * s + 4 * hf + 2] += d.z; gv[8 * s + 4 * hf + 3] += d.w;
                    }
        }
        const float eA = expf(a.A_log[h]);
        const float zscale = -eA * kLog2e;  // exp2(zscale z) = e^{-e^A z}
        const float gm2 = a.g_min * kLog2e;
        if constexpr (GENERAL) {
            // bounded gate g_min sigmoid(e^A z), or the unbounded v1 gate
            // -e^A softplus(z) (both evaluated, one kept: no divergent code)
            const bool softplus = (a.flags & kGateSoftplus) != 0;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float x = gv[v];
                // one exp2: e^{-e^A z} for the bounded gate, e^{-|z|} for softplus
                const float t = exp2_fast(softplus ? -fabsf(x) * kLog2e : zscale * x);
                const float gb = gm2 * __builtin_amdgcn_rcpf(1.0f + t);
                const float gs = -eA * (fmaxf(x, 0.f) * kLog2e + __builtin_amdgcn_logf(1.0f + t));
                gv[v] = valid ? (softplus ? gs : gb) : 0.f;
            }
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float g2 = gm2 * __builtin_amdgcn_rcpf(1.0f + exp2_fast(zscale * gv[v]));
                gv[v] = valid ? g2 : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) gv[v] = valid ? gv[v] * kLog2e : 0.f;
    }
    // block-local inclusive cumulative log2-decay L, one scan round over all
    // elements at a time so consecutive DPP operations are independent
#pragma unroll
    for (int sh = 0; sh < 4; ++sh) {
#pragma unroll
        for (int v = 0; v < NV; ++v) gv[v] += row_shift_add(gv[v], sh);
    }
    // A block whose decay exceeds 2^-kWideLog2 on some channel (an unbounded
    // gate, or a caller's log-decay) cannot use the factored diagonal product:
    // its column factor 2^-L would leave the float range.  Such a wave forms
    // the diagonal products element by element (phase C), the rest of the
    // chunk algebra only uses factors <= 1.
    bool wide = false;  // wave-uniform
    if constexpr (GENERAL) {
        float lmin = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (DK >= 32 || v % 8 < 4) lmin = fminf(lmin, gv[v]);  // channels that exist
        wide = __ballot(lmin < -kWideLog2) != 0;
    }
    if (active) {
        if (r == 15) {
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                *reinterpret_cast<float4*>(&s_tot[I][32 * s + 4 * gq]) =
                    make_float4(gv[8 * s], gv[8 * s + 1], gv[8 * s + 2], gv[8 * s + 3]);
                if (DK >= 32)
                    *reinterpret_cast<float4*>(&s_tot[I][32 * s + 16 + 4 * gq]) =
                        make_float4(gv[8 * s + 4], gv[8 * s + 5], gv[8 * s + 6], gv[8 * s + 7]);
            }
        }
        if (gq == 0) s_beta[16 * I + r] = beta;
    }
    lds_barrier();

    // ------------------------------------------------------------ phase B
    // Per (block, channel) decay factors, each computed once.
    for (int e = threadIdx.x; e < NCH * NBK * DK; e += 256) {
        const int sb = e / (NBK * DK), Ib = (e / DK) % NBK, c = e % DK;
        if (sb >= nsub) continue;
        float E = 0.f, GC = 0.f;
#pragma unroll
        for (int J = 0; J < NBK; ++J) {
            const float x = s_tot_all[sb][J][c];
            if (J < Ib) E += x;
            GC += x;
        }
        const float Ll = s_tot_all[sb][Ib][c];
        s_eE_all[sb][Ib][c] = exp2_fast(E);
        s_eLl_all[sb][Ib][c] = exp2_fast(Ll);
        s_eK_all[sb][Ib][c] = exp2_fast(GC - E - Ll);
#pragma unroll
        for (int J = 0; J + 1 < NBK; ++J) {
            if (J + 1 < Ib) {
                float gap = 0.f;  // <= 0: decay between the end of block J and the entry of block Ib
#pragma unroll
                for (int K = 0; K < NBK; ++K)
                    if (K > J && K < Ib) gap += s_tot_all[sb][K][c];
                s_pair_all[sb][pair_index(Ib, J)][c] = exp2_fast(gap);
            }
        }
        if (Ib == 0) {
            const size_t cb = (size_t)bh * a.wsNC + g * NCH + sb;  // workspace block of that chunk
            float* gam = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(a.ws) + cb * L.bytes + L.gamma_byte);
            gam[c] = exp2_fast(GC);
        }
    }
    lds_barrier();

    // ------------------------------------------------------------ phase C
    // Row operands (q, k scaled by exp(L)), diagonal column operand
    // (k scaled by exp(-L)), the chunk operands Kd, Qp, and K' for KpT.
    Frag<T> rkf[KSD], rqf[KSD];
    floatx4 akkR = {0.f, 0.f, 0.f, 0.f}, aqkR = akkR, akkC = akkR;  // diagonal block products
    if (active) {
        if (wide) {
            // Diagonal block element by element: entry (i, j) = sum_c x_ic k_jc
            // 2^(L_ic - L_jc), x = k or q, exponent clamped at 0 (positive only
            // above the diagonal, which phase D masks).  The lanes of group gq
            // hold the same channels for the block's 16 tokens, so token j's
            // values come from lane 16 gq + j; each lane sums its own channels,
            // then the four groups add their partial sums.
            // two passes of 8 columns bound the live accumulators
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float pk[8], pq[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float Lv = gv[v];
                    const float qh = qr[v / 4].get(v % 4) * rq;
                    const float kh = kr[v / 4].get(v % 4) * rk;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int src = (lane & 48) | (8 * half + j);
                        const float kj = __shfl(kh, src, 64), Lj = __shfl(Lv, src, 64);
                        const float ke = kj * exp2_fast(fminf(Lv - Lj, 0.f));
                        pk[j] = fmaf(kh, ke, pk[j]);
                        pq[j] = fmaf(qh, ke, pq[j]);
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pk[j] += __shfl_xor(pk[j], 16, 64);
                    pk[j] += __shfl_xor(pk[j], 32, 64);
                    pq[j] += __shfl_xor(pq[j], 16, 64);
                    pq[j] += __shfl_xor(pq[j], 32, 64);
                }
                // every lane of token r now holds row r at columns 8 half + j:
                // R layout picks columns 4 gq + i, C layout takes row 4 gq + i's
                // entry at column r
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int col = 8 * half + j;
                        if (col == 4 * gq + i) {
                            akkR[i] = pk[j];
                            aqkR[i] = pq[j];
                        }
                        const float tj = __shfl(pk[j], (lane & 48) | (4 * gq + i), 64);
                        if (col == r) akkC[i] = tj;
                    }
                }
            }
        }
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            float eE[8], eLl[8], eK[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int c = 32 * s + 16 * hf + 4 * gq;
                if (DK >= 32 || hf == 0) {
                    const float4 x = *reinterpret_cast<const float4*>(&s_eE[I][c]);
                    const float4 y = *reinterpret_cast<const float4*>(&s_eLl[I][c]);
                    const float4 z = *reinterpret_cast<const float4*>(&s_eK[I][c]);
                    eE[4 * hf] = x.x; eE[4 * hf + 1] = x.y; eE[4 * hf + 2] = x.z; eE[4 * hf + 3] = x.w;
                    eLl[4 * hf] = y.x; eLl[4 * hf + 1] = y.y; eLl[4 * hf + 2] = y.z; eLl[4 * hf + 3] = y.w;
                    eK[4 * hf] = z.x; eK[4 * hf + 1] = z.y; eK[4 * hf + 2] = z.z; eK[4 * hf + 3] = z.w;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) { eE[4 * hf + i] = 0.f; eLl[4 * hf + i] = 0.f; eK[4 * hf + i] = 0.f; }
                }
            }
            Frag<T> kd, qp, ob, kp, cdf;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int v = 8 * s + j;
                const float Lv = gv[v];
                const float e1 = exp2_fast(Lv);
                const float einv = exp2_fast(-Lv);
                const float qh = qr[v / 4].get(v % 4) * rq;
                const float kh = kr[v / 4].get(v % 4) * rk;
                const float rsq = qh * e1;
                const float rsk = kh * e1;
                const float cdg = kh * einv;
                // k exp(Ll - L): decay from the token to its block end (in one
                // exponent when 2^-L may overflow)
                float offv;
                if (wide) {
                    const int c = 32 * s + 16 * (j / 4) + 4 * gq + (j % 4);
                    offv = (DK >= 32 || j < 4) ? kh * exp2_fast(s_tot[I][c] - Lv) : 0.f;
                } else {
                    offv = cdg * eLl[j];
                }
                rqf[s].set(j, rsq);
                rkf[s].set(j, rsk);
                cdf.set(j, cdg);
                kd.set(j, rsk * eE[j]);
                qp.set(j, rsq * eE[j]);
                ob.set(j, offv);
                kp.set(j, offv * eK[j]);
            }
            if (!wide) {
                akkR = mma(cdf, rkf[s], akkR);   // R layout: row r, col 4gq+i
                aqkR = mma(cdf, rqf[s], aqkR);
                akkC = mma(rkf[s], cdf, akkC);   // C layout: row 4gq+i, col r
            }
            frag_store(kd, ws + L.kd + (size_t)(I * KSD + s) * 512, lane);
            frag_store(qp, ws + L.qp + (size_t)(I * KSD + s) * 512, lane);
            if constexpr (NBK > 1) {
                if (I < NBK - 1) frag_store(ob, &s_offb[I < NOFF ? I : 0][s][0], lane);
            }
            // KpT tiles by an exact identity product: mma(K' rows, E_R) is the
            // C-layout tile (tokens of block I) x (channels of block R), i.e. one
            // half of the A fragment of KpT for channel block R.
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int R = 2 * s + hf;
                if (R < NBD) {
                    Frag<T> e;
#pragma unroll
                    for (int j = 0; j < 8; ++j) e.set(j, (slot_index(gq, j) == 16 * hf + r) ? 1.f : 0.f);
                    floatx4 x = {0.f, 0.f, 0.f, 0.f};
                    x = mma(kp, e, x);
                    const float xv[4] = {x[0], x[1], x[2], x[3]};
                    T* tile = ws + L.kpt + (size_t)(R * KSC + I / 2) * 512;
                    half_store(tile, lane, I % 2, xv);
                    if (I % 2 == 0 && I + 1 >= NBK) {
                        const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
                        half_store(tile, lane, 1, zero4);
                    }
                }
            }
            // keep each step's table reads next to their use (bounds live registers)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    lds_barrier();

    // ------------------------------------------------------------ phase D
    floatx4 TdC = {0.f, 0.f, 0.f, 0.f}, TdR = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        const float4 bcol = *reinterpret_cast<const float4*>(&s_beta[16 * I + 4 * gq]);
        const float bc[4] = {bcol.x, bcol.y, bcol.z, bcol.w};
        float aq[4];
        floatx4 I4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 4 * gq + i;
            akkR[i] = (cc < r) ? akkR[i] * beta : 0.f;
            aq[i] = (cc <= r) ? aqkR[i] : 0.f;
            akkC[i] = (r < cc) ? akkC[i] * bc[i] : 0.f;
            I4[i] = (cc == r) ? 1.f : 0.f;
        }
        T* aqk_tile = ws + L.aqk + (size_t)(I * KSC + I / 2) * 512;
        half_store(aqk_tile, lane, I % 2, aq);
        if (I % 2 == 0) {
            const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
            half_store(aqk_tile, lane, 1, zero4);
        }
        // off-diagonal blocks J < I: entry (i, j) = sum_c rowside_I[i,c] pair[c] offb_J[j,c]
#pragma unroll
        for (int J = 0; J < NBK - 1; ++J) {
            if (J < I) {
                floatx4 ak = {0.f, 0.f, 0.f, 0.f}, aqo = ak;
#pragma unroll
                for (int s = 0; s < KSD; ++s) {
                    Frag<T> cof;
                    frag_load(cof, &s_offb[J][s][0], lane);
                    if (J + 1 < I) {
                        // columns rescaled by the decay between the blocks (<= 1)
                        const float* pr = &s_pair[pair_index(I, J)][32 * s];
                        const float4 p0 = *reinterpret_cast<const float4*>(pr + 4 * gq);
                        const float4 p1 = DK >= 32 ? *reinterpret_cast<const float4*>(pr + 16 + 4 * gq)
                                                   : make_float4(0.f, 0.f, 0.f, 0.f);
                        const float sc[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                        for (int j = 0; j < 8; ++j) cof.set(j, cof.get(j) * sc[j]);
                    }
                    ak = mma(cof, rkf[s], ak);
                    aqo = mma(cof, rqf[s], aqo);
                }
                float aqv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) { aqv[i] = aqo[i]; ak[i] *= beta; }
                *reinterpret_cast<float4*>(&s_akk[pair_index(I, J)][lane * 4]) = make_float4(ak[0], ak[1], ak[2], ak[3]);
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
        *reinterpret_cast<float4*>(&s_tdiag[I][lane * 4]) = make_float4(TdR[0], TdR[1], TdR[2], TdR[3]);
    }
    lds_barrier();

    // ------------------------------------------------------------ phase E
    // Wave J builds block column J of T = (I + A_kk)^-1:
    //   T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,  then writes R(T_IJ) Diag(beta).
    if (active) {
        const int J = I;
        const float4 bj = *reinterpret_cast<const float4*>(&s_beta[16 * J + 4 * gq]);
        auto write_tb = [&](int Ir, const floatx4& TR) {
            const float x[4] = {TR[0] * bj.x, TR[1] * bj.y, TR[2] * bj.z, TR[3] * bj.w};
            half_store(ws + L.tb + (size_t)(Ir * KSC + J / 2) * 512, lane, J % 2, x);
        };
        write_tb(J, TdR);
        if (J % 2 == 0) {
            const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
            half_store(ws + L.tb + (size_t)(J * KSC + J / 2) * 512, lane, 1, zero4);
        }
        floatx4 TcolC[NBK];
#pragma unroll
        for (int K = 0; K < NBK; ++K) TcolC[K] = TdC;
#pragma unroll
        for (int Ir = 1; Ir < NBK; ++Ir) {
            if (Ir > J) {
                floatx4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = 0; K < NBK - 1; ++K) {
                    if (K >= J && K < Ir) {
                        const float4 v4 = *reinterpret_cast<const float4*>(&s_akk[pair_index(Ir, K)][lane * 4]);
                        const floatx4 aR = {v4.x, v4.y, v4.z, v4.w};
                        X += mm16(aR, TcolC[K]);
                    }
                }
                const float4 t4 = *reinterpret_cast<const float4*>(&s_tdiag[Ir][lane * 4]);
                const floatx4 TiiR = {t4.x, t4.y, t4.z, t4.w};
                TcolC[Ir] = -mm16(TiiR, X);
                write_tb(Ir, -mm16(X, TiiR));
            }
        }
    }
}

struct InterArgs {
    const void* v;
    const float* S0;     // incoming state of the value strips (NULL: zero)
    const float* M0;     // incoming transition of the identity strips (NULL: identity)
    void* o; float* S_out; float* M_out; void* P_out;
    const void* ws;
    int T, H, Dv;
    int wsNC;            // chunk blocks per (b, h) in the workspace buffer, chunk c0 first
    int c0, nc;          // chunks [c0, c0 + nc) in this launch
    int n_m, n_strips, n_groups;
};

constexpr size_t kLdsBudget = 160 * 1024;  // LDS per CU on gfx950

// LDS ring of the inter-chunk kernel.  A slot holds one chunk block followed by
// the chunk's values for the workgroup's NS = 16-column strips
// ([C tokens][16 NS]).  Two copy waves fill the slots with global_load_lds,
// 1 KiB per instruction ("piece"); copy wave 0 issues the first kPer0 pieces
// of a chunk, copy wave 1 the rest (each streams a contiguous half).
template <typename T, int DK, int C, int NS>
struct InterRing {
    static constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    static constexpr int kVRow = 16 * NS * (int)sizeof(T);   // bytes of one token's staged values
    static constexpr size_t kVBytes = round_up((size_t)C * kVRow, 1024);
    static constexpr size_t kSlot = L.bytes + kVBytes;
    // output staging: two tiles of [C tokens][16 NS] (chunk parity), so each
    // output row leaves as one 16 NS-element segment instead of NS strips
    static constexpr int kORow = 16 * NS * (int)sizeof(T);  // bytes of one token's output row
    static constexpr size_t kOTile = (size_t)C * kORow;
    static constexpr size_t kOBytes = 2 * kOTile;
    static constexpr int kBlkPieces = (int)((L.bytes + 1023) / 1024);
    static constexpr int kVPieces = (int)(kVBytes / 1024);
    static constexpr int kPieces = kBlkPieces + kVPieces;
    static constexpr int kPer0 = (kPieces + 1) / 2;  // pieces per chunk of copy wave 0
    static constexpr int kPer1 = kPieces / 2;        // ... and of copy wave 1
    // as many slots as fit, up to 6, with the copies in flight countable by
    // vmcnt (at most kSlots - 2 chunks of one wave are waited over)
    // (a configuration whose one slot and tiles exceed the LDS is never launched)
    static constexpr bool kFits = kSlot + kOBytes <= kLdsBudget;
    static constexpr int kSlotsLds = kFits ? (int)((kLdsBudget - kOBytes) / kSlot) : 1;
    static constexpr int kSlotsVm = 2 + 63 / (kPer0 > 0 ? kPer0 : 1);
    static constexpr int kSlots = kSlotsLds < 6 ? (kSlotsLds < kSlotsVm ? kSlotsLds : kSlotsVm)
                                                : (6 < kSlotsVm ? 6 : kSlotsVm);
    static_assert(kSlots >= 1, "a chunk block must fit in LDS");
    static_assert(kSlots <= 2 || (kSlots - 2) * kPer0 < 64, "vmcnt range");
    static_assert(kVRow % 16 == 0 && 1024 % kVRow == 0, "value rows tile a piece");
    static_assert(kORow % 16 == 0, "output rows are whole 16-byte granules");
};

// Contraction steps s of the token-block products with row block Ib that
// touch the causal lower triangle (2 s <= Ib: step s spans blocks 2 s, 2 s + 1).
constexpr int lower_steps(int nbk, int ksc) {
    int t = 0;
    for (int ib = 0; ib < nbk; ++ib)
        for (int s = 0; s < ksc; ++s) t += (2 * s <= ib) ? 1 : 0;
    return t;
}

// Wait until at most m chunks of this copy wave's pieces (P per chunk) are in
// flight; loads complete in issue order.
template <int P, int MAXM>
__device__ __forceinline__ void wait_chunks(int m) {
    if constexpr (MAXM >= 3) {
        if (m >= 3) { wait_vmcnt<3 * P>(); return; }
    }
    if constexpr (MAXM >= 2) {
        if (m >= 2) { wait_vmcnt<2 * P>(); return; }
    }
    if constexpr (MAXM >= 1) {
        if (m >= 1) { wait_vmcnt<P>(); return; }
    }
    wait_vmcnt<0>();
}

// Inter-chunk kernel.  A workgroup serves NS = NW * SPW 16-column strips of one
// (b, h) with NW compute waves of SPW strips each, plus two copy waves:
//   * the copy waves keep up to kSlots - 1 chunks ahead in the LDS ring
//     (block and values), waiting only on their own loads;
//   * a compute wave holds its strips of S in fp32 registers, reads every
//     operand fragment from LDS once for all its strips, stores o directly,
//     and never waits on global loads.
// One fence-free barrier per chunk hands a slot over.
template <typename T, int DK, int C, int NW, int SPW>
__global__ __launch_bounds__(64 * (NW + 2)) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_inter_kernel(const InterArgs a) {
    constexpr int NS = NW * SPW;
    using Ring = InterRing<T, DK, C, NS>;
    constexpr BlockLayout L = Ring::L;
    constexpr int K = Ring::kSlots;
    constexpr bool kAhead = K >= 3;  // next chunk's operands are read during the current one
    // small bf16 blocks: the chunk's LDS reads are spread between its
    // matrix-core products (see the end of the loop body)
    constexpr bool kInterleave = C <= 32 && sizeof(T) == 2 && SPW == 1;
    constexpr int NBK = C / 16;
    constexpr int KSD = (DK + 31) / 32;
    constexpr int NBD = DK / 16;
    constexpr int KSC = (C + 31) / 32;
    extern __shared__ __align__(16) unsigned char s_raw[];
    // per chunk and strip: products (R, U, S update, O) and LDS reads
    // (KpT, gamma, Qp, Aqk, then Kd, Tb and the values of the next chunk)
    constexpr int kTri = lower_steps(NBK, KSC);
    constexpr int kMfmaPerChunk = NBK * KSD + kTri + NBD * KSC + NBK * KSD + kTri;
    constexpr int kDsPerChunk = NBD * KSC + NBD + NBK * KSD + kTri + NBK * KSD + kTri + 4 * NBK;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int gq = lane >> 4;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = bid % a.n_groups;
    const int bh = bid / a.n_groups;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int cend = a.c0 + a.nc;
    // value columns staged for this workgroup: strips [vs0, vs1) of the value part
    const int vs0 = max(0, grp * NS - a.n_m);
    const int vs1 = min(a.Dv / 16, grp * NS + NS - a.n_m);
    const int vcol0 = 16 * vs0;
    auto slot_of = [&](int n) -> unsigned char* { return s_raw + (size_t)((n - a.c0) % K) * Ring::kSlot; };

    if (w >= NW) {
        // ------------------------------------------------------ copy waves
        const int cw = w - NW;
        const unsigned char* gblk = reinterpret_cast<const unsigned char*>(a.ws) + (size_t)bh * a.wsNC * L.bytes;
        const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(a.v);
        constexpr int kLanesPerRow = Ring::kVRow / 16;
        constexpr int kTokPerPiece = 64 / kLanesPerRow;
        const int vcol = vcol0 + (lane % kLanesPerRow) * (16 / (int)sizeof(T));
        const int vcol_ld = vcol < 16 * vs1 ? vcol : 0;  // columns outside the range load any valid bytes
        // values: a wave-uniform 64-bit base per chunk plus a 32-bit lane offset
        const uint32_t tstride = (uint32_t)(a.H * a.Dv * (int)sizeof(T));  // bytes per token
        const unsigned char* vrow0 = vsrc + (((size_t)b * a.T * a.H + h) * a.Dv) * sizeof(T);
        const uint32_t vlane_tok = (uint32_t)(lane / kLanesPerRow);
        const uint32_t vlane_col = (uint32_t)(vcol_ld * (int)sizeof(T));
        auto issue = [&](int n) {
            unsigned char* slot = slot_of(n);
            const unsigned char* gb = gblk + (size_t)(n - a.c0) * L.bytes;
            const unsigned char* vb = vrow0 + (size_t)n * C * tstride;
            // token rows to load: those of this chunk inside the sequence (>= 1);
            // lanes past them (the chunk's tail, or a piece that spans more
            // tokens than a chunk holds) reload the last row, zeroed or unused later
            const uint32_t lim = (uint32_t)min(a.T - n * C, C);
#pragma unroll
            for (int p = 0; p < Ring::kPieces; ++p) {
                if ((p < Ring::kPer0) != (cw == 0)) continue;
                if (p < Ring::kBlkPieces) {
                    const int off = p * 1024 + lane * 16;
                    if (off < (int)L.bytes)
                        __builtin_amdgcn_global_load_lds(
                            (const __attribute__((address_space(1))) void*)(gb + off),
                            (__attribute__((address_space(3))) void*)(slot + p * 1024), 16, 0, 0);
                } else {
                    const int j = p - Ring::kBlkPieces;
                    uint32_t tok = (uint32_t)(j * kTokPerPiece) + vlane_tok;
                    tok = tok < lim ? tok : lim - 1;
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void*)(vb + (tok * tstride + vlane_col)),
                        (__attribute__((address_space(3))) void*)(slot + L.bytes + j * 1024), 16, 0, kCopyNT);
                }
            }
        };
        auto wait_for = [&](int m) {  // at most m chunks of this wave still in flight
            if (cw == 0) wait_chunks<Ring::kPer0, (K >= 2 ? K - 2 : 0)>(m);
            else wait_chunks<Ring::kPer1, (K >= 2 ? K - 2 : 0)>(m);
        };
        if (K == 1) {
            if (a.nc > 0) { issue(a.c0); wait_for(0); }
            lds_barrier();  // chunk c0 is in LDS
            for (int n = a.c0; n < cend; ++n) {
                lds_barrier();  // the compute waves are done with the slot
                if (n + 1 < cend) { issue(n + 1); wait_for(0); }
                lds_barrier();
            }
        } else {
            // kAhead: chunks n + 1 and n + 2 are in LDS at the barrier ending
            // chunk n (the compute waves read chunk n + 1's operands early);
            // otherwise chunk n + 1.
            constexpr int D = kAhead ? 2 : 1;
            int nis = a.c0;  // next chunk to issue
            for (; nis < cend && nis < a.c0 + K - 1; ++nis) issue(nis);
            if (a.nc > 0) wait_for(max(0, nis - a.c0 - D));
            lds_barrier();  // chunks c0 .. c0 + D - 1 are in LDS
            for (int n = a.c0; n < cend; ++n) {
                // the slot of chunk n - 1 was released at the previous barrier
                if (n + K - 1 < cend) issue(n + K - 1);
                if (n + D < cend) wait_for(min(K - 1 - D, cend - n - 1 - D));  // chunk n + D has landed
                lds_barrier();
            }
        }
        return;
    }

    // ------------------------------------------------------------ compute waves
    // Strip j of this wave: strip index grp * NS + w * SPW + j (wave-uniform).
    bool live[SPW], mstrip[SPW];
    int col0[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const int strip = grp * NS + w * SPW + j;
        live[j] = strip < a.n_strips;
        mstrip[j] = strip < a.n_m;
        col0[j] = (mstrip[j] ? strip : strip - a.n_m) * 16;
    }
    bool any_live = false;
#pragma unroll
    for (int j = 0; j < SPW; ++j) any_live = any_live || live[j];

    // incoming state of each strip: loaded (all loads in flight together), or
    // identity / zero
    floatx4 S[SPW][NBD];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        const float* sinit = live[j] ? (mstrip[j] ? a.M0 : a.S0) : nullptr;  // wave-uniform
        const int sw = mstrip[j] ? DK : a.Dv;
        const int col = col0[j] + r;
        if (sinit) {
#pragma unroll
            for (int R = 0; R < NBD; ++R)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[j][R][i] = sinit[((size_t)bh * DK + 16 * R + 4 * gq + i) * sw + col];
        } else {
#pragma unroll
            for (int R = 0; R < NBD; ++R)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[j][R][i] = (live[j] && mstrip[j] && 16 * R + 4 * gq + i == col) ? 1.f : 0.f;
        }
    }
    // the state is in registers before the loop: inside it the only vector
    // memory operations in flight are output stores, never waited for
    wait_vmcnt<0>();

    using Raw = typename RawBits<T>::type;
    uint32_t vlane[SPW], vmask[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        // byte offset of this lane's column within a staged value row
        // (strips without values read row 0 of the staging area and mask it)
        vlane[j] = (live[j] && !mstrip[j]) ? (uint32_t)((col0[j] - vcol0 + r) * (int)sizeof(T)) : 0u;
        vmask[j] = (live[j] && !mstrip[j]) ? 0xffffffffu : 0u;
    }

    // Outputs leave through the staging tiles: compute wave w stores tokens
    // [w C / NW, (w + 1) C / NW) of the previous chunk's tile, one 16-byte
    // granule per lane and step.  Granule g of the wave's rows covers token
    // g / kGpr, strip (g % kGpr) / kGps of the group, 16 bytes of it.
    constexpr int kEpg = 16 / (int)sizeof(T);      // elements per granule
    constexpr int kGps = 16 / kEpg;                // granules per strip row
    constexpr int kGpr = NS * kGps;                // granules per token row
    constexpr int kTpw = C / NW;                   // tokens stored per compute wave
    constexpr int kOSteps = (kTpw * kGpr + 63) / 64;
    unsigned char* s_otile = s_raw + (size_t)K * Ring::kSlot;
    unsigned char* gbase[NS];   // per strip of the group: output row of token 0 (b, h), or null
    uint32_t gstride[NS];       // bytes per token
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        const int strip = grp * NS + sl;
        const bool ms = strip < a.n_m;
        T* out = ms ? reinterpret_cast<T*>(a.P_out) : reinterpret_cast<T*>(a.o);
        const int out_w = ms ? DK : a.Dv;
        const int c0s = (ms ? strip : strip - a.n_m) * 16;
        gstride[sl] = (uint32_t)(a.H * out_w * (int)sizeof(T));
        gbase[sl] = (strip < a.n_strips && out)
                        ? reinterpret_cast<unsigned char*>(out) + (((size_t)b * a.T * a.H + h) * out_w + c0s) * sizeof(T)
                        : nullptr;
    }
    auto store_rows = [&](int m) {  // rows of chunk m's tile owned by this wave
        const unsigned char* tile = s_otile + (size_t)((m - a.c0) & 1) * Ring::kOTile + (size_t)w * kTpw * Ring::kORow;
#pragma unroll
        for (int st = 0; st < kOSteps; ++st) {
            const int gi = st * 64 + lane;
            const int tok = w * kTpw + gi / kGpr;
            const int sl = (gi % kGpr) / kGps;
            const int part = gi % kGps;
            unsigned char* base = nullptr;
            uint32_t stride = 0;
#pragma unroll
            for (int t = 0; t < NS; ++t)
                if (sl == t) { base = gbase[t]; stride = gstride[t]; }
            if (gi < kTpw * kGpr && base && m * C + tok < a.T) {
                const uint4 v = *reinterpret_cast<const uint4*>(tile + (size_t)gi * 16);
                *reinterpret_cast<uint4*>(base + (size_t)m * C * stride + (uint32_t)tok * stride + (uint32_t)(part * 16)) = v;
            }
        }
    };

    // Operands on the serial path (Kd, Tb and the values of a chunk) live in
    // registers from one chunk to the next: with kAhead they are read for
    // chunk n + 1 while chunk n's output is computed.
    Frag<T> Ak[NBK][KSD], At[NBK][KSC];
    uint32_t Vraw[SPW][NBK * 4];
    auto load_serial = [&](int n) {
        const unsigned char* cur = slot_of(n);
        const T* s_blk = reinterpret_cast<const T*>(cur);
        const unsigned char* s_val = cur + L.bytes;
#pragma unroll
        for (int J = 0; J < NBK; ++J)
#pragma unroll
            for (int s = 0; s < KSD; ++s) frag_load(Ak[J][s], s_blk + L.kd + (size_t)(J * KSD + s) * 512, lane);
#pragma unroll
        for (int Ib = 0; Ib < NBK; ++Ib)
#pragma unroll
            for (int s = 0; s < KSC; ++s)
                if (2 * s <= Ib) frag_load(At[Ib][s], s_blk + L.tb + (size_t)(Ib * KSC + s) * 512, lane);
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
#pragma unroll
            for (int J = 0; J < NBK; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Vraw[j][4 * J + i] =
                        (uint32_t)*reinterpret_cast<const Raw*>(s_val + (16 * J + 4 * gq + i) * Ring::kVRow + vlane[j]);
        }
    };

    lds_barrier();  // the first chunk(s) are in LDS
    if (kAhead && any_live && a.nc > 0) load_serial(a.c0);

    for (int n = a.c0; n < cend; ++n) {
        const unsigned char* cur = slot_of(n);
        const T* s_blk = reinterpret_cast<const T*>(cur);
        const float* s_gam = reinterpret_cast<const float*>(cur + L.gamma_byte);

        if (any_live) {
            if (!kAhead) load_serial(n);
            // the rest of chunk n's operands, read now, used after U
            Frag<T> Ap[NBD][KSC], Aq[NBK][KSD], Aa[NBK][KSC];
            float4 g4[NBD];
#pragma unroll
            for (int R = 0; R < NBD; ++R)
#pragma unroll
                for (int s = 0; s < KSC; ++s) frag_load(Ap[R][s], s_blk + L.kpt + (size_t)(R * KSC + s) * 512, lane);
#pragma unroll
            for (int R = 0; R < NBD; ++R) g4[R] = *reinterpret_cast<const float4*>(s_gam + 16 * R + 4 * gq);
#pragma unroll
            for (int Ib = 0; Ib < NBK; ++Ib) {
#pragma unroll
                for (int s = 0; s < KSD; ++s) frag_load(Aq[Ib][s], s_blk + L.qp + (size_t)(Ib * KSD + s) * 512, lane);
#pragma unroll
                for (int s = 0; s < KSC; ++s)
                    if (2 * s <= Ib) frag_load(Aa[Ib][s], s_blk + L.aqk + (size_t)(Ib * KSC + s) * 512, lane);
            }

            // Operand copy of the incoming state.
            Frag<T> Sf[SPW][KSD];
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int s = 0; s < KSD; ++s)
                    Sf[j][s] = (2 * s + 1 < NBD) ? frag_from_c<T>(S[j][2 * s], S[j][2 * s + 1])
                                                 : frag_from_c_lo<T>(S[j][2 * s]);
            // R = V - Kd S,  U = Tb R   (Tb is block lower triangular)
            Frag<T> Uf[SPW][KSC];
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                // the token blocks' product chains interleaved (independent
                // products between dependent ones).  Rows past the end of the
                // sequence hold finite copies of the last row: their U rows are
                // zero (beta = 0 puts zeros in Tb's rows and columns for them)
                floatx4 Rr[NBK];
#pragma unroll
                for (int J = 0; J < NBK; ++J) Rr[J] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSD; ++s)
#pragma unroll
                    for (int J = 0; J < NBK; ++J) Rr[J] = mma(Ak[J][s], Sf[j][s], Rr[J]);
#pragma unroll
                for (int J = 0; J < NBK; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Rr[J][i] = RawBits<T>::to_float((Raw)(Vraw[j][4 * J + i] & vmask[j])) - Rr[J][i];
                Frag<T> Rf[KSC];
#pragma unroll
                for (int s = 0; s < KSC; ++s)
                    Rf[s] = (2 * s + 1 < NBK) ? frag_from_c<T>(Rr[2 * s], Rr[2 * s + 1]) : frag_from_c_lo<T>(Rr[2 * s]);
                floatx4 U[NBK];
#pragma unroll
                for (int Ib = 0; Ib < NBK; ++Ib) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < KSC; ++s)
                        if (2 * s <= Ib) acc = mma(At[Ib][s], Rf[s], acc);
                    U[Ib] = acc;
                }
#pragma unroll
                for (int s = 0; s < KSC; ++s)
                    Uf[j][s] = (2 * s + 1 < NBK) ? frag_from_c<T>(U[2 * s], U[2 * s + 1]) : frag_from_c_lo<T>(U[2 * s]);
            }
            // S <- Diag(gamma) S + KpT U
#pragma unroll
            for (int j = 0; j < SPW; ++j)
#pragma unroll
                for (int R = 0; R < NBD; ++R) {
                    S[j][R][0] *= g4[R].x; S[j][R][1] *= g4[R].y; S[j][R][2] *= g4[R].z; S[j][R][3] *= g4[R].w;
#pragma unroll
                    for (int s = 0; s < KSC; ++s) S[j][R] = mma(Ap[R][s], Uf[j][s], S[j][R]);
                }
            // next chunk's serial operands, read while the output is computed
            // (the last chunk reads its own slot again: no branch in the loop body)
            if (kAhead) load_serial(n + 1 < cend ? n + 1 : n);
            // O^T = S^T Qp^T + U^T Aqk^T, stored.  A B fragment of S or U is
            // an A fragment of its transpose, and the A fragments of Qp and Aqk
            // are B fragments of theirs, so swapping the operands gives O^T:
            // lane (r, gq) holds value columns 4 gq .. 4 gq + 3 of token
            // 16 Ib + r, one 4-element store per token block.
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                floatx4 acc[NBK];
#pragma unroll
                for (int Ib = 0; Ib < NBK; ++Ib) acc[Ib] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KSD; ++s)
#pragma unroll
                    for (int Ib = 0; Ib < NBK; ++Ib) acc[Ib] = mma(Sf[j][s], Aq[Ib][s], acc[Ib]);
#pragma unroll
                for (int s = 0; s < KSC; ++s)
#pragma unroll
                    for (int Ib = 0; Ib < NBK; ++Ib)
                        if (2 * s <= Ib) acc[Ib] = mma(Uf[j][s], Aa[Ib][s], acc[Ib]);
                // one scheduling region from the loop top to here: issue the
                // chunk's LDS reads (this chunk's S-update and output operands,
                // then the next chunk's serial operands) between the products,
                // so the LDS streams while the matrix core works
                if constexpr (kInterleave) interleave_mfma_ds<kMfmaPerChunk, kDsPerChunk>();
                unsigned char* tile = s_otile + (size_t)((n - a.c0) & 1) * Ring::kOTile;
#pragma unroll
                for (int Ib = 0; Ib < NBK; ++Ib)
                    store4(reinterpret_cast<T*>(tile + (size_t)(16 * Ib + r) * Ring::kORow +
                                                (size_t)((w * SPW + j) * 16 + 4 * gq) * sizeof(T)),
                           acc[Ib]);
            }
        }
        // the previous chunk's outputs (its tile was completed before the last barrier)
        if (n > a.c0) store_rows(n - 1);
        if (K == 1) lds_barrier();  // done reading the single slot
        lds_barrier();              // the next chunk(s) are in LDS
    }
    if (a.nc > 0) store_rows(cend - 1);

#pragma unroll
    for (int j = 0; j < SPW; ++j) {
        float* dst = mstrip[j] ? a.M_out : a.S_out;
        const int dw = mstrip[j] ? DK : a.Dv;
        if (live[j] && dst) {
#pragma unroll
            for (int R = 0; R < NBD; ++R)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[((size_t)bh * DK + 16 * R + 4 * gq + i) * dw + col0[j] + r] = S[j][R][i];
        }
    }
}

// One instantiation of the inter kernel: NW compute waves of one strip each.
template <typename T, int DK, int C, int NW>
struct InterKernel {
    using Ring = InterRing<T, DK, C, NW>;
    static constexpr int kThreads = 64 * (NW + 2);
    static constexpr size_t kLds = (size_t)Ring::kSlots * Ring::kSlot + Ring::kOBytes;
    static const void* fn() { return reinterpret_cast<const void*>(kda_inter_kernel<T, DK, C, NW, 1>); }
    static hipError_t set_attributes() {
        // set on every call: the attribute is per device, and the call only records a limit
        return hipFuncSetAttribute(fn(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    }
    // workgroups of this kernel resident on device `dev` at once (CUs times
    // workgroups per CU), asked once per device; 0 when the runtime cannot say
    static int capacity(int dev) {
        constexpr int kMaxDev = 64;
        static std::atomic<int> cache[kMaxDev];
        if (!Ring::kFits || dev < 0 || dev >= kMaxDev) return 0;
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
        int cus = 0, per_cu = 0;
        if (set_attributes() != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn(), kThreads, kLds) != hipSuccess)
            return 0;
        v = cus * per_cu;
        cache[dev].store(v, std::memory_order_relaxed);
        return v;
    }
    static hipError_t launch(const InterArgs& ea, int BH, hipStream_t s) {
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, C, NW, 1>), dim3((unsigned)BH * ea.n_groups), dim3(kThreads),
                           kLds, s, ea);
        return hipGetLastError();
    }
};

// Launch configuration of the chunk kernels for one (T, DK, C).
//
// Compute waves per inter workgroup: the workgroups of one (b, h) all stream
// the same chunk blocks, and each compute wave reads every block fragment from
// LDS, so fewer waves per workgroup cost fewer LDS reads per strip but more
// workgroups.  The launch takes the fewest waves (1, 2 or 4) whose grid is
// resident on the device in one round; when none is, 4 (or fewer when the
// strips of a (b, h) fit in fewer).
template <typename T, int DK, int C>
struct ChunkLaunch {
    static constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    static constexpr int NCH = 64 / C;  // chunks per intra workgroup

    const ChunkArgs& a;
    int BH;
    int nw = 4;
    InterArgs ea{};

    explicit ChunkLaunch(const ChunkArgs& args) : a(args), BH(args.B * args.H) {
        ea.v = a.v; ea.o = a.o; ea.P_out = a.P_out;
        ea.T = a.T; ea.H = a.H; ea.Dv = a.Dv;
        ea.n_m = (a.M_out || a.P_out) ? DK / 16 : 0;
        ea.n_strips = ea.n_m + a.Dv / 16;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) dev = -1;
        const int caps[3] = {InterKernel<T, DK, C, 1>::capacity(dev), InterKernel<T, DK, C, 2>::capacity(dev),
                             InterKernel<T, DK, C, 4>::capacity(dev)};
        const bool fits[3] = {InterKernel<T, DK, C, 1>::Ring::kFits, InterKernel<T, DK, C, 2>::Ring::kFits,
                              InterKernel<T, DK, C, 4>::Ring::kFits};
        nw = 0;
        for (int i = 0, w = 1; i < 3 && !nw; ++i, w *= 2)
            if (fits[i] && (long long)BH * ((ea.n_strips + w - 1) / w) <= caps[i]) nw = w;
        if (!nw) {  // no grid resident in one round: the fewest workgroups (fewest waves on a tie)
            int best_g = 1 << 30;
            for (int i = 0, w = 1; i < 3; ++i, w *= 2) {
                const int g = (ea.n_strips + w - 1) / w;
                if (fits[i] && g < best_g) { best_g = g; nw = w; }
            }
        }
        ea.n_groups = (ea.n_strips + nw - 1) / nw;
    }
    hipError_t set_attributes() const {
        switch (nw) {
            case 1: return InterKernel<T, DK, C, 1>::set_attributes();
            case 2: return InterKernel<T, DK, C, 2>::set_attributes();
            default: return InterKernel<T, DK, C, 4>::set_attributes();
        }
    }
    // intra kernel over chunks [c0, c0 + nc) into the buffer `buf` of `per` chunks per (b, h)
    hipError_t intra(void* buf, int per, int c0, int nc, hipStream_t s) const {
        IntraArgs ia{a.q, a.k, a.z, a.beta_raw, a.A_log, buf, a.T, a.H, a.G, a.dt_bias, per, c0, nc, a.g_min, a.flags};
        const dim3 grid((unsigned)(BH * ((nc + NCH - 1) / NCH)));
        if ((a.flags & kGateSoftplus) || !(a.flags & kGateIn))
            hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, true>), grid, dim3(256), 0, s, ia);
        else
            hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, false>), grid, dim3(256), 0, s, ia);
        return hipGetLastError();
    }
    // inter kernel over the same chunks; the state enters from S0/M0 (first
    // slice) or the carry region, and leaves to S_out/M_out (last slice) or it
    hipError_t inter(void* buf, int per, int c0, int nc, bool first, bool last, float* S_scr, float* M_scr,
                     hipStream_t s) {
        ea.ws = buf; ea.wsNC = per; ea.c0 = c0; ea.nc = nc;
        ea.S0 = first ? a.S0 : S_scr;
        ea.M0 = first ? nullptr : M_scr;
        ea.S_out = last ? a.S_out : S_scr;
        ea.M_out = last ? a.M_out : M_scr;
        switch (nw) {
            case 1: return InterKernel<T, DK, C, 1>::launch(ea, BH, s);
            case 2: return InterKernel<T, DK, C, 2>::launch(ea, BH, s);
            default: return InterKernel<T, DK, C, 4>::launch(ea, BH, s);
        }
    }
};

template <typename T, int DK, int C>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t stream, hipEvent_t* ev, int n_ev) {
    ChunkLaunch<T, DK, C> cl(a);
    const hipError_t attr = cl.set_attributes();
    if (attr != hipSuccess) return attr;
    const int BH = cl.BH;
    const int per = slice_chunks(BH, a.NC, cl.L.bytes);
    // the kernels below index the workspace with this `per`: refuse a buffer
    // sized for anything else rather than write past it
    if (a.ws_bytes < chunk_workspace_bytes(sizeof(T), DK, a.Dv, C, (size_t)BH, (size_t)per, 1))
        return hipErrorInvalidValue;
    // one buffer of `per` chunks, reused by every slice (same stream), then the carry
    float* S_scr = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(a.ws) + (size_t)BH * per * cl.L.bytes);
    float* M_scr = S_scr + (size_t)BH * DK * a.Dv;

    int k = 0;  // kernels launched so far (event k + 1 is recorded after kernel k)
    auto mark = [&]() -> bool { return !ev || k + 1 >= n_ev || hipEventRecord(ev[++k], stream) == hipSuccess; };
    if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return hipErrorInvalidValue;

    const int nsl = a.NC > 0 ? (a.NC + per - 1) / per : 1;
    for (int sl = 0; sl < nsl; ++sl) {
        const int c0 = sl * per;
        const int nc = std::max(0, std::min(per, a.NC - c0));
        if (nc > 0) {
            const hipError_t e = cl.intra(a.ws, per, c0, nc, stream);
            if (e != hipSuccess) return e;
            if (!mark()) return hipErrorInvalidValue;
        }
        const hipError_t e = cl.inter(a.ws, per, c0, nc, sl == 0, sl == nsl - 1, S_scr, M_scr, stream);
        if (e != hipSuccess) return e;
        if (!mark()) return hipErrorInvalidValue;
    }
    return hipSuccess;
}

int chunk_kernel_count(int elem_bytes, int DK, int C, int BH, int NC) {
    const BlockLayout L = block_layout(elem_bytes, DK, C);
    if (NC <= 0) return 1;
    const int per = slice_chunks(BH, NC, L.bytes);
    return 2 * ((NC + per - 1) / per);
}

// Overlapped schedule over slices of the sequence: intra(s) on `s_main` writes
// buffer s % 2; inter(s) on `aux` reads it after intra(s) and carries the state
// to slice s + 1.  intra(s + 2) reuses the buffer once inter(s) is done.
// Events: sync[b] = intra into buffer b done, sync[2 + b] = inter of buffer b
// done, sync[4] = all inter work done (joined back into s_main).
template <typename T, int DK, int C>
static hipError_t launch_chunk_overlap_t(const ChunkArgs& a, hipStream_t s_main, hipStream_t aux, hipEvent_t* sync,
                                         hipEvent_t* tev, int n_tev) {
    ChunkLaunch<T, DK, C> cl(a);
    const hipError_t attr = cl.set_attributes();
    if (attr != hipSuccess) return attr;
    const int BH = cl.BH;
    const int per = overlap_slice_chunks(BH, a.NC, cl.L.bytes);
    if (a.ws_bytes < chunk_workspace_bytes(sizeof(T), DK, a.Dv, C, (size_t)BH, (size_t)per, 2))
        return hipErrorInvalidValue;
    const size_t buf_bytes = (size_t)BH * per * cl.L.bytes;
    unsigned char* ws = reinterpret_cast<unsigned char*>(a.ws);
    float* S_scr = reinterpret_cast<float*>(ws + 2 * buf_bytes);
    float* M_scr = S_scr + (size_t)BH * DK * a.Dv;
    auto rec = [&](int idx, hipStream_t s) -> bool {
        return !tev || idx >= n_tev || hipEventRecord(tev[idx], s) == hipSuccess;
    };
#define KDA_HIP(x) do { const hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)
    // the aux stream starts after everything already queued on the main stream
    KDA_HIP(hipEventRecord(sync[4], s_main));
    KDA_HIP(hipStreamWaitEvent(aux, sync[4], 0));
    const int nsl = a.NC > 0 ? (a.NC + per - 1) / per : 1;
    int k = 0;  // kernel index for the timing events
    for (int sl = 0; sl < nsl; ++sl) {
        const int c0 = sl * per;
        const int nc = std::max(0, std::min(per, a.NC - c0));
        const int b = sl & 1;
        void* buf = ws + b * buf_bytes;
        if (nc > 0) {
            if (sl >= 2) KDA_HIP(hipStreamWaitEvent(s_main, sync[2 + b], 0));  // inter(sl - 2) has read buffer b
            if (!rec(2 * k, s_main)) return hipErrorInvalidValue;
            KDA_HIP(cl.intra(buf, per, c0, nc, s_main));
            if (!rec(2 * k + 1, s_main)) return hipErrorInvalidValue;
            ++k;
            KDA_HIP(hipEventRecord(sync[b], s_main));
            KDA_HIP(hipStreamWaitEvent(aux, sync[b], 0));
        }
        if (!rec(2 * k, aux)) return hipErrorInvalidValue;
        KDA_HIP(cl.inter(buf, per, c0, nc, sl == 0, sl == nsl - 1, S_scr, M_scr, aux));
        if (!rec(2 * k + 1, aux)) return hipErrorInvalidValue;
        ++k;
        KDA_HIP(hipEventRecord(sync[2 + b], aux));
    }
    // the main stream resumes after the last inter kernel
    KDA_HIP(hipEventRecord(sync[4], aux));
    KDA_HIP(hipStreamWaitEvent(s_main, sync[4], 0));
#undef KDA_HIP
    return hipSuccess;
}

int chunk_overlap_kernel_count(int elem_bytes, int DK, int C, int BH, int NC) {
    const BlockLayout L = block_layout(elem_bytes, DK, C);
    if (NC <= 0) return 1;
    const int per = overlap_slice_chunks(BH, NC, L.bytes);
    return 2 * ((NC + per - 1) / per);
}

template <typename T, int DK>
static hipError_t launch_chunk_c(int C, const ChunkArgs& a, hipStream_t s, hipEvent_t* ev, int n_ev) {
    switch (C) {
        case 16: return launch_chunk_t<T, DK, 16>(a, s, ev, n_ev);
        case 32: return launch_chunk_t<T, DK, 32>(a, s, ev, n_ev);
        case 64: return launch_chunk_t<T, DK, 64>(a, s, ev, n_ev);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_chunk_d(int DK, int C, const ChunkArgs& a, hipStream_t s, hipEvent_t* ev, int n_ev) {
    switch (DK) {
        case 16: return launch_chunk_c<T, 16>(C, a, s, ev, n_ev);
        case 32: return launch_chunk_c<T, 32>(C, a, s, ev, n_ev);
        case 64: return launch_chunk_c<T, 64>(C, a, s, ev, n_ev);
        case 128: return launch_chunk_c<T, 128>(C, a, s, ev, n_ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s, hipEvent_t* ev, int n_ev) {
    return dt == 1 ? launch_chunk_d<bf16_t>(DK, C, a, s, ev, n_ev) : launch_chunk_d<float>(DK, C, a, s, ev, n_ev);
}

template <typename T, int DK>
static hipError_t launch_overlap_c(int C, const ChunkArgs& a, hipStream_t s, hipStream_t aux, hipEvent_t* sync,
                                   hipEvent_t* tev, int n_tev) {
    switch (C) {
        case 16: return launch_chunk_overlap_t<T, DK, 16>(a, s, aux, sync, tev, n_tev);
        case 32: return launch_chunk_overlap_t<T, DK, 32>(a, s, aux, sync, tev, n_tev);
        case 64: return launch_chunk_overlap_t<T, DK, 64>(a, s, aux, sync, tev, n_tev);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_overlap_d(int DK, int C, const ChunkArgs& a, hipStream_t s, hipStream_t aux,
                                   hipEvent_t* sync, hipEvent_t* tev, int n_tev) {
    switch (DK) {
        case 16: return launch_overlap_c<T, 16>(C, a, s, aux, sync, tev, n_tev);
        case 32: return launch_overlap_c<T, 32>(C, a, s, aux, sync, tev, n_tev);
        case 64: return launch_overlap_c<T, 64>(C, a, s, aux, sync, tev, n_tev);
        case 128: return launch_overlap_c<T, 128>(C, a, s, aux, sync, tev, n_tev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_overlap(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s, hipStream_t aux,
                                hipEvent_t* sync, hipEvent_t* tev, int n_tev) {
    return dt == 1 ? launch_overlap_d<bf16_t>(DK, C, a, s, aux, sync, tev, n_tev)
                   : launch_overlap_d<float>(DK, C, a, s, aux, sync, tev, n_tev);
}

}  // namespace kda
