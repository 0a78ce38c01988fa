// kda_chunk_kernels.h - the chunkwise KDA forward kernels on gfx950 and their
// launch configuration (included by kda_chunk.hip and kda_layer.hip).
//
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
#pragma once

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// cache policy of copies whose data is read once: non-temporal (the nt bit of
// the gfx950 cache-policy operand)
constexpr int kCopyNT = 2;
// cache policy of copies of data other workgroups write during the kernel:
// the sc1 bit, as the agent-scope atomic loads of the same data take it
constexpr int kCopyCoherent = 16;

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
    // fused input-side convolution (CONV instantiations): kernel-4 taps and
    // biases of the q and k channels ([Hk DK][4] / [Hk DK], biases nullable)
    // and the carried window [B][3][cstride] (nullable: zeros) whose rows hold
    // the q channels at offset 0 and the k channels at offset qk_off
    const float* cw_q; const float* cw_k; const float* cb_q; const float* cb_k;
    const void* cstate; int cstride, qk_off;
    // fused output side: the per-token partial sums of squares the inter
    // kernel exchanges between the workgroups of a (b, h), gss_n floats per
    // chunk-head ([B H][wsNC][gss_n]); this kernel marks those of its chunks
    // unwritten (-1) before the inter kernel runs.  NULL: none.
    float* gss = nullptr;
    int gss_n = 0;
};

__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// GENERAL: the kernel for the unbounded v1 gate and for caller-supplied
// log-decays (any g <= 0); the bounded in-kernel gate, which the library only
// accepts when the factored products stay in range, takes the plain kernel.
// CONV: q and k are the raw inputs of the layer's short convolution; the
// kernel forms SiLU(ShortConv_4(.)) of each before everything else.
template <typename T, int DK, int C, bool GENERAL, bool CONV = false>
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

    // The tail of each chunk block (KpT, Tb, Aqk, gamma: the tiles that
    // different waves write in halves) is assembled in LDS and leaves at the
    // end as whole 16-byte lane stores, so every line of the block is written
    // once and in full (bf16, chunks of at most 32 tokens, where the image
    // fits beside the phase arrays in the space of the input staging).
    constexpr bool kImg = kStage && C <= 32;
    constexpr size_t kImgBytes = L.bytes - L.kpt * sizeof(T);  // block bytes from KpT on
    static_assert(kImgBytes % 16 == 0, "whole 16-byte pieces");

    // per chunk of the workgroup:
    __shared__ __align__(16) float s_tot_all[NCH][NBK][DK];     // block totals of the log2 decay
    __shared__ float s_beta_all[NCH][C];
    __shared__ __align__(16) float4 s_cw[CONV ? 2 : 1][CONV ? DK : 1];  // conv taps of q, k channels
    __shared__ float s_cb[CONV ? 2 : 1][CONV ? DK : 1];
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
        __align__(16) unsigned char img[kImg ? NCH : 1][kImg ? kImgBytes : 16];  // block tails (kImg)
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

    if (a.gss) {  // this workgroup's chunks of the exchange area: not yet written
        float* p = a.gss + ((size_t)bh * a.wsNC + (size_t)g * NCH) * a.gss_n;
        for (int e = threadIdx.x; e < nsub * a.gss_n; e += 256) p[e] = -1.f;
    }

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
    // where this wave's block tail (from KpT on) is written: the LDS image
    // (kImg) or the workspace block itself
    T* tl = kImg ? reinterpret_cast<T*>(sh.ph.img[kImg ? sub : 0]) : ws + L.kpt;

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
            if constexpr (!CONV) {
                wait_vmcnt<0>();  // this wave's copies are in LDS (it reads only its own rows)
                asm volatile("" ::: "memory");
            }
        }
    }
    if constexpr (CONV) {
        // taps and biases of the head's q and k channels into LDS; every wave
        // waits for its copies, then a barrier makes all staged rows (the
        // previous block's rows are this block's window) and the taps visible
        if (threadIdx.x < 2 * DK) {
            const int tt = threadIdx.x / DK, c = threadIdx.x % DK;
            const float* cw = tt ? a.cw_k : a.cw_q;
            const float* cb = tt ? a.cb_k : a.cb_q;
            const float4 wv = reinterpret_cast<const float4*>(cw)[(size_t)hq * DK + c];
            const float bv = cb ? cb[(size_t)hq * DK + c] : 0.f;
            s_cw[tt][c] = wv;
            s_cb[tt][c] = bv;
        }
        wait_vmcnt<0>();
        lds_barrier();
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
    if constexpr (CONV) {
        // SiLU(ShortConv_4(x)) of q and k at this lane's token t = 16 I + r and
        // channels.  x[t - 3] comes from this wave's staged row r - 3, the
        // previous wave's row 13 + r, or (the workgroup's first three tokens,
        // and the fp32 path) global memory, the carried window or zero for
        // t - 3 < 0; x[t - 1] and x[t - 2] are the neighbouring lanes' x, or
        // their x[t - 3] where the row runs out.  Values are rounded to the
        // input type as if the convolution had been stored.
        const int tok0 = n * C + 16 * I;           // token of row 0 of this block
        const int tm3 = tok0 + r - 3;              // this lane's x[t - 3]
        Raw4<T> yq[2 * KSD], yk[2 * KSD];
#pragma unroll
        for (int s2 = 0; s2 < KSD; ++s2) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int c = 32 * s2 + 16 * hf + 4 * gq;
                const int e = 2 * s2 + hf;
                yq[e].zero();
                yk[e].zero();
                if (!active || !(DK >= 32 || hf == 0)) continue;
                bool done = false;
                if constexpr (kStage) {
                    const int rw = r >= 3 ? r - 3 : 13 + r;
                    const unsigned char* st = r >= 3 ? stage : (w > 0 ? sh.stage + (w - 1) * kStageWave : nullptr);
                    if (st) {
                        const int off = rw * RB + (((c / 8) ^ (rw % LPR)) * 16) + (c % 8) * 2;
                        yq[e].v = *reinterpret_cast<const uint2*>(st + off);
                        yk[e].v = *reinterpret_cast<const uint2*>(st + 16 * RB + off);
                        done = true;
                    }
                }
                if (!done) {
                    if (tm3 >= 0) {
                        const size_t rr = ((size_t)b * a.T + (tm3 < a.T ? tm3 : a.T - 1)) * Hk + hq;
                        yq[e].load(reinterpret_cast<const T*>(a.q) + rr * DK + c);
                        yk[e].load(reinterpret_cast<const T*>(a.k) + rr * DK + c);
                    } else if (a.cstate) {
                        const T* srow = reinterpret_cast<const T*>(a.cstate) + ((size_t)b * 3 + 3 + tm3) * a.cstride;
                        yq[e].load(srow + (size_t)hq * DK + c);
                        yk[e].load(srow + a.qk_off + (size_t)hq * DK + c);
                    }
                }
            }
        }
        auto conv_tensor = [&](Raw4<T> (&x)[2 * KSD], const Raw4<T> (&y)[2 * KSD], int tt) {
#pragma unroll
            for (int e = 0; e < 2 * KSD; ++e) {
                if (!(DK >= 32 || e % 2 == 0)) continue;  // channels that exist (the rest stay zero)
                Raw4<T> x1, x2;  // x[t - 1], x[t - 2]
#pragma unroll
                for (int wd = 0; wd < Raw4<T>::kWords; ++wd) {
                    const uint32_t xw = x[e].word(wd), yw = y[e].word(wd);
                    const uint32_t a1 = row_shr_word(xw, 1), b1 = row_shl_word(yw, 2);
                    const uint32_t a2 = row_shr_word(xw, 2), b2 = row_shl_word(yw, 1);
                    x1.set_word(wd, r >= 1 ? a1 : b1);
                    x2.set_word(wd, r >= 2 ? a2 : b2);
                }
                const int c = 32 * (e / 2) + 16 * (e % 2) + 4 * gq;
                float out[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    out[i] = silu_(conv4(s_cw[tt][c + i], s_cb[tt][c + i], y[e].get(i), x2.get(i), x1.get(i), x[e].get(i)));
                }
                x[e].set4(out);
            }
        };
        conv_tensor(qr, yq, 0);
        conv_tensor(kr, yk, 1);
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
            float* gam = kImg ? reinterpret_cast<float*>(sh.ph.img[kImg ? sb : 0] + (L.gamma_byte - L.kpt * sizeof(T)))
                              : reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(a.ws) + cb * L.bytes + L.gamma_byte);
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
                    T* tile = tl + kpt_offset(R, I / 2, KSC, NBK);
                    if (kpt_half(I / 2, NBK)) quarter_store(tile, lane, xv);  // no block I + 1: a half tile
                    else half_store(tile, lane, I % 2, xv);
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
        // diagonal block: a half tile for even I (block I + 1 of the step lies
        // above the diagonal), the second half of a full tile for odd I
        T* aqk_tile = tl + (L.aqk - L.kpt) + tri_offset(I, I / 2, KSC);
        if (I % 2 == 0) quarter_store(aqk_tile, lane, aq);
        else half_store(aqk_tile, lane, 1, aq);
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
                half_store(tl + (L.aqk - L.kpt) + tri_offset(I, J / 2, KSC), lane, J % 2, aqv);
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
            T* tile = tl + (L.tb - L.kpt) + tri_offset(Ir, J / 2, KSC);
            if (tri_half(Ir, J / 2)) quarter_store(tile, lane, x);  // diagonal block of an even row block
            else half_store(tile, lane, J % 2, x);
        };
        write_tb(J, TdR);
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
    if constexpr (kImg) {
        // the assembled block tails leave as whole 16-byte pieces
        lds_barrier();
        for (int sb = 0; sb < nsub; ++sb) {
            unsigned char* dst = reinterpret_cast<unsigned char*>(a.ws) +
                                 ((size_t)bh * a.wsNC + g * NCH + sb) * L.bytes + L.kpt * sizeof(T);
            for (int e = threadIdx.x; e < (int)(kImgBytes / 16); e += 256)
                *reinterpret_cast<uint4*>(dst + (size_t)e * 16) = *reinterpret_cast<const uint4*>(sh.ph.img[sb] + e * 16);
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
    // fused input-side convolution of v (CONV instantiations): taps [H Dv][4],
    // biases [H Dv] or NULL, carried window [B][3][cstride] or NULL with the
    // v channels at offset v_off of each row
    const float* cw_v; const float* cb_v; const void* cstate; int cstride, v_off;
    // fused output side (GATE instantiations): o receives
    // sigmoid(gate) * o / sqrt(mean o^2 + 1e-6) * gw per head row; gate
    // [B,T,H,Dv] in the value type, gw [Dv] or NULL (ones), gss the exchange
    // area of the per-token partial sums of squares ([B H][wsNC][n_groups][C],
    // marked -1 by the intra kernel)
    const void* gate; const float* gw; float* gss;
};

constexpr size_t kLdsBudget = 160 * 1024;  // LDS per CU on gfx950

// fused output side: the RMS norm's epsilon (inside the root, as the separate
// output-side kernel takes it) and the bound on polls of one partial sum
constexpr float kGateRmsEps = 1e-6f;
constexpr int kGateSpinLimit = 1 << 20;

// LDS ring of the inter-chunk kernel.  A slot holds one chunk block followed by
// the chunk's values for the workgroup's NS = 16-column strips
// ([C tokens][16 NS]).  Two copy waves fill the slots with global_load_lds,
// 1 KiB per instruction ("piece"); copy wave 0 issues the first kPer0 pieces
// of a chunk, copy wave 1 the rest (each streams a contiguous half).
// GATE (the fused output side): the slot of chunk n also carries the gate
// tile of chunk n - kGateLag (laid out as the values) and the exchange area of
// that chunk (partial sums of squares [C][kGateGroups] fp32, read past the
// caches), so the store waves that store chunk n - kGateLag's rows during
// chunk n find both in LDS.
template <typename T, int DK, int C, int NS, bool SPREAD = true, bool GATE = false>
struct InterRing {
    static constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    static constexpr int kVRow = 16 * NS * (int)sizeof(T);   // bytes of one token's staged values
    static constexpr size_t kVBytes = round_up((size_t)C * kVRow, 1024);
    static constexpr size_t kGBytes = GATE ? kVBytes : 0;                          // gate tile
    static constexpr size_t kPBytes = GATE ? round_up((size_t)kGateGroups * C * 4, 1024) : 0;  // exchange area
    static constexpr size_t kSlot = L.bytes + kVBytes + kGBytes + kPBytes;
    // output staging: tiles of [C tokens][16 NS] (a ring over chunks), so each
    // output row leaves as one 16 NS-element segment instead of NS strips:
    // two (a chunk's rows leave during the next chunk), or with GATE
    // kSlots + 4 (they leave kGateLag = kSlots + 3 chunks later) followed by
    // two sets (chunk parity) of the compute waves' per-lane partial sums of
    // squares [C tokens][NS strips x 4 lane groups]
    static constexpr int kORow = 16 * NS * (int)sizeof(T);  // bytes of one token's output row
    static constexpr size_t kOTile = (size_t)C * kORow;
    static constexpr size_t kSsBytes = GATE ? 2 * (size_t)C * NS * 4 * 4 : 0;
    // Bank-spread layouts (SPREAD).  A compute wave reads the values of
    // tokens 4 gq + i (i fixed per instruction) and writes output rows r, so
    // rows four apart must not share banks.  Values: a 1 KiB piece holds
    // kVTok token rows of kVGran 16-byte granules; granule g of row u of the
    // piece sits at granule position (u % 4) 16 + (u / 4) kVGran + g, so the
    // rows 4 gq + i of one read fall on distinct banks.  Outputs: the tile is
    // cut into 16-row blocks stored granule-column-major (granule og of row t
    // at position og 16 + t % 16), so the 16 rows one write touches are
    // distinct banks; with 8-byte writes (bf16) rows 8-15 of a block also
    // swap the two halves of their granules, so rows eight apart differ in
    // bank too.  Without SPREAD both keep plain row-major order: the fused
    // convolution reads seven value rows per token block at lane-dependent
    // offsets, and for it the plain layouts measured faster.
    static constexpr int kVGran = kVRow / 16;  // granules per staged value row
    static constexpr int kVTok = 64 / kVGran;  // value rows per piece
    static constexpr int kOGran = kORow / 16;  // granules per output row
    static_assert(kVTok % 4 == 0, "pieces hold whole groups of four rows");
    // LDS offset (from the values of the slot) of byte lb of value row t
    static __host__ __device__ constexpr uint32_t voff(int t, uint32_t lb) {
        if (!SPREAD) return (uint32_t)(t * kVRow) + lb;
        return (uint32_t)((t / kVTok) * 1024 +
                          ((((t % kVTok) & 3) * 16 + ((t % kVTok) >> 2) * kVGran + (int)(lb >> 4)) << 4)) +
               (lb & 15u);
    }
    // the row and granule that DMA lane L writes in its piece (the inverse of voff)
    static __device__ __forceinline__ int dma_row(int L) {
        return SPREAD ? 4 * ((L % 16) / kVGran) + L / 16 : L / kVGran;
    }
    static __device__ __forceinline__ int dma_granule(int L) { return SPREAD ? (L % 16) % kVGran : L % kVGran; }
    // LDS offset (from the tile) of byte ob of output row t
    static constexpr bool kSpread = SPREAD;
    static constexpr uint32_t kOHalf = (sizeof(T) == 2 && SPREAD) ? 8u : 0u;
    static __host__ __device__ constexpr uint32_t ooff(int t, uint32_t ob) {
        if (!SPREAD) return (uint32_t)(t * kORow) + ob;
        return (uint32_t)((t >> 4) * 16 * kORow + (((int)(ob >> 4) * 16 + (t & 15)) << 4)) +
               ((ob & 15u) ^ (((t >> 3) & 1) ? kOHalf : 0u));
    }
    static constexpr int kBlkPieces = (int)((L.bytes + 1023) / 1024);
    static constexpr int kVPieces = (int)(kVBytes / 1024);
    static constexpr int kPPieces = (int)(kPBytes / 1024);
    static constexpr int kPieces = kBlkPieces + kVPieces + (GATE ? kVPieces + kPPieces : 0);
    static constexpr int kPer0 = (kPieces + 1) / 2;  // pieces per chunk of copy wave 0
    static constexpr int kPer1 = kPieces / 2;        // ... and of copy wave 1
    // as many slots as fit, up to 6, with the copies in flight countable by
    // vmcnt (at most kSlots - 2 chunks of one wave are waited over); with
    // GATE every slot brings one more output tile
    // (a configuration whose one slot and tiles exceed the LDS is never launched)
    static constexpr size_t kFixed = (GATE ? 4 : 2) * kOTile + kSsBytes;
    static constexpr size_t kPerSlot = kSlot + (GATE ? kOTile : 0);
    static constexpr bool kFitsOne = kPerSlot + kFixed <= kLdsBudget;
    static constexpr int kSlotsLds = kFitsOne ? (int)((kLdsBudget - kFixed) / kPerSlot) : 1;
    static constexpr int kSlotsVm = 2 + 63 / (kPer0 > 0 ? kPer0 : 1);
    static constexpr int kSlots = kSlotsLds < 6 ? (kSlotsLds < kSlotsVm ? kSlotsLds : kSlotsVm)
                                                : (6 < kSlotsVm ? 6 : kSlotsVm);
    // GATE takes at least two slots (with one, the fused output side is not
    // offered and the call takes the separate output-side kernel)
    static constexpr bool kFits = kFitsOne && (!GATE || kSlots >= 2);
    // GATE: chunks between a chunk's products and its store.  The slot of
    // chunk n is copied from the start of chunk n - kSlots + 1 (the ring's
    // depth), so the partials of chunk n - kGateLag it carries were published
    // three chunks before: a group up to that far behind the others costs
    // them no read of the exchange area.
    static constexpr int kGateLag = kSlots + 3;
    static constexpr int kOT = GATE ? kGateLag + 1 : 2;  // output tiles
    static constexpr size_t kOBytes = kOT * kOTile + kSsBytes;
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
//
// GATE: the layer's output side is applied to each output row before it is
// stored ("KDA 模块交互式演示" §1.7 完整层; "Implémenter KDA" 'La porte de
// sortie de rang plein'): y = sigmoid(gate) * o / sqrt(mean o^2 + 1e-6) * gw
// over the head's Dv channels, which the n_groups workgroups of a (b, h)
// share.  NW store waves join the compute and copy waves.  Every compute lane
// writes the sum of squares of its four columns of each token of chunk n to
// LDS (o rounded to the output type first, as a stored o would be); during
// chunk n + 1 store wave 0 adds them up and publishes the workgroup's partial
// of each token to the exchange area.  The copy waves bring chunk m's gate
// tile and every group's partials for it into the slot of chunk m + D
// (D = kGateLag, three more than the ring's depth, so the copy starts well
// after the partials were published), and the store waves store chunk m's
// rows during chunk m + D from the tile kept since, off the compute waves'
// serial chunk step.  A partial not yet published when it was copied (a group
// more than three chunks behind) is read again from the exchange area until
// it is there.  A group waits only for partials of chunks well behind its
// own, which the others publish without waiting on anything later, so the
// wait ends whenever all workgroups of the (b, h) are resident together (the
// launch only takes this path when the whole grid is).  Each wait is also
// bounded: past the bound the row is written as NaN rather than hang.
template <typename T, int DK, int C, int NW, int SPW, bool CONV = false, bool GATE = false>
__global__ __launch_bounds__(64 * (NW + 2 + (GATE ? NW : 0))) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_inter_kernel(const InterArgs a) {
    constexpr int NS = NW * SPW;
    using Ring = InterRing<T, DK, C, NS, !CONV, GATE>;
    constexpr int kOT = Ring::kOT;       // output tiles: a chunk's rows leave 1 or (GATE) D chunks later
    constexpr int D = Ring::kGateLag;
    if constexpr (GATE && !Ring::kFits) return;  // never launched
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

    // Outputs leave through the staging tiles: output wave ow (compute wave
    // ow, or with GATE store wave ow) stores tokens [ow C / NW, (ow + 1) C / NW)
    // of a chunk's tile, one 16-byte
    // granule per lane and step: step st, lane l takes granule og = g / kTpw
    // of row g % kTpw of the wave's rows (g = 64 st + l; with the plain tile
    // granule g % kGpr of row g / kGpr), i.e. strip og / kGps of the group,
    // 16 bytes of it.
    constexpr int kEpg = 16 / (int)sizeof(T);      // elements per granule
    constexpr int kGps = 16 / kEpg;                // granules per strip row
    constexpr int kGpr = NS * kGps;                // granules per token row
    constexpr int kTpw = C / NW;                   // tokens stored per output wave
    // wave roles: compute waves [0, NW), with GATE store waves [NW, 2 NW),
    // then the two copy waves (so that, with waves dealt to the four SIMDs in
    // order, the store waves' arithmetic does not share a SIMD with a compute
    // wave at NW = 2)
    constexpr int kCopy0 = GATE ? 2 * NW : NW;
    const int ow = GATE ? w - NW : w;              // this wave's index among the output waves
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
        const unsigned char* tile = s_otile + (size_t)((unsigned)(m - a.c0) % (unsigned)kOT) * Ring::kOTile;
#pragma unroll
        for (int st = 0; st < kOSteps; ++st) {
            const int gi = st * 64 + lane;
            // (bank-spread tile: a granule column of the wave's rows per 16
            // lanes; plain tile: whole rows one after the other)
            const int tok = ow * kTpw + (Ring::kSpread ? gi % kTpw : gi / kGpr);
            const int og = Ring::kSpread ? gi / kTpw : gi % kGpr;
            const int sl = og / kGps;
            const int part = og % kGps;
            unsigned char* base = nullptr;
            uint32_t stride = 0;
#pragma unroll
            for (int t = 0; t < NS; ++t)
                if (sl == t) { base = gbase[t]; stride = gstride[t]; }
            if (gi < kTpw * kGpr && base && m * C + tok < a.T) {
                uint4 v = *reinterpret_cast<const uint4*>(tile + (Ring::ooff(tok, (uint32_t)og * 16) & ~15u));
                if (Ring::kOHalf && ((tok >> 3) & 1)) v = make_uint4(v.z, v.w, v.x, v.y);  // halves swapped in LDS
                *reinterpret_cast<uint4*>(base + (size_t)m * C * stride + (uint32_t)tok * stride + (uint32_t)(part * 16)) = v;
            }
        }
    };

    // Fused output side (GATE).  Exchange area of chunk m: the partial sums of
    // squares of its C tokens, token-major with room for kGateGroups groups
    // (one workgroup per 16 NS value columns of the head: at most Dv / 16 = 8).
    constexpr int kGMax = kGateGroups;
    // per-lane partials of the compute waves: [2 (chunk parity)][C tokens][NW waves x 4 lane groups]
    float* s_ss = reinterpret_cast<float*>(s_otile + (size_t)kOT * Ring::kOTile);
    auto gss_at = [&](int m, int grp_, int tok) -> float* {
        return a.gss + (((size_t)bh * a.wsNC + (size_t)(m - a.c0)) * C + tok) * kGMax + grp_;
    };
    bool gate_expired = false;  // a wait of this lane ran out (its rows are then NaN)
    // where granule st of this lane goes: token row, strip of the group, part of it
    auto granule = [&](int st, int& tok, int& sl, int& part) -> bool {
        const int gi = st * 64 + lane;
        tok = ow * kTpw + (Ring::kSpread ? gi % kTpw : gi / kGpr);
        const int og = Ring::kSpread ? gi / kTpw : gi % kGpr;
        sl = og / kGps;
        part = og % kGps;
        return gi < kTpw * kGpr && grp * NS + sl < a.n_strips;
    };
    float wv[GATE ? kOSteps : 1][GATE ? kEpg : 1];  // output weights of this lane's granules
    if constexpr (GATE) {
#pragma unroll
        for (int st = 0; st < kOSteps; ++st) {
            int tok, sl, part;
            const bool ok = granule(st, tok, sl, part);
            const int col = ok ? (grp * NS + sl) * 16 + part * kEpg : 0;
#pragma unroll
            for (int e = 0; e < kEpg; ++e) wv[st][e] = a.gw ? a.gw[col + e] : 1.f;
        }
        wait_vmcnt<0>();  // landed before the store waves' loop (see the convolution's taps)
    }
    // put this workgroup's partials of chunk m (the tile's rows, summed over
    // the compute waves' lanes in a fixed order) in the exchange area
    auto publish = [&](int m) {
        if (ow == 0 && lane < C) {
            const float4* ss = reinterpret_cast<const float4*>(s_ss + ((size_t)((m - a.c0) & 1) * C + lane) * NW * 4);
            float p = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float4 x = ss[ww];
                p += (x.x + x.y) + (x.z + x.w);
            }
            __hip_atomic_store(gss_at(m, grp, lane), p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    // partial p of group g for token tok of chunk m as copied; read again from
    // the exchange area while it is unpublished (-1; a NaN partial passes)
    auto settle = [&](float p, int m, int g, int tok) -> float {
        for (int it = 0; p < 0.f; ++it) {
            if (gate_expired || it >= kGateSpinLimit) {
                gate_expired = true;
                return __builtin_nanf("");
            }
            __builtin_amdgcn_s_sleep(2);
            p = __hip_atomic_load(gss_at(m, g, tok), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return p;
    };
    // chunk m's rows of this wave: o from its tile, normalised and gated
    auto emit_gated = [&](int m, int st, int tok, int sl, int part, const uint4& gt, float tot) {
        const unsigned char* tile = s_otile + (size_t)((unsigned)(m - a.c0) % (unsigned)kOT) * Ring::kOTile;
        unsigned char* base = nullptr;
        uint32_t stride = 0;
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (sl == t) { base = gbase[t]; stride = gstride[t]; }
        const int og = sl * kGps + part;
        uint4 v = *reinterpret_cast<const uint4*>(tile + (Ring::ooff(tok, (uint32_t)og * 16) & ~15u));
        if (Ring::kOHalf && ((tok >> 3) & 1)) v = make_uint4(v.z, v.w, v.x, v.y);  // halves swapped in LDS
        const float inv = __builtin_amdgcn_rsqf(tot * (1.f / (float)a.Dv) + kGateRmsEps);
        float y[kEpg];
#pragma unroll
        for (int e = 0; e < kEpg; ++e)
            y[e] = sigmoidf_(Gran16<T>::get(gt, e)) * Gran16<T>::get(v, e) * inv * wv[st][e];
        *reinterpret_cast<uint4*>(base + (size_t)m * C * stride + (uint32_t)tok * stride + (uint32_t)(part * 16)) =
            Gran16<T>::pack(y);
    };
    // chunk m = n - D during chunk n: gate and partials from the slot of chunk n.
    // All LDS reads go out together; the partials are summed without a branch
    // and read again from the exchange area only if one of them was copied
    // before its group published it.
    auto store_gated_lds = [&](int m, const unsigned char* slot) {
        const unsigned char* gtile = slot + L.bytes + Ring::kVBytes;
        const float* part_s = reinterpret_cast<const float*>(slot + L.bytes + 2 * Ring::kVBytes);
#pragma unroll
        for (int st = 0; st < kOSteps; ++st) {
            int tok, sl, part;
            if (granule(st, tok, sl, part) && m * C + tok < a.T) {
                const int og = sl * kGps + part;
                const uint4 gt = *reinterpret_cast<const uint4*>(gtile + Ring::voff(tok, (uint32_t)og * 16));
                const float4 p0 = *reinterpret_cast<const float4*>(part_s + tok * kGMax);
                const float4 p1 = *reinterpret_cast<const float4*>(part_s + tok * kGMax + 4);
                const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                float tot = 0.f, lo = 0.f;
#pragma unroll
                for (int g = 0; g < kGMax; ++g) {
                    const float x = g < a.n_groups ? pv[g] : 0.f;
                    tot += x;
                    lo = fminf(lo, x);
                }
                if (lo < 0.f) {  // copied before publication: wait for the late ones
                    tot = 0.f;
#pragma unroll
                    for (int g = 0; g < kGMax; ++g)
                        if (g < a.n_groups) tot += settle(pv[g], m, g, tok);
                }
                emit_gated(m, st, tok, sl, part, gt, tot);
            }
        }
    };
    // the last D chunks after the loop: their gates and partials are read
    // straight from memory, all requests in flight together
    constexpr int kDB = D;
    auto drain_gated = [&](int m0, int m1) {
        uint4 gpre[GATE ? kDB : 1][GATE ? kOSteps : 1];
        float ppre[GATE ? kDB : 1][GATE ? kOSteps : 1][GATE ? kGMax : 1];
#pragma unroll
        for (int i = 0; i < kDB; ++i) {
            const int m = m0 + i;
#pragma unroll
            for (int st = 0; st < kOSteps; ++st) {
                int tok, sl, part;
                if (m < m1 && granule(st, tok, sl, part) && m * C + tok < a.T) {
                    unsigned char* base = nullptr;
                    uint32_t stride = 0;
#pragma unroll
                    for (int t = 0; t < NS; ++t)
                        if (sl == t) { base = gbase[t]; stride = gstride[t]; }
                    const size_t off = (size_t)(base - reinterpret_cast<unsigned char*>(a.o)) + (size_t)m * C * stride +
                                       (uint32_t)tok * stride + (uint32_t)(part * 16);
                    gpre[i][st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(a.gate) + off);
#pragma unroll
                    for (int g = 0; g < kGMax; ++g)
                        if (g < a.n_groups)
                            ppre[i][st][g] =
                                __hip_atomic_load(gss_at(m, g, tok), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kDB; ++i) {
            const int m = m0 + i;
#pragma unroll
            for (int st = 0; st < kOSteps; ++st) {
                int tok, sl, part;
                if (m < m1 && granule(st, tok, sl, part) && m * C + tok < a.T) {
                    float tot = 0.f;
#pragma unroll
                    for (int g = 0; g < kGMax; ++g)
                        if (g < a.n_groups) tot += settle(ppre[i][st][g], m, g, tok);
                    emit_gated(m, st, tok, sl, part, gpre[i][st], tot);
                }
            }
        }
    };

    if (w >= kCopy0) {
        // ------------------------------------------------------ copy waves
        const int cw = w - kCopy0;
        const unsigned char* gblk = reinterpret_cast<const unsigned char*>(a.ws) + (size_t)bh * a.wsNC * L.bytes;
        const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(a.v);
        constexpr int kTokPerPiece = Ring::kVTok;
        // lane L writes granule position L of a piece: row Ring::dma_row(L)
        // of the piece, granule Ring::dma_granule(L) of the row
        const int vcol = vcol0 + Ring::dma_granule(lane) * (16 / (int)sizeof(T));
        const uint32_t vcol_b = (uint32_t)((vcol < 16 * vs1 ? vcol : 0) * (int)sizeof(T));  // columns outside the range load any valid bytes
        // values: a wave-uniform 64-bit base per chunk plus a 32-bit lane offset
        const uint32_t tstride = (uint32_t)(a.H * a.Dv * (int)sizeof(T));  // bytes per token
        const unsigned char* vrow0 = vsrc + (((size_t)b * a.T * a.H + h) * a.Dv) * sizeof(T);
        const uint32_t vlane_tok = (uint32_t)Ring::dma_row(lane);
        // gate rows of (b, h) (GATE), addressed like the values
        const unsigned char* grow0 = GATE ? reinterpret_cast<const unsigned char*>(a.gate) + (vrow0 - vsrc) : nullptr;
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
                } else if (p < Ring::kBlkPieces + Ring::kVPieces) {
                    const int j = p - Ring::kBlkPieces;
                    uint32_t tok = (uint32_t)(j * kTokPerPiece) + vlane_tok;
                    tok = tok < lim ? tok : lim - 1;
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void*)(vb + (tok * tstride + vcol_b)),
                        (__attribute__((address_space(3))) void*)(slot + L.bytes + j * 1024), 16, 0, kCopyNT);
                } else if constexpr (GATE) {
                    // chunk mg = n - D (chunk c0 before the first D chunks: loaded, unused)
                    const int mg = max(n - D, a.c0);
                    if (p < Ring::kBlkPieces + 2 * Ring::kVPieces) {
                        // its gate tile, staged like the values
                        const int j = p - Ring::kBlkPieces - Ring::kVPieces;
                        const uint32_t glim = (uint32_t)min(a.T - mg * C, C);
                        uint32_t tok = (uint32_t)(j * kTokPerPiece) + vlane_tok;
                        tok = tok < glim ? tok : glim - 1;
                        const unsigned char* gtb = grow0 + (size_t)mg * C * tstride;
                        __builtin_amdgcn_global_load_lds(
                            (const __attribute__((address_space(1))) void*)(gtb + (tok * tstride + vcol_b)),
                            (__attribute__((address_space(3))) void*)(slot + L.bytes + Ring::kVBytes + j * 1024), 16,
                            0, kCopyNT);
                    } else {
                        // every group's partials of it, past the caches (as the
                        // exchange area's coherent loads and stores go)
                        const int j = p - Ring::kBlkPieces - 2 * Ring::kVPieces;
                        const int off = j * 1024 + lane * 16;
                        if (off < kGateGroups * C * 4)
                            __builtin_amdgcn_global_load_lds(
                                (const __attribute__((address_space(1))) void*)(
                                    reinterpret_cast<const unsigned char*>(
                                        a.gss + ((size_t)bh * a.wsNC + (size_t)(mg - a.c0)) * (kGateGroups * C)) +
                                    off),
                                (__attribute__((address_space(3))) void*)(slot + L.bytes + 2 * Ring::kVBytes + j * 1024),
                                16, 0, kCopyCoherent);
                    }
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

    if constexpr (GATE) {
        if (w >= NW && w < kCopy0) {
            // ------------------------------------------------- store waves
            // During chunk n: publish chunk n - 1's partials (completed
            // before the last barrier) and store chunk n - D's rows with the
            // gate tile and partials that came in chunk n's slot; after the
            // loop, the last chunks.  The same barriers as the other waves.
            // (Placed after the copy waves' code: placed before it, the
            // compiler made every LDS read here wait for this wave's own
            // output stores, a full store latency per chunk.)
            lds_barrier();  // the first chunk(s) are in LDS
            for (int n = a.c0; n < cend; ++n) {
                if (n > a.c0) publish(n - 1);
                if (n - D >= a.c0) store_gated_lds(n - D, slot_of(n));
                if (K == 1) lds_barrier();
                lds_barrier();
            }
            if (a.nc > 0) {
                publish(cend - 1);
                drain_gated(max(a.c0, cend - D), cend);
            }
            return;
        }
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
    // offset of row 16 J + 4 gq + i: voff(4 gq, lb) + voff(16 J, 0) + 256 i
    uint32_t vlane_q[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) vlane_q[j] = Ring::voff(4 * gq, vlane[j]);

    // Operands on the serial path (Kd, Tb and the values of a chunk) live in
    // registers from one chunk to the next: with kAhead they are read for
    // chunk n + 1 while chunk n's output is computed.
    Frag<T> Ak[NBK][KSD], At[NBK][KSC];
    uint32_t Vraw[SPW][NBK * 4];
    // fused convolution of v: this lane's column's taps and bias per strip, and
    // the raw values of the three tokens before the chunk being read
    float4 cvw[SPW];
    float cvb[SPW];
    uint32_t vprev[SPW][3];
    if constexpr (CONV) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int col = (live[j] && !mstrip[j]) ? col0[j] + r : 0;
            const size_t ch = (size_t)h * a.Dv + col;
            cvw[j] = reinterpret_cast<const float4*>(a.cw_v)[ch];
            cvb[j] = a.cb_v ? a.cb_v[ch] : 0.f;
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const int tt = a.c0 * C - 3 + p;
                Raw x = 0;
                if (tt >= 0)
                    x = *reinterpret_cast<const Raw*>(reinterpret_cast<const T*>(a.v) +
                                                      (((size_t)b * a.T + tt) * a.H + h) * a.Dv + col);
                else if (a.cstate)
                    x = *reinterpret_cast<const Raw*>(reinterpret_cast<const T*>(a.cstate) +
                                                      ((size_t)b * 3 + 3 + tt) * a.cstride + a.v_off + ch);
                vprev[j][p] = (uint32_t)x;
            }
        }
        // these loads land before the loop too (a first use inside it would
        // put a wait on every chunk, behind that chunk's output stores)
        wait_vmcnt<0>();
    }
    // fused convolution: staging offsets of the rows 4 gq + p - 3 (p < 7)
    // relative to their 16-row block, and whether a row lies in the block before
    uint32_t crow[CONV ? 7 : 1];
    bool cprev[CONV ? 7 : 1];
    if constexpr (CONV) {
#pragma unroll
        for (int p = 0; p < 7; ++p) {
            const int x = 4 * gq + p - 3;
            cprev[p] = x < 0;
            crow[p] = Ring::voff(x < 0 ? 16 + x : x, 0);
        }
    }
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
                if (2 * s <= Ib) {
                    if (tri_half(Ib, s)) frag_load_half(At[Ib][s], s_blk + L.tb + tri_offset(Ib, s, KSC), lane);
                    else frag_load(At[Ib][s], s_blk + L.tb + tri_offset(Ib, s, KSC), lane);
                }
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            if constexpr (CONV) {
                // SiLU(ShortConv_4(v)) of tokens 16 J + 4 gq + i: the window
                // reaches three tokens back, into the previous chunk (vprev)
                // for the first rows; rounded to the input type as if stored
#pragma unroll
                for (int J = 0; J < NBK; ++J) {
                    float x[7];
#pragma unroll
                    for (int p = 0; p < 7; ++p) {
                        // row 16 J + 4 gq + p - 3: in block J, or (cprev[p]) at
                        // the end of block J - 1, or before the chunk (J = 0)
                        const uint32_t base = cprev[p] ? (J > 0 ? Ring::voff(16 * (J - 1), 0) : 0u) : Ring::voff(16 * J, 0);
                        const uint32_t raw = (uint32_t)*reinterpret_cast<const Raw*>(s_val + base + crow[p] + vlane[j]);
                        const uint32_t pv = vprev[j][p < 3 ? p : 2];
                        x[p] = RawBits<T>::to_float((Raw)((J == 0 && cprev[p]) ? pv : raw));
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const T yv = (T)silu_(conv4(cvw[j], cvb[j], x[i], x[i + 1], x[i + 2], x[i + 3]));
                        Vraw[j][4 * J + i] = (uint32_t)__builtin_bit_cast(Raw, yv);
                    }
                }
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    vprev[j][p] = (uint32_t)*reinterpret_cast<const Raw*>(s_val + Ring::voff(C - 3 + p, 0) + vlane[j]);
            } else {
#pragma unroll
                for (int J = 0; J < NBK; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Vraw[j][4 * J + i] =
                            (uint32_t)*reinterpret_cast<const Raw*>(s_val + Ring::voff(16 * J, 0) + 256 * i + vlane_q[j]);
            }
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
                for (int s = 0; s < KSC; ++s) {
                    if (kpt_half(s, NBK)) frag_load_half(Ap[R][s], s_blk + L.kpt + kpt_offset(R, s, KSC, NBK), lane);
                    else frag_load(Ap[R][s], s_blk + L.kpt + kpt_offset(R, s, KSC, NBK), lane);
                }
#pragma unroll
            for (int R = 0; R < NBD; ++R) g4[R] = *reinterpret_cast<const float4*>(s_gam + 16 * R + 4 * gq);
#pragma unroll
            for (int Ib = 0; Ib < NBK; ++Ib) {
#pragma unroll
                for (int s = 0; s < KSD; ++s) frag_load(Aq[Ib][s], s_blk + L.qp + (size_t)(Ib * KSD + s) * 512, lane);
#pragma unroll
                for (int s = 0; s < KSC; ++s)
                    if (2 * s <= Ib) {
                        if (tri_half(Ib, s)) frag_load_half(Aa[Ib][s], s_blk + L.aqk + tri_offset(Ib, s, KSC), lane);
                        else frag_load(Aa[Ib][s], s_blk + L.aqk + tri_offset(Ib, s, KSC), lane);
                    }
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
            float ssw[GATE ? NBK : 1];  // this lane's share of the tokens' sums of squares
#pragma unroll
            for (int Ib = 0; Ib < (GATE ? NBK : 1); ++Ib) ssw[Ib] = 0.f;
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
                unsigned char* tile = s_otile + (size_t)((unsigned)(n - a.c0) % (unsigned)kOT) * Ring::kOTile;
                const uint32_t opos = Ring::ooff(r, (uint32_t)(((w * SPW + j) * 16 + 4 * gq) * (int)sizeof(T)));
#pragma unroll
                for (int Ib = 0; Ib < NBK; ++Ib)
                    store4(reinterpret_cast<T*>(tile + Ring::ooff(16 * Ib, 0) + opos), acc[Ib]);
                if constexpr (GATE) {
#pragma unroll
                    for (int Ib = 0; Ib < NBK; ++Ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = to_f<T>(from_f<T>(acc[Ib][i]));  // as stored
                            ssw[Ib] = fmaf(x, x, ssw[Ib]);
                        }
                }
            }
            if constexpr (GATE) {
                // lane (r, gq) holds columns 4 gq .. 4 gq + 3 of token 16 Ib + r
                float* ss = s_ss + (size_t)((n - a.c0) & 1) * C * NW * 4 + w * 4 + gq;
#pragma unroll
                for (int Ib = 0; Ib < NBK; ++Ib) ss[(16 * Ib + r) * NW * 4] = ssw[Ib];
            }
        } else if constexpr (GATE) {
            float* ss = s_ss + (size_t)((n - a.c0) & 1) * C * NW * 4 + w * 4 + gq;
#pragma unroll
            for (int Ib = 0; Ib < NBK; ++Ib) ss[(16 * Ib + r) * NW * 4] = 0.f;
        }
        if constexpr (!GATE) {
            // the previous chunk's tile was completed before the last barrier
            if (n > a.c0) store_rows(n - 1);
        }
        if (K == 1) lds_barrier();  // done reading the single slot
        lds_barrier();              // the next chunk(s) are in LDS
    }
    if (!GATE && a.nc > 0) store_rows(cend - 1);  // (GATE: the store waves store)

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

// One instantiation of the inter kernel: NW compute waves of one strip each
// (CONV: with the fused convolution of v; GATE: with the fused output side).
template <typename T, int DK, int C, int NW, bool CONV = false, bool GATE = false>
struct InterKernel {
    using Ring = InterRing<T, DK, C, NW, !CONV, GATE>;
    static constexpr int kThreads = 64 * (NW + 2 + (GATE ? NW : 0));  // GATE: NW store waves
    static constexpr size_t kLds = (size_t)Ring::kSlots * Ring::kSlot + Ring::kOBytes;
    static const void* fn() { return reinterpret_cast<const void*>(kda_inter_kernel<T, DK, C, NW, 1, CONV, GATE>); }
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
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, C, NW, 1, CONV, GATE>), dim3((unsigned)BH * ea.n_groups), dim3(kThreads),
                           kLds, s, ea);
        return hipGetLastError();
    }
};

// Launch configuration of the chunk kernels for one (T, DK, C).
//
// Compute waves per inter workgroup: the workgroups of one (b, h) all stream
// the same chunk blocks, and each compute wave reads every block fragment from
// LDS, so fewer waves per workgroup cost fewer LDS reads per strip but more
// workgroups.  The launch takes the fewest waves (1, 2, 4, or for 2-byte
// elements without the fused output side 8) whose grid is resident on the
// device in one round; when none is, the most (or fewer when the strips of a
// (b, h) fit in fewer): every workgroup streams the whole block of each
// chunk, so fewer workgroups copy less.  GATE (the fused output side) needs the
// workgroups of a (b, h) resident together: `resident` says whether a grid
// of the exact instantiation fits in one round, and the caller takes another
// path when it does not.
template <typename T, int DK, int C, bool GATE = false>
struct ChunkLaunch {
    static constexpr BlockLayout L = block_layout(sizeof(T), DK, C);
    static constexpr int NCH = 64 / C;  // chunks per intra workgroup

    const ChunkArgs& a;
    int BH;
    int nw = 4;
    bool resident = false;
    InterArgs ea{};
    // eight compute waves: 2-byte elements only (four-byte value rows of
    // eight strips do not tile the ring's bank-spread pieces) and not with the
    // fused output side (its store waves would pass 1024 threads)
    static constexpr bool kNW8 = sizeof(T) == 2 && !GATE;

    template <int NW>
    static int capacity(int dev, bool conv) {
        if constexpr (NW == 8 && !kNW8) return 0;
        // the plain path sizes every launch by the instantiation without the
        // convolution (same LDS, one workgroup per CU at the sizes that fill
        // the device); the gated path asks the exact one
        else if (GATE && conv) return InterKernel<T, DK, C, NW, true, GATE>::capacity(dev);
        else return InterKernel<T, DK, C, NW, false, GATE>::capacity(dev);
    }
    template <int NW>
    static constexpr bool fits() {
        if constexpr (NW == 8 && !kNW8) return false;
        else return InterKernel<T, DK, C, NW, false, GATE>::Ring::kFits;
    }

    explicit ChunkLaunch(const ChunkArgs& args) : a(args), BH(args.B * args.H) {
        ea.v = a.v; ea.o = a.o; ea.P_out = a.P_out;
        ea.T = a.T; ea.H = a.H; ea.Dv = a.Dv;
        ea.n_m = (a.M_out || a.P_out) ? DK / 16 : 0;
        ea.n_strips = ea.n_m + a.Dv / 16;
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) dev = -1;
        const bool conv = a.conv_w != nullptr;
        const int caps[4] = {capacity<1>(dev, conv), capacity<2>(dev, conv), capacity<4>(dev, conv),
                             capacity<8>(dev, conv)};
        const bool fits[4] = {ChunkLaunch::fits<1>(), ChunkLaunch::fits<2>(), ChunkLaunch::fits<4>(),
                              ChunkLaunch::fits<8>()};
        nw = 0;
        for (int i = 0, w = 1; i < 4 && !nw; ++i, w *= 2)
            if (fits[i] && (long long)BH * ((ea.n_strips + w - 1) / w) <= caps[i]) nw = w;
        resident = nw != 0;
        if (!nw) {  // no grid resident in one round: the fewest workgroups (fewest waves on a tie)
            int best_g = 1 << 30;
            for (int i = 0, w = 1; i < 4; ++i, w *= 2) {
                const int g = (ea.n_strips + w - 1) / w;
                if (fits[i] && g < best_g) { best_g = g; nw = w; }
            }
        }
        if (!nw) nw = 4;  // no instantiation fits (GATE only: the caller takes the separate path)
        ea.n_groups = (ea.n_strips + nw - 1) / nw;
        if (a.conv_w) {
            const int Hk = a.H / a.G;
            ea.cw_v = a.conv_w + (size_t)2 * Hk * DK * 4;
            ea.cb_v = a.conv_b ? a.conv_b + (size_t)2 * Hk * DK : nullptr;
            ea.cstate = a.conv_state;
            ea.cstride = 2 * Hk * DK + a.H * a.Dv;
            ea.v_off = 2 * Hk * DK;
        }
        ea.gate = a.gate; ea.gw = a.gate_w; ea.gss = a.gss;
    }
    // floats of the output side's exchange area per chunk-head
    int gss_per_chunk() const { return kGateGroups * C; }

    template <bool CONV>
    hipError_t set_attributes_c() const {
        switch (nw) {
            case 1: return InterKernel<T, DK, C, 1, CONV, GATE>::set_attributes();
            case 2: return InterKernel<T, DK, C, 2, CONV, GATE>::set_attributes();
            case 8:
                if constexpr (kNW8) return InterKernel<T, DK, C, 8, CONV, GATE>::set_attributes();
                else return hipErrorInvalidValue;
            default: return InterKernel<T, DK, C, 4, CONV, GATE>::set_attributes();
        }
    }
    hipError_t set_attributes() const { return a.conv_w ? set_attributes_c<true>() : set_attributes_c<false>(); }
    // intra kernel over chunks [c0, c0 + nc) into the buffer `buf` of `per` chunks per (b, h)
    hipError_t intra(void* buf, int per, int c0, int nc, hipStream_t s) const {
        IntraArgs ia{a.q, a.k, a.z, a.beta_raw, a.A_log, buf, a.T, a.H, a.G, a.dt_bias, per, c0, nc, a.g_min, a.flags};
        ia.gss = a.gss;
        ia.gss_n = a.gss_n;
        const dim3 grid((unsigned)(BH * ((nc + NCH - 1) / NCH)));
        if (a.conv_w) {
            const int Hk = a.H / a.G;
            ia.cw_q = a.conv_w;
            ia.cw_k = a.conv_w + (size_t)Hk * DK * 4;
            ia.cb_q = a.conv_b;
            ia.cb_k = a.conv_b ? a.conv_b + (size_t)Hk * DK : nullptr;
            ia.cstate = a.conv_state;
            ia.cstride = 2 * Hk * DK + a.H * a.Dv;
            ia.qk_off = Hk * DK;
            if (a.wide_decay)
                hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, true, true>), grid, dim3(256), 0, s, ia);
            else
                hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, false, true>), grid, dim3(256), 0, s, ia);
        } else if (a.wide_decay) {
            hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, true>), grid, dim3(256), 0, s, ia);
        } else {
            hipLaunchKernelGGL((kda_intra_kernel<T, DK, C, false>), grid, dim3(256), 0, s, ia);
        }
        return hipGetLastError();
    }
    // inter kernel over the same chunks; the state enters from S0/M0 (first
    // slice) or the carry region, and leaves to S_out/M_out (last slice) or it
    template <bool CONV>
    hipError_t inter_c(hipStream_t s) const {
        switch (nw) {
            case 1: return InterKernel<T, DK, C, 1, CONV, GATE>::launch(ea, BH, s);
            case 2: return InterKernel<T, DK, C, 2, CONV, GATE>::launch(ea, BH, s);
            case 8:
                if constexpr (kNW8) return InterKernel<T, DK, C, 8, CONV, GATE>::launch(ea, BH, s);
                else return hipErrorInvalidValue;
            default: return InterKernel<T, DK, C, 4, CONV, GATE>::launch(ea, BH, s);
        }
    }
    hipError_t inter(void* buf, int per, int c0, int nc, bool first, bool last, float* S_scr, float* M_scr,
                     hipStream_t s) {
        ea.ws = buf; ea.wsNC = per; ea.c0 = c0; ea.nc = nc;
        ea.S0 = first ? a.S0 : S_scr;
        ea.M0 = first ? nullptr : M_scr;
        ea.S_out = last ? a.S_out : S_scr;
        ea.M_out = last ? a.M_out : M_scr;
        return a.conv_w ? inter_c<true>(s) : inter_c<false>(s);
    }
};

}  // namespace kda
