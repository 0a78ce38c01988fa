// kda_compose.hip - segment composition (KCP) and output correction on gfx950.
//
// kda_compose: the prefix scan of "KDA 模块交互式演示" §1.6 and "Implémenter KDA"
// Test 3, S_s = M_s S_{s-1} + S_tilde_s, in fp32 on the matrix cores.  One wave
// per (b, h, 16-column strip); the strip of S stays in accumulators across the
// segments and feeds the next product as its B operand directly.
//
// kda_fixup: o_t += P_t S_in for segments that were run from a zero state.
// Valid because the recurrence is affine in the incoming state ("Implémenter
// KDA", 'Que teste réellement le test 2').
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK>
__global__ __launch_bounds__(256) void kda_compose_kernel(const ComposeArgs a) {
    constexpr int NBD = DK / 16;
    constexpr int KSD = (DK + 31) / 32;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int nstrip = a.Dv / 16;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int BH = a.B * a.H;
    if (wid >= BH * nstrip) return;  // this kernel has no barriers
    const int strip = wid % nstrip;
    const int bh = wid / nstrip;
    const int col = strip * 16 + r;

    floatx4 S[NBD];
#pragma unroll
    for (int R = 0; R < NBD; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[R][i] = a.S_in ? a.S_in[((size_t)bh * DK + 16 * R + 4 * gq + i) * a.Dv + col] : 0.f;

    for (int sg = 0; sg < a.n_seg; ++sg) {
        const float* Ms = a.M + ((size_t)sg * BH + bh) * DK * DK;
        const float* St = a.S_tilde + ((size_t)sg * BH + bh) * DK * a.Dv;
        float* Sout = a.S_prefix + ((size_t)sg * BH + bh) * DK * a.Dv;
        Frag<float> Sf[KSD];
#pragma unroll
        for (int s = 0; s < KSD; ++s)
            Sf[s] = (2 * s + 1 < NBD) ? frag_from_c<float>(S[2 * s], S[2 * s + 1])
                                      : frag_from_c_lo<float>(S[2 * s]);
        floatx4 Sn[NBD];
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            floatx4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = St[(size_t)(16 * R + 4 * gq + i) * a.Dv + col];
            const float* mrow = Ms + (size_t)(16 * R + r) * DK;
#pragma unroll
            for (int s = 0; s < KSD; ++s) {
                Frag<float> A;
                load4(mrow + 32 * s + 4 * gq, &A.v[0]);
                if (32 * s + 16 < DK) load4(mrow + 32 * s + 16 + 4 * gq, &A.v[4]);
                else { A.v[4] = A.v[5] = A.v[6] = A.v[7] = 0.f; }
                acc = mma(A, Sf[s], acc);
            }
            Sn[R] = acc;
        }
#pragma unroll
        for (int R = 0; R < NBD; ++R) {
            S[R] = Sn[R];
#pragma unroll
            for (int i = 0; i < 4; ++i) Sout[(size_t)(16 * R + 4 * gq + i) * a.Dv + col] = Sn[R][i];
        }
    }
}

constexpr int kFixTokens = 256;  // tokens per wave in kda_fixup

template <typename T, int DK>
__global__ __launch_bounds__(256) void kda_fixup_kernel(const FixupArgs a) {
    constexpr int KSD = (DK + 31) / 32;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int nstrip = a.Dv / 16;
    const int ntile = (a.T_seg + kFixTokens - 1) / kFixTokens;
    const long long total = (long long)a.n_seg * a.B * a.H * nstrip * ntile;
    const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= total) return;  // no barriers in this kernel
    long long x = wid;
    const int tt = (int)(x % ntile); x /= ntile;
    const int strip = (int)(x % nstrip); x /= nstrip;
    const int h = (int)(x % a.H); x /= a.H;
    const int b = (int)(x % a.B); x /= a.B;
    const int sg = (int)x;
    const float* Sprev = sg ? a.S_prefix + (((size_t)(sg - 1) * a.B + b) * a.H + h) * DK * a.Dv
                            : (a.S_in ? a.S_in + ((size_t)b * a.H + h) * DK * a.Dv : nullptr);
    if (!Sprev) return;
    const int col = strip * 16 + r;

    Frag<T> Sf[KSD];
#pragma unroll
    for (int s = 0; s < KSD; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int rw = 32 * s + slot_index(gq, j);
            Sf[s].set(j, rw < DK ? Sprev[(size_t)rw * a.Dv + col] : 0.f);
        }

    const T* P = reinterpret_cast<const T*>(a.P);
    T* o = reinterpret_cast<T*>(a.o);
    const size_t seg_row0 = ((size_t)sg * a.B + b) * a.T_seg;
    for (int tb = 0; tb < kFixTokens / 16; ++tb) {
        const int tok0 = tt * kFixTokens + 16 * tb;
        if (tok0 >= a.T_seg) break;
        const int tr = tok0 + r;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            Frag<T> A;
            float tmp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) tmp[j] = 0.f;
            if (tr < a.T_seg) {
                const T* prow = P + ((seg_row0 + tr) * a.H + h) * DK;
                load4(prow + 32 * s + 4 * gq, &tmp[0]);
                if (32 * s + 16 < DK) load4(prow + 32 * s + 16 + 4 * gq, &tmp[4]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) A.set(j, tmp[j]);
            acc = mma(A, Sf[s], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = tok0 + 4 * gq + i;
            if (tok < a.T_seg) {
                T* dst = o + ((seg_row0 + tok) * a.H + h) * a.Dv + col;
                *dst = from_f<T>(to_f<T>(*dst) + acc[i]);
            }
        }
    }
}

hipError_t launch_compose(int DK, const ComposeArgs& a, hipStream_t s) {
    const long long waves = (long long)a.B * a.H * (a.Dv / 16);
    const unsigned grid = (unsigned)((waves + 3) / 4);
    switch (DK) {
        case 16: hipLaunchKernelGGL(kda_compose_kernel<16>, dim3(grid), dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL(kda_compose_kernel<32>, dim3(grid), dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL(kda_compose_kernel<64>, dim3(grid), dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(kda_compose_kernel<128>, dim3(grid), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_fixup_t(int DK, const FixupArgs& a, hipStream_t s) {
    const long long ntile = (a.T_seg + kFixTokens - 1) / kFixTokens;
    const long long waves = (long long)a.n_seg * a.B * a.H * (a.Dv / 16) * ntile;
    const unsigned grid = (unsigned)((waves + 3) / 4);
    switch (DK) {
        case 16: hipLaunchKernelGGL((kda_fixup_kernel<T, 16>), dim3(grid), dim3(256), 0, s, a); break;
        case 32: hipLaunchKernelGGL((kda_fixup_kernel<T, 32>), dim3(grid), dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL((kda_fixup_kernel<T, 64>), dim3(grid), dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL((kda_fixup_kernel<T, 128>), dim3(grid), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fixup(int dt, int DK, const FixupArgs& a, hipStream_t s) {
    return dt == 1 ? launch_fixup_t<bf16_t>(DK, a, s) : launch_fixup_t<float>(DK, a, s);
}

}  // namespace kda
