// kda_compose.hip - segment composition (KCP) and output correction on gfx950.
//
// kda_compose: the prefix scan of "KDA 模块交互式演示" §1.6 and "Implémenter KDA"
// Test 3, S_s = M_s S_{s-1} + S_tilde_s, in fp32 on the matrix cores.  One
// workgroup per (b, h, 16-column strip) whose waves split the state's rows and
// pass the strip to each other through LDS between segments.
//
// kda_fixup: o_t += P_t S_in for segments that were run from a zero state.
// Valid because the recurrence is affine in the incoming state ("Implémenter
// KDA", 'Que teste réellement le test 2').
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Row of the strip state in LDS: 16 floats, plus 16 more every 4 rows so that
// the four lane groups of a wave (rows 4 apart) fall in different banks.
__device__ __forceinline__ int strip_at(int row, int c) { return row * 16 + (row >> 2) * 16 + c; }

// One workgroup per (b, h, 16-column strip), one wave per 16-row block R of
// the state.  Wave R forms rows 16 R .. 16 R + 15 of S_s = M_s S_{s-1} +
// S_tilde_s from its 16 rows of M_s (read one segment ahead) and the whole
// strip of S_{s-1}, which the waves exchange through LDS: the new strip goes
// to buffer s & 1, one barrier, and every wave reads it back as the B operand
// of the next product.  (Two buffers: a wave writes buffer s & 1 only after
// the barrier of segment s - 1, which every wave passes after its reads of
// buffer (s - 2) & 1.)  Contraction slot j of step s is state row 32 s + 4 gq
// + j (j < 4) or 32 s + 16 + 4 gq + j - 4, in both operands.
template <int DK>
__global__ __launch_bounds__(512) void kda_compose_kernel(const ComposeArgs a) {
    constexpr int KSD = (DK + 31) / 32;
    constexpr int kRowsLds = DK + DK / 4;
    __shared__ float s_S[2][kRowsLds * 16];
    const int lane = threadIdx.x & 63;
    const int R = threadIdx.x >> 6;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int nstrip = a.Dv / 16;
    // the strips of one (b, h) on one XCD: they read the same M rows, which
    // that XCD's L2 then serves after the first
    const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int strip = bid % nstrip;
    const int bh = bid / nstrip;
    const int BH = a.B * a.H;
    const int col = strip * 16 + r;

    Frag<float> Sf[KSD];
#pragma unroll
    for (int s = 0; s < KSD; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r0 = 32 * s + 4 * gq + j, r1 = r0 + 16;
            Sf[s].v[j] = (a.S_in && r0 < DK) ? a.S_in[((size_t)bh * DK + r0) * a.Dv + col] : 0.f;
            Sf[s].v[4 + j] = (a.S_in && r1 < DK) ? a.S_in[((size_t)bh * DK + r1) * a.Dv + col] : 0.f;
        }

    auto load_segment = [&](int sg, Frag<float> (&A)[KSD], floatx4& acc) {
        const float* mrow = a.M + (((size_t)sg * BH + bh) * DK + 16 * R + r) * DK;
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            load4(mrow + 32 * s + 4 * gq, &A[s].v[0]);
            if (32 * s + 16 < DK) load4(mrow + 32 * s + 16 + 4 * gq, &A[s].v[4]);
            else A[s].v[4] = A[s].v[5] = A[s].v[6] = A[s].v[7] = 0.f;
        }
        const float* St = a.S_tilde + ((size_t)sg * BH + bh) * DK * a.Dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = St[(size_t)(16 * R + 4 * gq + i) * a.Dv + col];
    };

    Frag<float> A[KSD];
    floatx4 acc;
    load_segment(0, A, acc);
    for (int sg = 0; sg < a.n_seg; ++sg) {
        Frag<float> nA[KSD];
        floatx4 nacc;
        const bool more = sg + 1 < a.n_seg;  // uniform over the workgroup
        if (more) load_segment(sg + 1, nA, nacc);
#pragma unroll
        for (int s = 0; s < KSD; ++s) acc = mma(A[s], Sf[s], acc);
        float* Sout = a.S_prefix + ((size_t)sg * BH + bh) * DK * a.Dv;
        float* buf = s_S[sg & 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * R + 4 * gq + i;
            Sout[(size_t)row * a.Dv + col] = acc[i];
            buf[strip_at(row, r)] = acc[i];
        }
        __syncthreads();
        if (more) {
#pragma unroll
            for (int s = 0; s < KSD; ++s)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r0 = 32 * s + 4 * gq + j, r1 = r0 + 16;
                    Sf[s].v[j] = r0 < DK ? buf[strip_at(r0, r)] : 0.f;
                    Sf[s].v[4 + j] = r1 < DK ? buf[strip_at(r1, r)] : 0.f;
                }
#pragma unroll
            for (int s = 0; s < KSD; ++s) A[s] = nA[s];
            acc = nacc;
        }
    }
}

constexpr int kFixTokens = 512;  // tokens per workgroup in kda_fixup
constexpr int kFixBlocks = 2;    // 16-token blocks whose reads a fix-up wave has in flight together

// 4 * NST consecutive elements of one o row: the part of a row one fix-up lane
// owns, kept packed until it is used.
template <typename T, int NST> struct ORun {
    static constexpr int W = NST * (int)sizeof(T);  // 32-bit words
    uint32_t w[W];
    __device__ __forceinline__ void load(const T* p) {
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const uint4 u = reinterpret_cast<const uint4*>(p)[i];
                w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
            }
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            w[0] = u.x; w[1] = u.y;
        }
    }
    __device__ __forceinline__ floatx4 get(int q) const {
        if constexpr (sizeof(T) == 2)
            return floatx4{__uint_as_float(w[2 * q] << 16), __uint_as_float(w[2 * q] & 0xffff0000u),
                           __uint_as_float(w[2 * q + 1] << 16), __uint_as_float(w[2 * q + 1] & 0xffff0000u)};
        else
            return floatx4{__uint_as_float(w[4 * q]), __uint_as_float(w[4 * q + 1]),
                           __uint_as_float(w[4 * q + 2]), __uint_as_float(w[4 * q + 3])};
    }
    __device__ __forceinline__ void put(int q, const floatx4& x) {
        if constexpr (sizeof(T) == 2) {
            typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
            const bf16x2v lo = {(bf16_t)x[0], (bf16_t)x[1]}, hi = {(bf16_t)x[2], (bf16_t)x[3]};
            w[2 * q] = __builtin_bit_cast(uint32_t, lo);
            w[2 * q + 1] = __builtin_bit_cast(uint32_t, hi);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[4 * q + i] = __float_as_uint(x[i]);
        }
    }
    __device__ __forceinline__ void store(T* p) const {
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int i = 0; i < W / 4; ++i)
                reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
        } else {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        }
    }
};

// One workgroup per (segment, b, h, 512-token tile): four waves, NG groups
// of NST value strips of 16 columns times 4 / NG token sub-tiles.  The
// workgroup first copies S_prev of its (segment, b, h) into LDS transposed
// (one row of DK channels per value column, coalesced 16-byte reads of the
// fp32 state), then every wave takes S_prev^T of its group as matrix-core A
// operands and, per 16-token block, forms O^T = S^T P^T.  Both operands take
// channel 32 s + 8 gq + j in contraction slot (gq, j) of step s, so each lane
// reads 16 contiguous bytes of a P row (and of an LDS column).  Row m of
// strip q's A operand is value column 4 NST (m / 4) + 4 q + m % 4 of the
// group, which leaves lane (r, gq) of the output with the 4 NST consecutive
// columns from 4 NST gq on of token r: one contiguous read-modify-write per
// lane and token.
template <typename T, int DK, int NST, int NG>
__global__ __launch_bounds__(256) void kda_fixup_kernel(const FixupArgs a) {
    constexpr int KSD = (DK + 31) / 32;
    constexpr int NB = kFixBlocks;
    constexpr int SUB = 4 / NG;           // token sub-tiles per workgroup
    constexpr int DV = 16 * NST * NG;     // value columns
    constexpr int LD = DK + 8;            // elements per LDS column (16-byte aligned rows)
    extern __shared__ __align__(16) unsigned char fix_raw[];
    T* s_St = reinterpret_cast<T*>(fix_raw);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r = lane & 15;
    const int gq = lane >> 4;
    const int ntile = (a.T_seg + kFixTokens - 1) / kFixTokens;
    // head index fastest: the workgroups that run together read and write
    // whole token rows of P and o (all heads of the same tokens)
    long long x = blockIdx.x;
    const int h = (int)(x % a.H); x /= a.H;
    const int tt = (int)(x % ntile); x /= ntile;
    const int b = (int)(x % a.B); x /= a.B;
    const int sg = (int)x;
    const float* Sprev = sg ? a.S_prefix + (((size_t)(sg - 1) * a.B + b) * a.H + h) * DK * DV
                            : (a.S_in ? a.S_in + ((size_t)b * a.H + h) * DK * DV : nullptr);
    if (!Sprev) return;  // uniform over the workgroup, before its only barrier

    // S_prev^T into LDS: element (row, col) of the state at
    // s_St[col LD + (row ^ swz(col))].  The swizzle permutes the 8-row
    // granules of a column (so a granule stays 16 contiguous bytes), with a
    // different permutation for each group of four columns: the columns four
    // apart that one staging write touches, and the lanes of a fragment read
    // four columns apart, then fall on different banks.
    const auto swz = [](int col) { return 8 * ((col >> 2) % (DK / 8)); };
    for (int i = threadIdx.x; i < DK * DV / 4; i += 256) {
        const int row = i / (DV / 4), c4 = 4 * (i % (DV / 4));
        const float4 v = reinterpret_cast<const float4*>(Sprev + (size_t)row * DV)[c4 / 4];
        const int rs = row ^ swz(c4);  // the same for the four columns c4 .. c4 + 3
        s_St[(c4 + 0) * LD + rs] = (T)v.x;
        s_St[(c4 + 1) * LD + rs] = (T)v.y;
        s_St[(c4 + 2) * LD + rs] = (T)v.z;
        s_St[(c4 + 3) * LD + rs] = (T)v.w;
    }
    __syncthreads();

    const int grp = w % NG;
    const int sub = w / NG;
    const int col0 = grp * 16 * NST;
    Frag<T> Sf[NST][KSD];
#pragma unroll
    for (int q = 0; q < NST; ++q) {
        const int col = col0 + 4 * NST * (r >> 2) + 4 * q + (r & 3);
#pragma unroll
        for (int s = 0; s < KSD; ++s) {
            if (32 * s + 8 * gq < DK) frag_load_row8(Sf[q][s], s_St + col * LD + ((32 * s + 8 * gq) ^ swz(col)));
            else Sf[q][s].zero();
        }
    }

    const T* P = reinterpret_cast<const T*>(a.P);
    T* o = reinterpret_cast<T*>(a.o);
    const size_t seg_row0 = ((size_t)sg * a.B + b) * a.T_seg;
    constexpr int kSubTokens = kFixTokens / SUB;
    const int tbeg = tt * kFixTokens + sub * kSubTokens;
    const int tend = min(a.T_seg, tbeg + kSubTokens);
    for (int tok0 = tbeg; tok0 < tend; tok0 += 16 * NB) {
        // all reads of the NB blocks go out before any product
        Frag<T> Pf[NB][KSD];
        ORun<T, NST> run[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int tok = tok0 + 16 * u + r;
            if (tok < tend) {
                const size_t row = (seg_row0 + tok) * a.H + h;
                const T* prow = P + row * DK;
#pragma unroll
                for (int s = 0; s < KSD; ++s) {
                    if (32 * s + 8 * gq < DK) frag_load_row8(Pf[u][s], prow + 32 * s + 8 * gq);
                    else Pf[u][s].zero();
                }
                run[u].load(o + row * DV + col0 + 4 * NST * gq);
            }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int tok = tok0 + 16 * u + r;
            if (tok0 + 16 * u < tend) {  // wave-uniform: the products need every lane
#pragma unroll
                for (int q = 0; q < NST; ++q) {
                    floatx4 acc = run[u].get(q);
#pragma unroll
                    for (int s = 0; s < KSD; ++s) acc = mma(Sf[q][s], Pf[u][s], acc);
                    run[u].put(q, acc);
                }
                if (tok < tend) run[u].store(o + ((seg_row0 + tok) * a.H + h) * DV + col0 + 4 * NST * gq);
            }
        }
    }
}

hipError_t launch_compose(int DK, const ComposeArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)(a.B * a.H * (a.Dv / 16));
    const dim3 block(64 * (DK / 16));
    switch (DK) {
        case 16: hipLaunchKernelGGL(kda_compose_kernel<16>, dim3(grid), block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(kda_compose_kernel<32>, dim3(grid), block, 0, s, a); break;
        case 64: hipLaunchKernelGGL(kda_compose_kernel<64>, dim3(grid), block, 0, s, a); break;
        case 128: hipLaunchKernelGGL(kda_compose_kernel<128>, dim3(grid), block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int DK, int NST, int NG>
static hipError_t launch_fixup_g(const FixupArgs& a, hipStream_t s) {
    constexpr size_t kLds = (size_t)16 * NST * NG * (DK + 8) * sizeof(T);
    const auto fn = kda_fixup_kernel<T, DK, NST, NG>;
    // set on every call: the attribute is per device, and the call only records a limit
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    const long long ntile = (a.T_seg + kFixTokens - 1) / kFixTokens;
    const unsigned grid = (unsigned)((long long)a.n_seg * a.B * a.H * ntile);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(256), kLds, s, a);
    return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_fixup_v(const FixupArgs& a, hipStream_t s) {
    // strips per group: 4 (64 columns) where the value dimension allows, else all of it
    switch (a.Dv) {
        case 16: return launch_fixup_g<T, DK, 1, 1>(a, s);
        case 32: return launch_fixup_g<T, DK, 2, 1>(a, s);
        case 64: return launch_fixup_g<T, DK, 4, 1>(a, s);
        case 128: return launch_fixup_g<T, DK, 4, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_fixup_t(int DK, const FixupArgs& a, hipStream_t s) {
    switch (DK) {
        case 16: return launch_fixup_v<T, 16>(a, s);
        case 32: return launch_fixup_v<T, 32>(a, s);
        case 64: return launch_fixup_v<T, 64>(a, s);
        case 128: return launch_fixup_v<T, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fixup(int dt, int DK, const FixupArgs& a, hipStream_t s) {
    return dt == 1 ? launch_fixup_t<bf16_t>(DK, a, s) : launch_fixup_t<float>(DK, a, s);
}

}  // namespace kda
