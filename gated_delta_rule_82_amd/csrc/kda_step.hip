// kda_step.hip - single-token KDA decode on gfx950 ("KDA 模块交互式演示" §1.7
// kda_step; "Implémenter KDA" 'La forme récurrente de référence').
//
// One workgroup per (b, h) and group of DVW value columns (both reductions
// run over Dk, column by column, so column groups are independent).  The
// fp32 state is streamed once from HBM into registers and written back once;
// both reductions are taken from the same pass, because with
// S' = Diag(alpha) S and u = beta (v - S'^T k):
//     S_new = S' + k u^T,     o = S_new^T q = S'^T q + u (k . q).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename T, int DK, int DV, int DVW, int NTH>
__global__ __launch_bounds__(NTH) void kda_step_kernel(const StepArgs a) {
    constexpr int NSPLIT = DV / DVW;                   // workgroups per (b, h)
    constexpr int CG = DVW / 4;                        // float4 column groups
    constexpr int NT = (CG * DK < NTH) ? CG * DK : NTH;
    constexpr int RG = NT / CG;                        // row groups
    constexpr int RPT = DK / RG;                       // rows per thread
    constexpr int MC = (DK + 63) / 64;                 // channels per lane in the prep wave

    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ __align__(16) float s_red[2][RG][DVW];
    __shared__ float s_misc[2];

    const int bh = blockIdx.x / NSPLIT;
    const int col0 = (blockIdx.x % NSPLIT) * DVW;
    const int h = bh % a.H;
    const int tid = threadIdx.x;
    if (tid >= NT) return;  // NT is a multiple of 64; no thread past NT reaches a barrier
    const int cg = tid % CG;
    const int rg = tid / CG;

    float* Sp = a.S + (size_t)bh * DK * DV + col0;
    // the state is touched once per step: non-temporal loads and stores
    // (measured: 212 -> 195 us per B256 H32 D128 step, the loads carry it)
    float4 Sr[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sp + (size_t)(rg + RG * m) * DV) + cg);
        Sr[m] = make_float4(t[0], t[1], t[2], t[3]);
    }
    // this thread's four values, requested with the state so that no global
    // load waits after the reductions (the workgroup lives one memory latency)
    float vv[4];
    load4(reinterpret_cast<const T*>(a.v) + (size_t)bh * DV + col0 + 4 * cg, vv);

    if (tid < 64) {
        // value head h reads q/k head h / G of the same batch row
        const size_t bq = (size_t)(bh / a.H) * (a.H / a.G) + h / a.G;
        const T* q = reinterpret_cast<const T*>(a.q) + bq * DK;
        const T* k = reinterpret_cast<const T*>(a.k) + bq * DK;
        const T* z = reinterpret_cast<const T*>(a.z) + (size_t)bh * DK;
        float qv[MC], kv[MC], zv[MC];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int c = tid + 64 * m;
            const bool ok = c < DK;
            qv[m] = ok ? to_f<T>(q[c]) : 0.f;
            kv[m] = ok ? to_f<T>(k[c]) : 0.f;
            zv[m] = ok ? to_f<T>(z[c]) + ((a.dt_bias && (a.flags & kGateIn)) ? a.dt_bias[(size_t)h * DK + c] : 0.f) : 0.f;
            sq += qv[m] * qv[m];
            sk += kv[m] * kv[m];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            sq += __shfl_xor(sq, off, 64);
            sk += __shfl_xor(sk, off, 64);
        }
        const float rq = (a.flags & kQkL2) ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f;
        const float rk = (a.flags & kQkL2) ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
        const bool gate = (a.flags & kGateIn) != 0;
        const float hscale = gate ? expf(a.A_log[h]) : 0.f;
        float qk = 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int c = tid + 64 * m;
            if (c < DK) {
                const float qh = qv[m] * rq, kh = kv[m] * rk;
                // bounded gate, or the unbounded v1 gate -e^A softplus(z)
                const float x = zv[m];
                const float g = !gate ? x
                              : (a.flags & kGateSoftplus) ? -hscale * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))))
                                                          : a.g_min * sigmoidf_(hscale * x);
                s_q[c] = qh;
                s_k[c] = kh;
                s_a[c] = expf(g);
                qk += qh * kh;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off, 64);
        if (tid == 0) {
            const float braw = to_f<T>(reinterpret_cast<const T*>(a.beta_raw)[bh]);
            s_misc[0] = (a.flags & kBetaSig) ? sigmoidf_(braw) : braw;
            s_misc[1] = qk;
        }
    }
    __syncthreads();

    float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), ps = pr;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int rw = rg + RG * m;
        const float al = s_a[rw], kr = s_k[rw], qr = s_q[rw];
        float4 x = Sr[m];
        x.x *= al; x.y *= al; x.z *= al; x.w *= al;
        Sr[m] = x;
        pr.x += kr * x.x; pr.y += kr * x.y; pr.z += kr * x.z; pr.w += kr * x.w;
        ps.x += qr * x.x; ps.y += qr * x.y; ps.z += qr * x.z; ps.w += qr * x.w;
    }
    reinterpret_cast<float4*>(&s_red[0][rg][0])[cg] = pr;
    reinterpret_cast<float4*>(&s_red[1][rg][0])[cg] = ps;
    __syncthreads();

    float4 rr = make_float4(0.f, 0.f, 0.f, 0.f), ss = rr;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        const float4 x = reinterpret_cast<const float4*>(&s_red[0][j][0])[cg];
        const float4 y = reinterpret_cast<const float4*>(&s_red[1][j][0])[cg];
        rr.x += x.x; rr.y += x.y; rr.z += x.z; rr.w += x.w;
        ss.x += y.x; ss.y += y.y; ss.z += y.z; ss.w += y.w;
    }
    const float beta = s_misc[0], qk = s_misc[1];
    float4 u;
    u.x = beta * (vv[0] - rr.x);
    u.y = beta * (vv[1] - rr.y);
    u.z = beta * (vv[2] - rr.z);
    u.w = beta * (vv[3] - rr.w);
    if (rg == 0) {
        T* op = reinterpret_cast<T*>(a.o) + (size_t)bh * DV + col0 + 4 * cg;
        op[0] = from_f<T>(ss.x + u.x * qk);
        op[1] = from_f<T>(ss.y + u.y * qk);
        op[2] = from_f<T>(ss.z + u.z * qk);
        op[3] = from_f<T>(ss.w + u.w * qk);
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int rw = rg + RG * m;
        const float kr = s_k[rw];
        float4 x = Sr[m];
        x.x += kr * u.x; x.y += kr * u.y; x.z += kr * u.z; x.w += kr * u.w;
        const floatx4 t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(Sp + (size_t)rw * DV) + cg);
    }
}

template <typename T, int DK, int DV, int DVW, int NTH>
static hipError_t launch_step_x(const StepArgs& a, hipStream_t s) {
    constexpr int CG = DVW / 4;
    constexpr int NT = (CG * DK < NTH) ? CG * DK : NTH;
    hipLaunchKernelGGL((kda_step_kernel<T, DK, DV, DVW, NTH>), dim3((unsigned)(a.B * a.H * (DV / DVW))), dim3(NT), 0, s, a);
    return hipGetLastError();
}

// Dv = 128: one workgroup of 512 threads per (b, h), so each wave reads two
// whole 512-byte state rows per instruction and the workgroup one contiguous
// 64 KiB state (measured at B256 H32 D128: 189 us per step against 195 us
// with two 64-column workgroups per (b, h), 197 us with 256 threads, 194-199
// us for forms that keep three workgroups per CU resident instead of two).
// Smaller Dv: 64 columns at most per workgroup of 256 threads.
template <typename T, int DK, int DV>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
    if constexpr (DV == 128) return launch_step_x<T, DK, DV, 128, 512>(a, s);
    constexpr int DVW = DV > 64 ? 64 : DV;
    return launch_step_x<T, DK, DV, DVW, 256>(a, s);
}

template <typename T, int DK>
static hipError_t launch_step_v(int DV, const StepArgs& a, hipStream_t s) {
    switch (DV) {
        case 16: return launch_step_t<T, DK, 16>(a, s);
        case 32: return launch_step_t<T, DK, 32>(a, s);
        case 64: return launch_step_t<T, DK, 64>(a, s);
        case 128: return launch_step_t<T, DK, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_step_k(int DK, int DV, const StepArgs& a, hipStream_t s) {
    switch (DK) {
        case 16: return launch_step_v<T, 16>(DV, a, s);
        case 32: return launch_step_v<T, 32>(DV, a, s);
        case 64: return launch_step_v<T, 64>(DV, a, s);
        case 128: return launch_step_v<T, 128>(DV, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(int dt, int DK, int DV, const StepArgs& a, hipStream_t s) {
    return dt == 1 ? launch_step_k<bf16_t>(DK, DV, a, s) : launch_step_k<float>(DK, DV, a, s);
}

}  // namespace kda
