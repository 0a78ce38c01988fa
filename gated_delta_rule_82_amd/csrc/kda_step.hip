// kda_step.hip - single-token KDA decode on gfx950 ("KDA 模块交互式演示" §1.7
// kda_step; "Implémenter KDA" 'La forme récurrente de référence').
//
// The fp32 state is read from HBM once and written back once per step, and
// both reductions over Dk are taken from the same pass (column by column, so
// groups of value columns are independent), because with
// S' = Diag(alpha) S and u = beta (v - S'^T k):
//     S_new = S' + k u^T,     o = S_new^T q = S'^T q + u (k . q).
#include <atomic>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Raw per-head inputs of one step that the prep wave reads: lane l holds
// channels l + 64 m of q, k and z (zero past Dk) and lane 0 the raw beta.
template <typename T, int DK>
struct StepHeadRaw {
    static constexpr int MC = (DK + 63) / 64;
    T q[MC], k[MC], z[MC];
    T beta;
};

template <typename T, int DK>
__device__ __forceinline__ void step_load_head(const StepArgs& a, int bh, int lane, StepHeadRaw<T, DK>& r) {
    const int h = bh % a.H;
    // value head h reads q/k head h / G of the same batch row
    const size_t bq = (size_t)(bh / a.H) * (a.H / a.G) + h / a.G;
    const T* q = reinterpret_cast<const T*>(a.q) + bq * DK;
    const T* k = reinterpret_cast<const T*>(a.k) + bq * DK;
    const T* z = reinterpret_cast<const T*>(a.z) + (size_t)bh * DK;
#pragma unroll
    for (int m = 0; m < StepHeadRaw<T, DK>::MC; ++m) {
        const int c = lane + 64 * m;
        const bool ok = c < DK;
        r.q[m] = ok ? q[c] : from_f<T>(0.f);
        r.k[m] = ok ? k[c] : from_f<T>(0.f);
        r.z[m] = ok ? z[c] : from_f<T>(0.f);
    }
    if (lane == 0) r.beta = reinterpret_cast<const T*>(a.beta_raw)[bh];
}

// One wave prepares a head: normalised q and k, the decay alpha = e^g of
// every key channel, beta and q.k, into LDS (s_misc = {beta, q.k}).
template <typename T, int DK>
__device__ __forceinline__ void step_prep_head(const StepArgs& a, int bh, int lane, const StepHeadRaw<T, DK>& r,
                                               float* s_q, float* s_k, float* s_a, float* s_misc) {
    constexpr int MC = StepHeadRaw<T, DK>::MC;
    const int h = bh % a.H;
    float qv[MC], kv[MC], zv[MC];
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
        const int c = lane + 64 * m;
        qv[m] = to_f<T>(r.q[m]);
        kv[m] = to_f<T>(r.k[m]);
        zv[m] = (c < DK) ? to_f<T>(r.z[m]) + ((a.dt_bias && (a.flags & kGateIn)) ? a.dt_bias[(size_t)h * DK + c] : 0.f)
                         : 0.f;
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
        const int c = lane + 64 * m;
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
    if (lane == 0) {
        const float braw = to_f<T>(r.beta);
        s_misc[0] = (a.flags & kBetaSig) ? sigmoidf_(braw) : braw;
        s_misc[1] = qk;
    }
}

// The rest of a step for one thread that holds rows rg + RG m (m < RPT) of
// four state columns (col0 + 4 cg ..) in Sr, with the head prepared in LDS:
// decay the rows and form this thread's partial S'^T k and S'^T q into s_red
// (the caller then synchronises and calls step_finish).
template <int RG, int RPT, int DVW>
__device__ __forceinline__ void step_partials(float4 (&Sr)[RPT], int rg, int cg, const float* s_q, const float* s_k,
                                              const float* s_a, float (*s_red)[RG][DVW]) {
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
}

// Sum the partials, write o (row group 0) and the updated rows of the state.
template <typename T, int DK, int DV, int RG, int RPT, int DVW>
__device__ __forceinline__ void step_finish(const StepArgs& a, int bh, int col0, float4 (&Sr)[RPT], const float (&vv)[4],
                                            int rg, int cg, const float* s_k, const float* s_misc,
                                            const float (*s_red)[RG][DVW]) {
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
    static_assert(RG * RPT == DK, "the row groups cover Dk");
    float* Sp = a.S + (size_t)bh * DK * DV + col0;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int rw = rg + RG * m;
        const float kr = s_k[rw];
        float4 x = Sr[m];
        x.x += kr * u.x; x.y += kr * u.y; x.z += kr * u.z; x.w += kr * u.w;
        // the state is written once per step: non-temporal stores
        const floatx4 t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<floatx4*>(Sp + (size_t)rw * DV) + cg);
    }
}

// General shapes: one workgroup per (b, h) and group of DVW value columns
// (both reductions run over Dk column by column, so column groups are
// independent); the state goes from HBM to registers and back once.
template <typename T, int DK, int DV, int DVW, int NTH>
__global__ __launch_bounds__(NTH) void kda_step_kernel(const StepArgs a) {
    constexpr int NSPLIT = DV / DVW;                   // workgroups per (b, h)
    constexpr int CG = DVW / 4;                        // float4 column groups
    constexpr int NT = (CG * DK < NTH) ? CG * DK : NTH;
    constexpr int RG = NT / CG;                        // row groups
    constexpr int RPT = DK / RG;                       // rows per thread

    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ __align__(16) float s_red[2][RG][DVW];
    __shared__ float s_misc[2];

    const int bh = blockIdx.x / NSPLIT;
    const int col0 = (blockIdx.x % NSPLIT) * DVW;
    const int tid = threadIdx.x;
    if (tid >= NT) return;  // NT is a multiple of 64; no thread past NT reaches a barrier
    const int cg = tid % CG;
    const int rg = tid / CG;

    const float* Sp = a.S + (size_t)bh * DK * DV + col0;
    // non-temporal state loads (measured: 212 -> 195 us per B256 H32 D128
    // step with the earlier one-pass kernel)
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
        StepHeadRaw<T, DK> r;
        step_load_head<T, DK>(a, bh, tid, r);
        step_prep_head<T, DK>(a, bh, tid, r, s_q, s_k, s_a, s_misc);
    }
    __syncthreads();
    step_partials<RG, RPT, DVW>(Sr, rg, cg, s_q, s_k, s_a, s_red);
    __syncthreads();
    step_finish<T, DK, DV, RG, RPT, DVW>(a, bh, col0, Sr, vv, rg, cg, s_k, s_misc, s_red);
}

// Dk = Dv = 128: persistent workgroups, one per CU, each taking heads
// blockIdx.x, blockIdx.x + gridDim.x, ...  Two copy waves stream the next
// head's 64 KiB state into one of two LDS slots with global_load_lds while
// eight compute waves (512 threads, 8 rows of 4 columns each) finish the
// current head from the other slot and store it back; wave 0 also prepares
// the next head's q, k, decay and beta one head ahead (double-buffered), and
// every thread requests its next four values one head ahead.  Each head
// costs two barriers, and only the copy waves ever wait on the state's loads.
// (Measured at B256 H32 D128 on one MI355X: 174 us per step, 77.9 % of HBM
// peak, against 188 us for one 512-thread workgroup per (b, h) loading
// straight into registers and 177 us for an in-place torch multiply of the
// same state; the same kernel with non-temporal copies ran at 188 us.)
constexpr int kStepStreamThreads = 640;
constexpr int kStepStreamLds = 2 * 128 * 128 * 4;

template <typename T>
__global__ __launch_bounds__(kStepStreamThreads) void kda_step_stream_kernel(const StepArgs a) {
    constexpr int DK = 128, DV = 128;
    constexpr int CG = 32, RG = 16, RPT = 8;
    constexpr int kStateB = DK * DV * 4;
    extern __shared__ __align__(16) unsigned char s_slots[];  // two states
    __shared__ float s_q[2][DK], s_k[2][DK], s_a[2][DK];
    __shared__ __align__(16) float s_red[2][RG][DV];
    __shared__ float s_misc[2][2];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int G = gridDim.x;
    const int first = blockIdx.x;
    const int nbh = a.B * a.H;
    const int nmine = first < nbh ? (nbh - 1 - first) / G + 1 : 0;  // heads of this workgroup

    if (w >= 8) {
        // ------------------------------------------------------ copy waves
        // each streams half of a state: 32 pieces of 1 KiB (16 bytes per lane)
        const int cw = w - 8;
        auto issue = [&](int i) {
            const unsigned char* src = reinterpret_cast<const unsigned char*>(a.S + (size_t)(first + i * G) * DK * DV);
            unsigned char* slot = s_slots + (i & 1) * kStateB;
#pragma unroll
            for (int p = 0; p < 32; ++p) {
                const int pc = cw * 32 + p;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(src + pc * 1024 + lane * 16),
                    (__attribute__((address_space(3))) void*)(slot + pc * 1024), 16, 0, 0);
            }
        };
        if (nmine > 0) { issue(0); wait_vmcnt<0>(); }
        lds_barrier();  // head 0 is in its slot
        for (int i = 0; i < nmine; ++i) {
            // the slot of head i + 1 held head i - 1, read before the last barrier
            if (i + 1 < nmine) issue(i + 1);
            lds_barrier();
            wait_vmcnt<0>();
            lds_barrier();  // head i + 1 is in its slot
        }
        return;
    }

    // ------------------------------------------------------------ compute waves
    const int cg = tid % CG;
    const int rg = tid / CG;
    StepHeadRaw<T, DK> raw;
    T rv[4];
    auto load_next = [&](int i) {  // raw inputs of head i, one head ahead
        const int bh = first + i * G;
        const T* vp = reinterpret_cast<const T*>(a.v) + (size_t)bh * DV + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[e] = vp[e];
        if (w == 0) step_load_head<T, DK>(a, bh, lane, raw);
    };
    if (nmine > 0) {
        load_next(0);
        if (w == 0) step_prep_head<T, DK>(a, first, lane, raw, s_q[0], s_k[0], s_a[0], s_misc[0]);
    }
    lds_barrier();
    for (int i = 0; i < nmine; ++i) {
        const int bh = first + i * G;
        const int pb = i & 1;
        float vv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = to_f<T>(rv[e]);
        if (i + 1 < nmine) load_next(i + 1);
        const unsigned char* slot = s_slots + pb * kStateB;
        float4 Sr[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            Sr[m] = *reinterpret_cast<const float4*>(slot + ((size_t)(rg + RG * m) * DV + 4 * cg) * 4);
        step_partials<RG, RPT, DV>(Sr, rg, cg, s_q[pb], s_k[pb], s_a[pb], s_red);
        lds_barrier();
        step_finish<T, DK, DV, RG, RPT, DV>(a, bh, 0, Sr, vv, rg, cg, s_k[pb], s_misc[pb], s_red);
        // the other buffer's last readers finished before the barrier above
        if (w == 0 && i + 1 < nmine)
            step_prep_head<T, DK>(a, bh + G, lane, raw, s_q[pb ^ 1], s_k[pb ^ 1], s_a[pb ^ 1], s_misc[pb ^ 1]);
        lds_barrier();
    }
}

template <typename T, int DK, int DV, int DVW, int NTH>
static hipError_t launch_step_x(const StepArgs& a, hipStream_t s) {
    constexpr int CG = DVW / 4;
    constexpr int NT = (CG * DK < NTH) ? CG * DK : NTH;
    hipLaunchKernelGGL((kda_step_kernel<T, DK, DV, DVW, NTH>), dim3((unsigned)(a.B * a.H * (DV / DVW))), dim3(NT), 0, s, a);
    return hipGetLastError();
}

// Workgroups of the streamed kernel resident on the current device at once
// (CUs times workgroups per CU), asked once per device; 0 if unknown.
template <typename T>
static int step_stream_capacity() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kda_step_stream_kernel<T>),
                                                     kStepStreamThreads, kStepStreamLds) != hipSuccess)
        return 0;
    v = cus * per_cu;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

template <typename T>
static hipError_t launch_step_stream(const StepArgs& a, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(kda_step_stream_kernel<T>);
    // set on every call: the attribute is per device, and the call only records a limit
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kStepStreamLds);
    if (e != hipSuccess) return e;
    const int nbh = a.B * a.H;
    const int cap = step_stream_capacity<T>();
    // any grid is correct (a workgroup's heads are independent of the others');
    // one resident round is the fastest
    const int grid = nbh < (cap > 0 ? cap : 256) ? nbh : (cap > 0 ? cap : 256);
    hipLaunchKernelGGL((kda_step_stream_kernel<T>), dim3((unsigned)grid), dim3(kStepStreamThreads), kStepStreamLds, s, a);
    return hipGetLastError();
}

// Dv = 128 with Dk = 128: the streamed persistent kernel.  Other Dk with Dv =
// 128: one workgroup of 512 threads per (b, h), so each wave reads two whole
// 512-byte state rows per instruction.  Smaller Dv: 64 columns at most per
// workgroup of 256 threads.
template <typename T, int DK, int DV>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
    if constexpr (DK == 128 && DV == 128) return launch_step_stream<T>(a, s);
    else if constexpr (DV == 128) return launch_step_x<T, DK, DV, 128, 512>(a, s);
    else return launch_step_x<T, DK, DV, (DV > 64 ? 64 : DV), 256>(a, s);
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
