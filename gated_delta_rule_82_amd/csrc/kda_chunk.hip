// kda_chunk.hip - chunkwise KDA forward on gfx950: the launch sequence of
// kda_chunk_fwd (intra and inter kernels over slices of the sequence) and the
// built-in scratch of the allocation-free entry point.
#include "kda_chunk_kernels.h"

namespace kda {

template <typename T, int DK, int C>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t stream, hipEvent_t* ev, int n_ev) {
    ChunkLaunch<T, DK, C> cl(a);
    const hipError_t attr = cl.set_attributes();
    if (attr != hipSuccess) return attr;
    const int BH = cl.BH;
    const int per = slice_chunks(BH, a.NC, cl.L.bytes, a.slice_budget);
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

template <typename T, int DK, int C>
static hipError_t launch_intra_t(const ChunkArgs& a, void* buf, int per, int c0, int nc, hipStream_t s) {
    return ChunkLaunch<T, DK, C>(a).intra(buf, per, c0, nc, s);
}

hipError_t launch_chunk_intra(int dt, int DK, int C, const ChunkArgs& a, void* buf, int per, int c0, int nc,
                              hipStream_t s) {
#define KDA_INTRA_C(T, D)                                                        \
    switch (C) {                                                                 \
        case 16: return launch_intra_t<T, D, 16>(a, buf, per, c0, nc, s);        \
        case 32: return launch_intra_t<T, D, 32>(a, buf, per, c0, nc, s);        \
        case 64: return launch_intra_t<T, D, 64>(a, buf, per, c0, nc, s);        \
        default: return hipErrorInvalidValue;                                    \
    }
#define KDA_INTRA_D(T)                                                           \
    switch (DK) {                                                                \
        case 16: KDA_INTRA_C(T, 16)                                              \
        case 32: KDA_INTRA_C(T, 32)                                              \
        case 64: KDA_INTRA_C(T, 64)                                              \
        case 128: KDA_INTRA_C(T, 128)                                            \
        default: return hipErrorInvalidValue;                                    \
    }
    if (dt == 1) { KDA_INTRA_D(bf16_t) }
    KDA_INTRA_D(float)
#undef KDA_INTRA_D
#undef KDA_INTRA_C
}

int chunk_kernel_count(int elem_bytes, int DK, int C, int BH, int NC) {
    const BlockLayout L = block_layout(elem_bytes, DK, C);
    if (NC <= 0) return 1;
    const int per = slice_chunks(BH, NC, L.bytes);
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

// ------------------------------------------------------------ built-in scratch
// The per-chunk blocks of one slice and the carried state of the
// allocation-free entry point.  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels and copies take the address
// hipGetSymbolAddress returns for the current device, cached per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_pointer(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* cache[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!cache[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        cache[dev] = p;
    }
    *ptr = cache[dev];
    return hipSuccess;
}

}  // namespace kda
