// kda_layer.hip - the layer body on gfx950 (kda_layer_fwd): the chunk kernels
// with the layer's output side, sigmoid(gate) times the per-head RMS norm of
// o, applied in the inter kernel before each output row is stored
// ("KDA 模块交互式演示" §1.7 完整层; "Implémenter KDA" 'La porte de sortie de
// rang plein').  The workgroups of a (b, h) exchange per-token partial sums
// of squares through the workspace, which needs them all resident together;
// when the grid is not, the call runs the plain chunk kernels into y and the
// separate output-side kernel over y in place (the same result up to the
// summation order of the norm).
#include "kda_chunk_kernels.h"

namespace kda {

template <typename T, int DK, int C>
static hipError_t launch_layer_t(const ChunkArgs& args, hipStream_t stream) {
    const int dt = sizeof(T) == 2 ? 1 : 0;
    ChunkArgs a = args;
    ChunkLaunch<T, DK, C, true> cl(a);
    const int BH = cl.BH;
    const int per = slice_chunks(BH, a.NC, cl.L.bytes, a.slice_budget);
    if (a.ws_bytes < layer_workspace_bytes(sizeof(T), DK, a.Dv, C, (size_t)BH, (size_t)per))
        return hipErrorInvalidValue;
    if (!cl.resident) {
        ChunkArgs plain = args;
        plain.gate = nullptr;
        plain.gate_w = nullptr;
        hipError_t e = launch_chunk(dt, DK, C, plain, stream, nullptr, 0);
        if (e != hipSuccess || a.T == 0) return e;
        GateArgs ga{a.o, a.gate, a.gate_w, a.o, (size_t)a.B * a.T * a.H};
        return launch_output_gate(dt, a.Dv, ga, stream);
    }
    const hipError_t attr = cl.set_attributes();
    if (attr != hipSuccess) return attr;
    unsigned char* ws = reinterpret_cast<unsigned char*>(a.ws);
    float* S_scr = reinterpret_cast<float*>(ws + (size_t)BH * per * cl.L.bytes);
    float* M_scr = S_scr + (size_t)BH * DK * a.Dv;
    a.gss = reinterpret_cast<float*>(ws + layer_gss_offset(sizeof(T), DK, a.Dv, C, (size_t)BH, (size_t)per));
    a.gss_n = cl.gss_per_chunk();
    cl.ea.gss = a.gss;

    const int nsl = a.NC > 0 ? (a.NC + per - 1) / per : 1;
    for (int sl = 0; sl < nsl; ++sl) {
        const int c0 = sl * per;
        const int nc = std::max(0, std::min(per, a.NC - c0));
        if (nc > 0) {
            const hipError_t e = launch_chunk_intra(dt, DK, C, a, a.ws, per, c0, nc, stream);
            if (e != hipSuccess) return e;
        }
        const hipError_t e = cl.inter(a.ws, per, c0, nc, sl == 0, sl == nsl - 1, S_scr, M_scr, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int DK>
static hipError_t launch_layer_c(int C, const ChunkArgs& a, hipStream_t s) {
    switch (C) {
        case 16: return launch_layer_t<T, DK, 16>(a, s);
        case 32: return launch_layer_t<T, DK, 32>(a, s);
        case 64: return launch_layer_t<T, DK, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_layer_d(int DK, int C, const ChunkArgs& a, hipStream_t s) {
    switch (DK) {
        case 16: return launch_layer_c<T, 16>(C, a, s);
        case 32: return launch_layer_c<T, 32>(C, a, s);
        case 64: return launch_layer_c<T, 64>(C, a, s);
        case 128: return launch_layer_c<T, 128>(C, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_layer(int dt, int DK, int C, const ChunkArgs& a, hipStream_t s) {
    return dt == 1 ? launch_layer_d<bf16_t>(DK, C, a, s) : launch_layer_d<float>(DK, C, a, s);
}

}  // namespace kda
