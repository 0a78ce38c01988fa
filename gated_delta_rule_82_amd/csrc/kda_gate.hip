// kda_gate.hip - the layer's output side on gfx950: per-head RMS
// normalisation of the core's output under the full-rank sigmoid gate, the
// step before the output projection ("KDA 模块交互式演示" §1.7
// KimiDeltaAttention 完整层; "Implémenter KDA" 'La porte de sortie de rang
// plein', kda_output):
//
//   y[b,t,h,c] = sigmoid(gate[b,t,h,c]) * o[b,t,h,c] * weight[c]
//                / sqrt(mean_c' o[b,t,h,c']^2 + 1e-6)
//
// Pure bandwidth (o and gate read once, y written once).  A lane holds one
// 16-byte piece of a head row; the LPR lanes of a row reduce its sum of
// squares with xor shuffles inside their group, and a wave takes kRowsPerLane
// row groups with all their loads in flight before any arithmetic.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerLane = 4;
constexpr float kRmsEps = 1e-6f;

// 16 bytes of one row, widened to float.
template <typename T> struct Piece;
template <> struct Piece<bf16_t> {
    static constexpr int N = 8;
    uint4 raw;
    __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t wd = i < 2 ? raw.x : i < 4 ? raw.y : i < 6 ? raw.z : raw.w;
        return (i & 1) ? __uint_as_float(wd & 0xffff0000u) : __uint_as_float(wd << 16);
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[N]) {
        typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
        const bf16x8v o = {(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3],
                           (bf16_t)v[4], (bf16_t)v[5], (bf16_t)v[6], (bf16_t)v[7]};
        __builtin_nontemporal_store(o, reinterpret_cast<bf16x8v*>(p));
    }
};
template <> struct Piece<float> {
    static constexpr int N = 4;
    floatx4 v4;
    __device__ __forceinline__ void load(const float* p) { v4 = *reinterpret_cast<const floatx4*>(p); }
    __device__ __forceinline__ float get(int i) const { return v4[i]; }
    static __device__ __forceinline__ void store(float* p, const float (&v)[N]) {
        const floatx4 o = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<floatx4*>(p));
    }
};

}  // namespace

template <typename T, int DV>
__global__ __launch_bounds__(kThreads) void kda_output_gate_kernel(const GateArgs a) {
    constexpr int N = Piece<T>::N;   // elements per lane
    constexpr int LPR = DV / N;      // lanes per head row
    constexpr int RPW = 64 / LPR;    // rows per wave and step
    static_assert(LPR >= 1 && 64 % LPR == 0, "a head row spans a power-of-two lane group");
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR, part = lane % LPR;
    const size_t wave = ((size_t)blockIdx.x * kThreads + threadIdx.x) / 64;
    const size_t row0 = wave * (size_t)(RPW * kRowsPerLane) + sub;

    float w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = a.weight ? a.weight[part * N + i] : 1.f;

    Piece<T> po[kRowsPerLane], pg[kRowsPerLane];
#pragma unroll
    for (int u = 0; u < kRowsPerLane; ++u) {
        const size_t row = row0 + (size_t)u * RPW;
        if (row < a.rows) {
            const size_t off = row * DV + part * N;
            po[u].load(reinterpret_cast<const T*>(a.o) + off);
            pg[u].load(reinterpret_cast<const T*>(a.gate) + off);
        }
    }
#pragma unroll
    for (int u = 0; u < kRowsPerLane; ++u) {
        const size_t row = row0 + (size_t)u * RPW;
        if (row < a.rows) {  // uniform over the lane group of this row
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) ss = fmaf(po[u].get(i), po[u].get(i), ss);
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, LPR);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + kRmsEps);
            float y[N];
#pragma unroll
            for (int i = 0; i < N; ++i) y[i] = sigmoidf_(pg[u].get(i)) * po[u].get(i) * inv * w[i];
            Piece<T>::store(reinterpret_cast<T*>(a.y) + row * DV + part * N, y);
        }
    }
}

template <typename T, int DV>
static hipError_t launch_gate_t(const GateArgs& a, hipStream_t s) {
    constexpr int RPW = 64 / (DV / Piece<T>::N);
    const size_t rows_per_block = (size_t)(kThreads / 64) * RPW * kRowsPerLane;
    const size_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((kda_output_gate_kernel<T, DV>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_gate_d(int DV, const GateArgs& a, hipStream_t s) {
    switch (DV) {
        case 16: return launch_gate_t<T, 16>(a, s);
        case 32: return launch_gate_t<T, 32>(a, s);
        case 64: return launch_gate_t<T, 64>(a, s);
        case 128: return launch_gate_t<T, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_output_gate(int dt, int DV, const GateArgs& a, hipStream_t s) {
    return dt == 1 ? launch_gate_d<bf16_t>(DV, a, s) : launch_gate_d<float>(DV, a, s);
}

}  // namespace kda
