// kda_conv.hip - the layer's input side on gfx950: causal depthwise short
// convolution over the token axis, then SiLU ("KDA 模块交互式演示" §1.1
// ShortConv and §1.7 KimiDeltaAttention 完整层; "Implémenter KDA" 'La
// paramétrisation': kernel 4, then Swish).
//
//   y[b, t, c] = act(bias[c] + sum_{j=0..3} w[c, j] x[b, t - 3 + j, c])
//
// Tap 3 multiplies the current token (last tap 1 and the others 0 is the
// identity).  The three inputs before the first token come from a carried
// window (or are zero), and the last three inputs of the call leave in one.
//
// Pure bandwidth: every input is read once (plus a three-row halo per tile)
// and every output written once (non-temporal: nothing reads it back soon).
// A thread owns 8 consecutive channels (one 16-byte row piece in bf16) of one
// tile of kTile tokens, keeps the window in registers and has a whole tile's
// row loads in flight at once (bf16; fp32 in batches of 8 rows).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kTaps = 4;
constexpr int kTile = 32;     // tokens per thread
constexpr int kThreads = 256;
constexpr int kChan = 8;      // channels per thread

// Eight consecutive elements of one row, widened to float.
template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
    static constexpr int kBatch = 32;  // rows whose loads are in flight together (a whole tile)
    uint4 raw;
    // plain loads: the next tile's workgroup re-reads the last three rows as
    // its halo, which non-temporal loads would not keep (measured: 29 vs 32 us
    // per layer-sized tensor)
    __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { raw = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t wd = i < 2 ? raw.x : i < 4 ? raw.y : i < 6 ? raw.z : raw.w;
        return (i & 1) ? __uint_as_float(wd & 0xffff0000u) : __uint_as_float(wd << 16);
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[kChan]) {
        typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
        const bf16x8v o = {(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3],
                           (bf16_t)v[4], (bf16_t)v[5], (bf16_t)v[6], (bf16_t)v[7]};
        __builtin_nontemporal_store(o, reinterpret_cast<bf16x8v*>(p));
    }
};
template <> struct Row8<float> {
    static constexpr int kBatch = 8;
    floatx4 lo, hi;
    __device__ __forceinline__ void load(const float* p) {
        lo = reinterpret_cast<const floatx4*>(p)[0];
        hi = reinterpret_cast<const floatx4*>(p)[1];
    }
    __device__ __forceinline__ void zero() {
        lo = floatx4{0.f, 0.f, 0.f, 0.f};
        hi = lo;
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
    static __device__ __forceinline__ void store(float* p, const float (&v)[kChan]) {
        const floatx4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<floatx4*>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<floatx4*>(p) + 1);
    }
};

}  // namespace

// grid: x = channel blocks of kThreads * kChan, y = token tiles, z = batch
template <typename T>
__global__ __launch_bounds__(kThreads) void kda_short_conv_kernel(const ShortConvArgs a) {
    const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kChan;
    if (c0 >= a.C) return;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * kTile;
    const int t1 = min(t0 + kTile, a.T);
    const T* x = reinterpret_cast<const T*>(a.x) + (size_t)b * a.T * a.C + c0;
    T* y = reinterpret_cast<T*>(a.y) + (size_t)b * a.T * a.C + c0;

    float w[kChan][kTaps], bias[kChan];
#pragma unroll
    for (int i = 0; i < kChan; ++i) {
        const float4 t = reinterpret_cast<const float4*>(a.w)[c0 + i];
        w[i][0] = t.x; w[i][1] = t.y; w[i][2] = t.z; w[i][3] = t.w;
        bias[i] = a.bias ? a.bias[c0 + i] : 0.f;
    }

    // window: inputs t0 - 3, t0 - 2, t0 - 1 (from x, the carried window, or zero)
    float win[kTaps - 1][kChan];
#pragma unroll
    for (int j = 0; j < kTaps - 1; ++j) {
        const int t = t0 - (kTaps - 1) + j;
        Row8<T> r;
        if (t >= 0) r.load(x + (size_t)t * a.C);
        else if (a.state_in)
            r.load(reinterpret_cast<const T*>(a.state_in) + ((size_t)b * (kTaps - 1) + (kTaps - 1) + t) * a.C + c0);
        else r.zero();
#pragma unroll
        for (int i = 0; i < kChan; ++i) win[j][i] = r.get(i);
    }

    constexpr int NB = Row8<T>::kBatch;
    for (int tb = t0; tb < t1; tb += NB) {
        Row8<T> rows[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (tb + u < t1) rows[u].load(x + (size_t)(tb + u) * a.C);
            else rows[u].zero();
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (tb + u < t1) {
                float out[kChan];
#pragma unroll
                for (int i = 0; i < kChan; ++i) {
                    const float cur = rows[u].get(i);
                    const float s = conv4(make_float4(w[i][0], w[i][1], w[i][2], w[i][3]), bias[i], win[0][i],
                                          win[1][i], win[2][i], cur);
                    out[i] = a.silu ? silu_(s) : s;
                    win[0][i] = win[1][i];
                    win[1][i] = win[2][i];
                    win[2][i] = cur;
                }
                Row8<T>::store(y + (size_t)(tb + u) * a.C, out);
            }
        }
    }

    // the tile holding the last token hands the window on
    if (a.state_out && t0 + kTile >= a.T) {
        T* so = reinterpret_cast<T*>(a.state_out) + (size_t)b * (kTaps - 1) * a.C + c0;
#pragma unroll
        for (int j = 0; j < kTaps - 1; ++j) {
            float v[kChan];
#pragma unroll
            for (int i = 0; i < kChan; ++i) v[i] = win[j][i];
            Row8<T>::store(so + (size_t)j * a.C, v);
        }
    }
}

int short_conv_tile() { return kTile; }

hipError_t launch_short_conv(int dt, const ShortConvArgs& a, hipStream_t s) {
    const int cb = (a.C / kChan + kThreads - 1) / kThreads;
    const int tiles = a.T > 0 ? (a.T + kTile - 1) / kTile : 1;
    const dim3 grid((unsigned)cb, (unsigned)tiles, (unsigned)a.B);
    if (dt == 1)
        hipLaunchKernelGGL(kda_short_conv_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(kda_short_conv_kernel<float>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
