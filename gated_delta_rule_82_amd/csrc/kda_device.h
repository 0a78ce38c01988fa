// kda_device.h - device-side building blocks shared by the gfx950 KDA kernels.
//
// Matrix-core convention used throughout (wave64, one 16x16 output tile):
//
//   * C layout ("column owner"): lane l holds X[4*(l/16) + i][l % 16], i = 0..3.
//     This is the accumulator layout of v_mfma_f32_16x16x{32_bf16,4_f32}.
//   * Operand fragment for one 32-long contraction step: lane l supplies row
//     (l % 16) of A (or column (l % 16) of B) at 8 contraction slots
//         slot j < 4  -> index 4*(l/16) + j
//         slot j >= 4 -> index 16 + 4*(l/16) + (j - 4).
//     A and B use the same slot map, so the product is exact whatever order the
//     hardware sums the slots in.  The map is chosen so that two C-layout tiles
//     stacked along the contraction axis (rows 0..15 and 16..31) ARE the B
//     fragment of the next product: no data moves across lanes.
//   * R layout ("row owner"): lane l holds X[l % 16][4*(l/16) + i].  For 16x16
//     matrices, mm(R(X), C(Y)) = C(X Y) and mm(C(Y), R(X)) = R(X Y).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float sigmoidf_(float x) {
    // 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each);
    // a large negative x gives exp2 = +inf and the reciprocal 0.
    return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return (bf16_t)x; }

// Causal kernel-4 short convolution of one channel: bias + w.x x[t-3] +
// w.y x[t-2] + w.z x[t-1] + w.w x[t], summed in this order with fused
// multiply-adds (the standalone input-side kernel and the convolution fused
// into the chunk kernels share it, so they produce the same values).
__device__ __forceinline__ float conv4(const float4 w, float bias, float x3, float x2, float x1, float x0) {
    float s = bias;
    s = fmaf(w.x, x3, s);
    s = fmaf(w.y, x2, s);
    s = fmaf(w.z, x1, s);
    s = fmaf(w.w, x0, s);
    return s;
}
__device__ __forceinline__ float silu_(float s) { return s * sigmoidf_(s); }

// 32-bit word of lane (row position r - d) within each 16-lane DPP row, for
// d in {1, 2} (zero where it runs off the row), and of lane r + d.
__device__ __forceinline__ uint32_t row_shr_word(uint32_t x, int d) {
    return d == 1 ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true)
                  : (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row_shl_word(uint32_t x, int d) {
    return d == 1 ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x101, 0xF, 0xF, true)
                  : (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x102, 0xF, 0xF, true);
}

// Raw element bits, converted to float only when consumed.
template <typename T> struct RawBits;
template <> struct RawBits<bf16_t> {
    typedef uint16_t type;
    static __device__ __forceinline__ float to_float(uint16_t x) { return bf16_bits_to_float(x); }
};
template <> struct RawBits<float> {
    typedef uint32_t type;
    static __device__ __forceinline__ float to_float(uint32_t x) { return __uint_as_float(x); }
};

// One 16-byte granule of consecutive elements: element i widened to float,
// and N floats packed back (round to nearest even for bf16).
template <typename T> struct Gran16;
template <> struct Gran16<bf16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ float get(const uint4& g, int i) {
        const uint32_t wd = i < 2 ? g.x : i < 4 ? g.y : i < 6 ? g.z : g.w;
        return (i & 1) ? __uint_as_float(wd & 0xffff0000u) : __uint_as_float(wd << 16);
    }
    static __device__ __forceinline__ uint4 pack(const float (&x)[8]) {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wd[k] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[2 * k]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[2 * k + 1]) << 16);
        return make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
};
template <> struct Gran16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ float get(const uint4& g, int i) {
        return __uint_as_float(i == 0 ? g.x : i == 1 ? g.y : i == 2 ? g.z : g.w);
    }
    static __device__ __forceinline__ uint4 pack(const float (&x)[4]) {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
};

// Four consecutive elements kept as loaded (bf16: two packed registers) and
// widened to float where used, so they occupy half the registers until then.
template <typename T> struct Raw4;
template <> struct Raw4<bf16_t> {
    static constexpr int kWords = 2;
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = i < 2 ? v.x : v.y;
        return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
    __device__ __forceinline__ uint32_t word(int i) const { return i ? v.y : v.x; }
    __device__ __forceinline__ void set_word(int i, uint32_t x) { if (i) v.y = x; else v.x = x; }
    // four values rounded to bf16 (round to nearest even)
    __device__ __forceinline__ void set4(const float (&x)[4]) {
        v.x = (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[1]) << 16);
        v.y = (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[3]) << 16);
    }
};
template <> struct Raw4<float> {
    static constexpr int kWords = 4;
    float4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ float get(int i) const { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
    __device__ __forceinline__ uint32_t word(int i) const { return __float_as_uint(get(i)); }
    __device__ __forceinline__ void set_word(int i, uint32_t x) {
        const float f = __uint_as_float(x);
        if (i == 0) v.x = f; else if (i == 1) v.y = f; else if (i == 2) v.z = f; else v.w = f;
    }
    __device__ __forceinline__ void set4(const float (&x)[4]) { v = make_float4(x[0], x[1], x[2], x[3]); }
};

// Load 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32).
__device__ __forceinline__ void load4(const float* p, float out[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float out[4]) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = bf16_bits_to_float(v.x & 0xffffu);
    out[1] = bf16_bits_to_float(v.x >> 16);
    out[2] = bf16_bits_to_float(v.y & 0xffffu);
    out[3] = bf16_bits_to_float(v.y >> 16);
}

// ---------------------------------------------------------------- fragments

__host__ __device__ constexpr int slot_index(int grp, int j) {
    return j < 4 ? 4 * grp + j : 16 + 4 * grp + (j - 4);
}

template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    bf16x8 v;
    __device__ __forceinline__ void set(int j, float x) { v[j] = (bf16_t)x; }
    __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (bf16_t)0.0f;
    }
};
template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int j, float x) { v[j] = x; }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
};

// acc += A * B over one 32-long contraction step.
__device__ __forceinline__ floatx4 mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const Frag<float>& a, const Frag<float>& b, floatx4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}

// Load / store a fragment from a fragment-major tile (64 lanes x 8 elements).
__device__ __forceinline__ void frag_load(Frag<bf16_t>& f, const bf16_t* tile, int lane) {
    f.v = *reinterpret_cast<const bf16x8*>(tile + lane * 8);
}
__device__ __forceinline__ void frag_load(Frag<float>& f, const float* tile, int lane) {
    const float4* p = reinterpret_cast<const float4*>(tile + lane * 8);
    float4 a = p[0], b = p[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void frag_store(const Frag<bf16_t>& f, bf16_t* tile, int lane) {
    *reinterpret_cast<bf16x8*>(tile + lane * 8) = f.v;
}
__device__ __forceinline__ void frag_store(const Frag<float>& f, float* tile, int lane) {
    float4* p = reinterpret_cast<float4*>(tile + lane * 8);
    p[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
    p[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}

// Store 4 values into one half (slots 0..3 or 4..7) of a lane's fragment slot.
__device__ __forceinline__ void half_store(bf16_t* tile, int lane, int half, const float x[4]) {
    bf16_t* p = tile + lane * 8 + half * 4;
    uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[0]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[1]) << 16);
    uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[2]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (bf16_t)x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ void half_store(float* tile, int lane, int half, const float x[4]) {
    *reinterpret_cast<float4*>(tile + lane * 8 + half * 4) = make_float4(x[0], x[1], x[2], x[3]);
}

// Half tiles (64 lanes x 4 elements): a lane's slots 0..3, the other four zero.
__device__ __forceinline__ void quarter_store(bf16_t* tile, int lane, const float x[4]) {
    typedef __bf16 bf16x4q __attribute__((ext_vector_type(4)));
    const bf16x4q v = {(bf16_t)x[0], (bf16_t)x[1], (bf16_t)x[2], (bf16_t)x[3]};
    *reinterpret_cast<bf16x4q*>(tile + lane * 4) = v;
}
__device__ __forceinline__ void quarter_store(float* tile, int lane, const float x[4]) {
    *reinterpret_cast<float4*>(tile + lane * 4) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void frag_load_half(Frag<bf16_t>& f, const bf16_t* tile, int lane) {
    typedef __bf16 bf16x4q __attribute__((ext_vector_type(4)));
    const bf16x4q h = *reinterpret_cast<const bf16x4q*>(tile + lane * 4);
    const bf16_t z = (bf16_t)0.f;
    f.v = bf16x8{h[0], h[1], h[2], h[3], z, z, z, z};
}
__device__ __forceinline__ void frag_load_half(Frag<float>& f, const float* tile, int lane) {
    const float4 h = *reinterpret_cast<const float4*>(tile + lane * 4);
    f.v[0] = h.x; f.v[1] = h.y; f.v[2] = h.z; f.v[3] = h.w;
    f.v[4] = f.v[5] = f.v[6] = f.v[7] = 0.f;
}

// Load 8 consecutive elements into a fragment's slots 0..7 (16 bytes for
// bf16, 32 for fp32; p aligned to 16 bytes).
__device__ __forceinline__ void frag_load_row8(Frag<bf16_t>& f, const bf16_t* p) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void frag_load_row8(Frag<float>& f, const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// The same with non-temporal loads (data read once).
__device__ __forceinline__ void frag_load_row8_nt(Frag<bf16_t>& f, const bf16_t* p) {
    f.v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}
__device__ __forceinline__ void frag_load_row8_nt(Frag<float>& f, const float* p) {
    const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    const floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p) + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.v[i] = a[i]; f.v[4 + i] = b[i]; }
}

// Load 4 consecutive elements widened to float (p aligned to 8 / 16 bytes).
__device__ __forceinline__ floatx4 load4v(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ floatx4 load4v(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// Store 4 consecutive elements (one 8- or 16-byte store; p aligned to it).
__device__ __forceinline__ void store4(bf16_t* p, const floatx4& x) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = {(bf16_t)x[0], (bf16_t)x[1], (bf16_t)x[2], (bf16_t)x[3]};
    *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, const floatx4& x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// B fragment from two C-layout tiles stacked along the contraction axis.
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_c(const floatx4& lo, const floatx4& hi) {
    Frag<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.set(i, lo[i]); f.set(4 + i, hi[i]); }
    return f;
}
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_c_lo(const floatx4& lo) {
    Frag<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.set(i, lo[i]); f.set(4 + i, 0.0f); }
    return f;
}

// 16x16x16 fp32 product on the matrix core: acc = X * Y with X given as its
// 4 contraction slots per lane (R layout of X or C layout of Y^T, see header).
__device__ __forceinline__ floatx4 mm16(const floatx4& a, const floatx4& b) {
    floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------- lane ops

// One round of an inclusive prefix sum over the 16 lanes of each DPP row:
// x shifted down the row by 2^sh lanes (zero where it runs off the row).
__device__ __forceinline__ float row_shift_add(float x, int sh) {
    const int v = __float_as_int(x);
    switch (sh) {
        case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));
    }
}

// Sum over the four lane groups that share lane % 16.
__device__ __forceinline__ float group_sum4(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// s_waitcnt vmcnt(N) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Scheduling pattern for the rest of the current scheduling region: M
// matrix-core instructions, each followed by its even share of D LDS reads.
template <int M, int D, int I = 0>
__device__ __forceinline__ void interleave_mfma_ds() {
    if constexpr (I < M) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        constexpr int nr = D * (I + 1) / M - D * I / M;
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // nr DS reads
        interleave_mfma_ds<M, D, I + 1>();
    }
}

// Workgroup barrier without a memory fence: this wave's LDS operations are
// complete (lgkmcnt 0), then s_barrier.  Outstanding global loads are not
// waited for; the caller accounts for them with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Map a linear block index so that consecutive logical blocks share an XCD
// (blocks are dealt round-robin over the 8 XCDs of MI355X).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

}  // namespace kda
