// kda_api.cpp - the exported C ABI: host validation, sizing and dispatch.
//
// Every entry point validates all arguments before it enqueues anything, and
// validation itself makes no HIP call, so rejected calls are side-effect free
// and can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>


#include "../../include/kda.h"
#include "kda_bwd.h"

namespace {

constexpr double kBf16Max = 3.3895313892515355e38;  // (2 - 2^-7) * 2^127
constexpr double kF32Max = 3.4028234663852886e38;
constexpr double kHeadroom = 1024.0;
constexpr int kFactorTile = 16;  // token tile of the factored decay products

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(kda_dtype dt) { return dt == KDA_F32 || dt == KDA_BF16; }
// known bits only; the v1 gate selects the form of the in-kernel gate
bool flags_ok(unsigned f) {
    return (f & ~15u) == 0 && (!(f & KDA_GATE_SOFTPLUS) || (f & KDA_GATE_IN_KERNEL));
}
int elem_bytes(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

bool gmin_ok(float g_min) { return isfinite(g_min) && g_min < 0.0f; }
// the bound g_min is used by the bounded in-kernel gate only
bool gate_ok(float g_min, unsigned f) {
    if ((f & KDA_GATE_IN_KERNEL) && (f & KDA_GATE_SOFTPLUS)) return true;
    return gmin_ok(g_min);
}
// The chunked forward factors each 16-token tile's decay into two products
// that stay in range only while kda_safe_chunk_size(g_min, dt) >= 16; a
// stronger bounded gate, like the unbounded one and caller-supplied decays,
// takes the kernel that evaluates out-of-range tiles element by element.
bool wide_decay(float g_min, unsigned f, kda_dtype dt) {
    if (!(f & KDA_GATE_IN_KERNEL) || (f & KDA_GATE_SOFTPLUS)) return true;
    return kda_safe_chunk_size(g_min, dt) < kFactorTile;
}

// Checks a pointer that must be present; optional ones pass when NULL.
kda_status need(const void* p) {
    if (!p) return KDA_ERR_NULL;
    return aligned16(p) ? KDA_OK : KDA_ERR_ALIGN;
}
kda_status maybe(const void* p) { return (!p || aligned16(p)) ? KDA_OK : KDA_ERR_ALIGN; }

// Sizes the kernels index with 32-bit arithmetic: at most 2^24 (b, h) pairs,
// 2^30 tokens and 2^46 / 128 token rows.
bool sizes_ok(long long B, long long T, long long H) {
    if (B < 0 || T < 0 || H < 0) return false;
    const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
    return bh <= (1ull << 24) && T <= (1ll << 30) && bh * (unsigned long long)T * 128ull <= (1ull << 46);
}
int chunks_of(int T, int chunk) { return (int)(((long long)T + chunk - 1) / chunk); }

// Byte ranges [a, a + na) and [b, b + nb) share a byte (both non-empty).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

#define KDA_TRY(expr)                        \
    do {                                     \
        const kda_status st_ = (expr);       \
        if (st_ != KDA_OK) return st_;       \
    } while (0)

}  // namespace

extern "C" {

int kda_safe_chunk_size(float g_min, kda_dtype dt) {
    if (!gmin_ok(g_min) || !dtype_ok(dt)) return -1;
    const double mx = dt == KDA_BF16 ? kBf16Max : kF32Max;
    const double v = log(mx / kHeadroom) / (-(double)g_min);
    if (v >= 2147483647.0) return 2147483647;  // a vanishing bound: any tile is safe
    return v < 0 ? 0 : (int)floor(v);
}

static size_t workspace_bytes_impl(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt) {
    if (chunk == 0) chunk = 64;
    if (!sizes_ok(B, T, H) || !dim_ok(Dk) || !dim_ok(Dv) || !dtype_ok(dt)) return 0;
    if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
    if ((size_t)B * H == 0) return 0;
    const int BH = B * H, NC = chunks_of(T, chunk);
    const size_t blk = kda::block_layout(elem_bytes(dt), Dk, chunk).bytes;
    const int per = kda::slice_chunks(BH, NC, blk);
    return kda::chunk_workspace_bytes(elem_bytes(dt), Dk, Dv, chunk, (size_t)BH, (size_t)per, 1);
}

size_t kda_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt) {
    return workspace_bytes_impl(B, T, H, Dk, Dv, chunk, dt);
}

static size_t layer_workspace_impl(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt) {
    if (workspace_bytes_impl(B, T, H, Dk, Dv, chunk, dt) == 0) return 0;
    if (chunk == 0) chunk = 64;
    const int BH = B * H, NC = chunks_of(T, chunk);
    const size_t blk = kda::block_layout(elem_bytes(dt), Dk, chunk).bytes;
    const int per = kda::slice_chunks(BH, NC, blk);
    return kda::layer_workspace_bytes(elem_bytes(dt), Dk, Dv, chunk, (size_t)BH, (size_t)per);
}

size_t kda_layer_fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt) {
    return layer_workspace_impl(B, T, H, Dk, Dv, chunk, dt);
}

}  // extern "C"

static kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* S0,
                                 void* o, float* S_out, float* M_out, void* P_out,
                                 int B, int T, int H, int Dk, int Dv, int chunk,
                                 float g_min, unsigned flags, kda_dtype dt,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t* ev, int n_ev,
                                 int G = 1, const float* dt_bias = nullptr, bool noalloc = false,
                                 const float* conv_w = nullptr, const float* conv_b = nullptr,
                                 const void* conv_state = nullptr,
                                 const void* gate = nullptr, const float* gate_w = nullptr) {
    if (!dtype_ok(dt) || !flags_ok(flags)) return KDA_ERR_DTYPE;
    if (dt_bias && !(flags & KDA_GATE_IN_KERNEL)) return KDA_ERR_DTYPE;  // it biases the in-kernel gate
    if (chunk == 0) chunk = 64;
    if (B < 0 || T < 0 || H < 0 || !dim_ok(Dk) || !dim_ok(Dv)) return KDA_ERR_SHAPE;
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_SHAPE;
    if (!gate_ok(g_min, flags)) return KDA_ERR_GATE;
    if (!sizes_ok(B, T, H)) return KDA_ERR_SHAPE;
    if (B == 0 || H == 0) return KDA_OK;
    if (T > 0) {
        KDA_TRY(need(q)); KDA_TRY(need(k)); KDA_TRY(need(v)); KDA_TRY(need(z));
        KDA_TRY(need(beta_raw)); KDA_TRY(need(o));
        if (flags & KDA_GATE_IN_KERNEL) KDA_TRY(need(A_log));
        else KDA_TRY(maybe(A_log));
    }
    KDA_TRY(maybe(S0)); KDA_TRY(maybe(S_out)); KDA_TRY(maybe(M_out)); KDA_TRY(maybe(P_out));
    KDA_TRY(maybe(dt_bias));
    if (conv_w) { KDA_TRY(maybe(conv_b)); KDA_TRY(maybe(conv_state)); }
    if (gate) {
        // the layer body: y (in the o slot) is written while other workgroups
        // still read the inputs, so it may share no byte with any of them
        KDA_TRY(maybe(gate_w));
        const size_t eb = (size_t)elem_bytes(dt);
        const size_t rows = (size_t)B * T * H;
        const size_t ny = rows * Dv * eb;
        const struct { const void* p; size_t n; } ins[] = {
            {q, rows * Dk * eb}, {k, rows * Dk * eb}, {v, ny}, {z, rows * Dk * eb}, {beta_raw, rows * eb},
            {gate, ny}, {gate_w, gate_w ? (size_t)Dv * 4 : 0}, {A_log, A_log ? (size_t)H * 4 : 0},
            {S0, S0 ? (size_t)B * H * Dk * Dv * 4 : 0}, {S_out, S_out ? (size_t)B * H * Dk * Dv * 4 : 0},
            {workspace, workspace_bytes}};
        for (const auto& in : ins)
            if (in.p && overlaps(o, ny, in.p, in.n)) return KDA_ERR_SHAPE;
    }
    size_t slice_budget = kda::kSliceBytes;
    if (noalloc) {
        // one chunk block of every (b, h) and the carried state must fit the
        // built-in scratch; the sequence is then cut into slices that fit
        const size_t carry = kda::round_up((size_t)B * H * Dk * (Dk + Dv) * 4, 256);
        const size_t blk = kda::block_layout(elem_bytes(dt), Dk, chunk).bytes;
        if (carry + (size_t)B * H * blk > kda::kScratchBytes) return KDA_ERR_SCRATCH;
        if (kda::scratch_pointer(&workspace) != hipSuccess) return KDA_ERR_HIP;
        workspace_bytes = kda::kScratchBytes;
        slice_budget = kda::kScratchBytes - carry;
    }
    const size_t ws_need = noalloc ? 0
                           : gate ? layer_workspace_impl(B, T, H, Dk, Dv, chunk, dt)
                                  : workspace_bytes_impl(B, T, H, Dk, Dv, chunk, dt);
    if (ws_need > 0) {
        if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
            workspace_bytes < ws_need)
            return KDA_ERR_WORKSPACE;
    }
    kda::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta_raw = beta_raw; a.A_log = A_log; a.S0 = S0;
    a.o = o; a.S_out = S_out; a.M_out = M_out; a.P_out = P_out; a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.B = B; a.T = T; a.H = H; a.Dv = Dv; a.NC = chunks_of(T, chunk);
    a.g_min = g_min; a.flags = flags;
    a.G = G; a.dt_bias = dt_bias;
    a.wide_decay = wide_decay(g_min, flags, dt);
    a.slice_budget = slice_budget;
    a.conv_w = conv_w; a.conv_b = conv_b; a.conv_state = conv_state;
    a.gate = gate; a.gate_w = gate_w;
    if (gate) {
        const hipError_t e = kda::launch_layer(dt == KDA_BF16 ? 1 : 0, Dk, chunk, a, stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (ev) {
        const int need = kda::chunk_kernel_count(elem_bytes(dt), Dk, chunk, B * H, a.NC) + 1;
        if (n_ev < need) return KDA_ERR_NULL;
        for (int i = 0; i < need; ++i)
            if (!ev[i]) return KDA_ERR_NULL;
    }
    const hipError_t e = kda::launch_chunk(dt == KDA_BF16 ? 1 : 0, Dk, chunk, a, stream, ev, n_ev);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         void* o, float* S_out, float* M_out, void* P_out,
                         int B, int T, int H, int Dk, int Dv, int chunk,
                         float g_min, unsigned flags, kda_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, o, S_out, M_out, P_out, B, T, H, Dk, Dv,
                          chunk, g_min, flags, dt, workspace, workspace_bytes, stream, nullptr, 0);
}

kda_status kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* z,
                               const void* beta_raw, const float* A_log, const float* S0,
                               void* o, float* S_out, float* M_out, void* P_out,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               float g_min, unsigned flags, kda_dtype dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream,
                               hipEvent_t* events, int n_events) {
    if (!events) return KDA_ERR_NULL;
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, o, S_out, M_out, P_out, B, T, H, Dk, Dv,
                          chunk, g_min, flags, dt, workspace, workspace_bytes, stream, events, n_events);
}

kda_status kda_chunk_fwd_conv(const void* q, const void* k, const void* v, const void* z,
                              const void* beta_raw, const float* A_log, const float* S0,
                              const float* conv_w, const float* conv_b, const void* conv_state,
                              void* o, float* S_out, int B, int T, int H, int Dk, int Dv, int chunk,
                              float g_min, unsigned flags, kda_dtype dt,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B > 0 && H > 0) KDA_TRY(need(conv_w));
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, o, S_out, nullptr, nullptr, B, T, H, Dk, Dv,
                          chunk, g_min, flags, dt, workspace, workspace_bytes, stream, nullptr, 0, 1, nullptr, false,
                          conv_w, conv_b, conv_state);
}

kda_status kda_layer_fwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         const float* conv_w, const float* conv_b, const void* conv_state,
                         const void* gate, const float* gate_weight,
                         void* y, float* S_out, int B, int T, int H, int Dk, int Dv, int chunk,
                         float g_min, unsigned flags, kda_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B > 0 && H > 0 && T > 0) KDA_TRY(need(gate));
    // with T = 0 nothing reads the gate: y stands in for it so that the call
    // still takes the layer path (its workspace and validation)
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, y, S_out, nullptr, nullptr, B, T, H, Dk, Dv,
                          chunk, g_min, flags, dt, workspace, workspace_bytes, stream, nullptr, 0, 1, nullptr, false,
                          conv_w, conv_b, conv_state, gate ? gate : (const void*)y, gate_weight);
}

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* S0,
                                 void* o, float* S_out, float* M_out, void* P_out,
                                 int B, int T, int H, int Dk, int Dv, int chunk,
                                 float g_min, unsigned flags, kda_dtype dt, hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, o, S_out, M_out, P_out, B, T, H, Dk, Dv,
                          chunk, g_min, flags, dt, nullptr, 0, stream, nullptr, 0, 1, nullptr, true);
}

int kda_chunk_fwd_kernel_count(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt) {
    if (chunk == 0) chunk = 64;
    if (B <= 0 || H <= 0 || !sizes_ok(B, T, H) || !dim_ok(Dk) || !dim_ok(Dv) || !dtype_ok(dt)) return 0;
    if (chunk != 16 && chunk != 32 && chunk != 64) return 0;
    return kda::chunk_kernel_count(elem_bytes(dt), Dk, chunk, B * H, chunks_of(T, chunk));
}

}  // extern "C"

static kda_status step_impl(const void* q, const void* k, const void* v, const void* z,
                            const void* beta_raw, const float* A_log, const float* dt_bias, float* S, void* o,
                            int B, int H, int G, int Dk, int Dv, float g_min, unsigned flags,
                            kda_dtype dt, hipStream_t stream) {
    if (!dtype_ok(dt) || !flags_ok(flags)) return KDA_ERR_DTYPE;
    if (dt_bias && !(flags & KDA_GATE_IN_KERNEL)) return KDA_ERR_DTYPE;
    if (!sizes_ok(B, 1, H) || !dim_ok(Dk) || !dim_ok(Dv)) return KDA_ERR_SHAPE;
    if (!((flags & KDA_GATE_SOFTPLUS) || gmin_ok(g_min))) return KDA_ERR_GATE;
    if (B == 0 || H == 0) return KDA_OK;
    KDA_TRY(need(q)); KDA_TRY(need(k)); KDA_TRY(need(v)); KDA_TRY(need(z));
    KDA_TRY(need(beta_raw)); KDA_TRY(need(S)); KDA_TRY(need(o));
    if (flags & KDA_GATE_IN_KERNEL) KDA_TRY(need(A_log));
    else KDA_TRY(maybe(A_log));
    KDA_TRY(maybe(dt_bias));
    kda::StepArgs a{q, k, v, z, beta_raw, A_log, S, o, B, H, g_min, flags};
    a.G = G; a.dt_bias = dt_bias;
    return kda::launch_step(dt == KDA_BF16 ? 1 : 0, Dk, Dv, a, stream) == hipSuccess ? KDA_OK
                                                                                     : KDA_ERR_HIP;
}

extern "C" {

kda_status kda_step(const void* q, const void* k, const void* v, const void* z,
                    const void* beta_raw, const float* A_log, float* S, void* o,
                    int B, int H, int Dk, int Dv, float g_min, unsigned flags,
                    kda_dtype dt, hipStream_t stream) {
    return step_impl(q, k, v, z, beta_raw, A_log, nullptr, S, o, B, H, 1, Dk, Dv, g_min, flags, dt, stream);
}

// q/k head count Hk against HV value heads: HV a positive multiple of Hk.
static bool groups_ok(int Hk, int HV) { return Hk > 0 && HV >= Hk && HV % Hk == 0; }

kda_status kda_step_grouped(const void* q, const void* k, const void* v, const void* z,
                            const void* beta_raw, const float* A_log, const float* dt_bias,
                            float* S, void* o, int B, int H, int HV, int Dk, int Dv,
                            float g_min, unsigned flags, kda_dtype dt, hipStream_t stream) {
    if (B > 0 && !groups_ok(H, HV)) return KDA_ERR_SHAPE;
    return step_impl(q, k, v, z, beta_raw, A_log, dt_bias, S, o, B, HV, B > 0 ? HV / H : 1, Dk, Dv,
                     g_min, flags, dt, stream);
}

kda_status kda_chunk_fwd_grouped(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* dt_bias,
                                 const float* S0, void* o, float* S_out, float* M_out, void* P_out,
                                 int B, int T, int H, int HV, int Dk, int Dv, int chunk,
                                 float g_min, unsigned flags, kda_dtype dt,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B > 0 && !groups_ok(H, HV)) return KDA_ERR_SHAPE;
    return chunk_fwd_impl(q, k, v, z, beta_raw, A_log, S0, o, S_out, M_out, P_out, B, T, HV, Dk, Dv,
                          chunk, g_min, flags, dt, workspace, workspace_bytes, stream, nullptr, 0,
                          B > 0 ? HV / H : 1, dt_bias);
}

kda_status kda_segment_compose(int n_seg, const float* M, const float* S_tilde,
                               const float* S_in, float* S_prefix,
                               int B, int H, int Dk, int Dv, hipStream_t stream) {
    if (n_seg < 0 || !sizes_ok((long long)n_seg * B, 1, H) || !dim_ok(Dk) || !dim_ok(Dv)) return KDA_ERR_SHAPE;
    if (n_seg == 0 || B == 0 || H == 0) return KDA_OK;
    KDA_TRY(need(M)); KDA_TRY(need(S_tilde)); KDA_TRY(need(S_prefix)); KDA_TRY(maybe(S_in));
    // the waves of a (b, h) read M, S_tilde and S_in while others write S_prefix
    const size_t bh = (size_t)B * H;
    const size_t mb = (size_t)n_seg * bh * Dk * Dk * 4, sb = (size_t)n_seg * bh * Dk * Dv * 4;
    if (overlaps(S_prefix, sb, M, mb) || overlaps(S_prefix, sb, S_tilde, sb) ||
        (S_in && overlaps(S_prefix, sb, S_in, bh * Dk * Dv * 4)))
        return KDA_ERR_SHAPE;
    kda::ComposeArgs a{M, S_tilde, S_in, S_prefix, n_seg, B, H, Dv};
    return kda::launch_compose(Dk, a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward workspace: operators, chunk-start states, chunk-end adjoints, the
// per-chunk dA_log parts and, for grouped heads, the per-value-head q/k
// gradients and the per-chunk gate-bias parts; each region 256-byte aligned.
struct BwdWorkspace {
    size_t ops, states, adj, eu, w, dA, dqk, dbias, total;
};
static BwdWorkspace bwd_workspace(int B, int T, int HV, int Dk, int Dv, bool grouped, bool bias) {
    BwdWorkspace w{};
    const size_t NC = ((size_t)T + kda::kBwdChunk - 1) / kda::kBwdChunk;
    const size_t BHN = (size_t)B * HV * NC;
    w.ops = 0;
    w.states = kda::round_up(BHN * kda::bwd_op_bytes(4, Dk), 256);  // fp32 operands: the larger block
    w.adj = w.states + kda::round_up(BHN * Dk * Dv * 4, 256);
    w.eu = w.adj + kda::round_up(BHN * Dk * Dv * 4, 256);
    w.w = w.eu + kda::round_up(BHN * 2 * kda::kBwdChunk * Dv * 4, 256);
    w.dA = w.w + kda::round_up(BHN * kda::kBwdChunk * Dv * 4, 256);
    w.dqk = w.dA + kda::round_up(BHN * 4, 256);
    w.dbias = w.dqk + (grouped ? kda::round_up(2 * (size_t)B * T * HV * Dk * 4, 256) : 0);
    w.total = w.dbias + (bias ? kda::round_up(BHN * Dk * 4, 256) : 0);
    return w;
}

size_t kda_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv) {
    if (!sizes_ok(B, T, H) || !dim_ok(Dk) || !dim_ok(Dv)) return 0;
    return bwd_workspace(B, T, H, Dk, Dv, false, false).total;
}

size_t kda_chunk_bwd_grouped_workspace(int B, int T, int H, int HV, int Dk, int Dv, int with_bias) {
    if (!sizes_ok(B, T, H) || !sizes_ok(B, T, HV) || !dim_ok(Dk) || !dim_ok(Dv)) return 0;
    if (HV > 0 && !groups_ok(H, HV)) return 0;
    return bwd_workspace(B, T, HV, Dk, Dv, HV > H, with_bias != 0).total;
}

static kda_status chunk_bwd_impl(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* dt_bias,
                                 const float* S0, const void* dout, const float* dS_T,
                                 void* dq, void* dk, void* dv, void* dz, void* dbeta_raw,
                                 float* dA_log, float* ddt_bias, float* dS0,
                                 int B, int T, int H, int HV, int Dk, int Dv, float g_min, unsigned flags,
                                 kda_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!dtype_ok(dt) || !flags_ok(flags)) return KDA_ERR_DTYPE;
    if (dt_bias && !(flags & KDA_GATE_IN_KERNEL)) return KDA_ERR_DTYPE;  // it biases the in-kernel gate
    if (B < 0 || T < 0 || H < 0 || HV < 0 || !dim_ok(Dk) || !dim_ok(Dv)) return KDA_ERR_SHAPE;
    if (HV > 0 && !groups_ok(H, HV)) return KDA_ERR_SHAPE;
    if (!sizes_ok(B, T, HV)) return KDA_ERR_SHAPE;
    if (!gate_ok(g_min, flags)) return KDA_ERR_GATE;
    if (HV == 0) return KDA_OK;
    KDA_TRY(need(dA_log));
    if (dt_bias) { KDA_TRY(need(dt_bias)); KDA_TRY(need(ddt_bias)); }
    else KDA_TRY(maybe(ddt_bias));
    if (B > 0 && T > 0) {
        KDA_TRY(need(q)); KDA_TRY(need(k)); KDA_TRY(need(v)); KDA_TRY(need(z));
        KDA_TRY(need(beta_raw)); KDA_TRY(need(dout));
        KDA_TRY(need(dq)); KDA_TRY(need(dk)); KDA_TRY(need(dv)); KDA_TRY(need(dz));
        KDA_TRY(need(dbeta_raw));
    }
    if (flags & KDA_GATE_IN_KERNEL) KDA_TRY(need(A_log));
    else KDA_TRY(maybe(A_log));
    KDA_TRY(maybe(S0)); KDA_TRY(maybe(dS_T)); KDA_TRY(maybe(dS0));
    const BwdWorkspace w = bwd_workspace(B, T, HV, Dk, Dv, HV > H, dt_bias != nullptr);
    {
        // outputs may overlap neither an input, another output nor the workspace
        const size_t eb = (size_t)elem_bytes(dt), rows = (size_t)B * T, bhv = (size_t)B * HV;
        const struct { const void* p; size_t n; } in[] = {
            {q, rows * H * Dk * eb}, {k, rows * H * Dk * eb}, {v, rows * HV * Dv * eb},
            {z, rows * HV * Dk * eb}, {beta_raw, rows * HV * eb}, {A_log, (size_t)HV * 4},
            {dt_bias, (size_t)HV * Dk * 4}, {S0, bhv * Dk * Dv * 4}, {dout, rows * HV * Dv * eb},
            {dS_T, bhv * Dk * Dv * 4}, {workspace, w.total}};
        const struct { const void* p; size_t n; } out[] = {
            {dq, rows * H * Dk * eb}, {dk, rows * H * Dk * eb}, {dv, rows * HV * Dv * eb},
            {dz, rows * HV * Dk * eb}, {dbeta_raw, rows * HV * eb}, {dA_log, (size_t)HV * 4},
            {ddt_bias, dt_bias ? (size_t)HV * Dk * 4 : 0}, {dS0, bhv * Dk * Dv * 4}};
        for (const auto& o : out) {
            if (!o.p) continue;
            for (const auto& i : in)
                if (i.p && overlaps(o.p, o.n, i.p, i.n)) return KDA_ERR_SHAPE;
            for (const auto& o2 : out)
                if (&o2 != &o && o2.p && overlaps(o.p, o.n, o2.p, o2.n)) return KDA_ERR_SHAPE;
        }
    }
    if (w.total > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
                        workspace_bytes < w.total))
        return KDA_ERR_WORKSPACE;
    kda::BwdArgs a{};
    unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta_raw = beta_raw; a.A_log = A_log; a.S0 = S0;
    a.dout = dout; a.dS_T = dS_T;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dz = dz; a.dbeta_raw = dbeta_raw; a.dA_log = dA_log; a.dS0 = dS0;
    a.ops = ws + w.ops;
    a.states = reinterpret_cast<float*>(ws + w.states);
    a.adj = reinterpret_cast<float*>(ws + w.adj);
    a.eu = reinterpret_cast<float*>(ws + w.eu);
    a.w = reinterpret_cast<float*>(ws + w.w);
    // without the gate A_log may be NULL: the kernels still read a value (and
    // drop it) from a valid address, the workspace's
    if (!A_log) a.A_log = reinterpret_cast<const float*>(ws);
    a.dA_part = reinterpret_cast<float*>(ws + w.dA);
    a.B = B; a.T = T; a.H = HV; a.Dv = Dv; a.NC = chunks_of(T, kda::kBwdChunk);
    a.g_min = g_min; a.flags = flags;
    a.G = HV / (H > 0 ? H : 1);
    a.dt_bias = dt_bias;
    a.ddt_bias = ddt_bias;
    a.dqk_part = HV > H ? reinterpret_cast<float*>(ws + w.dqk) : nullptr;
    a.dbias_part = dt_bias ? reinterpret_cast<float*>(ws + w.dbias) : nullptr;
    return kda::launch_chunk_bwd(dt == KDA_BF16 ? 1 : 0, Dk, a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         const void* dout, const float* dS_T,
                         void* dq, void* dk, void* dv, void* dz, void* dbeta_raw,
                         float* dA_log, float* dS0,
                         int B, int T, int H, int Dk, int Dv, float g_min, unsigned flags,
                         kda_dtype dt, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return chunk_bwd_impl(q, k, v, z, beta_raw, A_log, nullptr, S0, dout, dS_T, dq, dk, dv, dz, dbeta_raw,
                          dA_log, nullptr, dS0, B, T, H, H, Dk, Dv, g_min, flags, dt, workspace,
                          workspace_bytes, stream);
}

kda_status kda_chunk_bwd_grouped(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* dt_bias,
                                 const float* S0, const void* dout, const float* dS_T,
                                 void* dq, void* dk, void* dv, void* dz, void* dbeta_raw,
                                 float* dA_log, float* ddt_bias, float* dS0,
                                 int B, int T, int H, int HV, int Dk, int Dv, float g_min, unsigned flags,
                                 kda_dtype dt, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return chunk_bwd_impl(q, k, v, z, beta_raw, A_log, dt_bias, S0, dout, dS_T, dq, dk, dv, dz, dbeta_raw,
                          dA_log, ddt_bias, dS0, B, T, H, HV, Dk, Dv, g_min, flags, dt, workspace,
                          workspace_bytes, stream);
}

kda_status kda_segment_fixup(int n_seg, const void* P, const float* S_in,
                             const float* S_prefix, void* o, int B, int T_seg,
                             int H, int Dk, int Dv, kda_dtype dt, hipStream_t stream) {
    if (!dtype_ok(dt)) return KDA_ERR_DTYPE;
    if (n_seg < 0 || B < 0 || !sizes_ok((long long)n_seg * B, T_seg, H) || !dim_ok(Dk) || !dim_ok(Dv))
        return KDA_ERR_SHAPE;
    if (n_seg == 0 || B == 0 || H == 0 || T_seg == 0) return KDA_OK;
    KDA_TRY(need(P)); KDA_TRY(need(o)); KDA_TRY(maybe(S_in));
    if (n_seg > 1) KDA_TRY(need(S_prefix));
    else KDA_TRY(maybe(S_prefix));
    kda::FixupArgs a{P, S_in, S_prefix, o, n_seg, B, T_seg, H, Dv};
    return kda::launch_fixup(dt == KDA_BF16 ? 1 : 0, Dk, a, stream) == hipSuccess ? KDA_OK
                                                                                  : KDA_ERR_HIP;
}

kda_status kda_short_conv(const void* x, const float* w, const float* bias,
                          const void* state_in, void* state_out, void* y,
                          int B, int T, int C, int silu, kda_dtype dt, hipStream_t stream) {
    if (!dtype_ok(dt)) return KDA_ERR_DTYPE;
    // channels counted as heads of at most 128 for the size bound
    if (C < 0 || C % 8 != 0 || !sizes_ok(B, T, C / 128 + 1)) return KDA_ERR_SHAPE;
    if (B == 0 || C == 0 || (T == 0 && !state_out)) return KDA_OK;
    KDA_TRY(need(w));
    KDA_TRY(maybe(state_in)); KDA_TRY(maybe(state_out));
    if (T > 0) { KDA_TRY(need(x)); KDA_TRY(need(y)); }
    const size_t eb = (size_t)elem_bytes(dt);
    const size_t xb = T > 0 ? (size_t)B * T * C * eb : 0, sb = (size_t)B * 3 * C * eb;
    // workgroups of different token tiles read x (and the window) while others
    // write y and the window out: no overlap, except the window updated in
    // place by a call whose tokens fit one tile
    if (overlaps(x, xb, y, xb)) return KDA_ERR_SHAPE;
    if (state_out && (overlaps(state_out, sb, x, xb) || overlaps(state_out, sb, y, xb))) return KDA_ERR_SHAPE;
    if (state_in && state_out && overlaps(state_in, sb, state_out, sb) &&
        (state_in != state_out || T > kda::short_conv_tile()))
        return KDA_ERR_SHAPE;
    kda::ShortConvArgs a{x, w, bias, state_in, state_out, y, B, T, C, silu ? 1 : 0};
    return kda::launch_short_conv(dt == KDA_BF16 ? 1 : 0, a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_gate(const void* o, const void* gate, const float* weight, void* y,
                           int B, int T, int H, int Dv, kda_dtype dt, hipStream_t stream) {
    if (!dtype_ok(dt)) return KDA_ERR_DTYPE;
    if (!sizes_ok(B, T, H) || !dim_ok(Dv)) return KDA_ERR_SHAPE;
    const size_t rows = (size_t)B * T * H;
    if (rows == 0) return KDA_OK;
    KDA_TRY(need(o)); KDA_TRY(need(gate)); KDA_TRY(need(y));
    // each element is read before it is written, so y may be o or gate
    // itself, but not a shifted view of either
    const size_t nb = rows * Dv * (size_t)elem_bytes(dt);
    if ((y != o && overlaps(y, nb, o, nb)) || (y != gate && overlaps(y, nb, gate, nb))) return KDA_ERR_SHAPE;
    kda::GateArgs a{o, gate, weight, y, rows};
    return kda::launch_output_gate(dt == KDA_BF16 ? 1 : 0, Dv, a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "unsupported or negative size";
        case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KDA_ERR_DTYPE: return "unknown dtype or switch bits";
        case KDA_ERR_GATE: return "g_min is not finite and negative";
        case KDA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case KDA_ERR_HIP: return "kernel launch failed";
        case KDA_ERR_SCRATCH: return "the sizes need more than the built-in scratch of kda_chunk_fwd_noalloc";
    }
    return "unknown status";
}

}  // extern "C"
