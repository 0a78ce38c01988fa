/*
 * kda.h - C ABI of the MI355X (gfx950) Kimi Delta Attention core.
 *
 * The operation is the gated delta rule with a bounded per-channel decay:
 *
 *   g_t  = g_min * sigmoid(exp(A_log[h]) * z_t)      per Dk channel
 *   S_t  = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   o_t  = S_t^T q_t
 *
 * with q, k L2-normalised and beta = sigmoid(beta_raw).  Decay is applied before
 * the delta erase and the readout uses the updated state ("Implémenter KDA",
 * 'La forme récurrente de référence' and its pitfalls).  The gate is the bounded
 * one of "线性注意力交互式演示" §1.2 Eq. 8 and "Implémenter KDA" 'La décroissance
 * bornée'.  The three switches mirror the in-kernel switches of "KDAAttention
 * 层", 'chunk_kda 内部做了什么'.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major buffers, 16-byte
 *    aligned.  Layouts: q, k, z [B,T,H,Dk]; v [B,T,H,Dv]; beta_raw [B,T,H];
 *    A_log [H] fp32; states [B,H,Dk,Dv] fp32; transitions [B,H,Dk,Dk] fp32.
 *    Decode tensors drop the T axis.  q, k, v, z, beta_raw and o share `dt`.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates, frees or synchronises; work is enqueued on `stream` (0 = null
 *    stream) and is asynchronous.
 *  - Arguments are validated on the host before anything is enqueued, so a
 *    rejected call writes nothing and makes no HIP call.  A failed launch
 *    returns KDA_ERR_HIP.  There is no global mutable state: concurrent calls
 *    are safe as long as they do not share output buffers or workspace.
 *  - Supported sizes: Dk, Dv in {16, 32, 64, 128}; chunk in {16, 32, 64}; any
 *    T >= 0 (a ragged tail chunk is padded with identity transitions).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,      /* a required pointer is NULL                         */
    KDA_ERR_SHAPE = 2,     /* unsupported or negative size, or bad chunk         */
    KDA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                   */
    KDA_ERR_DTYPE = 4,     /* unknown dtype or unknown switch bits               */
    KDA_ERR_GATE = 5,      /* g_min not finite or not negative (bounded gate)  */
    KDA_ERR_WORKSPACE = 6, /* workspace NULL, misaligned or too small           */
    KDA_ERR_HIP = 7,       /* a kernel launch failed                             */
    KDA_ERR_SCRATCH = 8    /* kda_chunk_fwd_noalloc: sizes beyond its scratch   */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Switch bits ("KDAAttention 层", 'three in_kernel switches'; all on by default).
 * With a bit clear the caller supplies the activated value in the same slot:
 * the already-normalised q/k, beta itself in place of beta_raw, or the
 * log-decay g (which must lie in [g_min, 0]) in place of the gate logit z.
 *
 * KDA_GATE_SOFTPLUS (only together with KDA_GATE_IN_KERNEL, KDA_ERR_DTYPE
 * otherwise) replaces the bounded gate by the unbounded KDA v1 gate
 * g = -exp(A_log[h]) * softplus(z) ("Implémenter KDA" 'La décroissance
 * bornée', the form the bounded gate replaces; "线性注意力交互式演示" Tab 3).
 * g_min is then not used.  The chunked form stays exact for any decay: a
 * 16-token block whose decay leaves the range of the factored products is
 * evaluated element by element in log space. */
enum {
    KDA_QK_L2NORM = 1u,
    KDA_BETA_SIGMOID = 2u,
    KDA_GATE_IN_KERNEL = 4u,
    KDA_FLAGS_DEFAULT = 7u,
    KDA_GATE_SOFTPLUS = 8u
};

/* Largest token tile whose factored inverse retention exp(-g_min * n) stays
 * below dtype_max / 2^10: floor(ln(dtype_max / 2^10) / -g_min)
 * ("KDA 模块交互式演示" §1.4 safe_chunk_size; Tab 9).  Returns 16 for g_min = -5
 * with either dtype, 8 for g_min = -10, and -1 for a non-finite or
 * non-negative g_min or an unknown dtype.  Host only; no HIP call.
 * kda_chunk_fwd factors the decay of 16-token tiles; when this returns less
 * than 16 for the call's bounded gate it evaluates every tile whose decay
 * leaves the factored range element by element (the path the unbounded v1
 * gate takes), so any finite negative g_min is accepted. */
int kda_safe_chunk_size(float g_min, kda_dtype dt);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 for invalid
 * sizes).  The workspace holds the per-chunk intermediates of the chunkwise
 * form and the state carried between slices; it must be 256-byte aligned.
 * Host only. */
size_t kda_chunk_fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk,
                               kda_dtype dt);

/* Chunkwise KDA forward ("KDA 模块交互式演示" §1.5 Eqs. 3-4 with the UT transform;
 * "Implémenter KDA" 'La forme par blocs').  Intra-chunk work is parallel,
 * the state is carried serially from chunk to chunk in fp32.
 *   S0     nullable: initial state [B,H,Dk,Dv] fp32; NULL means zero.
 *   o      [B,T,H,Dv], dtype dt (required when T > 0).
 *   S_out  nullable: final state [B,H,Dk,Dv] fp32; may alias S0 exactly.
 *   M_out  nullable: segment transition M = M_T ... M_1 [B,H,Dk,Dk] fp32 of the
 *          whole call ("Implémenter KDA" Test 2), for segment composition.
 *   P_out  nullable: correction rows [B,T,H,Dk], dtype dt, with
 *          o_t(S0) = o_t(0) + P_t S0 ("KDA 模块交互式演示" §1.6; the recurrence is
 *          affine in S0).  Requesting M_out or P_out doubles the state width.
 *   chunk  0 selects 64.
 * Returns KDA_OK or the first validation error. */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         void* o, float* S_out, float* M_out, void* P_out,
                         int B, int T, int H, int Dk, int Dv, int chunk,
                         float g_min, unsigned flags, kda_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Number of kernels one kda_chunk_fwd call launches for these sizes (0 for
 * invalid sizes).  The intra-chunk and inter-chunk kernels alternate over
 * slices of the sequence (one slice unless the per-chunk intermediates of
 * the whole sequence exceed 1 GiB); the workspace holds one slice.  Host only. */
int kda_chunk_fwd_kernel_count(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt);

/* Same computation and validation as kda_chunk_fwd, for measurement: events[0]
 * is recorded on `stream` before the first kernel and events[k + 1] after
 * kernel k (kernels alternate intra-chunk, inter-chunk), so the caller can time
 * each kernel with hipEventElapsedTime.  n_events must be at least
 * kda_chunk_fwd_kernel_count(...) + 1; KDA_ERR_NULL otherwise or if an event
 * is NULL. */
kda_status kda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* z,
                               const void* beta_raw, const float* A_log, const float* S0,
                               void* o, float* S_out, float* M_out, void* P_out,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               float g_min, unsigned flags, kda_dtype dt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream,
                               hipEvent_t* events, int n_events);

/* kda_chunk_fwd with the layer's input-side short convolution fused into it
 * ("KDA 模块交互式演示" §1.1 ShortConv and §1.7 完整层; "Implémenter KDA"
 * 'La paramétrisation'): q, k and v are the raw inputs of the convolution and
 * the core runs on
 *   x'[b,t,c] = SiLU(bias[c] + sum_{j=0..3} w[c,j] * x[b, t-3+j, c])
 * for each of q, k, v, with the values rounded to dt as if stored (so the
 * call equals kda_short_conv of each followed by kda_chunk_fwd, bit for bit).
 * The L2 norm of q', k' and every other switch act as in kda_chunk_fwd.
 *   conv_w      [H*Dk + H*Dk + H*Dv, 4] fp32 device: the taps of the q
 *               channels (head-major, [H][Dk]), then of the k channels, then
 *               of the v channels; tap 3 multiplies the current token.
 *   conv_b      [H*Dk + H*Dk + H*Dv] fp32 device (same channel order) or NULL.
 *   conv_state  [B, 3, H*Dk + H*Dk + H*Dv] dtype dt device or NULL (zeros):
 *               the three raw inputs before t = 0, oldest first (the window
 *               kda_short_conv hands on).  The window after the call is the
 *               last three raw inputs of (conv_state, x); the call does not
 *               write it.
 * Everything else as in kda_chunk_fwd without M_out and P_out (the same
 * workspace).  KDA_ERR_NULL without conv_w, KDA_ERR_ALIGN when conv_w,
 * conv_b or conv_state is not 16-byte aligned. */
kda_status kda_chunk_fwd_conv(const void* q, const void* k, const void* v, const void* z,
                              const void* beta_raw, const float* A_log, const float* S0,
                              const float* conv_w, const float* conv_b, const void* conv_state,
                              void* o, float* S_out, int B, int T, int H, int Dk, int Dv, int chunk,
                              float g_min, unsigned flags, kda_dtype dt,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The layer body without its projections ("KDA 模块交互式演示" §1.7
 * KimiDeltaAttention 完整层; "Implémenter KDA" 'La paramétrisation' and 'La
 * porte de sortie de rang plein'): the optional input-side convolution of
 * kda_chunk_fwd_conv, the chunkwise core of kda_chunk_fwd, and the output side
 * applied to each row of the core's output o before it is stored:
 *   y[b,t,h,c] = sigmoid(gate[b,t,h,c]) * o[b,t,h,c] * gate_weight[c]
 *                / sqrt(mean_c' o[b,t,h,c']^2 + 1e-6)
 * with o rounded to dt first (as kda_output_gate reads a stored o), so the
 * call equals kda_chunk_fwd(_conv) followed by kda_output_gate up to the
 * summation order of the norm.  o itself is never written to memory.
 *   conv_w, conv_b, conv_state  as in kda_chunk_fwd_conv; conv_w NULL: no
 *               convolution (q, k, v go to the core as given).
 *   gate        [B,T,H,Dv] dtype dt device (required when T > 0).
 *   gate_weight [Dv] fp32 device or NULL (ones), shared by the heads.
 *   y           [B,T,H,Dv] dtype dt device; it may overlap no input, S_out or
 *               the workspace (KDA_ERR_SHAPE).
 *   workspace   kda_layer_fwd_workspace bytes, 256-byte aligned: the chunk
 *               call's workspace plus an exchange area of 8 x chunk
 *               floats per chunk-head.
 * The workgroups that share a head's Dv channels exchange per-token partial
 * sums of squares through the workspace; when the device cannot hold all of
 * them at once the call runs the core into y and the output side over y in
 * place instead (same results).  The exchange counts on the device holding
 * the call's whole grid: calls of this entry point running at the same time
 * on one device (different streams) can share out its capacity so that
 * neither grid is whole, and their waits then run out after about a second
 * and write NaN rows; issue them in order on one stream.  Everything else as
 * kda_chunk_fwd without M_out and P_out. */
size_t kda_layer_fwd_workspace(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype dt);
kda_status kda_layer_fwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         const float* conv_w, const float* conv_b, const void* conv_state,
                         const void* gate, const float* gate_weight,
                         void* y, float* S_out, int B, int T, int H, int Dk, int Dv, int chunk,
                         float g_min, unsigned flags, kda_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, computation, validation and results as kda_chunk_fwd
 * without the workspace.  The per-chunk blocks and the state carried between
 * slices of the sequence live in a built-in device buffer of 64 MiB that every
 * GPU the library runs on holds until the process ends; the sequence is cut
 * into as many slices as that buffer requires.  The call allocates nothing
 * and calls no allocating routine; its first call on a device looks up that
 * device's buffer address.
 *   Limit: B * H * (blk + Dk * (Dk + Dv) * 4) <= 64 MiB, with blk the bytes
 *   of one chunk block (28 160 for bf16, Dk = 128, chunk 32; 59 904 at chunk
 *   64; 55 808 for fp32 at chunk 32), rounded as in kda_chunk_fwd_workspace;
 *   e.g. B * H <= 421 at Dk = Dv = 128, chunk 32, bf16.  Larger sizes return
 *   KDA_ERR_SCRATCH and enqueue nothing.
 *   Every call on a GPU uses that GPU's one buffer: calls that can overlap in
 *   time on one GPU (different streams, or host threads sharing a stream
 *   without ordering) race and give wrong results.  Calls issued in order on
 *   one stream are safe; nothing in the buffer needs to start at zero. */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* S0,
                                 void* o, float* S_out, float* M_out, void* P_out,
                                 int B, int T, int H, int Dk, int Dv, int chunk,
                                 float g_min, unsigned flags, kda_dtype dt, hipStream_t stream);

/* One decode step per (b,h), state updated IN PLACE ("KDA 模块交互式演示" §1.7
 * kda_step; "Implémenter KDA" reference step): decay, erase along k, write,
 * then read the updated state.  q, k, z [B,H,Dk]; v [B,H,Dv]; beta_raw [B,H];
 * S [B,H,Dk,Dv] fp32 in/out; o [B,H,Dv] dtype dt. */
kda_status kda_step(const void* q, const void* k, const void* v, const void* z,
                    const void* beta_raw, const float* A_log, float* S, void* o,
                    int B, int H, int Dk, int Dv, float g_min, unsigned flags,
                    kda_dtype dt, hipStream_t stream);

/* Grouped value heads and the per-dimension gate bias ("KDAAttention 层"
 * 完整数据流 and its parameter table: q, k [B,T,H,K]; v [B,T,HV,V]; g
 * [B,T,HV,K]; beta [B,T,HV]; A_log [HV]; dt_bias [HV,K]).  HV is a positive
 * multiple of H; value head hv reads q/k head hv / (HV / H).  Every other
 * argument is as in kda_chunk_fwd with H replaced by HV (z, beta_raw, A_log,
 * S0, o, S_out, M_out, P_out and the workspace, sized by
 * kda_chunk_fwd_workspace(B, T, HV, ...)).  dt_bias: [HV, Dk] fp32 device,
 * 16-byte aligned, added to z before the bounded gate, or NULL; it needs
 * KDA_GATE_IN_KERNEL (KDA_ERR_DTYPE otherwise).  KDA_ERR_SHAPE when HV is
 * not a positive multiple of H.  H == HV with dt_bias NULL is kda_chunk_fwd. */
kda_status kda_chunk_fwd_grouped(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* dt_bias,
                                 const float* S0, void* o, float* S_out, float* M_out, void* P_out,
                                 int B, int T, int H, int HV, int Dk, int Dv, int chunk,
                                 float g_min, unsigned flags, kda_dtype dt,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The decode step of kda_chunk_fwd_grouped: q, k [B,H,Dk]; v [B,HV,Dv]; z
 * [B,HV,Dk]; beta_raw [B,HV]; A_log [HV]; dt_bias [HV,Dk] or NULL; S
 * [B,HV,Dk,Dv] fp32 updated in place; o [B,HV,Dv]. */
kda_status kda_step_grouped(const void* q, const void* k, const void* v, const void* z,
                            const void* beta_raw, const float* A_log, const float* dt_bias,
                            float* S, void* o, int B, int H, int HV, int Dk, int Dv,
                            float g_min, unsigned flags, kda_dtype dt, hipStream_t stream);

/* Segment prefix scan ("KDA 模块交互式演示" §1.6 KCP; "Implémenter KDA" Test 3
 * and 'La loi de composition associative'): for s = 0..n_seg-1,
 *   S_prefix[s] = M[s] S_prev + S_tilde[s],  S_prev = (s ? S_prefix[s-1] : S_in).
 *   M [n_seg,B,H,Dk,Dk], S_tilde and S_prefix [n_seg,B,H,Dk,Dv], all fp32;
 *   S_in nullable [B,H,Dk,Dv] (NULL = zero).  S_prefix must not overlap the
 *   inputs (KDA_ERR_SHAPE). */
kda_status kda_segment_compose(int n_seg, const float* M, const float* S_tilde,
                               const float* S_in, float* S_prefix,
                               int B, int H, int Dk, int Dv, hipStream_t stream);

/* Output correction of segments run from a zero state (the affine split of
 * "Implémenter KDA" Test 2 applied to outputs): for every segment s and token t,
 *   o[s,b,t,h,:] += P[s,b,t,h,:] S_prev[s,b,h]   with
 *   S_prev[s] = (s ? S_prefix[s-1] : S_in)   (S_in NULL: segment 0 untouched).
 * P and o are segment-major [n_seg,B,T_seg,H,Dk] / [n_seg,B,T_seg,H,Dv] in dt
 * (a B = 1 sequence cut into equal segments already has this layout);
 * S_prefix [n_seg,B,H,Dk,Dv] fp32 as written by kda_segment_compose. */
kda_status kda_segment_fixup(int n_seg, const void* P, const float* S_in,
                             const float* S_prefix, void* o, int B, int T_seg,
                             int H, int Dk, int Dv, kda_dtype dt, hipStream_t stream);

/* The layer's input side for one of q, k, v ("KDA 模块交互式演示" §1.1
 * ShortConv and §1.7 完整层; "Implémenter KDA" 'La paramétrisation'): a causal
 * depthwise convolution of kernel 4 over the token axis, then SiLU when silu
 * is non-zero:
 *   y[b,t,c] = act(bias[c] + sum_{j=0..3} w[c,j] * x[b, t-3+j, c]).
 * Tap 3 multiplies the current token, so w[c] = (0,0,0,1) with no bias is the
 * identity the pages initialise to.
 *   x, y       [B,T,C] device, dtype dt, token-major (C = heads * head dim,
 *              the q/k/v layout above), C a multiple of 8; y must not
 *              overlap x.
 *   w          [C,4] fp32 device; bias [C] fp32 device or NULL (zero).
 *   state_in   [B,3,C] dtype dt device, the three inputs before t = 0, oldest
 *              first (a previous call's state_out), or NULL (zeros: the
 *              sequence starts here).
 *   state_out  [B,3,C] dtype dt device or NULL: receives the last three
 *              inputs of (state_in, x), the window the next call or the next
 *              decode token continues from.  It must not overlap x or y, and
 *              may be state_in itself (updated in place) only when T <= 32;
 *              otherwise it must not overlap state_in.
 * T = 0 copies state_in (or zeros) to state_out.  Errors: KDA_ERR_DTYPE,
 * KDA_ERR_SHAPE (negative size, C % 8, a forbidden overlap), KDA_ERR_NULL /
 * KDA_ERR_ALIGN (x, y, w, states: present and 16-byte aligned as required),
 * KDA_ERR_HIP.  Nothing is enqueued when an argument is rejected. */
kda_status kda_short_conv(const void* x, const float* w, const float* bias,
                          const void* state_in, void* state_out, void* y,
                          int B, int T, int C, int silu, kda_dtype dt, hipStream_t stream);

/* The layer's output side before its projection ("KDA 模块交互式演示" §1.7
 * 完整层; "Implémenter KDA" 'La porte de sortie de rang plein', kda_output):
 * per (b,t,h), over the head's Dv channels,
 *   y = sigmoid(gate) * o / sqrt(mean(o^2) + 1e-6) * weight[c].
 *   o, gate, y  [B,T,H,Dv] device, dtype dt; y may be o or gate itself (in
 *               place) but must not otherwise overlap them.
 *   weight      [Dv] fp32 device, shared by the heads, or NULL (ones).
 * Dv in {16,32,64,128}.  Errors: KDA_ERR_DTYPE, KDA_ERR_SHAPE (sizes, a
 * forbidden overlap), KDA_ERR_NULL / KDA_ERR_ALIGN (o, gate, y present and
 * 16-byte aligned), KDA_ERR_HIP.  Nothing is enqueued when an argument is
 * rejected. */
kda_status kda_output_gate(const void* o, const void* gate, const float* weight, void* y,
                           int B, int T, int H, int Dv, kda_dtype dt, hipStream_t stream);

/* Backward of kda_chunk_fwd (training).  The pages give the forward only; this
 * is its derivative, for a loss L with dL/do = dout and dL/dS_T = dS_T:
 *   dq, dk, dz [B,T,H,Dk] and dv [B,T,H,Dv], dbeta_raw [B,T,H]: device, dtype
 *              dt, the gradients with respect to the raw inputs through the
 *              switched activations (with a switch off, with respect to the
 *              activated quantity the caller passed in that slot);
 *   dA_log     [H] fp32 device: written (summed over batch and tokens; zero
 *              with the gate switch off);
 *   dS0        [B,H,Dk,Dv] fp32 device or NULL: the gradient with respect to
 *              the initial state.
 * Inputs as for kda_chunk_fwd (HV = H, no gate bias; every switch bit,
 * KDA_GATE_SOFTPLUS included); dout [B,T,H,Dv] dtype dt; dS_T [B,H,Dk,Dv]
 * fp32 or NULL (zero).  The arithmetic is fp32 in 32-token chunks, every decay
 * factor in one exponent (exact for any log-decay).  The workspace
 * (kda_chunk_bwd_workspace bytes, 256-byte aligned) holds the per-chunk
 * operators, the state at each chunk start and the state adjoint at each
 * chunk end.  Outputs may overlap neither an input, another output nor the
 * workspace (KDA_ERR_SHAPE).  Errors otherwise as kda_chunk_fwd. */
size_t kda_chunk_bwd_workspace(int B, int T, int H, int Dk, int Dv);
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* z,
                         const void* beta_raw, const float* A_log, const float* S0,
                         const void* dout, const float* dS_T,
                         void* dq, void* dk, void* dv, void* dz, void* dbeta_raw,
                         float* dA_log, float* dS0,
                         int B, int T, int H, int Dk, int Dv, float g_min, unsigned flags,
                         kda_dtype dt, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Backward of kda_chunk_fwd_grouped: q, k [B,T,H,Dk] read by HV = G H value
 * heads (value head hv reads q/k head hv / G), v, z, beta_raw, A_log, S0 and
 * dout per value head, dt_bias [HV,Dk] fp32 or NULL (added to the gate logit;
 * needs KDA_GATE_IN_KERNEL).  dq, dk [B,T,H,Dk] are the sums over the value
 * heads that read each q/k head; ddt_bias [HV,Dk] fp32 (required with a bias,
 * ignored without) is the logit gradient summed over batch and tokens; the
 * other outputs as kda_chunk_bwd, per value head.  Workspace:
 * kda_chunk_bwd_grouped_workspace(B, T, H, HV, Dk, Dv, dt_bias != NULL)
 * bytes (0 for invalid sizes).  Errors as kda_chunk_fwd_grouped. */
size_t kda_chunk_bwd_grouped_workspace(int B, int T, int H, int HV, int Dk, int Dv, int with_bias);
kda_status kda_chunk_bwd_grouped(const void* q, const void* k, const void* v, const void* z,
                                 const void* beta_raw, const float* A_log, const float* dt_bias,
                                 const float* S0, const void* dout, const float* dS_T,
                                 void* dq, void* dk, void* dv, void* dz, void* dbeta_raw,
                                 float* dA_log, float* ddt_bias, float* dS0,
                                 int B, int T, int H, int HV, int Dk, int Dv, float g_min, unsigned flags,
                                 kda_dtype dt, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
