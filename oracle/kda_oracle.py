"""fp64 CPU oracle for the Kimi Delta Attention (KDA) gated delta rule.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP path (no kernels, headers, helpers or constants) and imports nothing
from the product package.

Everything here is plain, slow and written to be checked by eye against the
pages it follows.  Citations name the page by its title and the section:

  [KDA-demo]     "【轻量化复刻大模型 / KIMI K3】KDA 模块交互式演示"
  [LinAttn-demo] "【轻量化复刻大模型】线性注意力交互式演示"
  [KDA-layer]    "KDAAttention 层" (notes, sec-05)
  [Impl-KDA]     "Implémenter KDA"

Layouts follow the pages' tensor statement ([LinAttn-demo] §1.2 "总体公式";
[KDA-layer] "完整数据流"): q, k, z are [B, T, H, Dk]; v is [B, T, H, Dv];
beta is [B, T, H]; A_log is [H]; states are [B, H, Dk, Dv].  All arithmetic
is float64.

Readings taken where the pages are silent or disagree (each also listed in
the design notes):
  * decay is applied BEFORE the delta erase ([Impl-KDA] "La forme récurrente
    de référence" and its first pitfall), although [KDA-demo] §1.3 and
    [LinAttn-demo] Eq. 1 write the erase against the un-decayed state;
  * the readout uses the post-update state, o_t = S_t^T q_t, with no 1/sqrt(Dk)
    scale ([KDA-demo] §1.3; [Impl-KDA] third pitfall);
  * the gate is g = g_min * sigmoid(exp(A_log[h]) * z) ([LinAttn-demo] Eq. 8,
    [Impl-KDA] "La décroissance bornée"; the parenthesis in [KDA-demo] §1.4 is
    garbled);
  * L2 normalisation divides by sqrt(sum x^2 + eps) with eps = 1e-6 (the
    pages give no epsilon);
  * the KDA v1 gate (switch bit 8) is g = -exp(A_log) * softplus(z): the form
    [Impl-KDA] states and the one whose dalpha/dz minimum (-1/4 at z = 0 for
    A_log = 0) [LinAttn-demo] Tab 3 plots; Eq. 7 of [LinAttn-demo], with
    exp(A_log) added inside the softplus, would move that minimum to z = -1;
  * with a switch off ([KDA-layer] "三个 in_kernel 开关") the caller supplies
    the activated quantity itself: the normalised q/k, beta in (0, 1), or the
    log-decay g in place of the gate logit z.

Every function below is pinned by tests that do not retype it (closed forms,
the pages' limit cases, exact rational arithmetic, the KCP identity and the
chunkwise form); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Switch bits, mirroring the three "in kernel" switches of [KDA-layer].
QK_L2NORM = 1
BETA_SIGMOID = 2
GATE_IN_KERNEL = 4
FLAGS_DEFAULT = QK_L2NORM | BETA_SIGMOID | GATE_IN_KERNEL
GATE_SOFTPLUS = 8  # with GATE_IN_KERNEL: the unbounded KDA v1 gate instead of the bounded one

G_MIN_DEFAULT = -5.0  # gate lower bound, [Impl-KDA] "La décroissance bornée"
L2_EPS = 1e-6


# ---------------------------------------------------------------------------
# Gates and normalisation
# ---------------------------------------------------------------------------

def sigmoid(x):
    """Logistic function in float64 ([KDA-layer] switch 2; [Impl-KDA])."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def l2_normalize(x, eps=L2_EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis ([KDA-demo] §1.3: q and k are
    L2-normalised; [KDA-layer] switch 1)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def bounded_log_decay(z, A_log, g_min=G_MIN_DEFAULT):
    """Bounded log-decay g = g_min * sigmoid(exp(A_log[h]) * z) per Dk channel.

    [LinAttn-demo] §1.2 Eq. 8 and [Impl-KDA] "La décroissance bornée".
    z is [..., H, Dk]; A_log is [H].  The result lies in (g_min, 0), so the
    retention alpha = exp(g) lies in (exp(g_min), 1).
    """
    z = np.asarray(z, dtype=np.float64)
    scale = np.exp(np.asarray(A_log, dtype=np.float64))[:, None]  # [H, 1]
    return g_min * sigmoid(scale * z)


def softplus(x):
    """log(1 + e^x) in float64, written as max(x, 0) + log1p(e^-|x|) so that
    neither tail overflows."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def softplus_log_decay(z, A_log):
    """The KDA v1 (Kimi Linear) gate g = -exp(A_log[h]) * softplus(z), per Dk
    channel ([Impl-KDA] "La décroissance bornée", which states the v1 form it
    replaces; [LinAttn-demo] Tab 3 plots alpha = exp(-softplus(z)) at A_log = 0
    and its gating paragraph writes g = -softplus(z)).
    Unbounded below: alpha = exp(g) reaches any value in (0, 1).  z is
    [..., H, Dk]; A_log is [H]."""
    z = np.asarray(z, dtype=np.float64)
    scale = np.exp(np.asarray(A_log, dtype=np.float64))[:, None]  # [H, 1]
    return -scale * softplus(z)


def prepare(q, k, z, beta_raw, A_log, g_min=G_MIN_DEFAULT, flags=FLAGS_DEFAULT):
    """Apply the switched activations of [KDA-layer] "chunk_kda 内部做了什么":
    L2-normalise q and k, squash beta by a sigmoid, and turn the gate logit
    into the bounded log-decay.  Returns (q_hat, k_hat, g, beta)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    beta_raw = np.asarray(beta_raw, dtype=np.float64)
    if flags & QK_L2NORM:
        q = l2_normalize(q)
        k = l2_normalize(k)
    beta = sigmoid(beta_raw) if flags & BETA_SIGMOID else beta_raw
    if flags & GATE_IN_KERNEL:
        g = softplus_log_decay(z, A_log) if flags & GATE_SOFTPLUS else bounded_log_decay(z, A_log, g_min)
    else:
        g = z
    return q, k, g, beta


# ---------------------------------------------------------------------------
# The recurrence (the plain definition)
# ---------------------------------------------------------------------------

def recurrent(q, k, v, g, beta, S0=None):
    """Token-by-token KDA recurrence; the definition every other form must meet.

    For each token, per (b, h) ([Impl-KDA] "La forme récurrente de référence",
    read with its pitfalls):
        S <- Diag(exp(g_t)) S            forget, channel by channel
        S <- S - beta_t k_t (k_t^T S)    erase the part aligned with k_t
        S <- S + beta_t k_t v_t^T        write the new association
        o_t = S^T q_t                    read the UPDATED state
    q, k, g: [B, T, H, Dk] (already activated); v: [B, T, H, Dv];
    beta: [B, T, H]; S0: [B, H, Dk, Dv] or None (zero state).
    Returns o [B, T, H, Dv] and the final state [B, H, Dk, Dv].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((B, T, H, Dv))
    for t in range(T):
        alpha = np.exp(g[:, t])                        # [B, H, Dk]
        S = alpha[..., None] * S                       # decay first
        kt = k[:, t]                                   # [B, H, Dk]
        proj = np.einsum("bhk,bhkv->bhv", kt, S)       # k^T S
        bt = beta[:, t][..., None]                     # [B, H, 1]
        S = S - kt[..., None] * (bt * proj)[..., None, :]
        S = S + kt[..., None] * (bt * v[:, t])[..., None, :]
        o[:, t] = np.einsum("bhk,bhkv->bhv", q[:, t], S)
    return o, S


def forward(q, k, v, z, beta_raw, A_log, S0=None, g_min=G_MIN_DEFAULT,
            flags=FLAGS_DEFAULT):
    """chunk_kda forward as a plain definition: switched activations
    ([KDA-layer]) followed by the recurrence.  Returns (o, S_final)."""
    qh, kh, g, beta = prepare(q, k, z, beta_raw, A_log, g_min, flags)
    return recurrent(qh, kh, v, g, beta, S0)


def step(S, q, k, v, z, beta_raw, A_log, g_min=G_MIN_DEFAULT, flags=FLAGS_DEFAULT):
    """One decode step ([KDA-demo] §1.7 lists kda_step as the single-token
    form of the core).  q, k, z: [B, H, Dk]; v: [B, H, Dv]; beta_raw: [B, H];
    S: [B, H, Dk, Dv].  Returns (o [B, H, Dv], S_new)."""
    o, S_new = forward(np.asarray(q)[:, None], np.asarray(k)[:, None],
                       np.asarray(v)[:, None], np.asarray(z)[:, None],
                       np.asarray(beta_raw)[:, None], A_log, S, g_min, flags)
    return o[:, 0], S_new


# ---------------------------------------------------------------------------
# Affine structure: transitions, segment fragments, composition (KCP)
# ---------------------------------------------------------------------------

def transition(k, beta, alpha):
    """Per-token transition M_t = (I - beta k k^T) Diag(alpha)
    ([Impl-KDA] Test 2, kda_transition).  k, alpha: [..., Dk]; beta: [...]."""
    k = np.asarray(k, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    Dk = k.shape[-1]
    eye = np.broadcast_to(np.eye(Dk), k.shape[:-1] + (Dk, Dk))
    proj = eye - beta[..., None, None] * (k[..., :, None] * k[..., None, :])
    return proj * alpha[..., None, :]          # right-multiply by Diag(alpha)


def segment_fragment(k, v, g, beta):
    """Fragment of one segment from a zero state ([Impl-KDA] Test 3):
    M = M_T ... M_1 (later tokens on the left) and S_tilde = run(segment, 0).
    Shapes as in `recurrent`; returns M [B,H,Dk,Dk], S_tilde [B,H,Dk,Dv]."""
    k = np.asarray(k, dtype=np.float64)
    B, T, H, Dk = k.shape
    q_dummy = np.zeros_like(k)
    _, S_tilde = recurrent(q_dummy, k, v, g, beta, None)
    M = np.broadcast_to(np.eye(Dk), (B, H, Dk, Dk)).copy()
    for t in range(T):
        Mt = transition(k[:, t], beta[:, t], np.exp(np.asarray(g)[:, t]))
        M = Mt @ M
    return M, S_tilde


def compose(fragments, S_in=None):
    """Prefix scan over segment fragments ([KDA-demo] §1.6; [Impl-KDA] Test 3):
    S <- M_s S + S_tilde_s for s = 1..n.  Returns the list of states after each
    segment.  fragments: sequence of (M, S_tilde) pairs."""
    out = []
    S = None
    for M, St in fragments:
        if S is None:
            S = np.zeros_like(St) if S_in is None else np.array(S_in, dtype=np.float64)
        S = M @ S + St
        out.append(S)
    return out


def compose_pair(second, first):
    """Associative composition law ([Impl-KDA] "La loi de composition
    associative"): (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2)."""
    M2, S2 = second
    M1, S1 = first
    return M2 @ M1, M2 @ S1 + S2


def readout_map(q, k, g, beta):
    """Readout map of one segment: P_t = q_t^T (M_t ... M_1), the row that the
    state before the segment reaches in o_t.  The recurrence is affine in its
    initial state ([Impl-KDA] 'Que teste réellement le test 2'), so a segment
    run from S0 reads o_t(S0) = o_t(0) + P_t S0 -- the output half of the
    KCP fix-up ([KDA-demo] §1.6).  q, k, g: [B, T, H, Dk]; beta: [B, T, H].
    Returns P [B, T, H, Dk]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T, H, Dk = k.shape
    M = np.broadcast_to(np.eye(Dk), (B, H, Dk, Dk)).copy()
    P = np.zeros((B, T, H, Dk))
    for t in range(T):
        M = transition(k[:, t], beta[:, t], np.exp(np.asarray(g)[:, t])) @ M
        P[:, t] = np.einsum("bhi,bhij->bhj", q[:, t], M)
    return P


def segment_fixup(o_zero, P, S_prefix, S_in=None):
    """Outputs of n segments run from their true incoming states: segment s
    reads o_zero[s] + P[s] S_prev, where S_prev is S_in (zero when None) for
    the first segment and the composed state after segment s - 1 otherwise.
    o_zero [n, B, Tseg, H, Dv]; P [n, B, Tseg, H, Dk]; S_prefix
    [n, B, H, Dk, Dv] (states after each segment, as `compose` returns)."""
    o_zero = np.asarray(o_zero, dtype=np.float64)
    out = o_zero.copy()
    for s in range(o_zero.shape[0]):
        if s == 0:
            if S_in is None:
                continue
            S_prev = np.asarray(S_in, dtype=np.float64)
        else:
            S_prev = np.asarray(S_prefix[s - 1], dtype=np.float64)
        out[s] += np.einsum("bthk,bhkv->bthv", np.asarray(P[s], dtype=np.float64), S_prev)
    return out


# ---------------------------------------------------------------------------
# Chunkwise form (model of the chunk algebra; used only to pin recurrent == chunk)
# ---------------------------------------------------------------------------

def chunkwise(q, k, v, g, beta, S0=None, chunk=64):
    """Chunkwise-parallel evaluation ([KDA-demo] §1.5 Eqs. 3-4, generalised to
    carry decay and the incoming state as in [Impl-KDA] "La forme par blocs",
    where the intra-chunk value is U - W S).

    Inside a chunk with incoming state S and local cumulative log-decay
    G_r = sum_{i<=r} g_i:
        A_kk[i, j] = beta_i sum_d k_id k_jd exp(G_id - G_jd)     (j <  i)
        A_qk[i, j] =        sum_d q_id k_jd exp(G_id - G_jd)     (j <= i)
        (I + A_kk) U = Diag(beta) (V - (K * exp(G)) S)           UT solve
        O = (Q * exp(G)) S + A_qk U
        S <- Diag(exp(G_C)) S + (K * exp(G_C - G))^T U
    The decay factors are formed element-wise from differences of G (never as
    1/gamma), so this model cannot overflow.  Shapes as in `recurrent`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    S = np.zeros((B, H, Dk, Dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((B, T, H, Dv))
    for b in range(B):
        for h in range(H):
            Sbh = S[b, h]
            for c0 in range(0, T, chunk):
                c1 = min(c0 + chunk, T)
                Q = q[b, c0:c1, h]
                K = k[b, c0:c1, h]
                V = v[b, c0:c1, h]
                bt = beta[b, c0:c1, h]
                G = np.cumsum(g[b, c0:c1, h], axis=0)          # [n, Dk]
                n = c1 - c0
                diff = G[:, None, :] - G[None, :, :]            # G_i - G_j
                lower_eq = np.tril(np.ones((n, n), dtype=bool))
                diff = np.where(lower_eq[..., None], diff, -np.inf)
                decay = np.exp(diff)                            # 0 above diagonal
                Akk = bt[:, None] * np.einsum("id,jd,ijd->ij", K, K, decay)
                Akk = np.tril(Akk, -1)
                Aqk = np.einsum("id,jd,ijd->ij", Q, K, decay)
                gam = np.exp(G)
                rhs = bt[:, None] * (V - (K * gam) @ Sbh)
                U = np.linalg.solve(np.eye(n) + Akk, rhs)
                o[b, c0:c1, h] = (Q * gam) @ Sbh + Aqk @ U
                Kc = K * np.exp(G[-1][None, :] - G)
                Sbh = np.exp(G[-1])[:, None] * Sbh + Kc.T @ U
            S[b, h] = Sbh
    return o, S


# ---------------------------------------------------------------------------
# Chunk-size safety bound
# ---------------------------------------------------------------------------

def safe_chunk_size(g_min, dtype_max, headroom=2.0 ** 10):
    """Largest tile n whose factored inverse retention exp(-g_min * n) stays
    below dtype_max / headroom: floor(ln(dtype_max / headroom) / (-g_min))
    ([KDA-demo] §1.4 safe_chunk_size; the pages leave the headroom open, 2^10
    is this project's reading).  g_min must be negative and finite."""
    if not (math.isfinite(g_min) and g_min < 0):
        raise ValueError("g_min must be finite and negative")
    val = math.log(dtype_max / headroom) / (-g_min)
    return max(0, int(math.floor(val)))


# ---------------------------------------------------------------------------
# Input side of the layer: short convolution and SiLU
# ([KDA-demo] §1.1 "ShortConv" and §1.7 "KimiDeltaAttention 完整层";
#  [Impl-KDA] "La paramétrisation")
# ---------------------------------------------------------------------------

SHORT_CONV_KERNEL = 4  # [Impl-KDA] "La paramétrisation": short_conv(..., kernel=4)


def short_conv(x, w, bias=None, state=None):
    """Causal depthwise convolution over the token axis ([KDA-demo] §1.1):
    each channel c mixes its own current and K - 1 previous inputs.

    x is [B, T, C]; w is [C, K]; bias is [C] or None.  Tap j of channel c
    multiplies x[t - (K - 1) + j, c], so tap K - 1 is the current token.  The
    pages write the sum over lags with w[c, lag] but also state that setting
    the LAST tap to 1 and the others to 0 makes the layer a no-op; only this
    indexing (the causal conv1d convention) makes both true, and it is the
    reading taken here.
    state is [B, K - 1, C], the K - 1 inputs that precede t = 0 (oldest
    first), or None for the pages' left zero padding ([KDA-demo] §1.1
    因果性); it is how a sequence continues across calls and how the decode
    step keeps its sliding window ([KDA-demo] §1.1 单步 decode).
    Returns (y [B, T, C], state_out [B, K - 1, C]): state_out holds the last
    K - 1 inputs of (state, x)."""
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[1]
    prev = np.zeros((B, K - 1, C)) if state is None else np.asarray(state, dtype=np.float64)
    xp = np.concatenate([prev, x], axis=1)  # row i of xp is token i - (K - 1)
    y = np.zeros((B, T, C))
    for t in range(T):
        for j in range(K):
            y[:, t] += w[:, j] * xp[:, t + j]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y, xp[:, T:].copy()


def silu(x):
    """SiLU (Swish) x * sigmoid(x) ([KDA-demo] §1.7; [Impl-KDA] swish)."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def conv_silu(x, w, bias=None, state=None):
    """SiLU(ShortConv(x)) for one of q, k, v ([KDA-demo] §1.7: the short
    convolution first, then SiLU; the L2 norm of q and k follows inside the
    core through its switch).  Returns (y, state_out) as short_conv."""
    y, st = short_conv(x, w, bias, state)
    return silu(y), st


# ---------------------------------------------------------------------------
# Output side of the layer: per-head RMS normalisation and sigmoid gate
# ([KDA-demo] §1.7 "KimiDeltaAttention 完整层" last line; [Impl-KDA] "La porte
# de sortie de rang plein", kda_output without its final projection)
# ---------------------------------------------------------------------------

RMS_EPS = 1e-6  # the pages give none; the same epsilon as the L2 norm


def head_rms_norm(o, weight=None, eps=RMS_EPS):
    """o / sqrt(mean(o^2) + eps) over each head's Dv channels (the last axis),
    times an optional per-channel weight [Dv] shared by the heads
    ([Impl-KDA] kda_output: RMSNorm par tête)."""
    o = np.asarray(o, dtype=np.float64)
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def output_gate(o, gate, weight=None, eps=RMS_EPS):
    """sigmoid(gate) * HeadRMSNorm(o): the full-rank output gate applied to the
    normalised heads, before the output projection ([KDA-demo] §1.7;
    [Impl-KDA] kda_output).  o and gate are [B, T, H, Dv]."""
    return sigmoid(gate) * head_rms_norm(o, weight, eps)


# ---------------------------------------------------------------------------
# Variants: grouped value heads and a per-dimension gate bias
# ([KDA-layer] "完整数据流": q, k [B, T, H, K] against v, g, beta [B, T, HV, ...],
#  A_log [HV] and dt_bias [HV, K] in its parameter table)
# ---------------------------------------------------------------------------

def group_heads(x, HV):
    """Give each of the HV value heads its q/k head: value head hv reads head
    hv // (HV // H) of x [B, T, H, D] (consecutive groups; the pages fix the
    shapes, not the assignment, and this is the reading taken)."""
    x = np.asarray(x, dtype=np.float64)
    H = x.shape[2]
    if HV % H:
        raise ValueError("HV must be a multiple of H")
    return np.repeat(x, HV // H, axis=2)


def biased_logit(z, dt_bias):
    """The gate logit with the per-dimension bias dt_bias [HV, K] added before
    the bounded gate ([KDA-layer] parameter table: dt_bias, per-dim gate
    bias)."""
    z = np.asarray(z, dtype=np.float64)
    return z if dt_bias is None else z + np.asarray(dt_bias, dtype=np.float64)


def forward_grouped(q, k, v, z, beta_raw, A_log, dt_bias=None, S0=None, g_min=G_MIN_DEFAULT,
                    flags=FLAGS_DEFAULT):
    """The layer core with HV value heads sharing H q/k heads and an optional
    gate bias (meaningful only with the gate computed in-kernel).  Shapes:
    q, k [B, T, H, Dk]; v [B, T, HV, Dv]; z [B, T, HV, Dk]; beta_raw
    [B, T, HV]; A_log [HV]; dt_bias [HV, Dk] or None."""
    if dt_bias is not None and not flags & GATE_IN_KERNEL:
        raise ValueError("dt_bias biases the in-kernel gate")
    HV = np.asarray(v).shape[2]
    return forward(group_heads(q, HV), group_heads(k, HV), v, biased_logit(z, dt_bias), beta_raw, A_log,
                   S0, g_min, flags)


def step_grouped(S, q, k, v, z, beta_raw, A_log, dt_bias=None, g_min=G_MIN_DEFAULT, flags=FLAGS_DEFAULT):
    """One decode step of forward_grouped: q, k [B, H, Dk]; v [B, HV, Dv];
    z [B, HV, Dk]; beta_raw [B, HV]; S [B, HV, Dk, Dv]."""
    if dt_bias is not None and not flags & GATE_IN_KERNEL:
        raise ValueError("dt_bias biases the in-kernel gate")
    HV = np.asarray(v).shape[1]
    qg = group_heads(np.asarray(q)[:, None], HV)[:, 0]
    kg = group_heads(np.asarray(k)[:, None], HV)[:, 0]
    return step(S, qg, kg, v, biased_logit(z, dt_bias), beta_raw, A_log, g_min, flags)


# ---------------------------------------------------------------------------
# Backward: the adjoint of the recurrence (the gradient of a scalar loss)
# ---------------------------------------------------------------------------
#
# The pages give no derivation of the backward pass; it is the derivative of
# the recurrence above, written out token by token in reverse (reverse-mode
# differentiation of `recurrent` and `prepare`), and pinned by finite
# differences of the forward.  For a loss L with dL/do_t = do_t and
# dL/dS_T = dS_T, and per token (P = Diag(alpha) S_prev, r = P^T k,
# u = beta (v - r), S = P + k u^T, o = S^T q):
#
#   Lam   = dS + q do^T                  adjoint of S_t, readout included
#   dq_hat= S do
#   w     = Lam^T k                      adjoint of u
#   dbeta = w . (v - r);   dv = beta w;   dr = -beta w
#   dP    = Lam + k dr^T
#   dk_hat= Lam u + P dr
#   dg    = rowsum(dP * P)               (= d alpha * alpha: d alpha = rowsum(dP * S_prev))
#   dS    <- Diag(alpha) dP              adjoint of S_{t-1}

def l2_normalize_backward(x, dy, eps=L2_EPS):
    """Gradient through y = x / sqrt(sum x^2 + eps) over the last axis:
    dx = dy / n - x (x . dy) / n^3."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    return dy / n - x * np.sum(x * dy, axis=-1, keepdims=True) / n ** 3


def backward(q, k, v, z, beta_raw, A_log, do, dS_T=None, S0=None, g_min=G_MIN_DEFAULT,
             flags=FLAGS_DEFAULT):
    """Gradients of L = sum(do * o) + sum(dS_T * S_T) for (o, S_T) =
    forward(q, k, v, z, beta_raw, A_log, S0, g_min, flags).

    Shapes as in `forward`; do is [B, T, H, Dv], dS_T [B, H, Dk, Dv] or None.
    Returns a dict with dq, dk, dz [B,T,H,Dk], dv [B,T,H,Dv], dbeta_raw
    [B,T,H], dA_log [H] and dS0 [B,H,Dk,Dv].  With a switch off the gradient
    is the one of the activated quantity the caller passed in that slot."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    beta_raw = np.asarray(beta_raw, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    qh, kh, g, beta = prepare(q, k, z, beta_raw, A_log, g_min, flags)
    B, T, H, Dk = kh.shape
    Dv = v.shape[-1]

    # forward again, keeping the state before each token
    S = np.zeros((B, H, Dk, Dv)) if S0 is None else np.array(S0, dtype=np.float64)
    S_prev = np.zeros((T, B, H, Dk, Dv))
    for t in range(T):
        S_prev[t] = S
        P = np.exp(g[:, t])[..., None] * S
        r = np.einsum("bhk,bhkv->bhv", kh[:, t], P)
        u = beta[:, t][..., None] * (v[:, t] - r)
        S = P + kh[:, t][..., None] * u[..., None, :]

    dqh = np.zeros_like(qh)
    dkh = np.zeros_like(kh)
    dg = np.zeros_like(g)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dS = np.zeros((B, H, Dk, Dv)) if dS_T is None else np.array(dS_T, dtype=np.float64)
    for t in reversed(range(T)):
        alpha = np.exp(g[:, t])
        P = alpha[..., None] * S_prev[t]
        kt = kh[:, t]
        r = np.einsum("bhk,bhkv->bhv", kt, P)
        e = v[:, t] - r
        bt = beta[:, t][..., None]
        u = bt * e
        S_t = P + kt[..., None] * u[..., None, :]
        Lam = dS + qh[:, t][..., None] * do[:, t][..., None, :]
        dqh[:, t] = np.einsum("bhkv,bhv->bhk", S_t, do[:, t])
        w = np.einsum("bhkv,bhk->bhv", Lam, kt)
        dbeta[:, t] = np.sum(w * e, axis=-1)
        dv[:, t] = bt * w
        dr = -bt * w
        dP = Lam + kt[..., None] * dr[..., None, :]
        dkh[:, t] = np.einsum("bhkv,bhv->bhk", Lam, u) + np.einsum("bhkv,bhv->bhk", P, dr)
        dg[:, t] = np.sum(dP * P, axis=-1)
        dS = alpha[..., None] * dP

    dq = l2_normalize_backward(q, dqh) if flags & QK_L2NORM else dqh
    dk = l2_normalize_backward(k, dkh) if flags & QK_L2NORM else dkh
    dbeta_raw = dbeta * beta * (1.0 - beta) if flags & BETA_SIGMOID else dbeta
    scale = np.exp(A_log)[:, None]                      # [H, 1]
    if flags & GATE_IN_KERNEL:
        if flags & GATE_SOFTPLUS:                        # g = -e^A softplus(z)
            dz = dg * (-scale * sigmoid(z))
            dA = np.sum(dg * g, axis=(0, 1, 3))
        else:                                            # g = g_min sigmoid(e^A z)
            s = sigmoid(scale * z)
            dsz = dg * g_min * s * (1.0 - s)             # dL / d(e^A z)
            dz = dsz * scale
            dA = np.sum(dsz * scale * z, axis=(0, 1, 3))
    else:
        dz = dg
        dA = np.zeros(H)
    return {"dq": dq, "dk": dk, "dv": dv, "dz": dz, "dbeta_raw": dbeta_raw, "dA_log": dA, "dS0": dS}


def backward_grouped(q, k, v, z, beta_raw, A_log, do, dt_bias=None, dS_T=None, S0=None,
                     g_min=G_MIN_DEFAULT, flags=FLAGS_DEFAULT):
    """Gradients of forward_grouped: q, k [B, T, H, Dk] feed HV = G H value
    heads (value head hv reads q/k head hv // G) and dt_bias [HV, Dk] is
    added to the gate logit.  The gradient of a q/k head is the sum over the
    value heads that read it; the bias gradient is the logit gradient summed
    over batch and tokens.  Returns the dict of `backward` with dq, dk
    [B, T, H, Dk] and, with a bias, ddt_bias [HV, Dk]."""
    if dt_bias is not None and not flags & GATE_IN_KERNEL:
        raise ValueError("dt_bias biases the in-kernel gate")
    q = np.asarray(q, dtype=np.float64)
    B, T, H, Dk = q.shape
    HV = np.asarray(v).shape[2]
    g = backward(group_heads(q, HV), group_heads(k, HV), v, biased_logit(z, dt_bias), beta_raw, A_log, do,
                 dS_T, S0, g_min, flags)
    G = HV // H
    g["dq"] = g["dq"].reshape(B, T, H, G, Dk).sum(axis=3)
    g["dk"] = g["dk"].reshape(B, T, H, G, Dk).sum(axis=3)
    if dt_bias is not None:
        g["ddt_bias"] = g["dz"].sum(axis=(0, 1))
    return g
