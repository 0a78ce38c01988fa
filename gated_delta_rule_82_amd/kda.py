"""Thin Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the current
stream.  There is no fallback: if libkda.so is missing or a call is rejected,
an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
QK_L2NORM, BETA_SIGMOID, GATE_IN_KERNEL = 1, 2, 4
FLAGS_DEFAULT = 7
GATE_SOFTPLUS = 8  # with GATE_IN_KERNEL: the unbounded KDA v1 gate -exp(A_log) softplus(z)

EXPORTS = (
    "kda_safe_chunk_size", "kda_chunk_fwd_workspace", "kda_chunk_fwd", "kda_chunk_fwd_timed",
    "kda_chunk_fwd_kernel_count", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_conv", "kda_layer_fwd_workspace",
    "kda_layer_fwd", "kda_step", "kda_chunk_fwd_grouped", "kda_step_grouped",
    "kda_segment_compose", "kda_segment_fixup", "kda_short_conv", "kda_output_gate",
    "kda_chunk_bwd_workspace", "kda_chunk_bwd", "kda_chunk_bwd_grouped_workspace", "kda_chunk_bwd_grouped",
    "kda_status_string",
)

_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libkda.so and declare the prototypes (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_delta_rule_82_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, U, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
    L.kda_safe_chunk_size.argtypes = [F, I]
    L.kda_safe_chunk_size.restype = I
    L.kda_chunk_fwd_workspace.argtypes = [I, I, I, I, I, I, I]
    L.kda_chunk_fwd_workspace.restype = S
    L.kda_chunk_fwd.argtypes = [P] * 11 + [I] * 6 + [F, U, I, P, S, P]
    L.kda_chunk_fwd.restype = I
    L.kda_chunk_fwd_timed.argtypes = [P] * 11 + [I] * 6 + [F, U, I, P, S, P, P, I]
    L.kda_chunk_fwd_timed.restype = I
    L.kda_chunk_fwd_kernel_count.argtypes = [I] * 7
    L.kda_chunk_fwd_kernel_count.restype = I
    L.kda_chunk_fwd_noalloc.argtypes = [P] * 11 + [I] * 6 + [F, U, I, P]
    L.kda_chunk_fwd_noalloc.restype = I
    L.kda_chunk_fwd_conv.argtypes = [P] * 12 + [I] * 6 + [F, U, I, P, S, P]
    L.kda_chunk_fwd_conv.restype = I
    L.kda_layer_fwd_workspace.argtypes = [I, I, I, I, I, I, I]
    L.kda_layer_fwd_workspace.restype = S
    L.kda_layer_fwd.argtypes = [P] * 14 + [I] * 6 + [F, U, I, P, S, P]
    L.kda_layer_fwd.restype = I
    L.kda_step.argtypes = [P] * 8 + [I] * 4 + [F, U, I, P]
    L.kda_step.restype = I
    L.kda_segment_compose.argtypes = [I, P, P, P, P, I, I, I, I, P]
    L.kda_segment_compose.restype = I
    L.kda_segment_fixup.argtypes = [I, P, P, P, P, I, I, I, I, I, I, P]
    L.kda_segment_fixup.restype = I
    L.kda_short_conv.argtypes = [P] * 6 + [I] * 5 + [P]
    L.kda_short_conv.restype = I
    L.kda_output_gate.argtypes = [P] * 4 + [I] * 5 + [P]
    L.kda_output_gate.restype = I
    L.kda_chunk_fwd_grouped.argtypes = [P] * 12 + [I] * 7 + [F, U, I, P, S, P]
    L.kda_chunk_fwd_grouped.restype = I
    L.kda_step_grouped.argtypes = [P] * 9 + [I] * 5 + [F, U, I, P]
    L.kda_step_grouped.restype = I
    L.kda_chunk_bwd_workspace.argtypes = [I] * 5
    L.kda_chunk_bwd_workspace.restype = S
    L.kda_chunk_bwd.argtypes = [P] * 16 + [I] * 5 + [F, U, I, P, S, P]
    L.kda_chunk_bwd.restype = I
    L.kda_chunk_bwd_grouped_workspace.argtypes = [I] * 7
    L.kda_chunk_bwd_grouped_workspace.restype = S
    L.kda_chunk_bwd_grouped.argtypes = [P] * 18 + [I] * 6 + [F, U, I, P, S, P]
    L.kda_chunk_bwd_grouped.restype = I
    L.kda_status_string.argtypes = [I]
    L.kda_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().kda_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise KDAError(fn, status, status_string(status))


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors must be contiguous device tensors")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def safe_chunk_size(g_min: float = -5.0, dtype: torch.dtype = torch.bfloat16) -> int:
    return load().kda_safe_chunk_size(g_min, _dt(dtype))


def workspace_bytes(B, T, H, Dk, Dv, chunk=64, dtype=torch.bfloat16) -> int:
    return load().kda_chunk_fwd_workspace(B, T, H, Dk, Dv, chunk, _dt(dtype))


def kernel_count(B, T, H, Dk, Dv, chunk=64, dtype=torch.bfloat16) -> int:
    """Kernels one chunk_fwd call launches (intra and inter alternate over slices)."""
    return load().kda_chunk_fwd_kernel_count(B, T, H, Dk, Dv, chunk, _dt(dtype))


def _event_handles(events):
    for e in events:
        if e.cuda_event == 0:  # torch creates the HIP event on its first record
            e.record()
    return (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])


def chunk_fwd(q, k, v, z, beta_raw, A_log, S0=None, *, chunk=64, g_min=-5.0,
              flags=FLAGS_DEFAULT, want_M=False, want_P=False, o=None, S_out=None,
              M_out=None, P_out=None, workspace=None, events=None, dt_bias=None):
    """Chunkwise KDA forward.  Returns (o, S_out) plus M and/or P when asked.

    `events` (optional): a list of torch.cuda.Event(enable_timing=True), at
    least kernel_count(...) + 1 (kda_chunk_fwd_timed): events[0] is recorded
    before the first kernel and events[k + 1] after kernel k.
    Grouped value heads (v, z, beta_raw with HV = a multiple of q's H heads)
    or a gate bias `dt_bias` [HV, Dk] fp32 run kda_chunk_fwd_grouped.
    """
    B, T, Hq, Dk = q.shape
    H = v.shape[2]
    Dv = v.shape[-1]
    grouped = Hq != H or dt_bias is not None
    if grouped and events is not None:
        raise ValueError("grouped heads / dt_bias run the plain call only")
    dt = q.dtype
    dev = q.device
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=dt, device=dev)
    if S_out is None:
        S_out = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    if want_M and M_out is None:
        M_out = torch.empty(B, H, Dk, Dk, dtype=torch.float32, device=dev)
    if want_P and P_out is None:
        P_out = torch.empty(B, T, H, Dk, dtype=dt, device=dev)
    need = workspace_bytes(B, T, H, Dk, Dv, chunk, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(S0),
            _ptr(o), _ptr(S_out), _ptr(M_out), _ptr(P_out),
            B, T, H, Dk, Dv, chunk, g_min, flags, _dt(dt),
            _ptr(workspace), workspace.numel(), _stream(dev))
    if grouped:
        gargs = (_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias), _ptr(S0),
                 _ptr(o), _ptr(S_out), _ptr(M_out), _ptr(P_out),
                 B, T, Hq, H, Dk, Dv, chunk, g_min, flags, _dt(dt),
                 _ptr(workspace), workspace.numel(), _stream(dev))
        _check("kda_chunk_fwd_grouped", load().kda_chunk_fwd_grouped(*gargs))
    elif events is None:
        _check("kda_chunk_fwd", load().kda_chunk_fwd(*args))
    else:
        evs = _event_handles(events)
        _check("kda_chunk_fwd_timed", load().kda_chunk_fwd_timed(*args, evs, len(events)))
    out = [o, S_out]
    if want_M:
        out.append(M_out)
    if want_P:
        out.append(P_out)
    return tuple(out)


def chunk_fwd_conv(q, k, v, z, beta_raw, A_log, conv_w, conv_b=None, conv_state=None, S0=None, *, chunk=64,
                   g_min=-5.0, flags=FLAGS_DEFAULT, o=None, S_out=None, workspace=None):
    """kda_chunk_fwd_conv: the core on SiLU(ShortConv_4(.)) of the raw q, k, v.
    conv_w [H*(2 Dk + Dv), 4] fp32 (q channels, then k, then v), conv_b the
    same channels or None, conv_state [B, 3, H*(2 Dk + Dv)] in the input
    dtype or None.  Returns (o, S_out)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=dt, device=dev)
    if S_out is None:
        S_out = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    need = workspace_bytes(B, T, H, Dk, Dv, chunk, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("kda_chunk_fwd_conv",
           load().kda_chunk_fwd_conv(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(S0),
                                     _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(o), _ptr(S_out),
                                     B, T, H, Dk, Dv, chunk, g_min, flags, _dt(dt),
                                     _ptr(workspace), workspace.numel(), _stream(dev)))
    return o, S_out


def layer_workspace_bytes(B, T, H, Dk, Dv, chunk=64, dtype=torch.bfloat16) -> int:
    return int(load().kda_layer_fwd_workspace(B, T, H, Dk, Dv, chunk, _dt(dtype)))


def layer_fwd(q, k, v, z, beta_raw, A_log, gate, gate_weight=None, S0=None, *, conv_w=None, conv_b=None,
              conv_state=None, chunk=64, g_min=-5.0, flags=FLAGS_DEFAULT, y=None, S_out=None, workspace=None):
    """kda_layer_fwd: the layer body without its projections, with the output
    side sigmoid(gate) * HeadRMSNorm(o) * gate_weight applied inside the core's
    output stores (and the input-side convolution when conv_w is given, as in
    chunk_fwd_conv).  gate [B,T,H,Dv] in the input dtype, gate_weight [Dv] fp32
    or None.  Returns (y, S_out)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if y is None:
        y = torch.empty(B, T, H, Dv, dtype=dt, device=dev)
    if S_out is None:
        S_out = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    need = layer_workspace_bytes(B, T, H, Dk, Dv, chunk, dt)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check("kda_layer_fwd",
           load().kda_layer_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(S0),
                                _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(gate), _ptr(gate_weight),
                                _ptr(y), _ptr(S_out), B, T, H, Dk, Dv, chunk, g_min, flags, _dt(dt),
                                _ptr(workspace), workspace.numel(), _stream(dev)))
    return y, S_out


def chunk_fwd_noalloc(q, k, v, z, beta_raw, A_log, S0=None, *, chunk=64, g_min=-5.0,
                      flags=FLAGS_DEFAULT, want_M=False, want_P=False, o=None, S_out=None,
                      M_out=None, P_out=None):
    """kda_chunk_fwd_noalloc: chunk_fwd without a workspace (the library's
    built-in device scratch; calls on one GPU must not overlap in time).
    Outputs not passed are allocated here by torch, before the call."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    if o is None:
        o = torch.empty(B, T, H, Dv, dtype=dt, device=dev)
    if S_out is None:
        S_out = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    if want_M and M_out is None:
        M_out = torch.empty(B, H, Dk, Dk, dtype=torch.float32, device=dev)
    if want_P and P_out is None:
        P_out = torch.empty(B, T, H, Dk, dtype=dt, device=dev)
    _check("kda_chunk_fwd_noalloc",
           load().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(S0),
                                        _ptr(o), _ptr(S_out), _ptr(M_out), _ptr(P_out),
                                        B, T, H, Dk, Dv, chunk, g_min, flags, _dt(dt), _stream(dev)))
    out = [o, S_out]
    if want_M:
        out.append(M_out)
    if want_P:
        out.append(P_out)
    return tuple(out)


def step(q, k, v, z, beta_raw, A_log, S, *, g_min=-5.0, flags=FLAGS_DEFAULT, o=None, dt_bias=None):
    """One decode step; S [B,HV,Dk,Dv] fp32 is updated in place.  Returns o.
    q, k have H heads, v, z, beta_raw HV (a multiple of H; grouped heads and
    dt_bias run kda_step_grouped)."""
    B, Hq, Dk = q.shape
    H = v.shape[1]
    Dv = v.shape[-1]
    if o is None:
        o = torch.empty(B, H, Dv, dtype=q.dtype, device=q.device)
    if Hq != H or dt_bias is not None:
        st = load().kda_step_grouped(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log),
                                     _ptr(dt_bias), _ptr(S), _ptr(o), B, Hq, H, Dk, Dv, g_min, flags,
                                     _dt(q.dtype), _stream(q.device))
        _check("kda_step_grouped", st)
        return o
    st = load().kda_step(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log),
                         _ptr(S), _ptr(o), B, H, Dk, Dv, g_min, flags, _dt(q.dtype),
                         _stream(q.device))
    _check("kda_step", st)
    return o


def segment_compose(M, S_tilde, S_in=None, *, S_prefix=None):
    """Prefix scan S_s = M_s S_{s-1} + S_tilde_s; M [n,B,H,Dk,Dk], S_tilde [n,B,H,Dk,Dv]."""
    n, B, H, Dk, Dv = S_tilde.shape
    if S_prefix is None:
        S_prefix = torch.empty_like(S_tilde)
    st = load().kda_segment_compose(n, _ptr(M), _ptr(S_tilde), _ptr(S_in), _ptr(S_prefix),
                                    B, H, Dk, Dv, _stream(S_tilde.device))
    _check("kda_segment_compose", st)
    return S_prefix


def segment_fixup(P, S_prefix, o, S_in=None):
    """o[s] += P[s] @ S_prev[s] in place; P [n,B,Tseg,H,Dk], o [n,B,Tseg,H,Dv]."""
    n, B, Tseg, H, Dk = P.shape
    Dv = o.shape[-1]
    st = load().kda_segment_fixup(n, _ptr(P), _ptr(S_in), _ptr(S_prefix), _ptr(o), B, Tseg,
                                  H, Dk, Dv, _dt(P.dtype), _stream(P.device))
    _check("kda_segment_fixup", st)
    return o


def bwd_workspace_bytes(B, T, H, Dk, Dv):
    return load().kda_chunk_bwd_workspace(B, T, H, Dk, Dv)


def chunk_bwd(q, k, v, z, beta_raw, A_log, dout, S0=None, dS_T=None, *, g_min=-5.0, flags=FLAGS_DEFAULT,
              want_dS0=True, workspace=None, dt_bias=None):
    """Backward of chunk_fwd: gradients of L = sum(dout * o) + sum(dS_T * S_T).
    Returns a dict dq, dk, dv, dz, dbeta_raw (input dtype), dA_log [H] and,
    when asked, dS0 [B,H,Dk,Dv] (fp32).  Grouped value heads (v with more
    heads than q) or a gate bias `dt_bias` run kda_chunk_bwd_grouped, which
    adds ddt_bias [HV, Dk] (fp32) when a bias is given."""
    B, T, Hq, Dk = q.shape
    H = v.shape[2]
    Dv = v.shape[-1]
    dt = q.dtype
    dev = q.device
    grouped = Hq != H or dt_bias is not None
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dz": torch.empty_like(z), "dbeta_raw": torch.empty_like(beta_raw),
         "dA_log": torch.empty(H, dtype=torch.float32, device=dev)}
    g["dS0"] = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev) if want_dS0 else None
    if dt_bias is not None:
        g["ddt_bias"] = torch.empty(H, Dk, dtype=torch.float32, device=dev)
    if grouped:
        need = load().kda_chunk_bwd_grouped_workspace(B, T, Hq, H, Dk, Dv, 1 if dt_bias is not None else 0)
    else:
        need = bwd_workspace_bytes(B, T, H, Dk, Dv)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if grouped:
        st = load().kda_chunk_bwd_grouped(
            _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(dt_bias), _ptr(S0), _ptr(dout),
            _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dz"]), _ptr(g["dbeta_raw"]),
            _ptr(g["dA_log"]), _ptr(g.get("ddt_bias")), _ptr(g["dS0"]),
            B, T, Hq, H, Dk, Dv, g_min, flags, _dt(dt), _ptr(workspace), workspace.numel(), _stream(dev))
        _check("kda_chunk_bwd_grouped", st)
    else:
        st = load().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta_raw), _ptr(A_log), _ptr(S0),
                                  _ptr(dout), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dz"]),
                                  _ptr(g["dbeta_raw"]), _ptr(g["dA_log"]), _ptr(g["dS0"]),
                                  B, T, H, Dk, Dv, g_min, flags, _dt(dt), _ptr(workspace), workspace.numel(),
                                  _stream(dev))
        _check("kda_chunk_bwd", st)
    return g


def short_conv(x, w, bias=None, *, state_in=None, state_out=None, silu=True, y=None):
    """y = SiLU(ShortConv(x)) (silu=False: the convolution alone) for x [B,T,C]
    (or [B,T,H,D], flattened to C = H*D); w [C,4] fp32 (tap 3 is the current
    token), bias [C] fp32 or None.  state_in / state_out [B,3,C] in x's dtype
    carry the last three inputs between calls (state_out may be state_in when
    T <= 32).  Returns y shaped like x."""
    shape = x.shape
    B, T = shape[0], shape[1]
    C = 1
    for d in shape[2:]:
        C *= d
    if y is None:
        y = torch.empty_like(x)
    st = load().kda_short_conv(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(state_out), _ptr(y),
                               B, T, C, 1 if silu else 0, _dt(x.dtype), _stream(x.device))
    _check("kda_short_conv", st)
    return y


def output_gate(o, gate, weight=None, *, y=None):
    """y = sigmoid(gate) * HeadRMSNorm(o) * weight for o, gate [B,T,H,Dv];
    weight [Dv] fp32 or None.  y may be o or gate (in place)."""
    B, T, H, Dv = o.shape
    if y is None:
        y = torch.empty_like(o)
    st = load().kda_output_gate(_ptr(o), _ptr(gate), _ptr(weight), _ptr(y), B, T, H, Dv,
                                _dt(o.dtype), _stream(o.device))
    _check("kda_output_gate", st)
    return y
