"""Thin ctypes binding of ``liblinattn.so`` (the C ABI of ``include/la.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity and their data pointers are handed to the library, which runs
every step on the GPU.  Outputs and workspaces that the caller does not pass
are allocated with torch (device memory is PyTorch's job here).  There is no
CPU fallback: a missing library or a tensor that is not on a GPU raises.

Functions named ``la_*`` mirror the C entry points one to one;
:func:`chunk_fwd`, :func:`chunk_fwd_varlen`, :func:`chunk_bwd` and
:func:`decode_step` are conveniences around them.
"""
from __future__ import annotations

import ctypes
import os

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_GATE_NONE, LA_GATE_GAMMA, LA_GATE_DIAG, LA_GATE_SCALAR = 0, 1, 2, 3
LA_F32, LA_BF16 = 0, 1
LA_PHI_IDENTITY, LA_PHI_ELU1 = 0, 1
LA_MAX_GAMMA_HEADS = 256

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "liblinattn.so")
_lib = None

# every symbol include/la.h declares
EXPORTED = (
    "la_chunk_fwd", "la_chunk_fwd_workspace_bytes", "la_chunk_fwd_segments",
    "la_decode_step", "la_status_string", "la_last_error_message",
    "la_version", "la_profile_begin", "la_profile_end", "la_profile_query",
    "la_chunk_bwd", "la_chunk_bwd_workspace_bytes", "la_chunk_bwd_chunk",
    "la_chunk_fwd_varlen", "la_chunk_fwd_varlen_workspace_bytes",
    "la_chunk_fwd_groupnorm", "la_delta_fwd", "la_delta_decode_step", "la_delta_chunk",
    "la_chunk_fwd_train", "la_chunk_train_states_bytes", "la_chunk_fwd_noalloc",
)
LA_NOALLOC_SCRATCH_BYTES = 64 << 20


class LaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class LaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "H", "L", "dk", "dv", "dtype", "phi", "normalize", "segments")]


class LaGroupNorm(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate", ctypes.c_void_p), ("eps", ctypes.c_float)]


def library_path() -> str:
    """Path of the library to load: LINATTN_LIBRARY if set, else the in-tree build."""
    return os.environ.get("LINATTN_LIBRARY") or _LIB_PATH


def load_library():
    """Load ``liblinattn.so`` (built by ``recurrent_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m recurrent_attention_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp = ctypes.POINTER(LaDesc)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.la_chunk_fwd.argtypes = [dp, vp, vp, vp, i, vp, vp, vp, i, vp, vp, vp, vp, sz, vp]
    lib.la_chunk_fwd.restype = i
    lib.la_chunk_fwd_noalloc.argtypes = [dp, vp, vp, vp, i, vp, vp, vp, i, vp, vp, vp, vp]
    lib.la_chunk_fwd_noalloc.restype = i
    lib.la_chunk_fwd_workspace_bytes.argtypes = [dp, i]
    lib.la_chunk_fwd_workspace_bytes.restype = sz
    lib.la_chunk_fwd_segments.argtypes = [dp, i]
    lib.la_chunk_fwd_segments.restype = i
    lib.la_chunk_fwd_groupnorm.argtypes = [dp, vp, vp, vp, i, vp, vp, vp, i,
                                            ctypes.POINTER(LaGroupNorm), vp, vp, vp, vp, sz, vp]
    lib.la_chunk_fwd_groupnorm.restype = i
    lib.la_delta_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.la_delta_fwd.restype = i
    lib.la_delta_decode_step.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp]
    lib.la_delta_decode_step.restype = i
    lib.la_delta_chunk.argtypes = [dp]
    lib.la_delta_chunk.restype = i
    lib.la_chunk_fwd_varlen.argtypes = [dp, vp, i, vp, vp, vp, i, vp, vp, vp, i, vp, vp, vp,
                                         vp, sz, vp]
    lib.la_chunk_fwd_varlen.restype = i
    lib.la_chunk_fwd_varlen_workspace_bytes.argtypes = [dp, i, i]
    lib.la_chunk_fwd_varlen_workspace_bytes.restype = sz
    lib.la_chunk_bwd.argtypes = [dp, vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                 vp]
    lib.la_chunk_fwd_train.argtypes = [dp, vp, vp, vp, i, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.la_chunk_fwd_train.restype = i
    lib.la_chunk_train_states_bytes.argtypes = [dp]
    lib.la_chunk_train_states_bytes.restype = sz
    lib.la_chunk_bwd.restype = i
    lib.la_chunk_bwd_workspace_bytes.argtypes = [dp]
    lib.la_chunk_bwd_workspace_bytes.restype = sz
    lib.la_chunk_bwd_chunk.argtypes = [dp]
    lib.la_chunk_bwd_chunk.restype = i
    lib.la_decode_step.argtypes = [dp, vp, vp, vp, i, vp, vp, vp, vp, vp]
    lib.la_decode_step.restype = i
    lib.la_status_string.argtypes = [i]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_last_error_message.argtypes = []
    lib.la_last_error_message.restype = ctypes.c_char_p
    lib.la_version.restype = i
    lib.la_profile_begin.restype = i
    lib.la_profile_end.restype = i
    lib.la_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(i),
                                     ctypes.POINTER(ctypes.c_double)]
    lib.la_profile_query.restype = i
    del fp
    _lib = lib
    return lib


def _check(status):
    if status != LA_OK:
        lib = load_library()
        raise LaError(status, lib.la_last_error_message().decode() or
                      lib.la_status_string(status).decode())


# ------------------------------------------------------------------ raw entry points

def make_desc(B, H, L, dk, dv, dtype=LA_BF16, phi=LA_PHI_IDENTITY,
              normalize=False, segments=0) -> LaDesc:
    return LaDesc(int(B), int(H), int(L), int(dk), int(dv), int(dtype), int(phi),
                  int(bool(normalize)), int(segments))


def la_chunk_fwd(desc, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk,
                 out, S_final, z_final, workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are ints (0 = NULL) or ctypes pointers."""
    return load_library().la_chunk_fwd(
        ctypes.byref(desc), q, k, v, int(gate_mode), gamma_or_log_alpha, S0, z0,
        int(chunk), out, S_final, z_final, workspace, int(workspace_bytes), stream)


def la_chunk_fwd_noalloc(desc, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk,
                         out, S_final, z_final, stream):
    """Raw call of the entry point that allocates nothing (its workspace is
    the library's static scratch array)."""
    return load_library().la_chunk_fwd_noalloc(
        ctypes.byref(desc), q, k, v, int(gate_mode), gamma_or_log_alpha, S0, z0,
        int(chunk), out, S_final, z_final, stream)


def la_chunk_fwd_groupnorm(desc, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk, gn,
                           out, S_final, z_final, workspace, workspace_bytes, stream):
    """Raw call; ``gn`` is a LaGroupNorm (or None for NULL)."""
    return load_library().la_chunk_fwd_groupnorm(
        ctypes.byref(desc), q, k, v, int(gate_mode), gamma_or_log_alpha, S0, z0, int(chunk),
        None if gn is None else ctypes.byref(gn), out, S_final, z_final, workspace,
        int(workspace_bytes), stream)


def la_delta_fwd(desc, q, k, v, beta, S0, out, S_final, stream):
    """Raw call; pointer arguments are ints (0 = NULL) or ctypes pointers."""
    return load_library().la_delta_fwd(ctypes.byref(desc), q, k, v, beta, S0, out, S_final,
                                       stream)


def la_delta_decode_step(desc, q, k, v, beta, S, out, stream):
    return load_library().la_delta_decode_step(ctypes.byref(desc), q, k, v, beta, S, out, stream)


def la_delta_chunk(desc) -> int:
    return int(load_library().la_delta_chunk(ctypes.byref(desc)))


def la_chunk_fwd_varlen(desc, cu_seqlens, max_seqlen, q, k, v, gate_mode,
                        gamma_or_log_alpha, S0, z0, chunk, out, S_final, z_final,
                        workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are ints (0 = NULL) or ctypes pointers."""
    return load_library().la_chunk_fwd_varlen(
        ctypes.byref(desc), cu_seqlens, int(max_seqlen), q, k, v, int(gate_mode),
        gamma_or_log_alpha, S0, z0, int(chunk), out, S_final, z_final, workspace,
        int(workspace_bytes), stream)


def la_chunk_fwd_varlen_workspace_bytes(desc, max_seqlen, chunk) -> int:
    return int(load_library().la_chunk_fwd_varlen_workspace_bytes(
        ctypes.byref(desc), int(max_seqlen), int(chunk)))


def la_chunk_bwd(desc, q, k, v, dout, gate_mode, gamma_or_log_alpha, S0, dS_final, states,
                 dq, dk, dv, dlog_alpha, dS0, workspace, workspace_bytes, stream):
    """Raw call; pointer arguments are ints (0 = NULL) or ctypes pointers."""
    return load_library().la_chunk_bwd(
        ctypes.byref(desc), q, k, v, dout, int(gate_mode), gamma_or_log_alpha, S0, dS_final,
        states, dq, dk, dv, dlog_alpha, dS0, workspace, int(workspace_bytes), stream)


def la_chunk_fwd_train(desc, q, k, v, gate_mode, gamma_or_log_alpha, S0, out, S_final, states,
                       states_bytes, workspace, workspace_bytes, stream):
    return load_library().la_chunk_fwd_train(
        ctypes.byref(desc), q, k, v, int(gate_mode), gamma_or_log_alpha, S0, out, S_final,
        states, int(states_bytes), workspace, int(workspace_bytes), stream)


def la_chunk_train_states_bytes(desc) -> int:
    return int(load_library().la_chunk_train_states_bytes(ctypes.byref(desc)))


def la_chunk_bwd_workspace_bytes(desc) -> int:
    return int(load_library().la_chunk_bwd_workspace_bytes(ctypes.byref(desc)))


def la_chunk_bwd_chunk(desc) -> int:
    return int(load_library().la_chunk_bwd_chunk(ctypes.byref(desc)))


def la_decode_step(desc, q, k, v, gate_mode, gate, S, z, out, stream):
    return load_library().la_decode_step(
        ctypes.byref(desc), q, k, v, int(gate_mode), gate, S, z, out, stream)


def la_chunk_fwd_workspace_bytes(desc, chunk) -> int:
    return int(load_library().la_chunk_fwd_workspace_bytes(ctypes.byref(desc), int(chunk)))


def la_chunk_fwd_segments(desc, chunk) -> int:
    return int(load_library().la_chunk_fwd_segments(ctypes.byref(desc), int(chunk)))


def la_status_string(status) -> str:
    return load_library().la_status_string(int(status)).decode()


def la_last_error_message() -> str:
    return load_library().la_last_error_message().decode()


def la_version() -> int:
    return int(load_library().la_version())


def la_profile_begin():
    _check(load_library().la_profile_begin())


def la_profile_end():
    _check(load_library().la_profile_end())


def la_profile_query(kernel: str):
    """(launches, total_ms) recorded for one kernel family since begin."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(load_library().la_profile_query(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


# ------------------------------------------------------------------ torch conveniences

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device}); there is no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t.data_ptr()


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _la_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32 (got {t.dtype})")


def _gamma_host(gamma, H):
    torch = _torch()
    g = torch.as_tensor(gamma, dtype=torch.float32).detach().cpu().reshape(-1)
    if g.numel() == 1:
        g = g.expand(H)
    g = g.contiguous()
    if g.numel() != H:
        raise ValueError(f"gamma needs {H} values (got {g.numel()})")
    return g


def chunk_fwd(q, k, v, gate_mode=LA_GATE_NONE, gamma=None, log_alpha=None,
              S0=None, z0=None, chunk=64, phi=LA_PHI_IDENTITY, normalize=False,
              segments=0, out=None, S_final=None, z_final=None,
              return_state=True, workspace=None, stream=None, groupnorm=None):
    """Chunkwise prefill.  q, k: [B,H,L,dk]; v: [B,H,L,dv] (bf16 or fp32, on
    the GPU).  Returns ``(out, S_final, z_final)``; the states are fp32 and
    z_final is None unless ``normalize``.  ``groupnorm`` = dict(weight=[H,dv]
    fp32 or None, bias=[H,dv] fp32 or None, gate=[B,H,L,dv] or None, eps)
    fuses the retention output epilogue (la_chunk_fwd_groupnorm)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _la_dtype(q)
    desc = make_desc(B, H, L, dk, dv, dt, phi, normalize, segments)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
    if return_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if return_state and normalize and z_final is None:
        z_final = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    need = la_chunk_fwd_workspace_bytes(desc, chunk)
    if need and workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g_arg = None
    g_keep = None
    if gate_mode == LA_GATE_GAMMA:
        g_keep = _gamma_host(gamma, H)
        g_arg = ctypes.c_void_p(g_keep.data_ptr())
    elif gate_mode in (LA_GATE_DIAG, LA_GATE_SCALAR):
        g_arg = _dev_ptr(log_alpha, "log_alpha", torch.float32,
                         (B, H, L, dk) if gate_mode == LA_GATE_DIAG else (B, H, L))
    ptrs = (_dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, L, dk)),
            _dev_ptr(v, "v", q.dtype, (B, H, L, dv)))
    mid = (gate_mode, g_arg, _dev_ptr(S0, "S0", torch.float32, (B, H, dk, dv)),
           _dev_ptr(z0, "z0", torch.float32, (B, H, dk)), chunk)
    tail = (_dev_ptr(out, "out", q.dtype, (B, H, L, dv)),
            _dev_ptr(S_final, "S_final", torch.float32, (B, H, dk, dv)),
            _dev_ptr(z_final, "z_final", torch.float32, (B, H, dk)),
            _dev_ptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream, dev))
    if groupnorm is None:
        st = la_chunk_fwd(desc, *ptrs, *mid, *tail)
    else:
        gn = LaGroupNorm(
            _dev_ptr(groupnorm.get("weight"), "groupnorm weight", torch.float32, (H, dv)),
            _dev_ptr(groupnorm.get("bias"), "groupnorm bias", torch.float32, (H, dv)),
            _dev_ptr(groupnorm.get("gate"), "groupnorm gate", q.dtype, (B, H, L, dv)),
            float(groupnorm.get("eps", 1e-5)))
        st = la_chunk_fwd_groupnorm(desc, *ptrs, *mid, gn, *tail)
    _check(st)
    del g_keep
    return out, S_final, z_final


def decode_step(q, k, v, S, z=None, gate_mode=LA_GATE_NONE, gamma=None,
                log_alpha=None, phi=LA_PHI_IDENTITY, out=None, stream=None):
    """One recurrent step.  q, k: [B,H,dk]; v: [B,H,dv]; S: [B,H,dk,dv] fp32
    (updated in place); z: [B,H,dk] fp32 or None (normalise iff given).
    Returns ``out`` [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    desc = make_desc(B, H, 1, dk, dv, _la_dtype(q), phi, z is not None, 0)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    g_arg = None
    g_keep = None
    if gate_mode == LA_GATE_GAMMA:
        g_keep = _gamma_host(gamma, H)
        g_arg = ctypes.c_void_p(g_keep.data_ptr())
    elif gate_mode in (LA_GATE_DIAG, LA_GATE_SCALAR):
        g_arg = _dev_ptr(log_alpha, "log_alpha", torch.float32,
                         (B, H, dk) if gate_mode == LA_GATE_DIAG else (B, H))
    st = la_decode_step(
        desc, _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, dk)),
        _dev_ptr(v, "v", q.dtype, (B, H, dv)),
        gate_mode, g_arg, _dev_ptr(S, "S", torch.float32, (B, H, dk, dv)),
        _dev_ptr(z, "z", torch.float32, (B, H, dk)),
        _dev_ptr(out, "out", q.dtype, (B, H, dv)), _stream_ptr(stream, q.device))
    _check(st)
    del g_keep
    return out


def chunk_fwd_varlen(q, k, v, cu_seqlens, max_seqlen=None, gate_mode=LA_GATE_NONE,
                     gamma=None, log_alpha=None, S0=None, z0=None, chunk=64,
                     phi=LA_PHI_IDENTITY, normalize=False, segments=0, out=None,
                     S_final=None, z_final=None, return_state=True, workspace=None,
                     stream=None):
    """Prefill of packed sequences.  q, k: [1,H,T,dk] (or [H,T,dk]); v:
    [1,H,T,dv]; cu_seqlens: int32 [N+1] on the GPU.  ``max_seqlen`` is the
    longest sequence (read from cu_seqlens when omitted, which copies it to
    the host).  Returns ``(out, S_final, z_final)`` with per-sequence states
    [N,H,dk,dv]."""
    torch = _torch()
    if q.dim() == 3:
        q, k, v = q[None], k[None], v[None]
        if log_alpha is not None and log_alpha.dim() == (3 if gate_mode == LA_GATE_DIAG else 2):
            log_alpha = log_alpha[None]
    one, H, T, dk = q.shape
    if one != 1:
        raise ValueError("packed sequences need q of shape [1,H,T,dk]")
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    N = cu_seqlens.numel() - 1
    if N < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    if max_seqlen is None:
        lens = cu_seqlens.diff()
        max_seqlen = max(1, int(lens.max().item()))
    dt = _la_dtype(q)
    desc = make_desc(N, H, T, dk, dv, dt, phi, normalize, segments)
    dev = q.device
    if out is None:
        out = torch.empty((1, H, T, dv), dtype=q.dtype, device=dev)
    if return_state and S_final is None:
        S_final = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if return_state and normalize and z_final is None:
        z_final = torch.empty((N, H, dk), dtype=torch.float32, device=dev)
    need = la_chunk_fwd_varlen_workspace_bytes(desc, max_seqlen, chunk)
    if need and workspace is None:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g_arg = None
    g_keep = None
    if gate_mode == LA_GATE_GAMMA:
        g_keep = _gamma_host(gamma, H)
        g_arg = ctypes.c_void_p(g_keep.data_ptr())
    elif gate_mode in (LA_GATE_DIAG, LA_GATE_SCALAR):
        g_arg = _dev_ptr(log_alpha, "log_alpha", torch.float32,
                         (1, H, T, dk) if gate_mode == LA_GATE_DIAG else (1, H, T))
    st = la_chunk_fwd_varlen(
        desc, _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)), max_seqlen,
        _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (1, H, T, dk)),
        _dev_ptr(v, "v", q.dtype, (1, H, T, dv)),
        gate_mode, g_arg, _dev_ptr(S0, "S0", torch.float32, (N, H, dk, dv)),
        _dev_ptr(z0, "z0", torch.float32, (N, H, dk)), chunk,
        _dev_ptr(out, "out", q.dtype, (1, H, T, dv)),
        _dev_ptr(S_final, "S_final", torch.float32, (N, H, dk, dv)),
        _dev_ptr(z_final, "z_final", torch.float32, (N, H, dk)),
        _dev_ptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream, dev))
    _check(st)
    del g_keep
    return out, S_final, z_final


def delta_fwd(q, k, v, beta, S0=None, out=None, S_final=None, return_state=True,
              stream=None):
    """Delta-rule prefill.  q, k: [B,H,L,dk]; v: [B,H,L,dv] (bf16 or fp32 on
    the GPU); beta: fp32 [B,H,L].  Returns ``(out, S_final)``."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    desc = make_desc(B, H, L, dk, dv, _la_dtype(q), LA_PHI_IDENTITY, False, 0)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
    if return_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    st = la_delta_fwd(
        desc, _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, L, dk)),
        _dev_ptr(v, "v", q.dtype, (B, H, L, dv)), _dev_ptr(beta, "beta", torch.float32, (B, H, L)),
        _dev_ptr(S0, "S0", torch.float32, (B, H, dk, dv)),
        _dev_ptr(out, "out", q.dtype, (B, H, L, dv)),
        _dev_ptr(S_final, "S_final", torch.float32, (B, H, dk, dv)), _stream_ptr(stream, dev))
    _check(st)
    return out, S_final


def delta_decode_step(q, k, v, beta, S, out=None, stream=None):
    """One delta-rule step.  q, k: [B,H,dk]; v: [B,H,dv]; beta: fp32 [B,H];
    S: fp32 [B,H,dk,dv] (updated in place).  Returns ``out`` [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    desc = make_desc(B, H, 1, dk, dv, _la_dtype(q), LA_PHI_IDENTITY, False, 0)
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    st = la_delta_decode_step(
        desc, _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, dk)),
        _dev_ptr(v, "v", q.dtype, (B, H, dv)), _dev_ptr(beta, "beta", torch.float32, (B, H)),
        _dev_ptr(S, "S", torch.float32, (B, H, dk, dv)), _dev_ptr(out, "out", q.dtype, (B, H, dv)),
        _stream_ptr(stream, q.device))
    _check(st)
    return out


def chunk_fwd_train(q, k, v, gate_mode=LA_GATE_NONE, gamma=None, log_alpha=None, S0=None,
                    phi=LA_PHI_IDENTITY, segments=0, stream=None):
    """Prefill that keeps its boundary states for :func:`chunk_bwd`.
    Returns ``(out, S_final, states)``."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    desc = make_desc(B, H, L, dk, dv, _la_dtype(q), phi, False, segments)
    dev = q.device
    out = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
    S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    nbytes = la_chunk_train_states_bytes(desc)
    states = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=dev)
    need = la_chunk_fwd_workspace_bytes(desc, la_chunk_bwd_chunk(desc))
    ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device=dev)
    g_arg = None
    g_keep = None
    if gate_mode == LA_GATE_GAMMA:
        g_keep = _gamma_host(gamma, H)
        g_arg = ctypes.c_void_p(g_keep.data_ptr())
    elif gate_mode in (LA_GATE_DIAG, LA_GATE_SCALAR):
        g_arg = _dev_ptr(log_alpha, "log_alpha", torch.float32,
                         (B, H, L, dk) if gate_mode == LA_GATE_DIAG else (B, H, L))
    st = la_chunk_fwd_train(
        desc, _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, L, dk)),
        _dev_ptr(v, "v", q.dtype, (B, H, L, dv)), gate_mode, g_arg,
        _dev_ptr(S0, "S0", torch.float32, (B, H, dk, dv)), _dev_ptr(out, "out"),
        _dev_ptr(S_final, "S_final"), _dev_ptr(states, "states"), states.numel() * 4,
        _dev_ptr(ws, "workspace"), ws.numel() * 4, _stream_ptr(stream, dev))
    _check(st)
    del g_keep
    return out, S_final, states


def chunk_bwd(q, k, v, dout, gate_mode=LA_GATE_NONE, gamma=None, log_alpha=None,
              S0=None, dS_final=None, phi=LA_PHI_IDENTITY, segments=0,
              workspace=None, stream=None, states=None):
    """Gradients of :func:`chunk_fwd` (no normaliser) for the loss
    ``sum(dout * out) + sum(dS_final * S_final)``.  Returns a dict with
    ``dq``, ``dk``, ``dv`` (dtype of q), ``dlog_alpha`` (fp32, DIAG and
    SCALAR gates, in the layout of log_alpha, else None) and ``dS0``
    (fp32).  ``states`` from :func:`chunk_fwd_train` skips the recompute of
    the forward states."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dt = _la_dtype(q)
    desc = make_desc(B, H, L, dk, dv, dt, phi, False, segments)
    dev = q.device
    dq = torch.empty((B, H, L, dk), dtype=q.dtype, device=dev)
    dkk = torch.empty((B, H, L, dk), dtype=q.dtype, device=dev)
    dvv = torch.empty((B, H, L, dv), dtype=q.dtype, device=dev)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    dla = None
    if gate_mode == LA_GATE_DIAG:
        dla = torch.empty((B, H, L, dk), dtype=torch.float32, device=dev)
    elif gate_mode == LA_GATE_SCALAR:
        dla = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    need = la_chunk_bwd_workspace_bytes(desc)
    if workspace is None and need:
        workspace = torch.empty(need // 4 + 4, dtype=torch.float32, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g_arg = None
    g_keep = None
    if gate_mode == LA_GATE_GAMMA:
        g_keep = _gamma_host(gamma, H)
        g_arg = ctypes.c_void_p(g_keep.data_ptr())
    elif gate_mode in (LA_GATE_DIAG, LA_GATE_SCALAR):
        g_arg = _dev_ptr(log_alpha, "log_alpha", torch.float32,
                         (B, H, L, dk) if gate_mode == LA_GATE_DIAG else (B, H, L))
    st = la_chunk_bwd(
        desc, _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype, (B, H, L, dk)),
        _dev_ptr(v, "v", q.dtype, (B, H, L, dv)), _dev_ptr(dout, "dout", q.dtype, (B, H, L, dv)),
        gate_mode, g_arg, _dev_ptr(S0, "S0", torch.float32, (B, H, dk, dv)),
        _dev_ptr(dS_final, "dS_final", torch.float32, (B, H, dk, dv)),
        _dev_ptr(states, "states"), _dev_ptr(dq, "dq"), _dev_ptr(dkk, "dk"), _dev_ptr(dvv, "dv"), _dev_ptr(dla, "dlog_alpha"),
        _dev_ptr(dS0, "dS0"), _dev_ptr(workspace, "workspace"), ws_bytes,
        _stream_ptr(stream, dev))
    _check(st)
    del g_keep
    return {"dq": dq, "dk": dkk, "dv": dvv, "dlog_alpha": dla, "dS0": dS0}


def chunk_bwd_workspace_bytes(B, H, L, dk, dv, dtype=LA_BF16, segments=0) -> int:
    return la_chunk_bwd_workspace_bytes(make_desc(B, H, L, dk, dv, dtype, 0, False, segments))


def chunk_fwd_workspace_bytes(B, H, L, dk, dv, chunk, dtype=LA_BF16,
                              normalize=False, segments=0) -> int:
    return la_chunk_fwd_workspace_bytes(
        make_desc(B, H, L, dk, dv, dtype, 0, normalize, segments), chunk)
