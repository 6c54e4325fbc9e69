"""Plain fp64 CPU oracle for the unified linear-attention recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library: the arithmetic lives in ``oracle.c`` (fp64, libm,
pthreads over (batch, head) pairs) and this module only marshals numpy arrays
through ctypes.

Forms (all compute the same function; see ``oracle.c`` for the citations):

* :func:`run`        -- the token-by-token recurrence, the definition.
* :func:`parallel`   -- the all-pairs masked form with direct decay products.
* :func:`chunkwise`  -- the chunkwise form with a ragged last chunk.
* :func:`backward`   -- reverse-mode derivative of the token loop (no
  normaliser): dq, dk, dv, d log_alpha, dS0 from dout and dS_final.
* :func:`delta_run`  -- the delta rule's token loop (DeltaNet recurrence).
* :func:`groupnorm_swish` -- retention's output epilogue (group norm over
  each token's head output, times swish of a gate), numpy fp64.

Layouts follow the GPU boundary: q, k ``[B,H,L,dk]``, v and out
``[B,H,L,dv]``, S ``[B,H,dk,dv]`` (rows indexed by the key channel), z
``[B,H,dk]``, gamma ``[H]``, log_alpha ``[B,H,L,dk]`` (diagonal gate) or
``[B,H,L]`` (scalar gate).  2-D ``[L,d]`` inputs are treated as B = H = 1.

The per-token scalar gate A_t = alpha_t I is, by definition, the diagonal
gate with every channel equal: its log-gate is repeated over the key
channels and run as the diagonal gate, and its gradient is the sum of the
diagonal gate's gradient over those channels (the chain rule of the
repetition).

Parity: every form is pinned by tests that do not call the oracle's own
formula (the pages' worked examples, closed forms, textbook masked matmuls,
chunk-size invariance and state hand-off invariants).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

GATE_NONE, GATE_GAMMA, GATE_DIAG, GATE_SCALAR = 0, 1, 2, 3
PHI_IDENTITY, PHI_ELU1 = 0, 1

# Planted mistakes (test-only), mirrored from oracle.c.
MUTATIONS = {
    "z_frozen": 1,
    "no_divide": 2,
    "read_before_update": 3,
    "transposed_state": 4,
    "decay_after_add": 5,
    "phi_on_v": 6,
    "gate_dropped": 7,
    "cross_off_by_one": 8,
    "state_off_by_one": 9,
    "gamma_squared": 10,
    "bwd_no_decay": 11,
    "bwd_dq_prev": 12,
    "delta_no_erase": 13,
    "delta_erase_after": 14,
}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# another build of oracle.c to load instead (the sanitizer build of the CPU
# tests); build() always writes _LIB
_LOAD = os.environ.get("ORACLE_LIBRARY") or _LIB
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
             "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LOAD == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LOAD)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        common = [i, i, i, i, i, i, dp, dp, i, i, dp, dp, dp, dp, dp]
        lib.oracle_run.argtypes = common + [dp, dp, dp, i]
        lib.oracle_parallel.argtypes = common + [dp, dp, dp]
        lib.oracle_chunkwise.argtypes = common + [i, dp, dp, dp, i]
        for f in (lib.oracle_run, lib.oracle_parallel, lib.oracle_chunkwise):
            f.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [i, i, i, i, i, i, dp, dp, i, dp, dp, dp, dp, dp, dp,
                                        dp, dp, dp, dp, dp, i, i]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_delta_run.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i, i]
        lib.oracle_delta_run.restype = ctypes.c_int
        lib.oracle_multiscale_decays.argtypes = [i, dp]
        lib.oracle_phi.argtypes = [i, ctypes.c_double]
        lib.oracle_phi.restype = ctypes.c_double
        lib.oracle_set_mutation.argtypes = [i]
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(q, k, v, gate_mode, gamma, log_alpha, S0, z0):
    q, k, v = _f64(q), _f64(k), _f64(v)
    two_d = q.ndim == 2
    if two_d:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4 or k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,L,dk] and v [B,H,L,dv]")
    B, H, L, dk = q.shape
    dv = v.shape[3]
    g = la = None
    if gate_mode == GATE_GAMMA:
        g = _f64(np.broadcast_to(np.asarray(gamma, dtype=np.float64).reshape(-1), (H,)))
    elif gate_mode == GATE_DIAG:
        la = _f64(log_alpha)
        if two_d and la.ndim == 2:
            la = la[None, None]
        la = np.ascontiguousarray(np.broadcast_to(la, (B, H, L, dk)))
    elif gate_mode == GATE_SCALAR:
        la = _f64(log_alpha)
        if two_d and la.ndim == 1:
            la = la[None, None]
        la = np.ascontiguousarray(np.broadcast_to(la.reshape(B, H, L)[..., None], (B, H, L, dk)))
    elif gate_mode != GATE_NONE:
        raise ValueError("unknown gate mode")
    S0 = _f64(S0)
    z0 = _f64(z0)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0.reshape(B, H, dk, dv))
    if z0 is not None:
        z0 = np.ascontiguousarray(z0.reshape(B, H, dk))
    return two_d, (B, H, L, dk, dv), q, k, v, g, la, S0, z0


def _finish(two_d, out, S, z):
    if two_d:
        return out[0, 0], S[0, 0], z[0, 0]
    return out, S, z


def _call(fn, extra_mid, extra_tail, q, k, v, gate_mode, gamma, log_alpha,
          phi, normalize, S0, z0):
    two_d, (B, H, L, dk, dv), q, k, v, g, la, S0, z0 = _prep(
        q, k, v, gate_mode, gamma, log_alpha, S0, z0)
    out = np.zeros((B, H, L, dv))
    S = np.zeros((B, H, dk, dv))
    z = np.zeros((B, H, dk))
    cmode = GATE_DIAG if gate_mode == GATE_SCALAR else int(gate_mode)
    args = [B, H, L, dk, dv, cmode, _ptr(g), _ptr(la), int(phi),
            int(bool(normalize)), _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0)]
    args += extra_mid + [_ptr(out), _ptr(S), _ptr(z)] + extra_tail
    rc = fn(*args)
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return _finish(two_d, out, S, z)


def run(q, k, v, gate_mode=GATE_NONE, gamma=None, log_alpha=None,
        phi=PHI_IDENTITY, normalize=False, S0=None, z0=None, nthreads=1):
    """Token-by-token recurrence. Returns ``(out, S_final, z_final)`` (fp64)."""
    lib = _load()
    return _call(lib.oracle_run, [], [int(nthreads)], q, k, v, gate_mode,
                 gamma, log_alpha, phi, normalize, S0, z0)


def parallel(q, k, v, gate_mode=GATE_NONE, gamma=None, log_alpha=None,
             phi=PHI_IDENTITY, normalize=False, S0=None, z0=None):
    """All-pairs masked form (tiny L only). Returns ``(out, S_final, z_final)``."""
    lib = _load()
    return _call(lib.oracle_parallel, [], [], q, k, v, gate_mode, gamma,
                 log_alpha, phi, normalize, S0, z0)


def chunkwise(q, k, v, chunk, gate_mode=GATE_NONE, gamma=None, log_alpha=None,
              phi=PHI_IDENTITY, normalize=False, S0=None, z0=None, nthreads=1):
    """Chunkwise form with chunk length ``chunk``."""
    lib = _load()
    return _call(lib.oracle_chunkwise, [int(chunk)], [int(nthreads)], q, k, v,
                 gate_mode, gamma, log_alpha, phi, normalize, S0, z0)


def backward(q, k, v, dout, gate_mode=GATE_NONE, gamma=None, log_alpha=None,
             phi=PHI_IDENTITY, S0=None, dS_final=None, checkpoint=64, nthreads=1):
    """Gradients of the token loop (no normaliser).

    ``dout`` is the gradient of the loss with respect to ``out`` and
    ``dS_final`` (optional) with respect to the final state.  Returns a dict
    with ``dq``, ``dk``, ``dv`` (fp64, the layouts of q, k, v), ``dlog_alpha``
    (diagonal and scalar gates, in the layout of log_alpha, else None) and
    ``dS0`` ``[B,H,dk,dv]`` (the gradient of the initial state, zero-state
    runs included).
    """
    lib = _load()
    two_d, (B, H, L, dk, dv), q, k, v, g, la, S0, _ = _prep(
        q, k, v, gate_mode, gamma, log_alpha, S0, None)
    do = _f64(dout)
    do = np.ascontiguousarray(do.reshape(B, H, L, dv))
    dSf = _f64(dS_final)
    if dSf is not None:
        dSf = np.ascontiguousarray(dSf.reshape(B, H, dk, dv))
    dq = np.zeros((B, H, L, dk))
    dk_ = np.zeros((B, H, L, dk))
    dv_ = np.zeros((B, H, L, dv))
    dla = np.zeros((B, H, L, dk)) if gate_mode in (GATE_DIAG, GATE_SCALAR) else None
    dS0 = np.zeros((B, H, dk, dv))
    cmode = GATE_DIAG if gate_mode == GATE_SCALAR else int(gate_mode)
    rc = lib.oracle_backward(B, H, L, dk, dv, cmode, _ptr(g), _ptr(la), int(phi),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(do), _ptr(dSf),
                             _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dS0),
                             int(checkpoint), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    if gate_mode == GATE_SCALAR:
        dla = dla.sum(axis=-1)
    res = {"dq": dq, "dk": dk_, "dv": dv_, "dlog_alpha": dla, "dS0": dS0}
    if two_d:
        res = {n: (a[0, 0] if a is not None else None) for n, a in res.items()}
    return res


def delta_run(q, k, v, beta, S0=None, use_delta=True, nthreads=1):
    """The delta rule's token loop: S_t = (I - beta_t k_t k_t^T) S_{t-1} +
    beta_t k_t v_t^T, o_t = q_t^T S_t.  q, k [B,H,L,dk], v [B,H,L,dv], beta
    [B,H,L] (2-D [L,d] / 1-D [L] inputs are one head).  Returns
    ``(out, S_final)`` in fp64."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    two_d = q.ndim == 2
    if two_d:
        q, k, v = q[None, None], k[None, None], v[None, None]
    B, H, L, dk = q.shape
    dv = v.shape[3]
    b = np.ascontiguousarray(_f64(beta).reshape(B, H, L))
    S0 = _f64(S0)
    if S0 is not None:
        S0 = np.ascontiguousarray(S0.reshape(B, H, dk, dv))
    out = np.zeros((B, H, L, dv))
    S = np.zeros((B, H, dk, dv))
    rc = lib.oracle_delta_run(B, H, L, dk, dv, _ptr(b), _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                              _ptr(out), _ptr(S), int(bool(use_delta)), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    if two_d:
        return out[0, 0], S[0, 0]
    return out, S


def groupnorm_swish(out, weight=None, bias=None, gate=None, eps=1e-5):
    """Retention's output epilogue, in fp64: each token's head output is
    normalised over its d_v channels (group norm, one group per head, biased
    variance), scaled and shifted per channel, then multiplied by
    swish(gate) = gate * sigmoid(gate).  out, gate [B,H,L,dv]; weight, bias
    [H,dv]."""
    o = _f64(out)
    mean = o.mean(axis=-1, keepdims=True)
    var = ((o - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (o - mean) / np.sqrt(var + eps)
    if weight is not None:
        y = y * _f64(weight)[None, :, None, :]
    if bias is not None:
        y = y + _f64(bias)[None, :, None, :]
    if gate is not None:
        g = _f64(gate)
        y = y * (g / (1.0 + np.exp(-g)))
    return y


def multiscale_decays(n: int) -> np.ndarray:
    """gamma_h = 1 - 2^(-5-h) for h = 0..n-1 (multi-scale retention)."""
    lib = _load()
    out = np.zeros(n)
    lib.oracle_multiscale_decays(int(n), _ptr(out))
    return out


def phi(kind: int, x: float) -> float:
    """The feature map as the oracle evaluates it (identity or elu+1)."""
    return _load().oracle_phi(int(kind), float(x))


@contextlib.contextmanager
def mutation(name: str):
    """Plant a known mistake in the oracle for the duration of the block.

    Used only by the mutation tests that show each pin catches a plausible
    error.  Not thread-safe with concurrent oracle calls.
    """
    lib = _load()
    lib.oracle_set_mutation(MUTATIONS[name])
    try:
        yield
    finally:
        lib.oracle_set_mutation(0)
