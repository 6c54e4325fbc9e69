"""Shared helpers for the GPU parity tests: run the HIP path and the fp64
oracle on the very same seeded tensors and compare them.

Error measure: for every (b,h) slice, max|gpu - ref| / max|ref| (normwise
relative error), reported as the maximum over slices.  Elementwise relative
error is meaningless where signed outputs cross zero.

Tolerances: 1e-4 for fp32 inputs and 2e-2 for bf16 inputs with fp32
accumulation, for outputs and final states alike.
"""
import numpy as np
import torch

import oracle
from recurrent_attention_amd import api

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def slice_rel_err(got, ref):
    """max over (b,h) of max|got-ref| / max|ref| for [B,H,...] arrays."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    B, H = ref.shape[:2]
    g = got.reshape(B * H, -1)
    r = ref.reshape(B * H, -1)
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    if not np.isfinite(g).all():
        return float("inf")
    return float((num / den).max())


def to_host64(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def run_pair(inp, gate_mode, chunk, phi=0, normalize=False, S0=None, z0=None,
             segments=0, device="cuda", nthreads=8, pairs=None):
    """Run the GPU prefill on ``inp`` (CPU tensors from workloads) and the
    oracle on the same values.  ``pairs`` restricts the oracle (and the
    comparison) to a list of flat (b*H + h) indices."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, L, dk = q.shape
    dq, dkk, dvv = (x.to(device) for x in (q, k, v))
    gated = gate_mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR)
    la_dev = inp["log_alpha"].to(device) if gated else None
    S0d = S0.to(device) if S0 is not None else None
    z0d = z0.to(device) if z0 is not None else None
    out, S, z = api.chunk_fwd(dq, dkk, dvv, gate_mode=gate_mode, gamma=inp["gamma"],
                              log_alpha=la_dev, S0=S0d, z0=z0d, chunk=chunk, phi=phi,
                              normalize=normalize, segments=segments)
    torch.cuda.synchronize()
    got = (to_host64(out), to_host64(S), to_host64(z) if normalize else None)

    def sel(x):
        if x is None:
            return None
        if pairs is None:
            return x
        flat = x.reshape((B * H,) + tuple(x.shape[2:]))
        return flat[pairs][:, None]   # [n, 1, ...]

    gam = None
    if gate_mode == api.LA_GATE_GAMMA:
        g = inp["gamma"].double().numpy()
        gam = g if pairs is None else None
    qn, kn, vn = (sel(to_host64(x)) for x in (q, k, v))
    lan = sel(to_host64(inp["log_alpha"])) if gated else None
    S0n = sel(to_host64(S0)) if S0 is not None else None
    z0n = sel(to_host64(z0)) if z0 is not None else None
    if pairs is not None and gate_mode == api.LA_GATE_GAMMA:
        # one pair per sample row: run each with its own head's gamma
        g = inp["gamma"].double().numpy()
        refs = [oracle.run(qn[i:i + 1], kn[i:i + 1], vn[i:i + 1], gate_mode=gate_mode,
                           gamma=[g[p % H]], phi=phi, normalize=normalize,
                           S0=None if S0n is None else S0n[i:i + 1],
                           z0=None if z0n is None else z0n[i:i + 1])
                for i, p in enumerate(pairs)]
        ref = tuple(np.concatenate([r[j] for r in refs]) for j in range(3))
    else:
        ref = oracle.run(qn, kn, vn, gate_mode=gate_mode, gamma=gam, log_alpha=lan,
                         phi=phi, normalize=normalize, S0=S0n, z0=z0n, nthreads=nthreads)
    got = tuple(sel(x) for x in got)
    return got, ref


def check(got, ref, dtype, what="", normalize=False):
    tol = TOL[dtype]
    e_out = slice_rel_err(got[0], ref[0])
    e_S = slice_rel_err(got[1], ref[1])
    errs = {"out": e_out, "S_final": e_S}
    if normalize:
        errs["z_final"] = slice_rel_err(got[2], ref[2])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{what}: errors {errs} exceed {tol}"
    return errs
