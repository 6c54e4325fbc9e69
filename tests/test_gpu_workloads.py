"""Parity at the full workload sizes, in the launch configuration the
benchmark times (automatic segments, chunk of the workload).

The GPU runs the whole workload; the fp64 oracle recomputes a seeded sample
of (b,h) pairs over their full length (a pair's outputs depend only on its
own tokens, so each sampled pair is an exact check of those outputs), or
every pair where that takes seconds.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_attention_amd import api, workloads
from parity_util import TOL, check, run_pair, slice_rel_err, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _prefill(name, pairs=None):
    w = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name, seed=0)
    got, ref = run_pair(inp, w.gate_mode, w.chunk, phi=w.phi, normalize=w.normalize,
                        pairs=pairs, nthreads=8)
    errs = check(got, ref, w.dtype, name, normalize=w.normalize)
    print(f"{name}: {errs}")


def test_linear_elu1_L64_d16_fp32_full():
    _prefill("linear_elu1_L64_d16_fp32")


def test_linear_elu1_B4H8_L2048_d64_full():
    _prefill("linear_elu1_B4H8_L2048_d64")


def test_retention_B2H16_L8192_d128_sampled():
    _prefill("retention_B2H16_L8192_d128", pairs=[0, 5, 16, 31])


def test_gla_B1H16_L32768_d128_sampled():
    _prefill("gla_B1H16_L32768_d128", pairs=[0, 7, 15])


def test_scalar_gate_B1H16_L32768_d128_sampled():
    _prefill("scalar_gate_B1H16_L32768_d128", pairs=[3, 12])


def _decode_setup(w, steps, with_z, phi):
    dev = torch.device("cuda", 0)
    S0, z0 = workloads.decode_state(w.B, w.H, w.dk, w.dv, seed=0, device=dev, with_z=with_z)
    q, k, v, _ = workloads.decode_tokens(w.B, w.H, w.dk, w.dv, steps, seed=1, device=dev)
    return dev, S0, z0, q, k, v


@pytest.mark.parametrize("with_z", [False, True])
def test_decode_retention_256x32_d128(with_z):
    """1000 steps on all 8192 pairs; the oracle follows 64 sampled pairs
    through every step, and all pairs through the first step."""
    w = workloads.WORKLOADS["decode_retention_256x32_d128"]
    steps = w.steps
    phi = api.LA_PHI_ELU1 if with_z else api.LA_PHI_IDENTITY
    dev, S0, z0, q, k, v = _decode_setup(w, steps, with_z, phi)
    gamma = torch.tensor(w.gamma, dtype=torch.float32)
    g64 = gamma.double().numpy()

    # first step, all pairs
    S = S0.clone()
    z = z0.clone() if with_z else None
    o1 = api.decode_step(q[0], k[0], v[0], S, z, gate_mode=api.LA_GATE_GAMMA,
                         gamma=gamma, phi=phi)
    torch.cuda.synchronize()
    ref = oracle.run(to_host64(q[0])[:, :, None], to_host64(k[0])[:, :, None],
                     to_host64(v[0])[:, :, None], gate_mode=oracle.GATE_GAMMA, gamma=g64,
                     phi=phi, normalize=with_z, S0=to_host64(S0),
                     z0=to_host64(z0) if with_z else None, nthreads=8)
    assert slice_rel_err(to_host64(o1)[:, :, None], ref[0]) <= TOL[torch.bfloat16]
    assert slice_rel_err(to_host64(S), ref[1]) <= TOL[torch.bfloat16]

    # all steps, sampled pairs
    S = S0.clone()
    z = z0.clone() if with_z else None
    outs = torch.empty((steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        api.decode_step(q[t], k[t], v[t], S, z, gate_mode=api.LA_GATE_GAMMA, gamma=gamma,
                        phi=phi, out=outs[t])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    flat = rng.choice(w.B * w.H, size=64, replace=False)
    bs, hs = flat // w.H, flat % w.H
    bi, hi = torch.as_tensor(bs), torch.as_tensor(hs)

    def pick(x):   # [steps,B,H,d] -> [64,1,steps,d]
        return to_host64(x[:, bi, hi].permute(1, 0, 2))[:, None]

    ref = oracle.run(pick(q), pick(k), pick(v), gate_mode=oracle.GATE_GAMMA,
                     gamma=[w.gamma[0]], phi=phi, normalize=with_z,
                     S0=to_host64(S0[bi, hi])[:, None],
                     z0=to_host64(z0[bi, hi])[:, None] if with_z else None, nthreads=8)
    got_o = to_host64(outs[:, bi, hi].permute(1, 0, 2))[:, None]
    errs = {"out": slice_rel_err(got_o, ref[0]), "S": slice_rel_err(to_host64(S[bi, hi])[:, None], ref[1])}
    if with_z:
        errs["z"] = slice_rel_err(to_host64(z[bi, hi])[:, None], ref[2])
    print(f"decode 1000 steps, 64 sampled pairs, z={with_z}: {errs}")
    assert all(e <= TOL[torch.bfloat16] for e in errs.values()), errs
