"""GPU parity with d_k != d_v: (d_k, d_v) = (64, 128) and (128, 64), the bf16
prefill (every gate, chunk lengths 16 to 64 with a ragged tail, several
segments, the normaliser with an initial state), its group-norm epilogue and
packed-sequence form, and the decode step in both types, each against the
fp64 oracle on the same seeded inputs (2e-2 for bf16 inputs, 1e-4 for fp32).
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_attention_amd import api, workloads
from parity_util import TOL, check, run_pair, slice_rel_err, to_host64

pytestmark = pytest.mark.gpu

NONE, GAMMA, DIAG, SCALAR = (api.LA_GATE_NONE, api.LA_GATE_GAMMA, api.LA_GATE_DIAG,
                              api.LA_GATE_SCALAR)
PAIRS = [(64, 128), (128, 64)]
BF = torch.bfloat16


def _inputs(B, H, L, dk, dv, dtype, mode, seed, state=False):
    inp = workloads.prefill_inputs(B, H, L, dk, dv, dtype, mode, seed=seed,
                                   scale_inputs=dtype != torch.float32, with_state=state)
    if mode == GAMMA:
        inp["gamma"] = torch.tensor(([0.9, 0.99, 0.5, 0.97] * H)[:H], dtype=torch.float32)
    return inp


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("C", [16, 48, 64])
def test_prefill_dk_ne_dv(dk, dv, mode, C):
    print(f"kv prefill dk={dk} dv={dv} mode={mode} C={C}", flush=True)
    inp = _inputs(1, 2, 5 * C + 7, dk, dv, BF, mode, seed=dk + C + mode)
    got, ref = run_pair(inp, mode, C, segments=3)
    check(got, ref, BF, f"dk={dk} dv={dv} C={C} mode={mode}")


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
def test_prefill_dk_ne_dv_normalised_with_state(dk, dv, mode):
    inp = _inputs(2, 2, 333, dk, dv, BF, mode, seed=7 + mode, state=True)
    got, ref = run_pair(inp, mode, 64, phi=api.LA_PHI_ELU1, normalize=True, S0=inp["S0"],
                        z0=inp["z0"], segments=0)
    check(got, ref, BF, f"normalised dk={dk} dv={dv} mode={mode}", normalize=True)


def test_prefill_dk_ne_dv_unsupported_beyond_its_builds():
    q = torch.zeros(1, 1, 128, 64, dtype=torch.float32, device="cuda")
    v = torch.zeros(1, 1, 128, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(api.LaError) as e:           # fp32 prefill: dk == dv only
        api.chunk_fwd(q, q, v)
    assert e.value.status == api.LA_ERR_UNSUPPORTED
    with pytest.raises(api.LaError) as e:           # the 128-token tile: dk == dv only
        api.chunk_fwd(q.to(BF), q.to(BF), v.to(BF), chunk=128)
    assert e.value.status == api.LA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("mode", [GAMMA, DIAG])
def test_groupnorm_epilogue_dk_ne_dv(dk, dv, mode):
    B, H, L = 2, 2, 3 * 64 + 5
    inp = _inputs(B, H, L, dk, dv, BF, mode, seed=31 + dk)
    gen = workloads.generator(32 + dk)
    w = 1.0 + 0.5 * torch.randn((H, dv), generator=gen)
    b = 0.3 * torch.randn((H, dv), generator=gen)
    gate = torch.randn((B, H, L, dv), generator=gen).to(BF)
    dev = "cuda"
    la = inp["log_alpha"].to(dev) if mode == DIAG else None
    out, S, _ = api.chunk_fwd(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), gate_mode=mode,
                              gamma=inp["gamma"], log_alpha=la, chunk=64, segments=2,
                              groupnorm=dict(weight=w.to(dev), bias=b.to(dev), gate=gate.to(dev),
                                             eps=1e-5))
    torch.cuda.synchronize()
    ref_o, ref_S, _ = oracle.run(*(to_host64(inp[x]) for x in ("q", "k", "v")), gate_mode=mode,
                                 gamma=inp["gamma"].double().numpy() if mode == GAMMA else None,
                                 log_alpha=to_host64(inp["log_alpha"]) if mode == DIAG else None,
                                 nthreads=8)
    ref = oracle.groupnorm_swish(ref_o, to_host64(w), to_host64(b), to_host64(gate), 1e-5)
    assert slice_rel_err(to_host64(out), ref) <= TOL[BF]
    assert slice_rel_err(to_host64(S), ref_S) <= TOL[BF]


@pytest.mark.parametrize("dk,dv", PAIRS)
def test_packed_sequences_dk_ne_dv(dk, dv):
    lens = [0, 150, 1, 64, 333]
    H = 2
    T = sum(lens)
    inp = _inputs(1, H, T, dk, dv, BF, DIAG, seed=41 + dk)
    dev = "cuda"
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    out, S, _ = api.chunk_fwd_varlen(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), cu,
                                     max(lens), gate_mode=DIAG,
                                     log_alpha=inp["log_alpha"].to(dev), chunk=64, segments=2)
    torch.cuda.synchronize()
    got_o, got_S = to_host64(out).reshape(H, T, dv), to_host64(S)
    for n, (a, e) in enumerate(zip(np.cumsum([0] + lens[:-1]), np.cumsum(lens))):
        if e == a:
            assert np.abs(got_S[n]).max() == 0.0
            continue
        sl = lambda x: to_host64(x)[:, :, a:e]
        ref_o, ref_S, _ = oracle.run(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), gate_mode=DIAG,
                                     log_alpha=sl(inp["log_alpha"]))
        assert slice_rel_err(got_o[None, :, a:e], ref_o) <= TOL[BF], n
        assert slice_rel_err(got_S[n][None], ref_S) <= TOL[BF], n


@pytest.mark.parametrize("dk,dv", PAIRS)
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode,normalize", [(GAMMA, False), (DIAG, True), (SCALAR, False),
                                            (NONE, True)])
def test_decode_dk_ne_dv(dk, dv, dt, mode, normalize):
    B, H, steps = 3, 2, 5
    phi = api.LA_PHI_ELU1 if normalize else api.LA_PHI_IDENTITY
    S0, z0 = workloads.decode_state(B, H, dk, dv, seed=dk + 3, with_z=normalize)
    q, k, v, la = workloads.decode_tokens(B, H, dk, dv, steps, seed=dk + 4, dtype=dt,
                                          scale_inputs=dt != torch.float32, gate=mode == DIAG)
    if mode == SCALAR:
        g = torch.randn((steps, B, H), generator=workloads.generator(dk + 5))
        la = torch.nn.functional.logsigmoid(g) / 16.0
    gamma = torch.tensor([0.97, 0.5], dtype=torch.float32)
    dev = "cuda"
    S = S0.to(dev).clone()
    z = z0.to(dev).clone() if normalize else None
    outs = []
    for t in range(steps):
        outs.append(api.decode_step(q[t].to(dev), k[t].to(dev), v[t].to(dev), S, z, gate_mode=mode,
                                    gamma=gamma,
                                    log_alpha=la[t].to(dev) if mode in (DIAG, SCALAR) else None,
                                    phi=phi))
    torch.cuda.synchronize()
    got_o = np.stack([to_host64(o) for o in outs], axis=2)
    perm = lambda x: to_host64(x).transpose(1, 2, 0, 3)
    ref = oracle.run(perm(q), perm(k), perm(v), gate_mode=mode,
                     gamma=gamma.double().numpy() if mode == GAMMA else None,
                     log_alpha=(perm(la) if mode == DIAG else
                                to_host64(la).transpose(1, 2, 0) if mode == SCALAR else None),
                     phi=phi, normalize=normalize, S0=to_host64(S0),
                     z0=to_host64(z0) if normalize else None)
    tol = TOL[dt]
    assert slice_rel_err(got_o, ref[0]) <= tol
    assert slice_rel_err(to_host64(S), ref[1]) <= tol
    if normalize:
        assert slice_rel_err(to_host64(z), ref[2]) <= tol
