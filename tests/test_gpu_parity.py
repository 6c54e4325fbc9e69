"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several chunks, several segments and a ragged tail.

Tolerance: normwise relative error per (b,h) slice <= 1e-4 for fp32 inputs
and <= 2e-2 for bf16 inputs (fp32 accumulation), for out, S_final, z_final.
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
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _inputs(B, H, L, d, dtype, mode, seed=0, gamma=None, state=False):
    inp = workloads.prefill_inputs(B, H, L, d, d, dtype, mode, seed=seed,
                                   scale_inputs=dtype != torch.float32,
                                   gamma=gamma, with_state=state)
    if mode == GAMMA and gamma is None:
        inp["gamma"] = torch.tensor(([0.9, 0.99, 0.5, 0.97] * H)[:H], dtype=torch.float32)
    return inp


# ------------------------------------------------------------------ prefill grid

GRID = [(dt, d, C, mode)
        for dt in ("f32", "bf16")
        for d in ((16, 32, 64, 128) if dt == "f32" else (32, 64, 128))
        for C in (16, 32, 64)
        for mode in (NONE, GAMMA, DIAG, SCALAR)]


@pytest.mark.parametrize("dt,d,C,mode", GRID)
def test_chunk_fwd_grid(dt, d, C, mode):
    dtype = DTYPES[dt]
    L = 5 * C + 7                           # 6 chunks, ragged tail
    inp = _inputs(1, 2, L, d, dtype, mode, seed=d + C + mode)
    got, ref = run_pair(inp, mode, C)
    check(got, ref, dtype, f"{dt} d={d} C={C} mode={mode}")


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunk_fwd_normalised_elu1_with_state(mode, dt):
    dtype = DTYPES[dt]
    inp = _inputs(2, 2, 333, 64, dtype, mode, seed=5, state=True)
    got, ref = run_pair(inp, mode, 64, phi=api.LA_PHI_ELU1, normalize=True,
                        S0=inp["S0"], z0=inp["z0"])
    check(got, ref, dtype, f"normalised {dt} mode={mode}", normalize=True)


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
def test_chunk_fwd_initial_state(mode):
    inp = _inputs(1, 4, 700, 128, torch.bfloat16, mode, seed=9, state=True)
    got, ref = run_pair(inp, mode, 64, S0=inp["S0"])
    check(got, ref, torch.bfloat16, f"S0 mode={mode}")


@pytest.mark.parametrize("segments", [1, 2, 3, 0, 11])
def test_segmentations_agree(segments):
    inp = _inputs(1, 2, 11 * 64 - 5, 128, torch.bfloat16, DIAG, seed=3, state=True)
    got, ref = run_pair(inp, DIAG, 64, S0=inp["S0"], segments=segments)
    check(got, ref, torch.bfloat16, f"segments={segments}")


@pytest.mark.parametrize("L", [1, 15, 16, 17, 63, 64, 65, 128])
@pytest.mark.parametrize("mode", [NONE, DIAG])
def test_edge_lengths(L, mode):
    inp = _inputs(2, 1, L, 64, torch.bfloat16, mode, seed=L, state=True)
    got, ref = run_pair(inp, mode, 64, phi=api.LA_PHI_ELU1, normalize=True,
                        S0=inp["S0"], z0=inp["z0"])
    check(got, ref, torch.bfloat16, f"L={L}", normalize=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gamma_limits_zero_and_one(dt):
    dtype = DTYPES[dt]
    inp = _inputs(1, 2, 200, 64, dtype, GAMMA, seed=1, gamma=[0.0, 1.0])
    got, ref = run_pair(inp, GAMMA, 32)
    check(got, ref, dtype, "gamma 0 and 1")
    # gamma = 0 keeps only the diagonal: o_t = (q_t . k_t) v_t
    q, k, v = (to_host64(inp[x])[0, 0] for x in ("q", "k", "v"))
    diag = (q * k).sum(axis=1, keepdims=True) * v
    assert np.abs(got[0][0, 0] - diag).max() <= TOL[dtype] * np.abs(diag).max() * 2


def test_diag_strong_gates_within_contract():
    inp = _inputs(1, 2, 300, 128, torch.bfloat16, DIAG, seed=4)
    g = torch.Generator().manual_seed(4)
    inp["log_alpha"] = -2.0 * torch.rand(inp["log_alpha"].shape, generator=g)
    got, ref = run_pair(inp, DIAG, 64)
    check(got, ref, torch.bfloat16, "strong gates, chunk 64")
    got, ref = run_pair(inp, DIAG, 16)
    check(got, ref, torch.bfloat16, "strong gates, chunk 16")


def test_many_heads_gamma():
    H = api.LA_MAX_GAMMA_HEADS
    gam = [1.0 - 2.0 ** (-1 - (h % 12)) for h in range(H)]
    inp = _inputs(1, H, 80, 32, torch.bfloat16, GAMMA, seed=2, gamma=gam)
    got, ref = run_pair(inp, GAMMA, 16)
    check(got, ref, torch.bfloat16, "H=256")


def test_in_place_state_and_determinism():
    inp = _inputs(1, 4, 1000, 128, torch.bfloat16, DIAG, seed=6, state=True)
    dev = "cuda"
    q, k, v, la = (inp[x].to(dev) for x in ("q", "k", "v", "log_alpha"))
    S = inp["S0"].to(dev).clone()
    out1, S1, _ = api.chunk_fwd(q, k, v, gate_mode=DIAG, log_alpha=la, S0=inp["S0"].to(dev))
    out2, _, _ = api.chunk_fwd(q, k, v, gate_mode=DIAG, log_alpha=la, S0=S, S_final=S)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(S, S1)
    out3, S3, _ = api.chunk_fwd(q, k, v, gate_mode=DIAG, log_alpha=la, S0=inp["S0"].to(dev))
    torch.cuda.synchronize()
    assert torch.equal(out1, out3) and torch.equal(S1, S3)


def test_resume_equals_one_pass():
    """Two prefills joined by S_final -> S0 equal one prefill of the whole."""
    inp = _inputs(1, 2, 640, 64, torch.bfloat16, GAMMA, seed=8)
    dev = "cuda"
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    g = inp["gamma"]
    full, Sf, _ = api.chunk_fwd(q, k, v, gate_mode=GAMMA, gamma=g)
    a, Sa, _ = api.chunk_fwd(q[:, :, :300].contiguous(), k[:, :, :300].contiguous(),
                             v[:, :, :300].contiguous(), gate_mode=GAMMA, gamma=g)
    b, Sb, _ = api.chunk_fwd(q[:, :, 300:].contiguous(), k[:, :, 300:].contiguous(),
                             v[:, :, 300:].contiguous(), gate_mode=GAMMA, gamma=g, S0=Sa)
    torch.cuda.synchronize()
    joined = torch.cat([a, b], dim=2)
    ref = oracle.run(*(to_host64(inp[x]) for x in ("q", "k", "v")), gate_mode=GAMMA,
                     gamma=g.double().numpy())
    # the split moves chunk boundaries, so bf16 operand rounding differs;
    # both runs are held to the oracle at the bf16 tolerance
    for o, S in ((joined, Sb), (full, Sf)):
        assert slice_rel_err(to_host64(o), ref[0]) <= 2e-2
        assert slice_rel_err(to_host64(S), ref[1]) <= 2e-2


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("normalize", [False, True])
def test_decode_steps(d, dt, mode, normalize):
    dtype = DTYPES[dt]
    if dtype == torch.bfloat16 and d < 32:
        pytest.skip("bf16 inputs need d >= 32")
    B, H, steps = 3, 4, 6
    phi = api.LA_PHI_ELU1 if normalize else api.LA_PHI_IDENTITY
    S0, z0 = workloads.decode_state(B, H, d, d, seed=d, with_z=normalize)
    q, k, v, la = workloads.decode_tokens(B, H, d, d, steps, seed=d + 1, dtype=dtype,
                                          scale_inputs=dtype != torch.float32,
                                          gate=mode == DIAG)
    if mode == SCALAR:
        # one gate per step, sequence and head
        g = torch.randn((steps, B, H), generator=workloads.generator(d + 2))
        la = torch.nn.functional.logsigmoid(g) / 16.0
    gamma = torch.tensor([0.97, 0.5, 1.0, 0.0], dtype=torch.float32)
    dev = "cuda"
    S = S0.to(dev).clone()
    z = z0.to(dev).clone() if normalize else None
    outs = []
    for t in range(steps):
        outs.append(api.decode_step(q[t].to(dev), k[t].to(dev), v[t].to(dev), S, z,
                                    gate_mode=mode, gamma=gamma,
                                    log_alpha=la[t].to(dev) if mode in (DIAG, SCALAR) else None,
                                    phi=phi))
    torch.cuda.synchronize()
    got_o = np.stack([to_host64(o) for o in outs], axis=2)       # [B,H,steps,d]
    perm = lambda x: to_host64(x).transpose(1, 2, 0, 3)          # [steps,B,H,d] -> [B,H,steps,d]
    ref = oracle.run(perm(q), perm(k), perm(v), gate_mode=mode,
                     gamma=gamma.double().numpy() if mode == GAMMA else None,
                     log_alpha=(perm(la) if mode == DIAG else
                                to_host64(la).transpose(1, 2, 0) if mode == SCALAR else None),
                     phi=phi,
                     normalize=normalize, S0=to_host64(S0),
                     z0=to_host64(z0) if normalize else None)
    tol = TOL[dtype]
    assert slice_rel_err(got_o, ref[0]) <= tol
    assert slice_rel_err(to_host64(S), ref[1]) <= tol
    if normalize:
        assert slice_rel_err(to_host64(z), ref[2]) <= tol


def test_prefill_then_decode_hand_off():
    """prefill(L) + decode(token L) == last row of prefill(L+1)."""
    L, d = 300, 128
    inp = _inputs(2, 2, L + 1, d, torch.bfloat16, DIAG, seed=12)
    dev = "cuda"
    q, k, v, la = (inp[x].to(dev) for x in ("q", "k", "v", "log_alpha"))
    full, _, _ = api.chunk_fwd(q, k, v, gate_mode=DIAG, log_alpha=la)
    _, S, _ = api.chunk_fwd(q[:, :, :L].contiguous(), k[:, :, :L].contiguous(),
                            v[:, :, :L].contiguous(), gate_mode=DIAG,
                            log_alpha=la[:, :, :L].contiguous())
    o = api.decode_step(q[:, :, L].contiguous(), k[:, :, L].contiguous(),
                        v[:, :, L].contiguous(), S, gate_mode=DIAG,
                        log_alpha=la[:, :, L].contiguous())
    torch.cuda.synchronize()
    ref = oracle.run(*(to_host64(inp[x]) for x in ("q", "k", "v")), gate_mode=DIAG,
                     log_alpha=to_host64(inp["log_alpha"]))
    assert slice_rel_err(to_host64(o)[:, :, None], ref[0][:, :, L:]) <= 2e-2
    assert slice_rel_err(to_host64(full)[:, :, L:], to_host64(o)[:, :, None]) <= 2e-2
