"""GPU parity of the packed-sequence prefill (la_chunk_fwd_varlen through
the C ABI) and of its hand-off to recurrent decoding, against the oracle's
token loop run on each sequence on its own.

Sequences of different lengths (empty, single-token, ragged, several
chunks, several segments) share each head's token axis; every sequence
starts from its own S0 (and z0) and returns its own S_final (and z_final).
Tolerance as for the prefill: normwise per (sequence, head) slice, 1e-4 for
fp32 inputs and 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_attention_amd import api, workloads
from parity_util import TOL, slice_rel_err, to_host64

pytestmark = pytest.mark.gpu

NONE, GAMMA, DIAG, SCALAR = (api.LA_GATE_NONE, api.LA_GATE_GAMMA, api.LA_GATE_DIAG,
                              api.LA_GATE_SCALAR)
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _packed(lens, H, d, dtype, mode, seed, state=True):
    """Packed inputs [1,H,T,d] plus per-sequence S0/z0 [N,H,...]."""
    T = int(sum(lens))
    inp = workloads.prefill_inputs(1, H, T, d, d, dtype, mode, seed=seed,
                                   scale_inputs=dtype != torch.float32)
    if mode == GAMMA:
        inp["gamma"] = torch.tensor(([0.9, 0.99, 0.5, 0.97] * H)[:H], dtype=torch.float32)
    gen = workloads.generator(seed + 500)
    N = len(lens)
    inp["S0"] = torch.randn((N, H, d, d), generator=gen) if state else None
    inp["z0"] = (1.0 + torch.randn((N, H, d), generator=gen).abs()) if state else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp["cu"] = torch.tensor(cu, dtype=torch.int32)
    return inp


def _run_gpu(inp, mode, chunk, phi=0, normalize=False, segments=0, max_seqlen=None):
    dev = "cuda"
    g = lambda x: None if x is None else x.to(dev)
    out, S, z = api.chunk_fwd_varlen(
        g(inp["q"]), g(inp["k"]), g(inp["v"]), g(inp["cu"]), max_seqlen=max_seqlen,
        gate_mode=mode, gamma=inp["gamma"], log_alpha=g(inp["log_alpha"]),
        S0=g(inp["S0"]), z0=g(inp["z0"]) if normalize else None, chunk=chunk, phi=phi,
        normalize=normalize, segments=segments)
    torch.cuda.synchronize()
    return to_host64(out), to_host64(S), (to_host64(z) if normalize else None)


def _run_oracle(inp, mode, phi=0, normalize=False):
    """Each sequence on its own: out [1,H,T,d], S [N,H,d,d], z [N,H,d]."""
    cu = inp["cu"].numpy()
    q, k, v = (to_host64(inp[x]) for x in ("q", "k", "v"))
    la = to_host64(inp["log_alpha"]) if mode in (DIAG, SCALAR) else None
    gam = inp["gamma"].double().numpy() if mode == GAMMA else None
    S0 = to_host64(inp["S0"])
    z0 = to_host64(inp["z0"])
    N = len(cu) - 1
    H, d = q.shape[1], q.shape[-1]
    out = np.zeros_like(v)
    S = np.zeros((N, H, d, d))
    z = np.zeros((N, H, d))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        s0 = None if S0 is None else S0[n:n + 1]
        zz = None if (z0 is None or not normalize) else z0[n:n + 1]
        if b == a:
            S[n] = 0.0 if s0 is None else s0[0]
            if normalize:
                z[n] = 0.0 if zz is None else zz[0]
            continue
        o, Sn, zn = oracle.run(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], gate_mode=mode,
                               gamma=gam, log_alpha=None if la is None else la[:, :, a:b],
                               phi=phi, normalize=normalize, S0=s0, z0=zz, nthreads=8)
        out[:, :, a:b] = o
        S[n] = Sn[0]
        if normalize:
            z[n] = zn[0]
    return out, S, (z if normalize else None)


def _seq_err(got, ref, cu):
    """max over sequences and heads of the normwise error of out."""
    e = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            e = max(e, slice_rel_err(got[:, :, a:b], ref[:, :, a:b]))
    return e


def _check(got, ref, cu, dtype, what, normalize=False):
    tol = TOL[dtype]
    errs = {"out": _seq_err(got[0], ref[0], cu), "S_final": slice_rel_err(got[1], ref[1])}
    if normalize:
        errs["z_final"] = slice_rel_err(got[2], ref[2])
    print(f"{what}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{what}: {errs} exceed {tol}"


LENS = [100, 0, 1, 64, 63, 65, 700, 17, 0, 300]


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt,d", [("f32", 16), ("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_varlen_matches_per_sequence_oracle(dt, d, mode):
    dtype = DTYPES[dt]
    inp = _packed(LENS, 2, d, dtype, mode, seed=d + mode)
    got = _run_gpu(inp, mode, 64)
    ref = _run_oracle(inp, mode)
    _check(got, ref, inp["cu"].numpy(), dtype, f"{dt} d={d} mode={mode}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("segments", [1, 3, 0])
def test_varlen_chunks_and_segments(chunk, segments):
    inp = _packed(LENS, 2, 64, torch.bfloat16, DIAG, seed=chunk + segments)
    got = _run_gpu(inp, DIAG, chunk, segments=segments)
    ref = _run_oracle(inp, DIAG)
    _check(got, ref, inp["cu"].numpy(), torch.bfloat16, f"chunk={chunk} segments={segments}")


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG])
def test_varlen_normalised_elu1(mode):
    inp = _packed(LENS, 2, 64, torch.float32, mode, seed=40 + mode)
    got = _run_gpu(inp, mode, 32, phi=api.LA_PHI_ELU1, normalize=True)
    ref = _run_oracle(inp, mode, phi=api.LA_PHI_ELU1, normalize=True)
    _check(got, ref, inp["cu"].numpy(), torch.float32, f"normalised mode={mode}", True)


def test_varlen_without_initial_state_and_max_seqlen_given():
    lens = [5, 129, 64]
    inp = _packed(lens, 3, 32, torch.bfloat16, DIAG, seed=9, state=False)
    got = _run_gpu(inp, DIAG, 64, max_seqlen=129)
    ref = _run_oracle(inp, DIAG)
    _check(got, ref, inp["cu"].numpy(), torch.bfloat16, "no S0")


def test_varlen_one_sequence_equals_the_dense_prefill():
    # a single packed sequence is the dense prefill of B = 1, bit for bit
    inp = _packed([777], 4, 128, torch.bfloat16, DIAG, seed=3)
    dev = "cuda"
    got = _run_gpu(inp, DIAG, 64, segments=3)
    out, S, _ = api.chunk_fwd(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                              gate_mode=DIAG, log_alpha=inp["log_alpha"].to(dev),
                              S0=inp["S0"].to(dev), chunk=64, segments=3)
    torch.cuda.synchronize()
    assert np.array_equal(got[0], to_host64(out))
    assert np.array_equal(got[1], to_host64(S))


def test_varlen_prefill_then_decode_hand_off():
    """Packed prefill of N prompts, then each sequence decodes 3 more tokens
    from its S_final with la_decode_step; the oracle runs prompt + tokens."""
    lens, H, d, steps = [40, 1, 200, 64, 0, 130], 2, 128, 3
    N = len(lens)
    inp = _packed(lens, H, d, torch.bfloat16, DIAG, seed=21)
    dev = "cuda"
    _, S, _ = _run_gpu(inp, DIAG, 64)
    S = torch.tensor(S, dtype=torch.float32, device=dev)
    qd, kd, vd, lad = workloads.decode_tokens(N, H, d, d, steps, seed=22, gate=True)
    outs = []
    for t in range(steps):
        o = api.decode_step(qd[t].to(dev), kd[t].to(dev), vd[t].to(dev), S, gate_mode=DIAG,
                            log_alpha=lad[t].to(dev))
        outs.append(to_host64(o))
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2)              # [N,H,steps,d]
    cu = inp["cu"].numpy()
    q, k, v, la = (to_host64(inp[x]) for x in ("q", "k", "v", "log_alpha"))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        cat = lambda x, y: np.concatenate([x[:, :, a:b], y[:, n][None].transpose(0, 2, 1, 3)], axis=2)
        qq = cat(q, to_host64(qd))
        kk = cat(k, to_host64(kd))
        vv = cat(v, to_host64(vd))
        ll = cat(la, to_host64(lad))
        ref, Sref, _ = oracle.run(qq, kk, vv, gate_mode=DIAG, log_alpha=ll,
                                  S0=to_host64(inp["S0"])[n:n + 1])
        e = slice_rel_err(got[n:n + 1], ref[:, :, b - a:])
        assert e <= 2e-2, (n, e)
        assert slice_rel_err(to_host64(S)[n:n + 1], Sref) <= 2e-2, n


@pytest.mark.parametrize("lens_kind", ["mixed", "equal"])
def test_varlen_many_sequences_launch_order(lens_kind):
    # more sequences than the ordering workgroup has threads, so the device
    # sort of the launch order loops; many equal chunk counts (ties) and
    # empty sequences.  The order must change no result.
    rng = np.random.default_rng(31)
    lens = (rng.integers(0, 41, size=1500) if lens_kind == "mixed" else np.full(1100, 32)).tolist()
    inp = _packed(lens, 2, 16, torch.float32, DIAG, seed=33)
    got = _run_gpu(inp, DIAG, 16)
    ref = _run_oracle(inp, DIAG)
    _check(got, ref, inp["cu"].numpy(), torch.float32, f"{len(lens)} sequences, {lens_kind}")
