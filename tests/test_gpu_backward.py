"""GPU parity of the chunkwise backward (la_chunk_bwd through the C ABI)
against the oracle's backward of the token loop, on the same seeded inputs.

The oracle's backward is pinned by finite differences of the pinned forward
(tests/test_oracle_backward.py).  Sizes span several chunks, several
segments and a ragged tail; the full-size workload (B=1, H=16, L=32768,
d=128, bf16, diagonal gate) is checked on sampled (b,h) slices, which the
oracle runs one by one.

Tolerance: normwise relative error per (b,h) slice, as for the forward:
1e-4 for fp32 inputs, 2e-2 for bf16 inputs (bf16 matrix-core operands,
fp32 accumulation and fp32 states), for dq, dk, dv, dlog_alpha and dS0.
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
GATED = (DIAG, SCALAR)
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dS0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _case(B, H, L, d, dtype, mode, seed=0, state=False, state_grad=True, gamma=None):
    inp = workloads.prefill_inputs(B, H, L, d, d, dtype, mode, seed=seed,
                                   scale_inputs=dtype != torch.float32,
                                   gamma=gamma, with_state=state)
    if mode == GAMMA and gamma is None:
        inp["gamma"] = torch.tensor(([0.9, 0.99, 0.5, 0.97] * H)[:H], dtype=torch.float32)
    inp.update(workloads.backward_inputs(B, H, L, d, d, dtype, seed=seed + 1000,
                                         scale_inputs=dtype != torch.float32,
                                         with_state_grad=state_grad))
    return inp


def _gpu_bwd(inp, mode, phi=0, segments=0):
    dev = "cuda"
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    g = api.chunk_bwd(t["q"], t["k"], t["v"], t["dout"], gate_mode=mode, gamma=inp["gamma"],
                      log_alpha=t["log_alpha"] if mode in GATED else None,
                      S0=t.get("S0"), dS_final=t["dS_final"], phi=phi, segments=segments)
    torch.cuda.synchronize()
    return {k: to_host64(v) for k, v in g.items()}


def _oracle_bwd(inp, mode, phi=0, pairs=None):
    """The oracle on all (b,h) slices, or on the flat indices ``pairs``."""
    f64 = {k: to_host64(v) if isinstance(v, torch.Tensor) else None
           for k, v in inp.items() if k != "gamma"}
    B, H = inp["q"].shape[:2]
    if pairs is None:
        return oracle.backward(
            f64["q"], f64["k"], f64["v"], f64["dout"], gate_mode=mode,
            gamma=None if inp["gamma"] is None else inp["gamma"].double().numpy(),
            log_alpha=f64["log_alpha"] if mode in GATED else None, phi=phi,
            S0=f64.get("S0"), dS_final=f64["dS_final"], nthreads=8)
    out = {k: [] for k in NAMES}
    for p in pairs:
        b, h = divmod(p, H)
        sl = lambda x: None if x is None else x[b:b + 1, h:h + 1]
        r = oracle.backward(
            sl(f64["q"]), sl(f64["k"]), sl(f64["v"]), sl(f64["dout"]), gate_mode=mode,
            gamma=None if inp["gamma"] is None else [float(inp["gamma"][h])],
            log_alpha=sl(f64["log_alpha"]) if mode in GATED else None, phi=phi,
            S0=sl(f64.get("S0")), dS_final=sl(f64["dS_final"]))
        for k in NAMES:
            out[k].append(r[k])
    return {k: (None if v[0] is None else np.concatenate(v)) for k, v in out.items()}


def _select(got, pairs):
    res = {}
    for k, x in got.items():
        if x is None:
            res[k] = None
            continue
        flat = x.reshape((-1,) + x.shape[2:])
        res[k] = flat[pairs][:, None]
    return res


def _check(got, ref, dtype, what):
    tol = TOL[dtype]
    errs = {}
    for k in NAMES:
        if ref[k] is None:
            assert got[k] is None, k
            continue
        errs[k] = slice_rel_err(got[k], ref[k])
    print(f"{what}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{what}: errors {errs} exceed {tol}"
    return errs


GRID = [(dt, d, mode)
        for dt in ("f32", "bf16")
        for d in ((16, 32, 64, 128) if dt == "f32" else (32, 64, 128))
        for mode in (NONE, GAMMA, DIAG, SCALAR)]


@pytest.mark.parametrize("dt,d,mode", GRID)
def test_chunk_bwd_grid(dt, d, mode):
    dtype = DTYPES[dt]
    C = api.la_chunk_bwd_chunk(api.make_desc(1, 2, 64, d, d, 1 if dt == "bf16" else 0))
    L = 5 * C + 7                           # 6 chunks, ragged tail
    inp = _case(1, 2, L, d, dtype, mode, seed=d + mode, state=True)
    got = _gpu_bwd(inp, mode)
    ref = _oracle_bwd(inp, mode)
    _check(got, ref, dtype, f"{dt} d={d} mode={mode}")


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunk_bwd_elu1_features(mode, dt):
    dtype = DTYPES[dt]
    inp = _case(2, 2, 333, 64, dtype, mode, seed=7, state=True)
    got = _gpu_bwd(inp, mode, phi=api.LA_PHI_ELU1)
    ref = _oracle_bwd(inp, mode, phi=api.LA_PHI_ELU1)
    _check(got, ref, dtype, f"elu1 {dt} mode={mode}")


@pytest.mark.parametrize("segments", [1, 2, 3, 0, 11])
def test_chunk_bwd_segmentations_agree(segments):
    inp = _case(1, 2, 11 * 64 - 5, 128, torch.bfloat16, DIAG, seed=3, state=True)
    got = _gpu_bwd(inp, DIAG, segments=segments)
    ref = _oracle_bwd(inp, DIAG)
    _check(got, ref, torch.bfloat16, f"segments={segments}")


@pytest.mark.parametrize("dt,d,mode", [("bf16", 128, DIAG), ("bf16", 128, SCALAR),
                                       ("bf16", 128, GAMMA), ("bf16", 64, NONE),
                                       ("f32", 64, DIAG), ("f32", 128, DIAG)])
def test_chunk_bwd_long_walk(dt, d, mode):
    # one segment per (b,h): the gradient kernel carries the state gradient
    # through every chunk of the sequence (96 chunks of 64 tokens, 192 of 32
    # for fp32 at d = 128), ending on a ragged chunk
    dtype = DTYPES[dt]
    inp = _case(1, 2, 96 * 64 - 17, d, dtype, mode, seed=21, state=True)
    got = _gpu_bwd(inp, mode, segments=1)
    ref = _oracle_bwd(inp, mode)
    _check(got, ref, dtype, f"long walk {dt} d={d} mode={mode}")


@pytest.mark.parametrize("L", [1, 31, 63, 64, 65, 129])
@pytest.mark.parametrize("mode", [NONE, DIAG, SCALAR])
def test_chunk_bwd_edge_lengths(L, mode):
    inp = _case(2, 1, L, 64, torch.bfloat16, mode, seed=L, state=True)
    got = _gpu_bwd(inp, mode, phi=api.LA_PHI_ELU1)
    ref = _oracle_bwd(inp, mode, phi=api.LA_PHI_ELU1)
    _check(got, ref, torch.bfloat16, f"L={L} mode={mode}")


@pytest.mark.parametrize("segments", [0, 1])
def test_chunk_bwd_without_state_or_state_gradient(segments):
    # S0 = NULL and dS_final = NULL: zero initial state, loss on out only;
    # with one segment the walk starts from no gradient at all
    inp = _case(1, 2, 300, 64, torch.float32, DIAG, seed=12, state=False, state_grad=False)
    got = _gpu_bwd(inp, DIAG, segments=segments)
    ref = _oracle_bwd(inp, DIAG)
    _check(got, ref, torch.float32, f"no S0, no dS_final, segments={segments}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunk_bwd_gamma_limits(dt):
    dtype = DTYPES[dt]
    inp = _case(1, 2, 200, 64, dtype, GAMMA, seed=1, gamma=[0.0, 1.0], state=True)
    got = _gpu_bwd(inp, GAMMA)
    ref = _oracle_bwd(inp, GAMMA)
    _check(got, ref, dtype, "gamma 0 and 1")


def test_chunk_bwd_is_linear_in_the_loss_gradients():
    # every gradient is linear in (dout, dS_final): the backward of a summed
    # loss is the sum of the backwards
    inp = _case(1, 2, 257, 64, torch.float32, DIAG, seed=21, state=True)
    a = _gpu_bwd(inp, DIAG)
    inp2 = dict(inp)
    extra = workloads.backward_inputs(1, 2, 257, 64, 64, torch.float32, seed=77,
                                      scale_inputs=False)
    inp2["dout"] = extra["dout"]
    inp2["dS_final"] = extra["dS_final"]
    b = _gpu_bwd(inp2, DIAG)
    inp3 = dict(inp)
    inp3["dout"] = inp["dout"] + extra["dout"]
    inp3["dS_final"] = inp["dS_final"] + extra["dS_final"]
    c = _gpu_bwd(inp3, DIAG)
    for k in NAMES:
        assert slice_rel_err(c[k], a[k] + b[k]) <= 1e-4, k


def test_chunk_bwd_scalar_gate_full_size_sampled():
    # the per-token scalar gate at the full size; the oracle checks one head
    inp = _case(1, 16, 32768, 128, torch.bfloat16, SCALAR, seed=33, state=True)
    got = _gpu_bwd(inp, SCALAR)
    pairs = [5]
    ref = _oracle_bwd(inp, SCALAR, pairs=pairs)
    _check(_select(got, pairs), ref, torch.bfloat16, "scalar gate, full size, sampled head")


def test_chunk_bwd_full_size_sampled():
    # the full-size gated workload, B=1 H=16 L=32768 d=128 bf16; the oracle
    # checks two sampled heads
    inp = _case(1, 16, 32768, 128, torch.bfloat16, DIAG, seed=31, state=True)
    got = _gpu_bwd(inp, DIAG)
    for k in NAMES:
        assert np.isfinite(got[k]).all(), k
    pairs = [0, 11]
    ref = _oracle_bwd(inp, DIAG, pairs=pairs)
    _check(_select(got, pairs), ref, torch.bfloat16, "full size, sampled heads")


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt,d", [("f32", 64), ("f32", 128), ("bf16", 128)])
def test_training_forward_states_feed_the_backward(dt, d, mode):
    # the training forward's outputs equal the plain prefill's, and the
    # backward from its stored boundary states matches the oracle
    dtype = DTYPES[dt]
    C = api.la_chunk_bwd_chunk(api.make_desc(1, 2, 64, d, d, 1 if dt == "bf16" else 0))
    inp = _case(1, 2, 7 * C + 5, d, dtype, mode, seed=40 + d + mode, state=True)
    dev = "cuda"
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    la = t["log_alpha"] if mode in GATED else None
    out, S, states = api.chunk_fwd_train(t["q"], t["k"], t["v"], gate_mode=mode,
                                         gamma=inp["gamma"], log_alpha=la, S0=t["S0"])
    out2, S2, _ = api.chunk_fwd(t["q"], t["k"], t["v"], gate_mode=mode, gamma=inp["gamma"],
                                log_alpha=la, S0=t["S0"], chunk=C)
    g = api.chunk_bwd(t["q"], t["k"], t["v"], t["dout"], gate_mode=mode, gamma=inp["gamma"],
                      log_alpha=la, S0=t["S0"], dS_final=t["dS_final"], states=states)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(S, S2)
    got = {k: to_host64(v) for k, v in g.items()}
    ref = _oracle_bwd(inp, mode)
    _check(got, ref, dtype, f"train states {dt} d={d} mode={mode}")
