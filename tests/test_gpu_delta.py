"""GPU parity of the delta rule (la_delta_fwd and la_delta_decode_step
through the C ABI) against the oracle's token loop, on the same seeded
inputs (unit-norm keys, write strengths beta = sigmoid(N(0,1))).

Tolerance as for the rest of the path: normwise per (b,h) slice, 1e-4 for
fp32 inputs and 2e-2 for bf16 inputs, for outputs and final states.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_attention_amd import api, workloads
from parity_util import TOL, slice_rel_err, to_host64

pytestmark = pytest.mark.gpu
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _run(inp, pairs=None):
    dev = "cuda"
    g = lambda x: None if x is None else x.to(dev)
    out, S = api.delta_fwd(g(inp["q"]), g(inp["k"]), g(inp["v"]), g(inp["beta"]),
                           S0=g(inp["S0"]))
    torch.cuda.synchronize()
    got_o, got_S = to_host64(out), to_host64(S)
    f = {k: to_host64(v) for k, v in inp.items() if v is not None}
    if pairs is None:
        ref_o, ref_S = oracle.delta_run(f["q"], f["k"], f["v"], f["beta"], S0=f.get("S0"),
                                        nthreads=8)
        return (got_o, got_S), (ref_o, ref_S)
    H = inp["q"].shape[1]
    go, gs, ro, rs = [], [], [], []
    for p in pairs:
        b, h = divmod(p, H)
        sl = lambda x: None if x is None else x[b:b + 1, h:h + 1]
        o, S_ = oracle.delta_run(sl(f["q"]), sl(f["k"]), sl(f["v"]), sl(f["beta"]),
                                 S0=sl(f.get("S0")))
        ro.append(o)
        rs.append(S_)
        go.append(got_o[b:b + 1, h:h + 1])
        gs.append(got_S[b:b + 1, h:h + 1])
    cat = lambda x: np.concatenate(x)
    return (cat(go), cat(gs)), (cat(ro), cat(rs))


def _check(got, ref, dtype, what):
    e = {"out": slice_rel_err(got[0], ref[0]), "S_final": slice_rel_err(got[1], ref[1])}
    print(f"{what}: " + ", ".join(f"{k} {v:.2e}" for k, v in e.items()))
    assert all(v <= TOL[dtype] for v in e.values()), f"{what}: {e}"


GRID = [(dt, d) for dt in ("f32", "bf16") for d in ((16, 32, 64, 128) if dt == "f32" else (32, 64, 128))]


@pytest.mark.parametrize("dt,d", GRID)
def test_delta_prefill_grid(dt, d):
    dtype = DTYPES[dt]
    C = api.la_delta_chunk(api.make_desc(1, 2, 64, d, d, 1 if dt == "bf16" else 0))
    inp = workloads.delta_inputs(2, 2, 5 * C + 7, d, d, dtype, seed=d, with_state=True)
    got, ref = _run(inp)
    _check(got, ref, dtype, f"delta {dt} d={d}")


@pytest.mark.parametrize("L", [1, 15, 16, 17, 63, 64, 65, 200])
def test_delta_edge_lengths(L):
    inp = workloads.delta_inputs(1, 3, L, 64, 64, torch.bfloat16, seed=L, with_state=True)
    got, ref = _run(inp)
    _check(got, ref, torch.bfloat16, f"delta L={L}")


# bf16 at d = 128 with 64-token chunks is the 8-wave layout: diagonal
# blocks solved two lanes per column on two waves, wave 0's output product
# formed by another wave; lengths from one token to ragged multi-chunk tails
@pytest.mark.parametrize("L", [1, 17, 64, 65, 130, 200])
def test_delta_edge_lengths_d128(L):
    inp = workloads.delta_inputs(1, 3, L, 128, 128, torch.bfloat16, seed=1000 + L, with_state=True)
    got, ref = _run(inp)
    _check(got, ref, torch.bfloat16, f"delta d=128 L={L}")


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_delta_write_strength_limits(beta):
    inp = workloads.delta_inputs(1, 2, 150, 64, 64, torch.float32, seed=7, with_state=True)
    inp["beta"] = torch.full_like(inp["beta"], beta)
    got, ref = _run(inp)
    _check(got, ref, torch.float32, f"delta beta={beta}")
    if beta == 0.0:   # nothing is written: the state stays S0
        assert np.abs(got[1] - to_host64(inp["S0"])).max() < 1e-5


def test_delta_unit_key_retrieval_on_the_gpu():
    # q = k, beta = 1: every output returns the value just written
    inp = workloads.delta_inputs(1, 2, 100, 64, 64, torch.float32, seed=8, with_state=True)
    inp["q"] = inp["k"].clone()
    inp["beta"] = torch.ones_like(inp["beta"])
    got, _ = _run(inp)
    assert slice_rel_err(got[0], to_host64(inp["v"])) <= 1e-4


def test_delta_workload_sampled():
    sp = workloads.DELTA_SPEC
    inp = workloads.delta_inputs(sp["B"], sp["H"], sp["L"], sp["d"], sp["d"], torch.bfloat16,
                                 seed=0)
    got, ref = _run(inp, pairs=[0, 37, 255])
    _check(got, ref, torch.bfloat16, "delta workload, sampled heads")


@pytest.mark.parametrize("dt,d", [("f32", 16), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_delta_decode_steps_and_hand_off(dt, d):
    """Prefill of L tokens, then 5 decode steps from its final state,
    against the oracle over all L + 5 tokens."""
    dtype = DTYPES[dt]
    L, steps = 70, 5
    inp = workloads.delta_inputs(3, 2, L + steps, d, d, dtype, seed=d + 3, with_state=True)
    dev = "cuda"
    pre = {k: (v[:, :, :L].contiguous() if (v is not None and v.dim() >= 3 and k != "S0") else v)
           for k, v in inp.items()}
    pre["beta"] = inp["beta"][:, :, :L].contiguous()
    g = lambda x: x.to(dev)
    _, S = api.delta_fwd(g(pre["q"]), g(pre["k"]), g(pre["v"]), g(pre["beta"]), S0=g(inp["S0"]))
    outs = []
    for t in range(L, L + steps):
        outs.append(to_host64(api.delta_decode_step(
            g(inp["q"][:, :, t].contiguous()), g(inp["k"][:, :, t].contiguous()),
            g(inp["v"][:, :, t].contiguous()), g(inp["beta"][:, :, t].contiguous()), S)))
    torch.cuda.synchronize()
    got = np.stack(outs, axis=2)
    f = {k: to_host64(v) for k, v in inp.items() if v is not None}
    ref_o, ref_S = oracle.delta_run(f["q"], f["k"], f["v"], f["beta"], S0=f["S0"], nthreads=8)
    tol = TOL[dtype]
    assert slice_rel_err(got, ref_o[:, :, L:]) <= tol
    assert slice_rel_err(to_host64(S), ref_S) <= tol


def test_delta_decode_from_scratch_equals_prefill():
    # decoding token by token from S0 gives the prefill's outputs
    inp = workloads.delta_inputs(2, 2, 40, 32, 32, torch.float32, seed=11, with_state=True)
    dev = "cuda"
    g = lambda x: x.to(dev)
    out, Sp = api.delta_fwd(g(inp["q"]), g(inp["k"]), g(inp["v"]), g(inp["beta"]),
                            S0=g(inp["S0"]))
    S = g(inp["S0"]).clone()
    outs = [to_host64(api.delta_decode_step(g(inp["q"][:, :, t].contiguous()),
                                            g(inp["k"][:, :, t].contiguous()),
                                            g(inp["v"][:, :, t].contiguous()),
                                            g(inp["beta"][:, :, t].contiguous()), S))
            for t in range(40)]
    torch.cuda.synchronize()
    assert slice_rel_err(np.stack(outs, axis=2), to_host64(out)) <= 1e-4
    assert slice_rel_err(to_host64(S), to_host64(Sp)) <= 1e-4
