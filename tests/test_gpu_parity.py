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

def _chunks(dt, d):
    """Chunk lengths built for a shape: multiples of 16 up to 64 everywhere,
    up to 128 where the 128-token tile fits the LDS (bf16 at d <= 64, fp32
    at d <= 32)."""
    big = d <= 64 if dt == "bf16" else d <= 32
    return (16, 32, 48, 64) + ((80, 96, 112, 128) if big else ())


GRID = [(dt, d, C, mode)
        for dt in ("f32", "bf16")
        for d in ((16, 32, 64, 128) if dt == "f32" else (32, 64, 128))
        for C in _chunks(dt, d)
        for mode in (NONE, GAMMA, DIAG, SCALAR)]


@pytest.mark.parametrize("dt,d,C,mode", GRID)
def test_chunk_fwd_grid(dt, d, C, mode):
    dtype = DTYPES[dt]
    L = 5 * C + 7                           # 6 chunks, ragged tail
    inp = _inputs(1, 2, L, d, dtype, mode, seed=d + C + mode)
    got, ref = run_pair(inp, mode, C)
    check(got, ref, dtype, f"{dt} d={d} C={C} mode={mode}")


# chunks shorter than their tile (48 in the 64-token tile; 80, 96, 112 in the
# 128-token one) with several segments, an initial state and the normaliser
@pytest.mark.parametrize("C", [48, 80, 112])
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
def test_chunk_shorter_than_its_tile(C, mode):
    dt = torch.bfloat16
    inp = _inputs(2, 2, 7 * C + 5, 64, dt, mode, seed=C + 60 + mode, state=True)
    got, ref = run_pair(inp, mode, C, phi=api.LA_PHI_ELU1, normalize=True, S0=inp["S0"],
                        z0=inp["z0"], segments=3)
    check(got, ref, dt, f"chunk {C} mode {mode}", normalize=True)


def test_chunk_128_unsupported_at_d128_bf16():
    inp = _inputs(1, 1, 256, 128, torch.bfloat16, NONE, seed=1)
    with pytest.raises(api.LaError) as e:
        api.chunk_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), chunk=128)
    assert e.value.status == api.LA_ERR_UNSUPPORTED


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunk_fwd_normalised_elu1_with_state(mode, dt):
    dtype = DTYPES[dt]
    inp = _inputs(2, 2, 333, 64, dtype, mode, seed=5, state=True)
    got, ref = run_pair(inp, mode, 64, phi=api.LA_PHI_ELU1, normalize=True,
                        S0=inp["S0"], z0=inp["z0"])
    check(got, ref, dtype, f"normalised {dt} mode={mode}", normalize=True)


# the normaliser's row sums over every lane-group width (1 to 16 lanes a row:
# the workgroup's threads over the rows of the tile) and, where the tile has
# more rows than the workgroup threads (d = 16 in the 128-token tile), more
# than one row a thread
NORM_TILES = [("f32", 16, 128), ("f32", 16, 80), ("f32", 16, 16), ("f32", 32, 96),
              ("f32", 32, 16), ("bf16", 32, 128), ("bf16", 64, 112), ("bf16", 64, 16),
              ("bf16", 128, 16), ("bf16", 128, 32), ("f32", 128, 64)]


@pytest.mark.parametrize("dt,d,C", NORM_TILES)
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
def test_chunk_fwd_normalised_every_row_width(dt, d, C, mode):
    dtype = DTYPES[dt]
    inp = _inputs(1, 2, 4 * C + 9, d, dtype, mode, seed=d + C + 17 * mode, state=True)
    got, ref = run_pair(inp, mode, C, phi=api.LA_PHI_ELU1, normalize=True, S0=inp["S0"],
                        z0=inp["z0"], segments=2)
    check(got, ref, dtype, f"normalised {dt} d={d} C={C} mode={mode}", normalize=True)


@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
def test_chunk_fwd_initial_state(mode):
    inp = _inputs(1, 4, 700, 128, torch.bfloat16, mode, seed=9, state=True)
    got, ref = run_pair(inp, mode, 64, S0=inp["S0"])
    check(got, ref, torch.bfloat16, f"S0 mode={mode}")


# 11 chunks: 1 to 11 chunks a segment, odd and even counts (the scalar-gate
# state pass alternates two tile sets by chunk parity)
@pytest.mark.parametrize("segments", [1, 2, 3, 0, 11])
@pytest.mark.parametrize("mode", [DIAG, SCALAR])
def test_segmentations_agree(segments, mode):
    inp = _inputs(1, 2, 11 * 64 - 5, 128, torch.bfloat16, mode, seed=3, state=True)
    got, ref = run_pair(inp, mode, 64, S0=inp["S0"], segments=segments)
    check(got, ref, torch.bfloat16, f"segments={segments} mode={mode}")


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


# Gates far past the half-chunk range of a single chunk-wide reference: every
# factor above one is now confined to half a 16-token block, so the kernel
# holds while any 8 consecutive log-gates of a channel sum to more than about
# -88.  -3 per token puts a half chunk of 64 at -96 (beyond fp32 for a
# chunk-wide reference); -7 per token, drawn between -3.5 and -10.5, puts
# 8 tokens down to -84.
@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("level", [-3.0, -5.0, -7.0])
@pytest.mark.parametrize("mode", [DIAG, SCALAR])
def test_strong_gates_beyond_half_chunk(C, level, mode):
    dt = torch.bfloat16
    inp = _inputs(1, 2, 5 * C + 7, 128, dt, mode, seed=40 + C, state=True)
    g = torch.Generator().manual_seed(41)
    shape = inp["log_alpha"].shape
    # around the level, from 0.5x to 1.5x, so the channels decay differently
    inp["log_alpha"] = level * (0.5 + torch.rand(shape, generator=g))
    got, ref = run_pair(inp, mode, C, S0=inp["S0"])
    check(got, ref, dt, f"log-gates near {level} per token, chunk {C}, mode {mode}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_exercise_gates_0_95_and_0_1(dt):
    # the gate values of "Module 22", "Exercise 3: You are the gate": a high
    # gate (0.95, the state holds) at some positions and a low one (0.1)
    # elsewhere; here chosen at random per token and channel
    dtype = DTYPES[dt]
    inp = _inputs(2, 2, 3 * 64 + 21, 64, dtype, DIAG, seed=44, state=True)
    g = torch.Generator().manual_seed(45)
    pick = torch.rand(inp["log_alpha"].shape, generator=g) < 0.5
    inp["log_alpha"] = torch.where(pick, torch.tensor(0.95).log(), torch.tensor(0.1).log())
    for C in (16, 64):
        got, ref = run_pair(inp, DIAG, C, S0=inp["S0"])
        check(got, ref, dtype, f"0.95/0.1 gates, chunk {C}")


def _strong_in_ranges(inp, ranges, level, seed):
    """log-gates of `level` (times 0.5..1.5) on the given (head, t0, t1)
    token ranges of every batch entry, the workload's mild gates elsewhere."""
    g = torch.Generator().manual_seed(seed)
    la = inp["log_alpha"].clone()
    for h, t0, t1 in ranges:
        sl = la[:, h, t0:t1]
        la[:, h, t0:t1] = level * (0.5 + torch.rand(sl.shape, generator=g))
    inp["log_alpha"] = la


# Strong gates in a few segments only: the main pass hands just those
# segments to the sub-chunk kernel (a flag per segment); the others keep the
# chunk-middle factors.  With one segment per (b,h) a whole head is handed
# over, with the automatic plan (16 segments of one chunk) single chunks.
@pytest.mark.parametrize("segments", [1, 0])
@pytest.mark.parametrize("mode", [DIAG, SCALAR])
def test_strong_gates_in_some_segments(mode, segments):
    dt = torch.bfloat16
    inp = _inputs(2, 3, 1000, 128, dt, mode, seed=46, state=True)
    _strong_in_ranges(inp, [(1, 300, 400), (2, 990, 1000)], -6.0, seed=47)
    got, ref = run_pair(inp, mode, 64, S0=inp["S0"], segments=segments)
    check(got, ref, dt, f"strong gates in some segments, mode {mode}, segments {segments}")


@pytest.mark.parametrize("mode", [DIAG, SCALAR])
def test_strong_gates_with_normaliser(mode):
    dt = torch.bfloat16
    inp = _inputs(2, 2, 333, 64, dt, mode, seed=48, state=True)
    _strong_in_ranges(inp, [(0, 0, 333), (1, 100, 200)], -5.0, seed=49)
    got, ref = run_pair(inp, mode, 64, phi=api.LA_PHI_ELU1, normalize=True, S0=inp["S0"],
                        z0=inp["z0"])
    check(got, ref, dt, f"strong gates, normalised, mode {mode}", normalize=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_strong_gates_with_groupnorm_epilogue(dt):
    dtype = DTYPES[dt]
    inp, w, b, gate = _gn_case(2, 2, 5 * 64 + 7, 64, dtype, DIAG, seed=50)
    _strong_in_ranges(inp, [(0, 0, 327), (1, 64, 200)], -5.0, seed=51)
    got, S, ref, ref_S = _gn_run(inp, DIAG, w, b, gate, 1e-5)
    assert slice_rel_err(got, ref) <= TOL[dtype]
    assert slice_rel_err(S, ref_S) <= TOL[dtype]


def test_strong_gates_training_forward():
    # the forward that keeps its boundary states: out, S_final and every
    # boundary state against the oracle's token loop
    dt = torch.bfloat16
    inp = _inputs(1, 2, 700, 64, dt, DIAG, seed=52, state=True)
    _strong_in_ranges(inp, [(1, 128, 400)], -5.0, seed=53)
    dev = "cuda"
    out, S, states = api.chunk_fwd_train(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                         gate_mode=DIAG, log_alpha=inp["log_alpha"].to(dev),
                                         S0=inp["S0"].to(dev))
    torch.cuda.synchronize()
    ref = oracle.run(*(to_host64(inp[x]) for x in ("q", "k", "v")), gate_mode=DIAG,
                     log_alpha=to_host64(inp["log_alpha"]), S0=to_host64(inp["S0"]))
    assert slice_rel_err(to_host64(out), ref[0]) <= TOL[dt]
    assert slice_rel_err(to_host64(S), ref[1]) <= TOL[dt]
    C = api.la_chunk_bwd_chunk(api.make_desc(1, 2, 700, 64, 64, api.LA_BF16))
    nslots = -(-700 // C) + 1          # the state before every chunk, then the final one (bf16)
    st = to_host64(states.view(torch.bfloat16)[: 2 * nslots * 64 * 64]).reshape(1, 2, nslots, 64, 64)
    for c in (1, 3, 5, 7):   # the state after c chunks = the state of a prefill of c*C tokens
        n = c * C
        ref_c = oracle.run(*(to_host64(inp[x])[:, :, :n] for x in ("q", "k", "v")), gate_mode=DIAG,
                           log_alpha=to_host64(inp["log_alpha"])[:, :, :n],
                           S0=to_host64(inp["S0"]))[1]
        assert slice_rel_err(st[:, :, c], ref_c) <= TOL[dt], c


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


# ------------------------------------------------------------------ retention output epilogue

def _gn_case(B, H, L, d, dtype, mode, seed, with_affine=True, with_gate=True):
    inp = _inputs(B, H, L, d, dtype, mode, seed=seed)
    gen = workloads.generator(seed + 99)
    w = (1.0 + 0.5 * torch.randn((H, d), generator=gen)) if with_affine else None
    b = 0.3 * torch.randn((H, d), generator=gen) if with_affine else None
    gate = torch.randn((B, H, L, d), generator=gen).to(dtype) if with_gate else None
    return inp, w, b, gate


def _gn_run(inp, mode, w, b, gate, eps, phi=0, normalize=False, segments=0):
    dev = "cuda"
    g = lambda x: None if x is None else x.to(dev)
    la = g(inp["log_alpha"]) if mode in (DIAG, SCALAR) else None
    out, S, _ = api.chunk_fwd(g(inp["q"]), g(inp["k"]), g(inp["v"]), gate_mode=mode,
                              gamma=inp["gamma"], log_alpha=la, chunk=64, phi=phi,
                              normalize=normalize, segments=segments,
                              groupnorm=dict(weight=g(w), bias=g(b), gate=g(gate), eps=eps))
    torch.cuda.synchronize()
    ref_o, ref_S, _ = oracle.run(
        *(to_host64(inp[x]) for x in ("q", "k", "v")), gate_mode=mode,
        gamma=inp["gamma"].double().numpy() if mode == GAMMA else None,
        log_alpha=to_host64(inp["log_alpha"]) if mode in (DIAG, SCALAR) else None,
        phi=phi, normalize=normalize, nthreads=8)
    ref = oracle.groupnorm_swish(ref_o, None if w is None else to_host64(w),
                                 None if b is None else to_host64(b),
                                 None if gate is None else to_host64(gate), eps)
    return to_host64(out), to_host64(S), ref, ref_S


@pytest.mark.parametrize("segments", [1, 0])
@pytest.mark.parametrize("mode", [NONE, GAMMA, DIAG, SCALAR])
@pytest.mark.parametrize("dt,d", [("f32", 16), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_groupnorm_swish_epilogue(dt, d, mode, segments):
    # one segment: six chunks in one workgroup; automatic: one chunk each
    dtype = DTYPES[dt]
    inp, w, b, gate = _gn_case(2, 2, 5 * 64 + 7, d, dtype, mode, seed=d + mode)
    got, S, ref, ref_S = _gn_run(inp, mode, w, b, gate, 1e-5, segments=segments)
    tol = TOL[dtype]
    e = slice_rel_err(got, ref)
    print(f"groupnorm {dt} d={d} mode={mode}: out {e:.2e}")
    assert e <= tol
    assert slice_rel_err(S, ref_S) <= tol    # the state is unaffected


def test_groupnorm_without_gate_and_affine_and_with_normaliser():
    inp, w, b, gate = _gn_case(1, 3, 200, 64, torch.float32, NONE, seed=5, with_affine=False,
                               with_gate=False)
    got, _, ref, _ = _gn_run(inp, NONE, w, b, gate, 1e-3, phi=api.LA_PHI_ELU1, normalize=True)
    assert slice_rel_err(got, ref) <= 1e-4
    # plain standardisation: every token's head output has mean 0
    assert np.abs(got.mean(axis=-1)).max() < 1e-4


def test_groupnorm_retention_workload_sampled():
    # the retention workload (B=2, H=16, L=8192, d=128, bf16, multi-scale
    # gamma) with the epilogue; the oracle checks three sampled heads
    name = "retention_B2H16_L8192_d128"
    wl = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name, seed=0)
    gen = workloads.generator(404)
    H, d = wl.H, wl.dv
    w = 1.0 + 0.5 * torch.randn((H, d), generator=gen)
    b = 0.3 * torch.randn((H, d), generator=gen)
    gate = torch.randn((wl.B, H, wl.L, d), generator=gen).to(torch.bfloat16)
    dev = "cuda"
    out, _, _ = api.chunk_fwd(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                              gate_mode=GAMMA, gamma=inp["gamma"], chunk=64,
                              groupnorm=dict(weight=w.to(dev), bias=b.to(dev),
                                             gate=gate.to(dev), eps=1e-5))
    torch.cuda.synchronize()
    got = to_host64(out)
    for pair in (0, 9, 31):
        bb, h = divmod(pair, H)
        sl = lambda x: to_host64(x)[bb:bb + 1, h:h + 1]
        o, _, _ = oracle.run(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), gate_mode=GAMMA,
                             gamma=[float(inp["gamma"][h])])
        ref = oracle.groupnorm_swish(o, to_host64(w)[h:h + 1], to_host64(b)[h:h + 1],
                                     sl(gate), 1e-5)
        e = slice_rel_err(got[bb:bb + 1, h:h + 1], ref)
        print(f"retention groupnorm pair {pair}: {e:.2e}")
        assert e <= TOL[torch.bfloat16]
