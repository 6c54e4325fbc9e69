"""Guard bands around every buffer the library writes.

Each output (and each workspace) is the middle of a larger allocation whose
4 KiB on either side hold a sentinel bit pattern (a NaN that no kernel
produces); outputs start out filled with it too.  After each call through
the C ABI the bands must be untouched, every output element must have been
overwritten, and the outputs must equal bit for bit those of the same call
into buffers of their exact size (the kernels are deterministic, so a
difference would be a race or a stray write).  Cases cover the ragged tail,
several segments, chunks shorter than their tile, the sub-chunk path of
strong gates, packed sequences, the decode steps, the delta rule and the
backward.
"""
import ctypes

import pytest
import torch

from recurrent_attention_amd import api, workloads

pytestmark = pytest.mark.gpu

GUARD = 4096                                   # bytes on either side
SENT = {2: 0x7FA5, 4: 0x7FA5A5A5}              # NaN bit patterns (bf16, fp32)
IVIEW = {2: torch.int16, 4: torch.int32}
DEV = "cuda"


class Guarded:
    """A tensor of ``shape`` in the middle of a sentinel-filled allocation."""

    def __init__(self, shape, dtype, init=None):
        self.esz = torch.empty((), dtype=dtype).element_size()
        self.n = 1
        for s in shape:
            self.n *= s
        self.g = GUARD // self.esz
        self.buf = torch.empty(self.g + self.n + self.g, dtype=dtype, device=DEV)
        self.buf.view(IVIEW[self.esz]).fill_(SENT[self.esz])
        self.t = self.buf[self.g:self.g + self.n].view(shape)
        if init is not None:
            self.t.copy_(init)

    @property
    def ptr(self):
        return self.t.data_ptr()

    def check(self, what, written=True):
        torch.cuda.synchronize()
        iv = self.buf.view(IVIEW[self.esz])
        s = SENT[self.esz]
        lo, hi = iv[:self.g], iv[self.g + self.n:]
        assert bool((lo == s).all()), f"{what}: write before the buffer"
        assert bool((hi == s).all()), f"{what}: write past the end of the buffer"
        if written:
            left = int((iv[self.g:self.g + self.n] == s).sum())
            assert left == 0, f"{what}: {left} of {self.n} elements never written"


def workspace(nbytes):
    return Guarded((max(nbytes, 4) // 4,), torch.float32)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _gate(mode, inp, H, keep):
    if mode == api.LA_GATE_GAMMA:
        g = torch.tensor([0.9 + 0.09 * (h % 3) / 2 for h in range(H)], dtype=torch.float32)
        keep.append(g)
        return ctypes.c_void_p(g.data_ptr()), [float(x) for x in g]
    if mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR):
        return inp["log_alpha"].data_ptr(), None
    return None, None


PREFILL = [
    # (B, H, L, d, dtype, mode, chunk, phi, normalize, segments)
    (1, 2, 5 * 64 + 7, 128, torch.bfloat16, api.LA_GATE_DIAG, 64, 0, False, 3),
    (2, 3, 300, 64, torch.bfloat16, api.LA_GATE_NONE, 48, 1, True, 0),
    (1, 2, 400, 32, torch.float32, api.LA_GATE_GAMMA, 128, 0, False, 2),
    (2, 2, 333, 128, torch.bfloat16, api.LA_GATE_SCALAR, 16, 0, False, 4),
    (1, 3, 250, 16, torch.float32, api.LA_GATE_NONE, 16, 1, True, 0),
    (1, 2, 700, 64, torch.bfloat16, api.LA_GATE_DIAG, 112, 0, False, 2),
]


@pytest.mark.parametrize("case", range(len(PREFILL)))
def test_prefill_guard_bands(case):
    B, H, L, d, dt, mode, chunk, phi, normalize, segments = PREFILL[case]
    print(f"canary prefill {PREFILL[case]}", flush=True)
    inp = workloads.prefill_inputs(B, H, L, d, d, dt, mode, seed=900 + case, device=DEV,
                                   with_state=True)
    keep = []
    gate, gamma = _gate(mode, inp, H, keep)
    S0 = inp["S0"]
    z0 = (1.0 + inp["z0"].abs()) if normalize else None
    la = inp["log_alpha"] if mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR) else None
    ref = api.chunk_fwd(inp["q"], inp["k"], inp["v"], gate_mode=mode, gamma=gamma, log_alpha=la,
                        S0=S0, z0=z0, chunk=chunk, phi=phi, normalize=normalize,
                        segments=segments)
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16 if dt == torch.bfloat16 else api.LA_F32,
                         phi, normalize, segments)
    need = api.la_chunk_fwd_workspace_bytes(desc, chunk)
    out = Guarded((B, H, L, d), dt)
    S = Guarded((B, H, d, d), torch.float32)
    z = Guarded((B, H, d), torch.float32) if normalize else None
    ws = workspace(need)
    st = api.la_chunk_fwd(desc, inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                          mode, gate, S0.data_ptr(), None if z0 is None else z0.data_ptr(), chunk,
                          out.ptr, S.ptr, None if z is None else z.ptr, ws.ptr, need, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out")
    S.check("S_final")
    ws.check("workspace", written=False)
    assert torch.equal(out.t, ref[0]) and torch.equal(S.t, ref[1])
    if normalize:
        z.check("z_final")
        assert torch.equal(z.t, ref[2])


def test_strong_gate_sub_chunk_path_guard_bands():
    # log-gates of -5 per token: every segment goes to the sub-chunk kernel
    B, H, L, d = 1, 2, 4 * 64 + 9, 128
    inp = workloads.prefill_inputs(B, H, L, d, d, torch.bfloat16, api.LA_GATE_DIAG, seed=950,
                                   device=DEV)
    la = torch.full_like(inp["log_alpha"], -5.0)
    ref = api.chunk_fwd(inp["q"], inp["k"], inp["v"], gate_mode=api.LA_GATE_DIAG, log_alpha=la,
                        chunk=64, segments=2)
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 2)
    need = api.la_chunk_fwd_workspace_bytes(desc, 64)
    out, S, ws = Guarded((B, H, L, d), torch.bfloat16), Guarded((B, H, d, d), torch.float32), \
        workspace(need)
    st = api.la_chunk_fwd(desc, inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                          api.LA_GATE_DIAG, la.data_ptr(), None, None, 64, out.ptr, S.ptr, None,
                          ws.ptr, need, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out")
    S.check("S_final")
    ws.check("workspace", written=False)
    assert torch.equal(out.t, ref[0]) and torch.equal(S.t, ref[1])


def test_groupnorm_and_noalloc_guard_bands():
    B, H, L, d = 2, 2, 3 * 64 + 5, 128
    inp = workloads.prefill_inputs(B, H, L, d, d, torch.bfloat16, api.LA_GATE_GAMMA, seed=960,
                                   device=DEV)
    keep = []
    gate, gamma = _gate(api.LA_GATE_GAMMA, inp, H, keep)
    gen = workloads.generator(961, DEV)
    gnw = 1.0 + 0.5 * torch.randn((H, d), generator=gen, device=DEV)
    gnb = 0.3 * torch.randn((H, d), generator=gen, device=DEV)
    sg = torch.randn((B, H, L, d), generator=gen, device=DEV).to(torch.bfloat16)
    ref = api.chunk_fwd(inp["q"], inp["k"], inp["v"], gate_mode=api.LA_GATE_GAMMA, gamma=gamma,
                        chunk=64, segments=2,
                        groupnorm=dict(weight=gnw, bias=gnb, gate=sg, eps=1e-5))
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 2)
    need = api.la_chunk_fwd_workspace_bytes(desc, 64)
    out, S, ws = Guarded((B, H, L, d), torch.bfloat16), Guarded((B, H, d, d), torch.float32), \
        workspace(need)
    gn = api.LaGroupNorm(gnw.data_ptr(), gnb.data_ptr(), sg.data_ptr(), 1e-5)
    st = api.la_chunk_fwd_groupnorm(desc, inp["q"].data_ptr(), inp["k"].data_ptr(),
                                    inp["v"].data_ptr(), api.LA_GATE_GAMMA, gate, None, None, 64,
                                    gn, out.ptr, S.ptr, None, ws.ptr, need, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out")
    S.check("S_final")
    ws.check("workspace", written=False)
    assert torch.equal(out.t, ref[0]) and torch.equal(S.t, ref[1])
    # the entry point without a workspace, plain output
    ref2 = api.chunk_fwd(inp["q"], inp["k"], inp["v"], gate_mode=api.LA_GATE_GAMMA, gamma=gamma,
                         chunk=64, segments=2)
    out2, S2 = Guarded((B, H, L, d), torch.bfloat16), Guarded((B, H, d, d), torch.float32)
    st = api.la_chunk_fwd_noalloc(desc, inp["q"].data_ptr(), inp["k"].data_ptr(),
                                  inp["v"].data_ptr(), api.LA_GATE_GAMMA, gate, None, None, 64,
                                  out2.ptr, S2.ptr, None, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out2.check("out (no-alloc)")
    S2.check("S_final (no-alloc)")
    assert torch.equal(out2.t, ref2[0]) and torch.equal(S2.t, ref2[1])


def test_varlen_guard_bands():
    lens = [0, 37, 300, 1, 129, 64]
    H, d, chunk = 2, 64, 64
    T = sum(lens)
    inp = workloads.prefill_inputs(1, H, T, d, d, torch.bfloat16, api.LA_GATE_DIAG, seed=970,
                                   device=DEV)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int32,
                      device=DEV)
    N, maxlen = len(lens), max(lens)
    ref = api.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], cu, maxlen,
                               gate_mode=api.LA_GATE_DIAG, log_alpha=inp["log_alpha"],
                               chunk=chunk, segments=2)
    desc = api.make_desc(N, H, T, d, d, api.LA_BF16, 0, False, 2)
    need = api.la_chunk_fwd_varlen_workspace_bytes(desc, maxlen, chunk)
    out, S, ws = Guarded((1, H, T, d), torch.bfloat16), Guarded((N, H, d, d), torch.float32), \
        workspace(need)
    st = api.la_chunk_fwd_varlen(desc, cu.data_ptr(), maxlen, inp["q"].data_ptr(),
                                 inp["k"].data_ptr(), inp["v"].data_ptr(), api.LA_GATE_DIAG,
                                 inp["log_alpha"].data_ptr(), None, None, chunk, out.ptr, S.ptr,
                                 None, ws.ptr, need, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out")
    S.check("S_final")
    ws.check("workspace", written=False)
    assert torch.equal(out.t, ref[0].view(1, H, T, d)) and torch.equal(S.t, ref[1])


@pytest.mark.parametrize("d,dt,normalize", [(128, torch.bfloat16, True), (16, torch.float32, False),
                                            (64, torch.bfloat16, False)])
def test_decode_guard_bands(d, dt, normalize):
    B, H = 5, 3
    S0, z0 = workloads.decode_state(B, H, d, d, seed=980, device=DEV, with_z=normalize)
    q, k, v, la = workloads.decode_tokens(B, H, d, d, 1, seed=981, device=DEV, dtype=dt, gate=True)
    q, k, v, la = q[0], k[0], v[0], la[0]
    phi = 1 if normalize else 0
    Sr = S0.clone()
    zr = z0.clone() if normalize else None
    ref = api.decode_step(q, k, v, Sr, zr, gate_mode=api.LA_GATE_DIAG, log_alpha=la, phi=phi)
    desc = api.make_desc(B, H, 1, d, d, api.LA_BF16 if dt == torch.bfloat16 else api.LA_F32,
                         phi, normalize, 0)
    S = Guarded((B, H, d, d), torch.float32, init=S0)
    z = Guarded((B, H, d), torch.float32, init=z0) if normalize else None
    out = Guarded((B, H, d), dt)
    st = api.la_decode_step(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), api.LA_GATE_DIAG,
                            la.data_ptr(), S.ptr, None if z is None else z.ptr, out.ptr,
                            _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    S.check("S")
    out.check("out")
    assert torch.equal(S.t, Sr) and torch.equal(out.t, ref)
    if normalize:
        z.check("z")
        assert torch.equal(z.t, zr)


def test_delta_guard_bands():
    B, H, L, d = 2, 2, 3 * 64 + 11, 128
    inp = workloads.delta_inputs(B, H, L, d, d, torch.bfloat16, seed=990, device=DEV,
                                 with_state=True)
    ref = api.delta_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], S0=inp["S0"])
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 0)
    out, S = Guarded((B, H, L, d), torch.bfloat16), Guarded((B, H, d, d), torch.float32)
    st = api.la_delta_fwd(desc, inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                          inp["beta"].data_ptr(), inp["S0"].data_ptr(), out.ptr, S.ptr, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out")
    S.check("S_final")
    assert torch.equal(out.t, ref[0]) and torch.equal(S.t, ref[1])
    # one decode step from the final state
    q1, k1, v1 = (x[:, :, -1].contiguous() for x in (inp["q"], inp["k"], inp["v"]))
    b1 = inp["beta"][:, :, -1].contiguous()
    Sr = ref[1].clone()
    o1 = api.delta_decode_step(q1, k1, v1, b1, Sr)
    ddesc = api.make_desc(B, H, 1, d, d, api.LA_BF16, 0, False, 0)
    Sg, og = Guarded((B, H, d, d), torch.float32, init=ref[1]), Guarded((B, H, d), torch.bfloat16)
    st = api.la_delta_decode_step(ddesc, q1.data_ptr(), k1.data_ptr(), v1.data_ptr(),
                                  b1.data_ptr(), Sg.ptr, og.ptr, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    Sg.check("S")
    og.check("out")
    assert torch.equal(Sg.t, Sr) and torch.equal(og.t, o1)


@pytest.mark.parametrize("mode,d", [(api.LA_GATE_DIAG, 128), (api.LA_GATE_GAMMA, 64),
                                    (api.LA_GATE_SCALAR, 32)])
def test_train_and_backward_guard_bands(mode, d):
    B, H, L = 1, 2, 3 * 64 + 21
    dt = torch.bfloat16
    inp = workloads.prefill_inputs(B, H, L, d, d, dt, mode, seed=1000 + d, device=DEV,
                                   with_state=True)
    grads = workloads.backward_inputs(B, H, L, d, d, dt, seed=1001, device=DEV,
                                      with_state_grad=True)
    keep = []
    gate, gamma = _gate(mode, inp, H, keep)
    la = inp["log_alpha"] if mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR) else None
    S0, dS = inp["S0"], grads["dS_final"]
    rout, rS, rstates = api.chunk_fwd_train(inp["q"], inp["k"], inp["v"], gate_mode=mode,
                                            gamma=gamma, log_alpha=la, S0=S0, segments=2)
    ref = api.chunk_bwd(inp["q"], inp["k"], inp["v"], grads["dout"], gate_mode=mode,
                        gamma=gamma, log_alpha=la, S0=S0, dS_final=dS, segments=2,
                        states=rstates)
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 2)
    # the training forward into guarded outputs and a guarded state buffer
    nst = api.la_chunk_train_states_bytes(desc)
    fneed = api.la_chunk_fwd_workspace_bytes(desc, api.la_chunk_bwd_chunk(desc))
    out, Sf = Guarded((B, H, L, d), dt), Guarded((B, H, d, d), torch.float32)
    states, fws = workspace(nst), workspace(fneed)
    st = api.la_chunk_fwd_train(desc, inp["q"].data_ptr(), inp["k"].data_ptr(),
                                inp["v"].data_ptr(), mode, gate, S0.data_ptr(), out.ptr, Sf.ptr,
                                states.ptr, nst, fws.ptr, fneed, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    out.check("out (train)")
    Sf.check("S_final (train)")
    states.check("states", written=False)
    assert torch.equal(out.t, rout) and torch.equal(Sf.t, rS)
    nw = nst // 4
    assert torch.equal(states.t[:nw].view(torch.int32), rstates[:nw].view(torch.int32))
    fws.check("workspace (train)", written=False)
    # the backward from those states, every gradient guarded
    bneed = api.la_chunk_bwd_workspace_bytes(desc)
    gq, gk, gv = (Guarded((B, H, L, d), dt) for _ in range(3))
    gla = None
    if mode == api.LA_GATE_DIAG:
        gla = Guarded((B, H, L, d), torch.float32)
    elif mode == api.LA_GATE_SCALAR:
        gla = Guarded((B, H, L), torch.float32)
    gS0, bws = Guarded((B, H, d, d), torch.float32), workspace(bneed)
    st = api.la_chunk_bwd(desc, inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                          grads["dout"].data_ptr(), mode, gate, S0.data_ptr(), dS.data_ptr(),
                          states.ptr, gq.ptr, gk.ptr, gv.ptr, None if gla is None else gla.ptr,
                          gS0.ptr, bws.ptr, bneed, _stream())
    assert st == api.LA_OK, api.la_last_error_message()
    for name, gbuf in (("dq", gq), ("dk", gk), ("dv", gv), ("dS0", gS0)):
        gbuf.check(name)
        assert torch.equal(gbuf.t, ref[name]), name
    if gla is not None:
        gla.check("dlog_alpha")
        assert torch.equal(gla.t, ref["dlog_alpha"])
    bws.check("workspace (backward)", written=False)
