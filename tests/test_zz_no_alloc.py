"""The prefill entry point that allocates nothing (la_chunk_fwd_noalloc),
called through the C ABI: its segment workspace is the library's static
scratch array instead of a caller buffer.  On the same inputs it must give
what la_chunk_fwd gives with a workspace of its own -- the same kernels on
the same segment plan, so bit for bit, which is tighter than the parity
tolerance -- on consecutive calls that reuse the scratch, the second one
smaller than the first (so it runs over slots the first call left
behind)."""
import ctypes

import pytest
import torch

from recurrent_attention_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(fn_noalloc, inp, mode, gamma, chunk, phi, normalize, segments, S0, z0):
    """One prefill through the raw C entry points; returns out, S_final, z_final."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    desc = api.make_desc(B, H, L, dk, dv, api.LA_BF16 if q.dtype == torch.bfloat16 else api.LA_F32,
                         phi, normalize, segments)
    out = torch.full((B, H, L, dv), float("nan"), dtype=q.dtype, device=dev)
    S = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    z = torch.full((B, H, dk), float("nan"), dtype=torch.float32, device=dev) if normalize else None
    keep = None
    if mode == api.LA_GATE_GAMMA:
        keep = torch.tensor(gamma, dtype=torch.float32)
        g = ctypes.c_void_p(keep.data_ptr())
    elif mode in (api.LA_GATE_DIAG, api.LA_GATE_SCALAR):
        g = inp["log_alpha"].data_ptr()
    else:
        g = None
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    head = (desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), mode, g, _ptr(S0), _ptr(z0), chunk,
            out.data_ptr(), S.data_ptr(), _ptr(z))
    if fn_noalloc:
        st = api.la_chunk_fwd_noalloc(*head, sp)
    else:
        need = api.la_chunk_fwd_workspace_bytes(desc, chunk)
        ws = torch.empty(max(need // 4, 4), dtype=torch.float32, device=dev)
        st = api.la_chunk_fwd(*head, ws.data_ptr(), ws.numel() * 4, sp)
    assert st == api.LA_OK, api.la_last_error_message()
    torch.cuda.synchronize()
    del keep
    return out, S, z


CASES = [
    # (B, H, L, d, mode, chunk, phi, normalize, segments): the first of each
    # pair fills many scratch slots, the second is smaller
    [(1, 16, 4096 + 37, 128, api.LA_GATE_DIAG, 64, 0, False, 0),
     (1, 4, 1000, 64, api.LA_GATE_DIAG, 64, 0, False, 3)],
    [(2, 8, 3000, 64, api.LA_GATE_NONE, 64, 1, True, 0),
     (1, 2, 700, 32, api.LA_GATE_NONE, 32, 1, True, 5)],
    [(2, 16, 2048, 128, api.LA_GATE_GAMMA, 64, 0, False, 0),
     (1, 3, 333, 128, api.LA_GATE_SCALAR, 16, 0, False, 4)],
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_workspace_entry_point(case):
    dev = "cuda"
    for n, (B, H, L, d, mode, chunk, phi, normalize, segments) in enumerate(CASES[case]):
        print(f"no-alloc case {case}.{n}: B={B} H={H} L={L} d={d} mode={mode} chunk={chunk} "
              f"segments={segments}", flush=True)
        inp = workloads.prefill_inputs(B, H, L, d, d, torch.bfloat16, mode, seed=70 + 3 * case + n,
                                       device=dev, with_state=True)
        gamma = [0.9 + 0.09 * (h % 2) for h in range(H)] if mode == api.LA_GATE_GAMMA else None
        S0 = inp["S0"]
        z0 = (1.0 + inp["z0"].abs()) if normalize else None
        desc = api.make_desc(B, H, L, d, d, api.LA_BF16, phi, normalize, segments)
        # the case exercises the scratch: more than one segment per (b,h)
        assert api.la_chunk_fwd_segments(desc, chunk) > 1
        assert api.la_chunk_fwd_workspace_bytes(desc, chunk) <= api.LA_NOALLOC_SCRATCH_BYTES
        ref = _call(False, inp, mode, gamma, chunk, phi, normalize, segments, S0, z0)
        got = _call(True, inp, mode, gamma, chunk, phi, normalize, segments, S0, z0)
        for a, b in zip(got, ref):
            if b is None:
                assert a is None
                continue
            assert torch.isfinite(b.float()).all()
            assert torch.equal(a, b)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    dev = "cuda"
    # 64 x 16 heads x 8 segments at d = 128: 8192 slots of 66 KB
    B, H, L, d = 64, 16, 512, 128
    desc = api.make_desc(B, H, L, d, d, api.LA_BF16, 0, False, 8)
    assert api.la_chunk_fwd_workspace_bytes(desc, 64) > api.LA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = api.la_chunk_fwd_noalloc(desc, q.data_ptr(), q.data_ptr(), q.data_ptr(), 0, None, None,
                                  None, 64, out.data_ptr(), None, None, sp)
    assert st == api.LA_ERR_UNSUPPORTED
    assert "scratch" in api.la_last_error_message()
