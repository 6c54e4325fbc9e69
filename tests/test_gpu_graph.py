"""The library's launches captured in a HIP graph and replayed.

A caller that captures its step into a graph must get, on every replay,
exactly what the direct call gives: the prefill (state pass, segment scan
and main pass: no allocation and no memset inside) and the in-place decode
step.  Each replay runs after eager work and a synchronisation of the
program's own, and its outputs are compared bit for bit with the direct
call's on the same inputs."""
import pytest
import torch

from recurrent_attention_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


def test_prefill_graph_replays_equal_the_direct_call():
    dev = "cuda"
    inp = workloads.prefill_inputs(1, 4, 3000, 128, 128, torch.bfloat16, api.LA_GATE_DIAG,
                                   seed=41, device=dev)
    q, k, v, la = inp["q"], inp["k"], inp["v"], inp["log_alpha"]
    out_ref, S_ref, _ = api.chunk_fwd(q, k, v, gate_mode=api.LA_GATE_DIAG, log_alpha=la, chunk=64)
    torch.cuda.synchronize()
    assert api.la_chunk_fwd_segments(
        api.make_desc(1, 4, 3000, 128, 128, api.LA_BF16, 0, False, 0), 64) > 1
    out = torch.empty_like(out_ref)
    S = torch.empty_like(S_ref)
    desc = api.make_desc(1, 4, 3000, 128, 128, api.LA_BF16, 0, False, 0)
    need = api.la_chunk_fwd_workspace_bytes(desc, 64)
    ws = torch.empty(need // 4 + 4, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        api.chunk_fwd(q, k, v, gate_mode=api.LA_GATE_DIAG, log_alpha=la, chunk=64, out=out,
                      S_final=S, workspace=ws, stream=side)
    for i in range(4):
        # the program's own eager work between replays
        out.fill_(float(i + 1))
        S.zero_()
        junk = (q.float() * (i + 1)).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, out_ref), f"replay {i}: out differs"
        assert torch.equal(S, S_ref), f"replay {i}: S_final differs"


def test_decode_graph_replays_equal_direct_steps():
    dev = "cuda"
    nseq, H, d, steps = 8, 4, 128, 5
    S0, _ = workloads.decode_state(nseq, H, d, d, seed=43, device=dev)
    qd, kd, vd, lad = workloads.decode_tokens(nseq, H, d, d, 1, seed=44, device=dev, gate=True)
    q, k, v, la = qd[0], kd[0], vd[0], lad[0]
    S_dir = S0.clone()
    S_gr = S0.clone()
    out_gr = torch.empty((nseq, H, d), dtype=torch.bfloat16, device=dev)
    # capture one step; replays continue the same state in place
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    S_cap = S0.clone()
    with torch.cuda.graph(g, stream=side):
        api.decode_step(q, k, v, S_cap, gate_mode=api.LA_GATE_DIAG, log_alpha=la, out=out_gr,
                        stream=side)
    S_cap.copy_(S0)            # capture does not run the step; start from S0
    for i in range(steps):
        o_dir = api.decode_step(q, k, v, S_dir, gate_mode=api.LA_GATE_DIAG, log_alpha=la)
        torch.cuda.synchronize()
        out_gr.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_gr, o_dir), f"step {i}: out differs"
        assert torch.equal(S_cap, S_dir), f"step {i}: state differs"
    del S_gr
