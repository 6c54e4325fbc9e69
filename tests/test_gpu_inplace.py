"""In-place final states: the ABI lets S_final (and z_final) alias S0 (and
z0) for the prefill and the delta rule's prefill.  The aliased call must
give what the out-of-place call gives, bit for bit, with one segment per
(b,h) (the main pass reads its initial state before it writes the final
one) and with several (the segment scan reads S0 before the main pass
runs)."""
import pytest
import torch

from recurrent_attention_amd import api, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    api.load_library()


@pytest.mark.parametrize("segments", [1, 0])
@pytest.mark.parametrize("mode,normalize,phi", [(api.LA_GATE_DIAG, False, 0),
                                                 (api.LA_GATE_GAMMA, False, 0),
                                                 (api.LA_GATE_NONE, True, 1)])
def test_prefill_final_state_in_place(mode, normalize, phi, segments):
    dev = "cuda"
    B, H, L, d = 2, 4, 1000, 64
    inp = workloads.prefill_inputs(B, H, L, d, d, torch.bfloat16, mode, seed=51, device=dev,
                                   with_state=True)
    gamma = [0.9, 0.99, 0.5, 0.97] if mode == api.LA_GATE_GAMMA else None
    S0 = inp["S0"].to(dev)
    z0 = (1.0 + inp["z0"].abs()).to(dev) if normalize else None
    kw = dict(gate_mode=mode, gamma=gamma, log_alpha=inp.get("log_alpha"), chunk=64, phi=phi,
              normalize=normalize, segments=segments)
    out_ref, S_ref, z_ref = api.chunk_fwd(inp["q"], inp["k"], inp["v"], S0=S0, z0=z0, **kw)
    S = S0.clone()
    z = z0.clone() if normalize else None
    out, S_ret, z_ret = api.chunk_fwd(inp["q"], inp["k"], inp["v"], S0=S, z0=z, S_final=S,
                                      z_final=z, **kw)
    torch.cuda.synchronize()
    assert S_ret.data_ptr() == S.data_ptr()
    assert torch.equal(out, out_ref)
    assert torch.equal(S, S_ref)
    if normalize:
        assert torch.equal(z, z_ref)


def test_delta_final_state_in_place():
    dev = "cuda"
    inp = workloads.delta_inputs(2, 4, 700, 64, 64, torch.bfloat16, seed=52, device=dev,
                                 with_state=True)
    out_ref, S_ref = api.delta_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], S0=inp["S0"])
    S = inp["S0"].clone()
    out, _ = api.delta_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], S0=S, S_final=S)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    assert torch.equal(S, S_ref)
