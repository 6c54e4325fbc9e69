"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before anything is
enqueued (fake, never-dereferenced pointers are enough for that)."""
import ctypes
import os
import re

import pytest

from recurrent_attention_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

A = 0x10000          # a 16-byte aligned fake device address
MIS = 0x10004        # a misaligned one


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(api.EXPORTED) == _declared()


def test_library_exports_every_declared_symbol():
    lib = api.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    assert api.la_version() == 1


def test_status_strings():
    assert api.la_status_string(0) == "ok"
    assert "invalid" in api.la_status_string(1)
    assert "unsupported" in api.la_status_string(2)
    assert "HIP" in api.la_status_string(3)


def _desc(**kw):
    base = dict(B=1, H=2, L=100, dk=64, dv=64, dtype=api.LA_BF16, phi=0,
                normalize=False, segments=0)
    base.update(kw)
    return api.make_desc(**base)


def _chunk(desc, gate_mode=0, gate=None, S0=None, z0=None, chunk=64, out=A,
           S_final=None, z_final=None, ws=None, ws_bytes=0, q=A, k=A, v=A):
    return api.la_chunk_fwd(desc, q, k, v, gate_mode, gate, S0, z0, chunk, out,
                            S_final, z_final, ws, ws_bytes, None)


def _gamma(vals):
    arr = (ctypes.c_float * len(vals))(*vals)
    return ctypes.cast(arr, ctypes.c_void_p), arr


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, api.LA_ERR_INVALID), ("H", -1, api.LA_ERR_INVALID),
    ("L", 0, api.LA_ERR_INVALID), ("dk", 0, api.LA_ERR_INVALID),
    ("dtype", 7, api.LA_ERR_INVALID), ("phi", 3, api.LA_ERR_INVALID),
    ("normalize", 2, api.LA_ERR_INVALID), ("segments", -1, api.LA_ERR_INVALID),
    ("dk", 48, api.LA_ERR_UNSUPPORTED), ("dv", 32, api.LA_ERR_UNSUPPORTED),
])
def test_chunk_rejects_bad_descriptor(field, value, status):
    d = _desc(**{field: value})
    assert _chunk(d) == status
    assert api.la_last_error_message() != ""


def test_chunk_rejects_null_descriptor():
    lib = api.load_library()
    st = lib.la_chunk_fwd(None, A, A, A, 0, None, None, None, 64, A, None, None,
                          None, 0, None)
    assert st == api.LA_ERR_INVALID


def test_bf16_needs_dk_32():
    assert _chunk(_desc(dk=16, dv=16)) == api.LA_ERR_UNSUPPORTED
    assert "dk >= 32" in api.la_last_error_message()


def test_bf16_decode_takes_d16():
    # the decode step runs on the vector units: bf16 at d = 16 passes the
    # host checks (a NULL S is the first thing refused after them)
    d = _desc(dk=16, dv=16, L=1)
    assert api.la_decode_step(d, A, A, A, 0, None, None, None, A, None) == api.LA_ERR_INVALID
    assert "non-NULL" in api.la_last_error_message()
    # the delta rule's decode is built for bf16 at d >= 32 only
    assert api.la_delta_decode_step(d, A, A, A, A, A, A, None) == api.LA_ERR_UNSUPPORTED


def _noalloc(desc, chunk=64, gate_mode=0, gate=None, q=A, out=A):
    return api.la_chunk_fwd_noalloc(desc, q, A, A, gate_mode, gate, None, None, chunk, out,
                                    None, None, None)


def test_noalloc_validates_on_the_host():
    # every argument check of la_chunk_fwd runs before the scratch is touched
    assert _noalloc(_desc(B=0)) == api.LA_ERR_INVALID
    assert _noalloc(_desc(), q=None) == api.LA_ERR_INVALID
    assert _noalloc(_desc(), q=MIS) == api.LA_ERR_INVALID
    assert _noalloc(_desc(), chunk=8) == api.LA_ERR_UNSUPPORTED
    assert _noalloc(_desc(), gate_mode=api.LA_GATE_DIAG) == api.LA_ERR_INVALID


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # 64 x 16 heads x 8 segments of 66 KB each at d = 128
    d = _desc(B=64, H=16, L=512, dk=128, dv=128, segments=8)
    assert api.la_chunk_fwd_workspace_bytes(d, 64) > api.LA_NOALLOC_SCRATCH_BYTES
    assert _noalloc(d) == api.LA_ERR_UNSUPPORTED
    assert "scratch" in api.la_last_error_message()


@pytest.mark.parametrize("chunk", [0, 8, 24, 144, -16])
def test_chunk_rejects_unsupported_chunk(chunk):
    assert _chunk(_desc(), chunk=chunk) == api.LA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dk,dtype,chunk,ok", [
    (64, api.LA_BF16, 48, True), (64, api.LA_BF16, 128, True), (128, api.LA_BF16, 112, False),
    (128, api.LA_BF16, 64, True), (32, api.LA_F32, 96, True), (64, api.LA_F32, 80, False)])
def test_chunk_lengths_by_shape(dk, dtype, chunk, ok):
    # multiples of 16 up to 64 everywhere; above 64 where the 128-token tile
    # is built (bf16 at dk <= 64, fp32 at dk <= 32)
    d = _desc(dk=dk, dv=dk, dtype=dtype, L=1000)
    assert (api.la_chunk_fwd_segments(d, chunk) > 0) == ok
    st = _chunk(d, chunk=chunk, q=None)          # NULL q: refused after the chunk check
    assert st == (api.LA_ERR_INVALID if ok else api.LA_ERR_UNSUPPORTED)


def test_chunk_rejects_null_and_misaligned_pointers():
    d = _desc(L=64)
    assert _chunk(d, q=None) == api.LA_ERR_INVALID
    assert _chunk(d, out=None) == api.LA_ERR_INVALID
    assert _chunk(d, k=MIS) == api.LA_ERR_INVALID
    assert "aligned" in api.la_last_error_message()
    assert _chunk(d, S0=MIS) == api.LA_ERR_INVALID


def test_chunk_gate_validation():
    d = _desc(L=64, H=2)
    assert _chunk(d, gate_mode=api.LA_GATE_GAMMA, gate=None) == api.LA_ERR_INVALID
    p, keep = _gamma([0.5, 1.5])
    assert _chunk(d, gate_mode=api.LA_GATE_GAMMA, gate=p) == api.LA_ERR_INVALID
    assert "outside [0, 1]" in api.la_last_error_message()
    p, keep = _gamma([0.5, float("nan")])
    assert _chunk(d, gate_mode=api.LA_GATE_GAMMA, gate=p) == api.LA_ERR_INVALID
    p, keep = _gamma([-0.1, 0.5])
    assert _chunk(d, gate_mode=api.LA_GATE_GAMMA, gate=p) == api.LA_ERR_INVALID
    assert _chunk(d, gate_mode=api.LA_GATE_DIAG, gate=None) == api.LA_ERR_INVALID
    assert _chunk(d, gate_mode=api.LA_GATE_DIAG, gate=MIS) == api.LA_ERR_INVALID
    assert _chunk(d, gate_mode=5, gate=A) == api.LA_ERR_INVALID
    big = _desc(L=64, H=257)
    p, keep = _gamma([0.5] * 257)
    assert _chunk(big, gate_mode=api.LA_GATE_GAMMA, gate=p) == api.LA_ERR_UNSUPPORTED


def test_chunk_normaliser_contract():
    d = _desc(L=64, normalize=False)
    assert _chunk(d, z0=A) == api.LA_ERR_INVALID
    assert _chunk(d, z_final=A) == api.LA_ERR_INVALID


def test_chunk_workspace_contract():
    d = _desc(B=1, H=1, L=4096, segments=4)
    need = api.la_chunk_fwd_workspace_bytes(d, 64)
    assert need == 1 * 1 * 4 * (64 * 64 + 2 * 64) * 4 + 16   # slots, then 4 segment flags
    assert _chunk(d, ws=None) == api.LA_ERR_INVALID
    assert _chunk(d, ws=A, ws_bytes=need - 4) == api.LA_ERR_INVALID
    assert _chunk(d, ws=MIS, ws_bytes=need) == api.LA_ERR_INVALID
    too_many = _desc(L=100, segments=3)   # 2 chunks of 64
    assert _chunk(too_many) == api.LA_ERR_INVALID


@pytest.mark.parametrize("B,H,L,chunk,segments,P", [
    (1, 16, 32768, 64, 0, 16),    # 16 pairs -> 16 segments of 32 chunks
    (2, 16, 8192, 64, 0, 8),
    (4, 8, 2048, 64, 0, 8),
    (1, 1, 64, 16, 0, 1),         # 4 chunks: one segment (at least 4 chunks each)
    (1, 1, 160, 16, 0, 2),        # 10 chunks: two segments of 5
    (1, 1, 64, 16, 6, 4),         # asked for: never more segments than chunks
    (1, 1, 100, 64, 5, 2),
    (256, 1, 100, 16, 0, 1),
    (1, 1, 1000, 64, 3, 3),       # 16 chunks: 6 + 6 + 4
    (1, 1, 1000, 64, 5, 4),       # 16 chunks: cps 4 -> 4 segments
])
def test_segment_plan(B, H, L, chunk, segments, P):
    d = _desc(B=B, H=H, L=L, segments=segments)
    assert api.la_chunk_fwd_segments(d, chunk) == P
    ws = api.la_chunk_fwd_workspace_bytes(d, chunk)
    # segment slots (several segments only), then one int32 flag per
    # segment, each part rounded up to 16 bytes
    flags = -(-B * H * P * 4 // 16) * 16
    assert ws == (0 if P == 1 else B * H * P * (64 * 64 + 128) * 4) + flags


def test_decode_validation():
    d = _desc(L=2)
    st = api.la_decode_step(d, A, A, A, 0, None, A, None, A, None)
    assert st == api.LA_ERR_INVALID and "L == 1" in api.la_last_error_message()
    d = _desc(L=1, normalize=True)
    assert api.la_decode_step(d, A, A, A, 0, None, A, None, A, None) == api.LA_ERR_INVALID
    d = _desc(L=1, normalize=False)
    assert api.la_decode_step(d, A, A, A, 0, None, A, A, A, None) == api.LA_ERR_INVALID
    assert api.la_decode_step(d, A, A, A, 0, None, None, None, A, None) == api.LA_ERR_INVALID
    assert api.la_decode_step(d, A, A, A, 0, None, MIS, None, A, None) == api.LA_ERR_INVALID
    p, keep = _gamma([2.0, 0.5])
    assert api.la_decode_step(d, A, A, A, api.LA_GATE_GAMMA, p, A, None, A,
                              None) == api.LA_ERR_INVALID


def test_profile_interface_without_launches():
    api.la_profile_begin()
    assert api.la_profile_query("chunk_main") == (0, 0.0)
    api.la_profile_end()
    with pytest.raises(api.LaError):
        api.la_profile_query("no_such_kernel")


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        api.chunk_fwd(q, q, q)


def _bwd(desc, gate_mode=0, gate=None, S0=None, dSf=None, dla=None, dS0=None,
         ws=A, ws_bytes=1 << 40, q=A, k=A, v=A, do=A, dq=A, dk=A, dv=A):
    return api.la_chunk_bwd(desc, q, k, v, do, gate_mode, gate, S0, dSf, None, dq, dk, dv,
                            dla, dS0, ws, ws_bytes, None)


def test_bwd_chunk_and_workspace_size():
    # states at every chunk boundary: (nchunks + 1) d x d per (b,h) in the
    # input element type (the state before each chunk and the final one),
    # plus the fp32 segment slots
    d = _desc(B=1, H=2, L=1000, dk=64, dv=64, dtype=api.LA_BF16, segments=1)
    assert api.la_chunk_bwd_chunk(d) == 64
    assert api.la_chunk_bwd_workspace_bytes(d) == 2 * (16 + 1) * 64 * 64 * 2
    d = _desc(B=1, H=2, L=1000, dk=64, dv=64, dtype=api.LA_F32, segments=4)
    assert api.la_chunk_bwd_workspace_bytes(d) == (
        2 * (16 + 1) * 64 * 64 * 4 + 2 * 4 * (64 * 64 + 128) * 4)
    f32_128 = _desc(dk=128, dv=128, dtype=api.LA_F32)
    assert api.la_chunk_bwd_chunk(f32_128) == 32
    assert api.la_chunk_bwd_workspace_bytes(_desc(L=0)) == 0


def test_bwd_validation():
    d = _desc(L=128)
    assert _bwd(_desc(L=128, normalize=True)) == api.LA_ERR_UNSUPPORTED
    assert _bwd(_desc(L=0)) == api.LA_ERR_INVALID
    for name in ("q", "k", "v", "do", "dq", "dk", "dv"):
        assert _bwd(d, **{name: None}) == api.LA_ERR_INVALID
        assert _bwd(d, **{name: MIS}) == api.LA_ERR_INVALID
    assert _bwd(d, S0=MIS) == api.LA_ERR_INVALID
    assert _bwd(d, dSf=MIS) == api.LA_ERR_INVALID
    assert _bwd(d, dS0=MIS) == api.LA_ERR_INVALID
    # the gate gradient goes with the diagonal gate and nothing else
    assert _bwd(d, gate_mode=api.LA_GATE_DIAG, gate=A, dla=None) == api.LA_ERR_INVALID
    assert _bwd(d, gate_mode=api.LA_GATE_NONE, dla=A) == api.LA_ERR_INVALID
    p, keep = _gamma([0.5, 1.5])
    assert _bwd(d, gate_mode=api.LA_GATE_GAMMA, gate=p) == api.LA_ERR_INVALID
    need = api.la_chunk_bwd_workspace_bytes(d)
    assert _bwd(d, ws=None) == api.LA_ERR_INVALID
    assert _bwd(d, ws_bytes=need - 4) == api.LA_ERR_INVALID
    assert _bwd(d, ws=MIS) == api.LA_ERR_INVALID
    assert _bwd(_desc(L=128, segments=3)) == api.LA_ERR_INVALID   # 2 chunks



def _varlen(desc, cu=A, max_seqlen=64, chunk=64, ws=None, ws_bytes=0, q=A, out=A):
    return api.la_chunk_fwd_varlen(desc, cu, max_seqlen, q, A, A, 0, None, None, None, chunk,
                                   out, None, None, ws, ws_bytes, None)


def test_varlen_validation():
    d = _desc(B=3, H=2, L=300)
    assert _varlen(d, cu=None) == api.LA_ERR_INVALID
    assert _varlen(d, cu=A + 2) == api.LA_ERR_INVALID          # not 4-byte aligned
    assert _varlen(d, max_seqlen=0) == api.LA_ERR_INVALID
    assert _varlen(d, max_seqlen=301) == api.LA_ERR_INVALID
    assert _varlen(d, q=None) == api.LA_ERR_INVALID
    assert _varlen(d, chunk=40) == api.LA_ERR_UNSUPPORTED
    assert _varlen(_desc(B=3, H=2, L=300, segments=3), max_seqlen=100) == api.LA_ERR_INVALID
    assert _varlen(_desc(B=0, H=2, L=300)) == api.LA_ERR_INVALID


def test_varlen_workspace_plans_for_the_longest_sequence():
    # 3 sequences x 2 heads, longest 1000 tokens (16 chunks of 64): the
    # automatic plan gives every (sequence, head) ceil(256 / 6) = 43
    # segments, at most 16 / 4 = 4 (4 chunks or more each)
    d = _desc(B=3, H=2, L=1500)
    need = api.la_chunk_fwd_varlen_workspace_bytes(d, 1000, 64)
    # segment slots, the segment flags (int32), then the launch order of the
    # 3 sequences (int32), each 16-byte rounded
    assert need == 3 * 2 * 4 * (64 * 64 + 2 * 64) * 4 + 3 * 2 * 4 * 4 + 16
    # one segment each: the flags and the order array
    d1 = _desc(B=3, H=2, L=1500, segments=1)
    assert api.la_chunk_fwd_varlen_workspace_bytes(d1, 1000, 64) == 32 + 16
    assert _varlen(d1, max_seqlen=1000, ws=None) == api.LA_ERR_INVALID
    assert api.la_chunk_fwd_varlen_workspace_bytes(d, 1501, 64) == 0   # invalid
    assert _varlen(d, max_seqlen=1000, ws=None) == api.LA_ERR_INVALID
    assert _varlen(d, max_seqlen=1000, ws=A, ws_bytes=need - 16) == api.LA_ERR_INVALID


def test_groupnorm_validation():
    d = _desc(L=128)
    gn = api.LaGroupNorm(None, None, None, 1e-5)
    call = lambda g, chunk=64, desc=d: api.la_chunk_fwd_groupnorm(
        desc, A, A, A, 0, None, None, None, chunk, g, A, None, None, None, 0, None)
    assert call(None) == api.LA_ERR_INVALID
    assert call(gn, chunk=32) == api.LA_ERR_UNSUPPORTED
    assert call(api.LaGroupNorm(None, None, None, 0.0)) == api.LA_ERR_INVALID
    assert call(api.LaGroupNorm(MIS, None, None, 1e-5)) == api.LA_ERR_INVALID
    assert call(api.LaGroupNorm(None, None, MIS, 1e-5)) == api.LA_ERR_INVALID
    assert call(gn, desc=_desc(L=0)) == api.LA_ERR_INVALID


def test_delta_validation():
    d = _desc(L=100)
    fwd = lambda desc, q=A, beta=A, out=A, S0=None: api.la_delta_fwd(desc, q, A, A, beta, S0,
                                                                     out, None, None)
    assert fwd(_desc(L=100, phi=1)) == api.LA_ERR_UNSUPPORTED
    assert fwd(_desc(L=100, normalize=True)) == api.LA_ERR_UNSUPPORTED
    assert fwd(_desc(L=100, dk=48, dv=48)) == api.LA_ERR_UNSUPPORTED
    assert fwd(d, q=None) == api.LA_ERR_INVALID
    assert fwd(d, beta=None) == api.LA_ERR_INVALID
    assert fwd(d, beta=MIS) == api.LA_ERR_INVALID
    assert fwd(d, S0=MIS) == api.LA_ERR_INVALID
    dec = lambda desc, S=A: api.la_delta_decode_step(desc, A, A, A, A, S, A, None)
    assert dec(_desc(L=2)) == api.LA_ERR_INVALID
    assert dec(_desc(L=1), S=None) == api.LA_ERR_INVALID
    assert api.la_delta_chunk(_desc(dk=128, dv=128, dtype=api.LA_F32)) == 32
    assert api.la_delta_chunk(_desc(dk=128, dv=128, dtype=api.LA_BF16)) == 64


def test_train_forward_validation():
    d = _desc(L=1000, dk=64, dv=64, dtype=api.LA_BF16)
    # states: (ceil(1000/64) + 1) boundary states per (b,h), bf16
    assert api.la_chunk_train_states_bytes(d) == 2 * 17 * 64 * 64 * 2
    call = lambda desc, states=A, nbytes=1 << 40: api.la_chunk_fwd_train(
        desc, A, A, A, 0, None, None, A, None, states, nbytes, A, 1 << 40, None)
    assert call(_desc(L=1000, normalize=True)) == api.LA_ERR_UNSUPPORTED
    assert call(d, states=None) == api.LA_ERR_INVALID
    assert call(d, states=MIS) == api.LA_ERR_INVALID
    assert call(d, nbytes=100) == api.LA_ERR_INVALID
    assert api.la_chunk_bwd(d, A, A, A, A, 0, None, None, None, MIS, A, A, A, None, None, A,
                            1 << 40, None) == api.LA_ERR_INVALID


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_dk_ne_dv_pairs(dk, dv):
    # the bf16 prefill (chunks up to 64) and the decode step in either type
    d = _desc(dk=dk, dv=dv, L=1000)
    P = api.la_chunk_fwd_segments(d, 64)
    assert P == 4          # 16 chunks, 2 pairs: ceil(256 / 2) segments, at most 16 / 4
    assert api.la_chunk_fwd_workspace_bytes(d, 64) == 2 * P * (dk * dv + 2 * dk) * 4 + 2 * P * 4
    assert api.la_chunk_fwd_workspace_bytes(d, 128) == 0
    assert _chunk(d, chunk=128) == api.LA_ERR_UNSUPPORTED
    assert _chunk(_desc(dk=dk, dv=dv, dtype=api.LA_F32)) == api.LA_ERR_UNSUPPORTED
    for dt in (api.LA_BF16, api.LA_F32):
        dd = _desc(dk=dk, dv=dv, L=1, dtype=dt)
        assert api.la_decode_step(dd, A, A, A, 0, None, None, None, A, None) == api.LA_ERR_INVALID
        assert "non-NULL" in api.la_last_error_message()
    # the backward, the training forward and the delta rule need dk == dv
    assert _bwd(d) == api.LA_ERR_UNSUPPORTED
    assert api.la_chunk_bwd_workspace_bytes(d) == 0
    assert api.la_chunk_train_states_bytes(d) == 0
    assert api.la_delta_fwd(d, A, A, A, A, None, A, None, None) == api.LA_ERR_UNSUPPORTED


def test_other_dk_dv_pairs_unsupported():
    assert _chunk(_desc(dk=32, dv=64)) == api.LA_ERR_UNSUPPORTED
    assert api.la_decode_step(_desc(dk=32, dv=64, L=1), A, A, A, 0, None, A, None, A,
                              None) == api.LA_ERR_UNSUPPORTED
    assert api.la_decode_step(_desc(dk=128, dv=16, L=1), A, A, A, 0, None, A, None, A,
                              None) == api.LA_ERR_UNSUPPORTED
