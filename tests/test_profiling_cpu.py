"""The kernel-family names of the profiling summaries cover every kernel the
library builds: each chunk_kernel instantiation in the built library (its
host-side symbols, demangled) falls into exactly the family its template
flags say (outputs -> chunk_main, or chunk_sub with the sub-chunk path;
state-only -> chunk_store when it stores every boundary state, else
chunk_state), and the other kernels into theirs.
A kernel left out of every family would drop out of the trace tables."""
import os
import re
import shutil
import subprocess

import pytest

from recurrent_attention_amd import api
from recurrent_attention_amd.profiling import family

_CFG = re.compile(r"la::chunk_kernel<la::ChunkCfg<\d+, \d+, \d+, \w+, \d, (\w+), \d+>, "
                  r"(\w+), (\w+), (\w+), (\w+), (\w+)>")


def _kernel_names():
    lib = api.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-C", "--defined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    names = set()
    for line in out.splitlines():
        m = re.search(r"void (la::\w+<.*>\(la::\w+\))$", line)
        if m:
            names.add("void " + m.group(1))
    return names


def test_every_chunk_kernel_has_its_family():
    names = [n for n in _kernel_names() if "la::chunk_kernel<" in n]
    assert len(names) > 100
    seen = set()
    for n in names:
        m = _CFG.search(n)
        assert m, n
        sonly, _elu1, _rev, store, _epi, sub = m.groups()
        want = (("chunk_sub" if sub == "true" else "chunk_main") if sonly == "false"
                else ("chunk_store" if store == "true" else "chunk_state"))
        assert family(n) == want, (n, family(n))
        seen.add(want)
    assert seen == {"chunk_main", "chunk_sub", "chunk_state", "chunk_store"}


def test_other_kernels_have_their_families():
    names = _kernel_names()
    want = {"la::state_scan_kernel<": "state_scan", "la::bwd_kernel<": "chunk_bwd",
            "la::delta_chunk_kernel<": "delta_chunk", "la::delta_decode_kernel<": "delta_decode",
            "la::decode_kernel<": "decode"}
    for prefix, fam in want.items():
        hits = [n for n in names if prefix in n]
        assert hits, prefix
        for n in hits:
            assert family(n) == fam, (n, family(n))
    assert family("void la::(anonymous namespace)::seq_order_kernel(int const*, int, int, int, int, int*)") == "seq_order"


def test_trace_table_groups_launch_shapes(tmp_path):
    # one kernel run with two grids (two parts of a program) gives two rows,
    # each with the mean and median of its own dispatches; the copy and
    # unknown kernels drop out
    from recurrent_attention_amd.profiling import trace_table
    name = "void la::decode_kernel<128, 128, true, 1>(la::DecodeParams)"
    rows = [(name, 8192 * 512, 512, 0, 100_000), (name, 8192 * 512, 512, 0, 120_000),
            (name, 32 * 512, 512, 0, 7_000), ("__amd_rocclr_copyBuffer", 64, 64, 0, 9),
            ("void other(int)", 64, 64, 0, 9)]
    path = tmp_path / "t_kernel_trace.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n")
        for n, g, w, a, b in rows:
            f.write(f'"{n}",{g},{w},{a},{b}\n')
    out = trace_table(str(path)).splitlines()
    assert len(out) == 4
    assert "| 32 x 512 | 1 | 7.00 | 7.00 | 7.00 | 7.00 |" in out[2]
    assert "| 8192 x 512 | 2 | 110.00 | 110.00 | 100.00 | 120.00 |" in out[3]


def test_derived_counter_ratios():
    from recurrent_attention_amd.profiling import derived
    # GRBM summed over 8 XCDs: 8000 -> 1000 busy cycles per XCD; 256 CUs x 4
    # SIMDs x 1000 cycles = 1.024e6 SIMD-cycles, a quarter of them in MFMA
    cs = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 256000.0,
          "SQ_INSTS_VALU_MFMA_MOPS_BF16": 10.0, "SQ_LDS_BANK_CONFLICT": 5.0,
          "SQ_LDS_IDX_ACTIVE": 50.0}
    d = derived(cs)
    assert d["mfma_busy_pct"] == 25.0
    assert d["bf16_flops"] == 5120.0
    assert d["lds_conflict_pct"] == 10.0
    assert derived({}) == {}
