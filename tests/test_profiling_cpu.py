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
