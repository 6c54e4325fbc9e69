"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run on the CPU only.

* ``oracle.c`` built by gcc with ``-fsanitize=address,undefined`` runs the
  oracle's pin tests (every form: token loop, all-pairs, chunkwise,
  backward, delta rule) in a process that preloads gcc's sanitizer runtimes
  and loads that build through ``ORACLE_LIBRARY``.
* ``la_api.hip`` (the C ABI: argument validation, workspace planning, the
  launch set-up) built by hipcc with the sanitizers on its host pass only
  (``-Xarch_host`` before each ``-fsanitize=``), linked with the kernels of
  the regular build, runs the C-ABI tests in a process that preloads clang's
  sanitizer runtime and loads that build through ``LINATTN_LIBRARY``.

Undefined behaviour aborts (``-fno-sanitize-recover``).  Each side also runs
one planted out-of-bounds read of the caller's memory, to show that the
sanitizer is live in that process: it must stop the run with an ASan report.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
ORACLE_SAN = os.path.join(OUT, "liboracle_san.so")
LIB_SAN = os.path.join(OUT, "liblinattn_san.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _gcc_runtimes():
    libs = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
            for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in libs):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    return ":".join(libs)


def _clang_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    return found[-1]


def _build_oracle():
    os.makedirs(OUT, exist_ok=True)
    src = os.path.join(ROOT, "oracle", "oracle.c")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-pthread", "-Wall",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-o", ORACLE_SAN, src, "-lm"])


def _build_library():
    sys.path.insert(0, ROOT)
    from recurrent_attention_amd import build as B
    B.build(incremental=True)                       # the kernels of the regular build
    os.makedirs(OUT, exist_ok=True)
    obj = os.path.join(OUT, "la_api_san.o")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined",
                 "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    cflags = [f for f in B.CFLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.check_call([HIPCC] + cflags + host_san +
                          ["-c", os.path.join(B.CSRC, "la_api.hip"), "-o", obj],
                          stderr=subprocess.DEVNULL)
    kernels = [o for o in sorted(glob.glob(os.path.join(B.BUILD, "*.o")))
               if os.path.basename(o) != "la_api.o"]
    subprocess.check_call([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", LIB_SAN,
                           obj] + kernels)


def _run(cmd, env_extra):
    env = dict(os.environ)
    env.update(SAN_OPTS)
    env.update(env_extra)
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_oracle_under_address_and_ub_sanitizers():
    pre = _gcc_runtimes()
    _build_oracle()
    env = {"LD_PRELOAD": pre, "ORACLE_LIBRARY": ORACLE_SAN}
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_oracle_pins.py", "tests/test_oracle_backward.py",
              "tests/test_oracle_delta.py"], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
    # the sanitized build is the one loaded, and a read past the end of the
    # caller's q (the token loop told L = 9 for 8 tokens) is caught
    probe = (
        "import ctypes, numpy as np, oracle\n"
        "lib = oracle._load()\n"
        "maps = open('/proc/self/maps').read()\n"
        "assert 'liboracle_san.so' in maps and 'libasan' in maps, 'not the sanitized build'\n"
        "dp = ctypes.POINTER(ctypes.c_double)\n"
        "q = np.zeros((8, 4)); k = np.zeros((9, 4)); v = np.zeros((9, 4))\n"
        "out = np.zeros((9, 4)); S = np.zeros((4, 4))\n"
        "p = lambda a: a.ctypes.data_as(dp)\n"
        "print('probe: loaded', flush=True)\n"
        "lib.oracle_run(1, 1, 9, 4, 4, 0, None, None, 0, 0, p(q), p(k), p(v), None, None,\n"
        "               p(out), p(S), None, 1)\n")
    r = _run([sys.executable, "-c", probe], env)
    assert "probe: loaded" in r.stdout, r.stderr[-3000:]
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def test_c_abi_host_code_under_address_and_ub_sanitizers():
    pre = _clang_runtime()
    _build_library()
    env = {"LD_PRELOAD": pre, "LINATTN_LIBRARY": LIB_SAN}
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_abi_cpu.py"], env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
    # the sanitized build is the one loaded, and the validation's read of a
    # per-head decay array shorter than the heads it is told of is caught
    probe = (
        "import ctypes, numpy as np\n"
        "from recurrent_attention_amd import api\n"
        "api.load_library()\n"
        "maps = open('/proc/self/maps').read()\n"
        "assert 'liblinattn_san.so' in maps and 'clang_rt.asan' in maps, 'not the sanitized build'\n"
        "d = api.make_desc(1, 64, 100, 64, 64, api.LA_BF16, 0, False, 0)\n"
        "g = np.full(1, 0.9, dtype=np.float32)\n"
        "print('probe: loaded', flush=True)\n"
        "api.la_chunk_fwd(d, 0x10000, 0x10000, 0x10000, api.LA_GATE_GAMMA,\n"
        "                 ctypes.c_void_p(g.ctypes.data), None, None, 64, 0x10000,\n"
        "                 None, None, None, 0, None)\n")
    r = _run([sys.executable, "-c", probe], env)
    assert "probe: loaded" in r.stdout, r.stderr[-3000:]
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
