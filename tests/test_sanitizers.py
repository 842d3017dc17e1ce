"""CPU-only: the oracle's C code and the C ABI's host-side argument checks run
under AddressSanitizer + UndefinedBehaviorSanitizer.

Each part builds its own sanitized copy (in a temporary directory) and runs
in a child process with the sanitizer runtime preloaded: gcc's for the
oracle (built with gcc, as the oracle always is), clang's for the library's
host code (hipcc is clang; the device code is compiled as usual and never
runs here).  Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_sparse_attention_mxfp4_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _run_child(script, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", textwrap.dedent(script)], env=env, capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "child done" in r.stdout, out[-4000:]
    return out


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


ORACLE_SCRIPT = """
import ctypes
import numpy as np
import oracle
assert hasattr(ctypes.CDLL(None), "__asan_init") and hasattr(ctypes.CDLL(None), "__ubsan_handle_add_overflow")
oracle.lib()

rng = np.random.default_rng(7)
# quantize: rows of random bf16 (finite), some slots out of the pool (skipped)
x = (rng.standard_normal((37, 512)).astype(np.float32) * 3).view(np.uint32)
x = ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)
pool = np.zeros((2, oracle.PAGE_BYTES), np.uint8)
slots = np.arange(37, dtype=np.int64)
slots[5] = 10_000
oracle.quantize_kv(x, slots, pool)
# indexer: two sequences, ragged, T = 2; Full, Reindex, and the causal form
B, T, HI = 2, 2, 8
n = np.array([300, 77], np.int32)
pt = np.array([[0, 1, 2, 3, 4], [5, 6, -1, -1, -1]], np.int32)
kidx = rng.integers(0, 256, (7, 64, 128), dtype=np.uint8)
kidx[(kidx & 0x7F) == 0x7F] = 0  # no NaN codes
q = rng.integers(0, 256, (B, T, HI, 128), dtype=np.uint8)
q[(q & 0x7F) == 0x7F] = 0
w = rng.standard_normal((B, T, HI)).astype(np.float32)
tk, pl, pn = oracle.index_full(q, w, kidx, pt, n, 16, 8)
rt = oracle.index_reindex(q, w, kidx, pt, n, pl, pn, 16)
nv = np.array([[10, 300], [0, 77]], np.int32)
oracle.index_full(q, w, kidx, pt, n, 16, 8, n_visible=nv)
# attention over a few dequantized rows
rows = rng.standard_normal((40, 512))
qa = rng.standard_normal((16, 512))
oracle.attention(qa, 0.04, rows)
# compressor
c = x[:32]
z = x[32:36].repeat(8, axis=0)
oracle.compress(c, z, 4)
print("child done")
"""

ABI_SCRIPT = """
import ctypes, os
assert hasattr(ctypes.CDLL(None), "__asan_init") and hasattr(ctypes.CDLL(None), "__ubsan_handle_add_overflow")
L = ctypes.CDLL(os.environ["CSA2_SAN_LIB"])
P = ctypes.c_void_p
X = P(0x1000)
INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3
i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
L.csa2_status_str.restype = ctypes.c_char_p
for st in (0, -1, -2, -3, -4, -5, 12345):
    assert L.csa2_status_str(st)
L.csa2_workspace_bytes.restype = sz
for op in (1, 2, 3, 99):
    for B, T in ((1, 1), (4, 1), (32, 2), (0, 1)):
        L.csa2_workspace_bytes(op, B, T, 64, 262144, 2048)
def full(q=X, max_n=64, B=1, T=1, HI=4, topk=8, pb=16, ot=X, ws=X, wsb=1 << 30):
    return L.csa2_index_full(q, X, X, i64(1), X, 1, X, max_n, B, T, HI, topk, pb, ot, X, X, ws, sz(wsb), None)
assert full(q=None) == INVALID
assert full(ot=None) == INVALID
assert full(B=0) == INVALID
assert full(topk=0) == INVALID
assert full(HI=6) == UNSUPPORTED
assert full(T=257) == UNSUPPORTED
assert full(B=300, T=256) == UNSUPPORTED
assert full(topk=32, pb=16) == UNSUPPORTED
assert full(max_n=262145) == UNSUPPORTED
assert full(ws=None) == WORKSPACE
assert full(wsb=16) == WORKSPACE
assert L.csa2_index_full_noalloc(None, X, X, i64(1), X, 1, X, 64, 1, 1, 4, 8, 16, X, X, X, None) == INVALID
assert L.csa2_index_full_causal(X, X, X, i64(1), X, 1, X, None, 64, 1, 1, 4, 8, 16, X, X, X, X, sz(1 << 30),
                                None) == INVALID
assert L.csa2_index_reindex(X, X, X, i64(1 << 26), X, 1, X, 1, 1, 4, X, X, 16, 8, X, X, sz(1 << 30),
                            None) == UNSUPPORTED
assert L.csa2_index_reindex(None, X, X, i64(1), X, 1, X, 1, 1, 4, X, X, 16, 8, X, X, sz(1 << 30),
                            None) == INVALID
assert L.csa2_test_select_path(3) == INVALID
assert L.csa2_test_select_path(0) == 0
print("child done")
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    ubsan = _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "libcsa2_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-fPIC", "-shared",
                           os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-o", lib, "-lm"])
    _run_child(ORACLE_SCRIPT, {
        "CSA2_ORACLE_LIB": lib,
        "LD_PRELOAD": f"{asan}:{ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "2",
    })


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_argument_checks_under_asan_ubsan(tmp_path):
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not (os.path.isabs(rt) and os.path.exists(rt)):
        pytest.skip("clang ASan runtime not found")
    sys.path.insert(0, os.path.join(ROOT, "compressed_sparse_attention_mxfp4_amd"))
    import build as csa2_build  # the library's own flags and sources
    lib = str(tmp_path / "libcsa2_san.so")
    cmd = [HIPCC] + csa2_build.flags() + [
        "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
        "-Xarch_host", "-shared-libsan"] + [os.path.join(CSRC, s) for s in csa2_build.SOURCES] + ["-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    _run_child(ABI_SCRIPT, {
        "CSA2_SAN_LIB": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
