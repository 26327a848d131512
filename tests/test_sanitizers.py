"""Sanitizer leg (CPU): the oracle and the host-side record code built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code only),
then exercised in a child process with the ASan runtime preloaded.

- The oracle (oracle/trace_oracle.c) runs the whole pin suite
  (tests/test_oracle_pins.py) through TRACE_ORACLE_LIB.
- The record code (precision_numerics_block_amd/csrc/trace_record.cpp)
  seals, checks, writes and reads records built by hand from the documented
  layout, and rejects damaged ones (flipped bits, bad header fields, short
  buffers, truncated, foreign and missing files); XXH64 is compared with the
  xxhash package.  Its size helper comes from the product library, loaded
  first with global symbols; the record functions are the sanitized build's.

Any sanitizer report fails the child (UBSan with halt_on_error, ASan on its
first error; leak detection is off because the interpreter itself keeps
allocations alive at exit)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _asan_runtime():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc / g++ not available")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no ASan runtime for gcc")
    return path


def _env(extra):
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(extra)
    return env


def _clean(r):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle

    lib = str(tmp_path / "liboracle_san.so")
    flags = [f for f in oracle.GCC_FLAGS if not f.startswith("-O")]
    subprocess.check_call(["gcc", *SAN, *flags, os.path.join(ROOT, "oracle", "trace_oracle.c"), "-o", lib, "-lm"])
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       env=_env({"TRACE_ORACLE_LIB": lib}), cwd=ROOT, capture_output=True, text=True, timeout=900)
    _clean(r)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]


RECORD_CHILD = r'''
import ctypes, os, struct, sys
import numpy as np
import xxhash

root, san_lib, prod_lib, tmp = sys.argv[1:5]
ctypes.CDLL(prod_lib, mode=ctypes.RTLD_GLOBAL)          # trace_guidance_bytes
L = ctypes.CDLL(san_lib)
vp, sz, i64, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
L.trace_record_bytes.restype, L.trace_record_bytes.argtypes = sz, [i64, i32, i32]
L.trace_record_seal.restype, L.trace_record_seal.argtypes = i32, [vp, sz]
L.trace_record_check.restype = i32
L.trace_record_check.argtypes = [vp, sz, ctypes.POINTER(i64), ctypes.POINTER(i32), ctypes.POINTER(i32)]
L.trace_record_write.restype, L.trace_record_write.argtypes = i32, [ctypes.c_char_p, vp, sz]
L.trace_record_read.restype, L.trace_record_read.argtypes = i32, [ctypes.c_char_p, vp, sz, ctypes.POINTER(sz)]
L.trace_xxh64.restype, L.trace_xxh64.argtypes = ctypes.c_uint64, [vp, sz]
HDR = struct.Struct("<IIqiiQQQQII")
p = lambda a: ctypes.c_void_p(a.ctypes.data)

def build(n, k, G, sealed, seed):
    rng = np.random.default_rng(seed)
    off = (n // 16 + 255) // 256 * 256
    stream = rng.integers(0, 256, off + n * k // 8, dtype=np.uint8)
    g = rng.random(G).astype(np.float32)
    g_area = (4 * G + 63) // 64 * 64
    payload = np.zeros(g_area + stream.size, np.uint8)
    payload[: 4 * G] = g.view(np.uint8)
    payload[g_area:] = stream
    h = xxhash.xxh64(payload.tobytes()).intdigest() if sealed else 0
    head = HDR.pack(0x44475254, 1, n, k, G, stream.size, off, payload.size, h, 1 if sealed else 0, 0)
    return np.concatenate([np.frombuffer(head, np.uint8), payload])

def check(rec):
    n, k, G = i64(), i32(), i32()
    return L.trace_record_check(p(rec), rec.size, ctypes.byref(n), ctypes.byref(k), ctypes.byref(G)), \
        (n.value, k.value, G.value)

rng = np.random.default_rng(1)
for ln in (0, 1, 3, 7, 8, 31, 32, 33, 63, 64, 65, 1000, 65537):
    b = rng.integers(0, 256, max(ln, 1), dtype=np.uint8)[:ln].copy()
    assert L.trace_xxh64(p(b) if ln else None, ln) == xxhash.xxh64(b.tobytes()).intdigest(), ln
for k, G in ((1, 1), (2, 1), (3, 1), (4, 1), (2, 3)):
    n = 16 * 300 * G
    rec = build(n, k, G, False, k + G)
    assert rec.size == L.trace_record_bytes(n, k, G)
    assert check(rec)[0] != 0                               # not sealed
    assert L.trace_record_seal(p(rec), rec.size) == 0
    assert np.array_equal(rec, build(n, k, G, True, k + G))
    assert check(rec) == (0, (n, k, G))
good = build(16 * 300, 2, 1, True, 9)
for pos in (64, 134, good.size - 1):
    bad = good.copy(); bad[pos] ^= 0x10
    assert check(bad)[0] == -8
for idx, value in ((0, 0x12345678), (1, 2), (3, 3), (2, 16 * 301), (5, 1 << 40), (7, 7)):
    vals = list(HDR.unpack(good[:64].tobytes())); vals[idx] = value
    bad = good.copy(); bad[:64] = np.frombuffer(HDR.pack(*vals), np.uint8)
    assert check(bad)[0] != 0, idx
for cut in (0, 10, 63, 64, good.size - 1):
    part = good[:cut].copy()
    assert check(part)[0] != 0, cut
path = os.path.join(tmp, "g.trg").encode()
assert L.trace_record_write(path, p(good), good.size) == 0
back = np.zeros(good.size + 100, np.uint8); got = sz()
assert L.trace_record_read(path, p(back), back.size, ctypes.byref(got)) == 0 and got.value == good.size
assert np.array_equal(back[: good.size], good)
raw = open(path, "rb").read()
for name, data in (("trunc.trg", raw[:-5]), ("junk.trg", b"\x00" * 200), ("head.trg", raw[:40])):
    q = os.path.join(tmp, name).encode(); open(q, "wb").write(data)
    assert L.trace_record_read(q, p(back), back.size, ctypes.byref(got)) != 0, name
assert L.trace_record_read(os.path.join(tmp, "missing.trg").encode(), p(back), back.size, ctypes.byref(got)) == -9
small = np.zeros(good.size - 1, np.uint8)
assert L.trace_record_read(path, p(small), small.size, ctypes.byref(got)) != 0
print("records ok")
'''


def test_record_code_under_sanitizers(tmp_path):
    prod = os.path.join(ROOT, "precision_numerics_block_amd", "libtrace_quant.so")
    if not os.path.exists(prod):
        pytest.skip("libtrace_quant.so is not built")
    lib = str(tmp_path / "librecord_san.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-Wl,-Bsymbolic", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "precision_numerics_block_amd", "csrc", "trace_record.cpp"), "-o", lib,
                           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")])
    child = tmp_path / "records_child.py"
    child.write_text(RECORD_CHILD)
    r = subprocess.run([sys.executable, str(child), ROOT, lib, prod, str(tmp_path)], env=_env({}), cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    _clean(r)
    assert "records ok" in r.stdout
