"""The host code under the address and undefined-behaviour sanitizers (CPU
only, no GPU code involved): the host part of the C ABI (size checks, level
table validation, workspace sizes, status strings: csrc/host_checks.cpp)
and both oracles are built with -fsanitize=address,undefined by gcc/g++ and
exercised in a child process that has the sanitizer runtime preloaded --
the oracle pins, and the host checks on valid, invalid and fuzzed inputs,
extreme sizes included.  Any report aborts the child and fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]

_CHILD = r"""
import ctypes, sys
sys.path[:0] = [{root!r}, {tests!r}]
import numpy as np

# host part of the C ABI
lib = ctypes.CDLL({host!r})
p, i64 = ctypes.c_void_p, ctypes.c_int64
lib.msda_validate_host.argtypes = [p, p] + [i64] * 7
lib.msda3d_validate_host.argtypes = [p, p] + [i64] * 7
SIZES = ("msda_backward_workspace_size", "msda_backward_fused_workspace_size",
         "msda3d_backward_workspace_size", "msda_backward_workspace_min",
         "msda_backward_fused_workspace_min", "msda3d_backward_workspace_min")
for f in SIZES:
    getattr(lib, f).argtypes = [i64] * 7
    getattr(lib, f).restype = ctypes.c_size_t
lib.msda_status_string.argtypes = [ctypes.c_int]
lib.msda_status_string.restype = ctypes.c_char_p
for code in range(-10, 3):
    assert lib.msda_status_string(code)
ptr = lambda a: a.ctypes.data_as(p)
r = np.random.Generator(np.random.PCG64(77))
extremes = [0, 1, 2, 3, 7, 8, 31, 255, 4096, 1 << 20, (1 << 31) - 1, 1 << 31, (1 << 40), -1,
            -(1 << 40), (1 << 62)]
n = 0
for trial in range(4000):
    dims3 = trial % 2 == 1
    L = int(r.integers(1, 17)) if trial % 5 else int(r.choice([0, 17, 1, 16]))
    ext = r.integers(-2, 40, (max(L, 1), 3 if dims3 else 2)).astype(np.int64)
    if trial % 7 == 0:
        ext[r.integers(0, max(L, 1))] = r.choice(extremes)
    sizes = ext.prod(axis=1)
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
    if trial % 3 == 0:
        starts = starts + r.integers(-1, 2, starts.shape)
    Nv = int(sizes.sum()) if trial % 4 else int(r.choice(extremes))
    B, Nq, M, D, K = (int(r.choice(extremes)) if r.random() < 0.2 else int(v)
                      for v in (2, 300, 8, 32, 4))
    fn = lib.msda3d_validate_host if dims3 else lib.msda_validate_host
    fn(ptr(ext), ptr(starts), B, Nv, Nq, M, D, L, K)
    for f in SIZES:
        getattr(lib, f)(B, Nv, Nq, M, D, L, K)
    n += 1
for dims in [(2, 22223, 22223, 8, 32, 4, 4), (4, 22223, 22223, 8, 32, 4, 8),
             ((1 << 40), 80, 16, 2, 8, 2, 2), (1, (1 << 40), 16, 2, 8, 2, 2),
             (1, 80, (1 << 40), 2, 8, 2, 2), (1, 80, 16, (1 << 30), 8, 2, 2),
             (1, 80, 16, 2, 8, 2, (1 << 40)), (1 << 30, 1, 1, 1, 4, 1, 1)]:
    for f in SIZES:
        getattr(lib, f)(*dims)
print("host checks:", n, "fuzzed calls", flush=True)

# the oracles, against their pins
import oracle, oracle.volume as ov
from oracle_pins import ALL_PINS
from volume_pins import ALL_VOLUME_PINS
orc = oracle.OracleLib({orc!r})
for pin in ALL_PINS:
    pin(orc)
vol = ov.VolumeLib({vol!r})
for pin in ALL_VOLUME_PINS:
    pin(vol)
print("oracle pins:", len(ALL_PINS) + len(ALL_VOLUME_PINS), flush=True)
print("SANITIZED_OK", flush=True)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's address-sanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    import oracle.volume
    from scale_deformable_attention_04_amd import build as hip_build
    host = hip_build.build_host_sanitized()
    orc = oracle.build(out=str(tmp_path / "liboracle_san.so"), extra=SAN)
    vol = oracle.volume.build(out=str(tmp_path / "liboracle3d_san.so"), extra=SAN)
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), host=host, orc=orc,
                         vol=vol)
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "SANITIZED_OK" in res.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
