"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. The oracle's C part (oracle/csa.c), driven on seeded inputs with ragged
   sizes (a context-row count and a reduction length that are not multiples
   of 64, ties and exact zeros among the scores): the sanitized build reports
   nothing and writes exactly the bytes of the ordinary build, whose values are
   the oracle's own (checked through oracle.csa).
2. The C ABI's argument validation (sl_api.cpp, host pass sanitized; the
   kernels' objects plain), driven by tests/sanitize/abi_driver.cpp with a
   host-built handle and only malformed calls, so nothing reaches the device.
"""
import glob
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import csa

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
ORACLE_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _write_inputs(path, rng, T=150, D=203, T_c=97, k=8, C=130, n=41):
    x = rng.standard_normal((T, D)).astype(np.float32)
    x[3, :] = 0.0                                   # an all-zero context row
    rows = np.sort(rng.choice(T, T_c, replace=False)).astype(np.int32)
    WA_t = (rng.standard_normal((2 * k, D)) * 0.1).astype(np.float32)
    WB0 = (rng.standard_normal((k, C)) * 0.3).astype(np.float32)
    WB1 = (rng.standard_normal((k, C)) * 0.3).astype(np.float32)
    WB0[:, 5] = WB0[:, 9]                           # two channels with equal scores
    WB1[:, 5] = WB1[:, 9]
    WB0[:, 17] = 0.0                                # an exactly zero score
    with open(path, "wb") as f:
        np.array([T, D, T_c, k, C, n], np.int64).tofile(f)
        for a in (x, rows, WA_t, WB0, WB1):
            a.tofile(f)
    return x, rows, WA_t, WB0, WB1, n


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_c_under_sanitizers(tmp_path, rng):
    src = [os.path.join(HERE, "sanitize", "csa_driver.c"), os.path.join(ROOT, "oracle", "csa.c")]
    plain, san = str(tmp_path / "plain"), str(tmp_path / "san")
    _run(["gcc"] + ORACLE_FLAGS + ["-o", plain] + src + ["-lm"])
    _run(["gcc"] + ORACLE_FLAGS + ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                   "-fno-sanitize-recover=all", "-o", san] + src + ["-lm"])
    inp = str(tmp_path / "in.bin")
    x, rows, WA_t, WB0, WB1, n = _write_inputs(inp, rng)
    _run([plain, inp, str(tmp_path / "out_plain.bin")])
    r = _run([san, inp, str(tmp_path / "out_san.bin")], env=SAN_ENV)
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    a = (tmp_path / "out_plain.bin").read_bytes()
    b = (tmp_path / "out_san.bin").read_bytes()
    assert a == b
    # the driver's outputs are the oracle's
    xa = np.frombuffer(a, np.float32, count=len(rows) * WA_t.shape[0]).reshape(len(rows), -1)
    want = csa.stage1(x, rows, WA_t)
    assert np.array_equal(xa.view(np.uint32), np.asarray(want, np.float32).view(np.uint32))
    off = xa.size * 4 + 3 * WB0.shape[1] * 4 + xa.size * 4
    cnt = int(np.frombuffer(a, np.int64, count=1, offset=off)[0])
    idx = np.frombuffer(a, np.int32, count=cnt, offset=off + 8)
    assert np.array_equal(idx, csa.select(csa.ssq_l2(want, WB0), n))


def _objects():
    objs = [p for p in glob.glob(os.path.join(ROOT, "_build", "*.o"))
            if os.path.basename(p) != "sl_api.cpp.o"]
    from contextual_sparsity_lora_amd import build as lib_build
    need = [os.path.join(ROOT, "_build", s + ".o") for s in lib_build.SOURCES if s != "sl_api.cpp"]
    if any(not os.path.exists(p) for p in need):
        lib_build.build()
    return need


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_abi_validation_under_sanitizers(tmp_path):
    from contextual_sparsity_lora_amd import build as lib_build
    hipcc = lib_build.HIPCC
    # Enum-typed parameters reach the library as plain integers from C and
    # Python callers; a value outside an enum's list is an argument error that
    # validation must reject (the driver passes such values), so C++'s own
    # rule on enum ranges (-fsanitize=enum) is left out.
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize=enum",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    flags = lib_build.FLAGS + san
    api_o, drv_o = str(tmp_path / "sl_api.o"), str(tmp_path / "driver.o")
    _run([hipcc] + flags + ["-x", "hip", "-c", os.path.join(ROOT, "contextual_sparsity_lora_amd", "csrc",
                                                           "sl_api.cpp"), "-o", api_o])
    _run([hipcc] + flags + ["-x", "hip", "-c", os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-o", drv_o])
    exe = str(tmp_path / "abi_driver")
    clang = "/opt/rocm/llvm/bin/clang++"
    _run([clang, "-fsanitize=address,undefined", "-o", exe, drv_o, api_o] + _objects()
         + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
    assert "0 failed" in r.stdout, r.stdout
