"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

Two host code bases are rebuilt with ASan and UBSan (no recovery: the first
report aborts the run) and exercised by the existing CPU tests in a child
process that preloads the sanitizer runtime:

* the fp64 oracle (oracle/*.c, gcc -fsanitize=address,undefined), under the
  oracle pins and the gradient pins;
* the C-ABI validation layer (csrc/kda_api.hip: host code built with clang
  -fsanitize=address,undefined through hipcc's -Xarch_host, linked with the
  library's other objects), under the ABI tests, every one of which stops
  in validation before any HIP call.

Device code is never built with a sanitizer.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_delta_rule_17_amd")
OUT = os.path.join(ROOT, "oracle", "_build", "sanitize")


def _run_child(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "-m", "not gpu"] + tests
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    return tail


def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "libkda_oracle_san.so")
    src = [os.path.join(ROOT, "oracle", f) for f in ("kda_recurrence.c", "kda_backward.c")]
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared",
                    "-std=c99", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-DKDA_MUTANT=0"] + src + ["-o", lib, "-lm"], check=True)
    rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                         check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    out = _run_child(["tests/test_oracle_pins.py", "tests/test_oracle_chunkwise.py",
                      "tests/test_oracle_backward.py", "tests/test_oracle_varlen.py",
                      "tests/test_oracle_grouped.py"],
                     {"LD_PRELOAD": " ".join(rt), "KDA_ORACLE_LIBRARY": lib})
    assert "passed" in out


def test_abi_validation_under_asan_ubsan():
    objs_dir = os.path.join(PKG, "_build")
    srcs = sorted(f for f in os.listdir(os.path.join(PKG, "csrc")) if f.endswith(".hip"))
    if not all(os.path.exists(os.path.join(objs_dir, f + ".o")) for f in srcs):
        from gated_delta_rule_17_amd.build import build
        build(verbose=False)
    from gated_delta_rule_17_amd.build import ARCH, FLAGS, HIPCC
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "kda_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1"]
    subprocess.run([HIPCC] + flags + san + ["-c", os.path.join(PKG, "csrc", "kda_api.hip"),
                                            "-o", api_o], check=True, capture_output=True)
    lib = os.path.join(OUT, "libkda_san.so")
    others = [os.path.join(objs_dir, f + ".o") for f in srcs if f != "kda_api.hip"]
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib, api_o] + others,
                   check=True, capture_output=True)
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.fail(f"clang ASan runtime not found: {rt}")
    out = _run_child(["tests/test_abi.py"], {"LD_PRELOAD": rt, "KDA_LIBRARY": lib})
    assert "passed" in out
