"""The CPU tier under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle: oracle.c built with -fsanitize=address,undefined
  (oracle/build.py: build_sanitized) and loaded in place of liboracle.so by
  a child pytest run of the oracle's pin tests, with the AddressSanitizer
  runtime preloaded. Any invalid access or undefined operation aborts it.
* The C ABI's host code: api.cpp and prefill_plan.cpp (argument checks, the
  decode and prefill plans, workspace layouts, tuning overrides) built for
  the host with the same sanitizers and linked with recording stubs of the
  HIP runtime and the kernel launches (tests/host_sanitize), then driven
  through every entry point over a grid of shapes, sizes and bad arguments.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _san_env(extra_preload):
    env = dict(os.environ)
    # the sanitizer runtime must come first; anything already preloaded stays
    env["LD_PRELOAD"] = " ".join(x for x in (extra_preload, os.environ.get("LD_PRELOAD")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@pytest.mark.timeout(900)
def test_oracle_pins_under_asan_and_ubsan():
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import build
    lib = build.build_sanitized()
    env = _san_env(asan)
    env["ORACLE_LIB"] = lib
    env["ORACLE_THREADS"] = "4"
    # the child really runs the instrumented library with the runtime loaded
    probe = ("import oracle; L = oracle.lib(); "
             "assert L._name.endswith('liboracle_asan.so'), L._name; "
             "maps = open('/proc/self/maps').read(); assert 'libasan' in maps; print('ok')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]
    files = ["tests/test_oracle_attention.py", "tests/test_oracle_codec.py",
             "tests/test_oracle_e5m2.py", "tests/test_oracle_dynamic.py",
             "tests/test_oracle_fp8attn.py", "tests/test_oracle_prefill.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not slow and not gpu",
                        "-p", "no:cacheprovider", *files], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=800)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


@pytest.mark.timeout(600)
def test_host_abi_under_asan_and_ubsan(tmp_path):
    if _gcc_runtime("libasan.so") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    csrc = os.path.join(ROOT, "fp8_kv_cache_write_amd", "csrc")
    here = os.path.join(ROOT, "tests", "host_sanitize")
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(csrc, "api.cpp"), os.path.join(csrc, "prefill_plan.cpp"),
           os.path.join(here, "stubs.cpp"), os.path.join(here, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = _san_env(None)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout, r.stderr[-3000:])
    assert "host checks passed" in r.stdout
