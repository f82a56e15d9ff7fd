"""Host code under address and undefined-behaviour sanitizers (CPU only).

* The oracle's C functions, compiled with gcc -fsanitize=address,undefined,
  driven on small inputs by tests/sanitize/oracle_main.c (which also checks a
  few closed forms).
* librssm's host-side ABI code (api.cpp), its host half compiled with the
  same sanitizers (device code untouched), linked with the kernel objects of
  the regular build and driven through validation paths that launch nothing
  (tests/sanitize/abi_main.cpp).

Skipped where a compiler or the sanitizer runtime is missing, and the ABI
part where a GPU is visible (the stand-in pointers are only safe where
nothing can run).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off"] + SAN +
                   [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_main.c"),
                    "-o", exe, "-lm"], str(tmp_path))
    if rc != 0 and "asan" in out.lower():
        pytest.skip("sanitizer runtime not available: " + out[-300:])
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "ok" in out and "runtime error" not in out, out


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="host-only test with stand-in pointers")
def test_abi_host_code_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    from linear_attention_decode_replayssm_amd import build as hip_build
    objs = [os.path.join(ROOT, "_build", os.path.splitext(n)[0] + ".o")
            for n in hip_build.SOURCES if n.endswith(".hip")]
    if not os.path.exists(hipcc) or not all(os.path.exists(o) for o in objs) or \
            not os.path.exists(os.path.join(rocm, "lib", "llvm", "bin", "clang++")):
        pytest.skip("hipcc or the regular build's kernel objects are missing")
    host_san = []
    for f in SAN:                      # host half only: each flag behind -Xarch_host
        host_san += ["-Xarch_host", f]
    csrc = os.path.join(ROOT, "linear_attention_decode_replayssm_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    api_o = str(tmp_path / "api_san.o")
    rc, out = _run([hipcc, "-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san + inc +
                   ["-c", os.path.join(csrc, "api.cpp"), "-o", api_o], str(tmp_path))
    assert rc == 0, out
    # the driver is plain C++: the host compiler of the same toolchain
    clangxx = os.path.join(rocm, "lib", "llvm", "bin", "clang++")
    main_o = str(tmp_path / "abi_main.o")
    rc, out = _run([clangxx, "-O1", "-std=c++17"] + SAN + inc +
                   ["-c", os.path.join(HERE, "abi_main.cpp"), "-o", main_o], str(tmp_path))
    assert rc == 0, out
    exe = str(tmp_path / "abi_san")
    rc, out = _run([hipcc, "-O1", "--offload-arch=gfx950"] + host_san +
                   [main_o, api_o] + objs + ["-o", exe], str(tmp_path))
    if rc != 0 and "asan" in out.lower():
        pytest.skip("sanitizer runtime not available: " + out[-300:])
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "ok" in out and "runtime error" not in out, out
