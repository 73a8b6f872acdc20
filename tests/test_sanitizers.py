"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The oracle (oracle/linattn_oracle.c) with its core pins as a C program
  (tests/sanitize/oracle_pins.c): gcc, -fsanitize=address,undefined, no recovery.
* The C ABI's host side (efficient_attention_amd/csrc/la_api.hip compiled for the host only)
  driven through every entry point's error paths and valid plans by tests/sanitize/abi_host.cpp,
  whose stand-ins for the kernel launchers check the plans they are handed.  clang (hipcc) with
  the sanitizers on the host compilation only; the few HIP runtime entry points the host code
  calls are stand-ins too, so nothing touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise AssertionError("%s failed (%d):\n%s\n%s" % (cmd[0], r.returncode, r.stdout[-4000:], r.stderr[-4000:]))
    return r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_pins")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-o", exe, os.path.join(SAN, "oracle_pins.c"),
          os.path.join(ROOT, "oracle", "linattn_oracle.c"), "-lm"], tmp_path)
    out = _run([exe], tmp_path)
    assert "oracle pins OK" in out


def test_abi_host_paths_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "efficient_attention_amd", "csrc")]
    host = [HIPCC, "--cuda-host-only", "-x", "hip", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer"]
    api_o, drv_o = str(tmp_path / "la_api.o"), str(tmp_path / "abi_host.o")
    _run(host + san + inc + ["-c", os.path.join(ROOT, "efficient_attention_amd", "csrc", "la_api.hip"),
                             "-o", api_o], tmp_path)
    _run(host + san + inc + ["-c", os.path.join(SAN, "abi_host.cpp"), "-o", drv_o], tmp_path)
    # the host object refers to the device image it would be linked with; give it an empty one
    syms = _run(["nm", "-u", api_o], tmp_path).split()
    stub = tmp_path / "image_stub.c"
    stub.write_text("".join("const char %s[16] = {0};\n" % s for s in syms if s.startswith("__hip_fatbin_")))
    stub_o = str(tmp_path / "image_stub.o")
    _run([CLANG, "-c", str(stub), "-o", stub_o], tmp_path)
    exe = str(tmp_path / "abi_host")
    _run([CLANG + "++", "-fsanitize=address,undefined", "-o", exe, api_o, drv_o, stub_o], tmp_path)
    out = _run([exe], tmp_path)
    assert "host ABI paths OK" in out
