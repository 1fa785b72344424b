"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The packer (pack.cpp) and the C ABI (abi.cpp) are compiled with both sanitizers on the host side (UB made
fatal) and linked with the kernels' objects of the regular build into a small executable
(tests/sanitize/host_driver.cpp). It packs 300 random size lists in every mode, reads every host accessor into
buffers of exactly the documented sizes, packs stack levels, and runs the argument checks of the device entry
points (which return before any launch). The run must exit 0 with no sanitizer report; leaks are reported
too.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "directional_mdlstm_handwriting_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _kernel_objects():
    objs = sorted(os.path.join(BUILD, f + ".o") for f in os.listdir(CSRC) if f.endswith(".hip"))
    if not all(os.path.exists(o) for o in objs):
        import __graft_entry__
        __graft_entry__._build_module().build()
    return objs


@pytest.mark.slow
def test_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    objs = _kernel_objects()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    host = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "pack.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-x", "c++", "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        host.append(obj)
    exe = str(tmp_path / "host_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], *host, *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # verify_asan_link_order=0: the environment may preload libraries ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in r.stdout
