"""The host-side argument checks of the C ABI under the host AddressSanitizer
and UndefinedBehaviorSanitizer (no GPU needed).

The library (csrc/blk.hip, csrc/attn.hip) is compiled with both sanitizers
on its host code (the device code is built as usual, without them), linked
with the C driver tests/abi_sanitize.c, and the driver calls every entry
point with arguments the library must refuse before any launch.  Any
sanitizer report makes the run fail (halt_on_error)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "backward_gpt_block_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# sanitizers for the host pass only; the sanitizer runtime is linked
# statically into the driver
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(900)
def test_abi_checks_under_host_sanitizers(tmp_path):
    from backward_gpt_block_amd.build import FLAGS, UNITS
    objs, procs = [], []
    for unit, extra in UNITS:   # both translation units compile at once
        obj = str(tmp_path / unit.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *extra, "-Xarch_host", "-O1", "-Xarch_host", "-g", *SAN, "-c",
               os.path.join(CSRC, unit), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{' '.join(cmd)}\n{err}"
    exe = str(tmp_path / "abi_sanitize")
    _run([HIPCC, "--offload-arch=gfx950", "-x", "c++", os.path.join(ROOT, "tests", "abi_sanitize.c"),
          "-x", "none", *objs, *SAN, "-Xarch_host", "-static-libsan", "-o", exe])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout
