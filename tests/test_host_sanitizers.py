"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Every csrc/*.hip is compiled with both sanitizers on its host side only (the kernels
are compiled as usual and never launched: there is no GPU here), linked with
tests/host_sanitize/abi_fuzz.cpp, and run.  The driver calls every C-ABI entry point
with well-formed arguments on fake device addresses, with each argument broken in
turn and with seeded random combinations of broken arguments; it exits non-zero on a
status outside the documented codes, and either sanitizer aborts it on an invalid
access, an integer overflow, a division by zero or a bad conversion in the host code.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bounded_decode_attention_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_fuzz.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# each sanitizer flag applies to the host compilation only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
COMMON = ["--offload-arch=gfx950", "-O2", "-Xarch_host", "-g", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]

pytestmark = pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC),
                                reason="hipcc not available")


def _build(tmp):
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(tmp, os.path.basename(src)[:-4] + ".o")
        procs.append(subprocess.Popen([HIPCC] + COMMON + SAN + ["-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        objs.append(obj)
    drv = os.path.join(tmp, "abi_fuzz.o")
    procs.append(subprocess.Popen([HIPCC, "-O2", "-g", "-std=c++17"] + SAN +
                                  ["-I", os.path.join(ROOT, "include"), "-c", DRIVER, "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate(timeout=600)[0].decode(errors="replace")
        assert p.returncode == 0, out[-4000:]
    exe = os.path.join(tmp, "abi_fuzz")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + ["-o", exe, drv] + objs,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    return exe


def test_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = _build(str(tmp_path))
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "50000"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("calls=")]
    assert line, r.stdout
    fields = dict(kv.split("=") for kv in line[0].split())
    # every entry point was reached with arguments that pass validation, and the
    # broken ones were rejected before any device work
    assert int(fields["entry_points"]) >= 30
    assert int(fields["edevice"]) > 0 and int(fields["rejected"]) > 0
