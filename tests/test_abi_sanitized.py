"""The C ABI's argument validation and dispatch, built for the host alone under
AddressSanitizer and UndefinedBehaviorSanitizer and run on the CPU.

abi.hip and lm_codebook.hip are compiled with --cuda-host-only; the kernel
launchers and the few HIP runtime calls they reach are replaced by the
recording stand-ins of tests/host_abi/stubs.hip, so no GPU and no HIP runtime
is needed.  tests/host_abi/driver.hip calls every entry point with valid and
malformed arguments and checks the return codes, the launches and the
host-side outputs; any sanitizer report aborts the run."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rotated_bit_quantized_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_abi")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src, obj, cuid):
    cmd = [HIPCC, "--cuda-host-only", f"-cuid={cuid}", "-O1", "-g", "-std=c++17", "-I" + CSRC,
           "-I" + os.path.join(ROOT, "include"), "-I" + HERE, "-c", src, "-o", obj] + SAN
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not present")
def test_abi_validation_under_sanitizers(tmp_path):
    objs = []
    for name, src in (("abi", os.path.join(CSRC, "abi.hip")), ("lmc", os.path.join(CSRC, "lm_codebook.hip")),
                      ("stubs", os.path.join(HERE, "stubs.hip")), ("driver", os.path.join(HERE, "driver.hip"))):
        obj = str(tmp_path / f"{name}.o")
        _compile(src, obj, name)
        objs.append(obj)
    # the host-only objects name the device-code image they would register;
    # it is never read, so a zero-filled stand-in of that name is enough
    syms = set()
    for obj in objs:
        out = subprocess.run(["nm", "-u", obj], capture_output=True, text=True, check=True).stdout
        syms.update(re.findall(r"\b(__hip_fatbin_\w+)", out))
    fat = tmp_path / "fatbin.cpp"
    fat.write_text("".join(f'extern "C" {{ unsigned char {s}[64] = {{0}}; }}\n' for s in sorted(syms)))
    fat_o = str(tmp_path / "fatbin.o")
    subprocess.run([CLANG, "-c", str(fat), "-o", fat_o], check=True)
    exe = str(tmp_path / "abi_check")
    link = [CLANG, "-fsanitize=address,undefined", "-o", exe] + objs + [fat_o]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # verify_asan_link_order=0: the environment may preload a library of its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "cases passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
