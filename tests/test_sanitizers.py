"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two instrumented builds, each exercised in a child process that preloads its
compiler's sanitizer runtime (Python itself is not instrumented):

* the fp64 oracle, built by gcc with -fsanitize=address,undefined, running
  every oracle pin;
* libks built for the host only (hipcc --offload-host-only: no device code is
  compiled, and nothing is launched), with the sanitizers on the host pass
  (-Xarch_host before each -fsanitize=), running the C ABI tests: argument
  validation, chain planning, workspace sizes and plan descriptions.

Any sanitizer report aborts the child (-fno-sanitize-recover=all), which
fails the test.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "kronecker_sparse_structured_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

SAN = ["-fsanitize=address", "-fsanitize=undefined"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(script: str, preload: str, tmp) -> subprocess.CompletedProcess:
    env = dict(os.environ, **ENV_SAN)
    # reports go to files in tmp (read back by _report)
    env["ASAN_OPTIONS"] += ":log_path=" + str(tmp / "asan")
    env["UBSAN_OPTIONS"] += ":log_path=" + str(tmp / "ubsan")
    env["LD_PRELOAD"] = preload
    env["PYTHONPATH"] = os.pathsep.join([ROOT, TESTS, env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, "-c", script], cwd=str(tmp), env=env, capture_output=True, text=True,
                          timeout=600)


def _report(proc, tmp) -> str:
    logs = "".join(open(os.path.join(str(tmp), f)).read()[:6000] for f in sorted(os.listdir(str(tmp)))
                   if f.startswith(("asan.", "ubsan.")))
    return "exit %d\n--- sanitizer reports ---\n%s\n--- stdout ---\n%s\n--- stderr ---\n%s" % (
        proc.returncode, logs, proc.stdout[-4000:], proc.stderr[-3000:])


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = str(tmp_path / "libks_oracle_asan.so")
    oracle.build(force=True, out=lib, extra_flags=["-g", "-fno-omit-frame-pointer", *SAN,
                                                   "-fno-sanitize-recover=all"])
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    script = (
        "import sys, pytest, oracle\n"
        "oracle._lib = oracle.load(%r)\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
        % (lib, os.path.join(TESTS, "test_oracle_pins.py")))
    proc = _child(script, runtime, tmp_path)
    assert proc.returncode == 0, _report(proc, tmp_path)
    assert "passed" in proc.stdout


def _clang_runtime() -> str:
    out = subprocess.run([os.path.join(ROCM, "llvm", "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        # older layouts name the runtime by target directory
        for root, _, files in os.walk(os.path.join(ROCM, "llvm", "lib", "clang")):
            if "libclang_rt.asan-x86_64.so" in files:
                return os.path.join(root, "libclang_rt.asan-x86_64.so")
        return ""
    return path


def test_libks_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    runtime = _clang_runtime()
    if not runtime:
        pytest.skip("clang's AddressSanitizer runtime not found")
    flags = ["--offload-host-only", "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
             "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    for f in SAN + ["-fno-sanitize-recover=all"]:
        flags += ["-Xarch_host", f]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        proc = subprocess.run([HIPCC, *flags, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        assert proc.returncode == 0, "compile %s failed:\n%s" % (src, proc.stderr[-4000:])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    # A host-only object still names the code-object bundle its device pass
    # would have embedded; give each one an empty bundle (the bundler's
    # magic and zero entries). No kernel is ever launched from this build.
    names = set()
    for obj in objs:
        out = subprocess.run(["nm", "-u", obj], capture_output=True, text=True, check=True).stdout
        names.update(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", out))
    stub = tmp_path / "empty_bundles.c"
    stub.write_text("".join(
        'const char %s[32] __attribute__((aligned(4096))) = "__CLANG_OFFLOAD_BUNDLE__";\n' % n
        for n in sorted(names)))
    stub_obj = str(tmp_path / "empty_bundles.o")
    subprocess.run(["gcc", "-c", "-fPIC", str(stub), "-o", stub_obj], check=True)
    objs.append(stub_obj)
    lib = str(tmp_path / "libks_asan.so")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *objs, "-o", lib]
    for f in SAN:
        link[1:1] = ["-Xarch_host", f]
    proc = subprocess.run(link, capture_output=True, text=True)
    assert proc.returncode == 0, "link failed:\n%s" % proc.stderr[-4000:]
    script = (
        "import sys, pytest\n"
        "from kronecker_sparse_structured_amd import libks\n"
        "libks.LIB_PATH = %r\n"
        "libks.load(%r)\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
        % (lib, lib, os.path.join(TESTS, "test_abi_cpu.py")))
    proc = _child(script, runtime, tmp_path)
    assert proc.returncode == 0, _report(proc, tmp_path)
    assert "passed" in proc.stdout
