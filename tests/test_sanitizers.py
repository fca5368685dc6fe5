"""CPU runs of the fp64 oracle and of the library's host code under
AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined and
  its pin tests (test_oracle.py, test_oracle_book.py, test_golden.py) run
  against that build in a child process with gcc's ASan runtime preloaded.
* The library's host code -- every argument check, the page layout, the
  workspace size, the path and launch choices, all in gdn_api.cpp -- is
  recompiled with hipcc, sanitizers on the host side only (-Xarch_host), and
  linked with the device objects of the normal build; test_abi.py runs
  against it with clang's ASan runtime preloaded.  No GPU is touched.

Each run starts with a canary: a heap overflow built with the same flags must
be reported, so a sanitizer that is silently inactive fails the test.
Leak checking is off (the interpreter itself holds memory until exit).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CANARY = "#include <stdlib.h>\nint main(void) { volatile char* p = malloc(8); p[8] = 1; return p[0]; }\n"


def _env(runtime: str) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def _check_canary(compile_cmd, exe):
    r = _run(compile_cmd)
    assert r.returncode == 0, r.stderr
    r = _run([exe])
    # either sanitizer may report the overflow first
    reported = "heap-buffer-overflow" in r.stderr or "runtime error:" in r.stderr
    assert r.returncode != 0 and reported, "sanitizer inactive"


def _clean(r):
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    runtime = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = tmp_path / "canary.c"
    src.write_text(CANARY)
    _check_canary(["gcc", "-O1", "-g", *SAN, str(src), "-o", str(tmp_path / "canary")], str(tmp_path / "canary"))

    lib = tmp_path / "liboracle_san.so"
    r = _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN, "-o", str(lib),
              os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"])
    assert r.returncode == 0, r.stderr
    driver = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle.oracle as O; O._LIB_PATH = %r\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_oracle.py',\n"
        "                  'tests/test_oracle_book.py', 'tests/test_golden.py'])\n"
        "assert O.lib()._name == %r, O.lib()._name\n"
        "sys.exit(int(rc))\n" % (ROOT, os.path.join(ROOT, "tests"), str(lib), str(lib)))
    _clean(_run([sys.executable, "-c", driver], env=_env(runtime)))


def test_host_api_under_address_and_undefined_sanitizers(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    objs = sorted(glob.glob(os.path.join(ROOT, "linear_attention_ssm_gdn_amd", "_build", "*.o")))
    dev_objs = [o for o in objs if os.path.basename(o) != "gdn_api.o"]
    if not rts or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    if len(dev_objs) + 1 != len(objs) or not dev_objs:
        pytest.skip("the library's objects are not built (run __graft_entry__.build())")
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    src = tmp_path / "canary.cpp"
    src.write_text(CANARY.replace("malloc(8)", "(char*)malloc(8)"))
    _check_canary([HIPCC, "-O1", "-g", *host_san, str(src), "-o", str(tmp_path / "canary")],
                  str(tmp_path / "canary"))

    obj = tmp_path / "gdn_api_san.o"
    r = _run([HIPCC, "--offload-arch=gfx950", "-mcode-object-version=5", "-O1", "-g", "-std=c++17", "-fPIC",
              "-fvisibility=hidden", *host_san, "-I" + os.path.join(ROOT, "include"), "-c",
              os.path.join(ROOT, "linear_attention_ssm_gdn_amd", "csrc", "gdn_api.cpp"), "-o", str(obj)])
    assert r.returncode == 0, r.stderr
    lib = tmp_path / "libgdn_san.so"
    r = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, "-o", str(lib), str(obj), *dev_objs])
    assert r.returncode == 0, r.stderr
    driver = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import linear_attention_ssm_gdn_amd._lib as L; L.LIB_PATH = %r\n"
        "import pytest\n"
        "rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py'])\n"
        "assert L.load()._name == %r, L.load()._name\n"
        "sys.exit(int(rc))\n" % (ROOT, os.path.join(ROOT, "tests"), str(lib), str(lib)))
    _clean(_run([sys.executable, "-c", driver], env=_env(rts[-1])))
