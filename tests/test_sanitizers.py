"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

* The oracle (``oracle/linattn_oracle.c``) is rebuilt with gcc's ASan and UBSan
  and its pins run against that build (the sanitizer runtimes preloaded into
  the test's own Python), so any out-of-bounds access, use after free,
  overflow or undefined operation in it fails the test.
* The C ABI's host code (argument checks, plan, workspace arithmetic) is
  rebuilt with clang's ASan and UBSan on the host side only and
  ``tests/test_abi.py`` runs against it: every validation path of every entry
  point, none of which launches a kernel.
* A planted out-of-bounds write in a copy of the oracle must be reported, so a
  silent harness cannot pass.
"""
import hashlib
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "linattn_oracle.c")
API_SRC = os.path.join(ROOT, "linear_attention_phi_amd", "csrc", "api.hip")
ORACLE_PINS = ["test_oracle.py", "test_oracle_delta.py", "test_oracle_backward.py", "test_oracle_lowp.py",
               "test_oracle_snapshots.py"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_oracle(src_text, out_dir):
    src = os.path.join(out_dir, "oracle_san.c")
    with open(src, "w") as f:
        f.write(src_text)
    lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN_FLAGS, "-o", lib, src, "-lm"],
                   check=True)
    return lib


def run_pytest(files, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", **env_extra)
    # -s: the sanitizer reports go to the process's stderr, not through pytest's capture
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                           *[os.path.join(ROOT, "tests", f) for f in files]],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def sanitizer_report(r):
    text = r.stdout + r.stderr
    return "AddressSanitizer" in text or "runtime error:" in text


def gcc_preload():
    return gcc_runtime("libasan.so") + ":" + gcc_runtime("libubsan.so")


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = build_oracle(open(ORACLE_SRC).read(), str(tmp_path))
    r = run_pytest(ORACLE_PINS, {"LD_PRELOAD": gcc_preload(), "LINATTN_ORACLE_LIB": lib})
    assert r.returncode == 0 and not sanitizer_report(r), (r.stdout + r.stderr)[-4000:]


def test_the_harness_reports_a_planted_overflow(tmp_path):
    src = open(ORACLE_SRC).read()
    site = "                ot[j] = num[j] / (den + eps);\n"
    assert src.count(site) == 1
    bad = src.replace(site, site + "            ot[Dv] = ot[0];\n")  # one element past the output row
    lib = build_oracle(bad, str(tmp_path))
    r = run_pytest(["test_oracle.py"], {"LD_PRELOAD": gcc_preload(), "LINATTN_ORACLE_LIB": lib})
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stdout + r.stderr


def build_abi_library():
    """liblinattn.so with clang's ASan and UBSan on the host side (cached by source hash)."""
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "linear_attention_phi_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            h.update(f.encode() + open(os.path.join(d, f), "rb").read())
    out_dir = os.path.join(tempfile.gettempdir(), "linattn_sanitize_" + h.hexdigest()[:16])
    lib = os.path.join(out_dir, "liblinattn_san.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(out_dir, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "hipcc")
    host = []
    for flag in ["-O1", "-g", *SAN_FLAGS]:
        host += ["-Xarch_host", flag]
    tmp = lib + ".tmp%d" % os.getpid()
    # device code unoptimized (never launched here; this keeps the build short)
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O0", "-std=c++17", "-fPIC", "-shared", *host,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-o", tmp, API_SRC], check=True, capture_output=True)
    os.replace(tmp, lib)
    return lib


def clang_asan_runtime():
    hipcc = os.environ.get("HIPCC", "hipcc")
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path):
        # the runtime sits with the compiler's resource directory
        res = subprocess.run([hipcc, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
        path = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path


def test_c_abi_validation_under_asan_and_ubsan():
    rt = clang_asan_runtime()
    if not os.path.exists(rt):
        pytest.skip(f"clang ASan runtime not found ({rt})")
    lib = build_abi_library()
    r = run_pytest(["test_abi.py"], {"LD_PRELOAD": rt, "LINATTN_ABI_LIB": lib})
    assert r.returncode == 0 and not sanitizer_report(r), (r.stdout + r.stderr)[-4000:]
