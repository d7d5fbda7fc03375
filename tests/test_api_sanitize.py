"""The C-ABI argument validation (aware_tiling_amd/csrc/api.cpp) built for
the host with AddressSanitizer and UndefinedBehaviorSanitizer, its kernel
launchers replaced by stubs (tests/sanitize/api_stubs.cpp) that only count
launches, and driven by tests/sanitize/api_driver.cpp over a grid of extreme
arguments: negative, zero, boundary and INT64 extremes for every size,
non-finite scales, null and misaligned pointers, short workspaces, an
out-of-range dtype.  The run must be free of overflow and invalid access,
and a call may launch only when every pointer is valid.  Each mutant below
weakens one check in a copy of api.cpp; the driver must reject every one.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "aware_tiling_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or
                                not os.path.isdir("/opt/rocm/include"),
                                reason="g++ or the HIP headers not available")


def _build_and_run(api_cpp, tmp_path, name):
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{CSRC}",
           api_cpp, os.path.join(SAN, "api_stubs.cpp"), os.path.join(SAN, "api_driver.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_api_validation_clean_under_sanitizers(tmp_path):
    r = _build_and_run(os.path.join(CSRC, "api.cpp"), tmp_path, "api_driver")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api validation:" in r.stdout


MUTANTS = [
    ("shape_unbounded_d",
     "if (n > (int64_t(1) << 24) || d > (int64_t(1) << 16) || bh > (int64_t(1) << 20)) return false;",
     "if (n > (int64_t(1) << 24) || bh > (int64_t(1) << 20)) return false;"),
    ("fwd_null_pointers_accepted",
     "  if (!Q || !K || !V || !O) return ATTN_ERR_INVALID_ARG;\n"
     "  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;\n"
     "  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;\n"
     "  hipStream_t s = static_cast<hipStream_t>(stream);\n"
     "  if (dtype == ATTN_BF16)\n",
     "  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ATTN_ERR_INVALID_ARG;\n"
     "  if (lse && !aligned16(lse)) return ATTN_ERR_INVALID_ARG;\n"
     "  hipStream_t s = static_cast<hipStream_t>(stream);\n"
     "  if (dtype == ATTN_BF16)\n"),
    ("misaligned_accepted", "& 15u) == 0; }", "& 7u) == 0; }"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_api_mutant_caught(name, old, new, tmp_path):
    text = open(os.path.join(CSRC, "api.cpp")).read()
    assert text.count(old) == 1, f"mutation site not found once: {old}"
    # The copy sits in the source directory's place for its includes.
    mutant = tmp_path / "api.cpp"
    mutant.write_text(text.replace(old, new))
    r = _build_and_run(str(mutant), tmp_path, "api_driver_" + name)
    assert r.returncode != 0, f"mutant {name} not caught: {r.stdout}"
