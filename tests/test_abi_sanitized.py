"""The C ABI's host layer under AddressSanitizer and UBSan (CPU only).

api.hip and rope_tables.hip (argument checks, launch planning, workspace
sizes, camera tokens, RoPE tables) are compiled with the sanitizers on their
host code only (-Xarch_host; device code is built as usual), linked with the
other objects of the regular build into tests/asan/abi_host_check.cpp, and
run.  That program feeds exactly-sized input arrays and canary-guarded
outputs to every host-only function and to the rejected-argument paths of
the device entry points, none of which reaches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segment_causal_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SANITIZED = ("api.hip", "rope_tables.hip")
REGULAR = ("kv_quant.hip", "rope3d.hip", "seg_attn.hip", "cam_xattn.hip", "w8a16.hip", "seg_attn_bwd.hip")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and ROCm clang++")
def test_abi_host_layer_under_asan_and_ubsan():
    from segment_causal_attention_amd import build as B
    os.makedirs(OUT, exist_ok=True)
    regular = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in REGULAR]
    if not all(os.path.exists(o) for o in regular):
        B.build()
    objs = []
    for s in SANITIZED:
        o = os.path.join(OUT, s.replace(".hip", ".o"))
        rc, out = _run([HIPCC, *B.FLAGS, "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-I",
                        os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, s), "-o", o])
        assert rc == 0, out
        objs.append(o)
    drv = os.path.join(OUT, "abi_host_check.o")
    host_san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    rc, out = _run([CLANG, "-std=c++17", "-O1", "-g", *host_san, "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "asan", "abi_host_check.cpp"), "-o", drv])
    assert rc == 0, out
    exe = os.path.join(OUT, "abi_host_check")
    rc, out = _run([CLANG, *host_san, drv, *objs, *regular, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "abi host checks passed" in out, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
