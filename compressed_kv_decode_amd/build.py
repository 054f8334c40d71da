"""Build libtqkv.so for gfx950 in-tree (compressed_kv_decode_amd/libtqkv.so).

    python -m compressed_kv_decode_amd.build            # compile + link
    python -m compressed_kv_decode_amd.build --check-c  # also compile tqkv.h as C99

Every HIP source is compiled by hipcc for gfx950 only, with packed fp32
instructions disabled (the compiler would otherwise form v_pk_* fp32 ops
from ordinary float code).
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtqkv.so")
SOURCES = ["tq_host.cpp", "tq_append.hip", "tq_decode.hip", "tq_promote.hip", "tq_probe.hip", "tq_mips.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def check_c_header() -> None:
    """The public header must compile as plain C99 without HIP headers."""
    src = os.path.join(BUILD, "hdr_check.c")
    os.makedirs(BUILD, exist_ok=True)
    with open(src, "w") as f:
        f.write('#include "tqkv.h"\nint main(void) { tq_config c; (void)c; return (int)tq_version() & 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                        "-c", src, "-o", os.path.join(BUILD, "hdr_check.o")], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("tqkv.h does not compile as C99:\n" + r.stderr)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--check-c", action="store_true")
    a = ap.parse_args()
    build()
    if a.check_c:
        check_c_header()
        print("tqkv.h compiles as C99")
    sys.exit(0)
