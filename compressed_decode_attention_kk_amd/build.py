"""Build the gfx950 shared library libkk.so in place (hipcc, no torch extension).

    python -m compressed_decode_attention_kk_amd.build
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkk.so")
# the decode kernel's variants are separate translation units so that they
# compile in parallel (the three-row-block one takes the longest)
SOURCES = ["kk_decode_full3.hip", "kk_decode_full12.hip", "kk_decode_lean.hip", "kk_decode_gqa.hip",
           "kk_decode.hip", "kk_host.cpp", "kk_write.hip", "kk_epilogue.hip", "kk_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (the kernels only use packed fp16 math)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-fPIC", "-shared"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noisy = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    return res.returncode, "\n".join(noisy)


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compiles every source to an object (in parallel, in a temporary
    folder), then links libkk.so in place."""
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with tempfile.TemporaryDirectory(prefix="kk_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        failed = [(s, log) for s, (rc, log) in zip(SOURCES, results) if rc != 0]
        for s, log in failed:
            sys.stderr.write(f"--- {s}\n{log}\n")
        if failed:
            raise RuntimeError("hipcc failed building libkk.so: " + ", ".join(s for s, _ in failed))
        if verbose:
            for s, (_, log) in zip(SOURCES, results):
                if log:
                    print(f"--- {s}\n{log}")
        rc, log = _run([HIPCC, *LINK_FLAGS, *objs, "-o", LIB + ".tmp"], verbose)
        if rc != 0:
            sys.stderr.write(log + "\n")
            raise RuntimeError("hipcc failed linking libkk.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
