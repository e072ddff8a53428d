"""Build libmoeq.so in-tree with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoeq.so")

SOURCES = ["api.hip", "quantize.hip", "router.hip", "route.hip", "permute.hip", "gemm_decode.hip", "gemm_prefill.hip", "dequant.hip", "combine.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def hip_runtime_dir() -> str:
    """Directory of the HIP runtime the process uses for device memory and streams.

    The library links the same libamdhip64 as torch (torch ships its own copy): one HIP
    runtime per process, so torch's pointers, streams and events are valid in libmoeq.
    """
    import torch
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    if os.path.exists(os.path.join(d, "libamdhip64.so")):
        return d
    return "/opt/rocm/lib"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    # one hipcc per source, a few at a time (each is a separate process)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 8)) as ex:
        for f in [ex.submit(_run, [HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o], verbose)
                  for s, o in zip(SOURCES, objs)]:
            f.result()
    rt = hip_runtime_dir()
    tmp = LIB + ".tmp"
    # plain host link (no implicit -lamdhip64): the device code objects are embedded in the
    # host objects and registered by their constructors
    # --no-undefined: a kernel whose host stub is missing fails here, not at load time
    _run([CLANGXX, "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp,
          os.path.join(rt, "libamdhip64.so"), f"-Wl,-rpath,{rt}"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
