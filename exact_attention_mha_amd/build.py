"""Build the gfx950 attention library in-tree with hipcc.

    python -m exact_attention_mha_amd.build

compiles every csrc/*.hip translation unit for gfx950 and links
exact_attention_mha_amd/libmha_gfx950.so. Cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmha_gfx950.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# Where matrix-core results land (ordinary VGPRs or accumulation registers)
# is left to the compiler; kernels steer it with their launch bounds.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    """Compile all translation units in parallel and link the shared library.

    Returns the library path. Raises RuntimeError with the compiler output on
    failure. Always rebuilds.
    """
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    tmp = tempfile.mkdtemp(prefix="mha_build_")
    try:
        procs = []
        objs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        errors = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = out.decode(errors="replace")
            if pr.returncode != 0:
                errors.append(f"{src}:\n{text}")
            elif verbose and text.strip():
                print(text)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp_lib = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
