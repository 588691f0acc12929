"""Build libfa.so in-tree with hipcc for gfx950.

    python -m long_context_decode_fourier_amd.build

Every HIP source under csrc/ and the C-ABI host file are compiled (one object
each, in parallel) and linked into one shared library next to this file.
Packed-fp32 instructions are disabled for all device code (the compiler still
vectorises everything else).
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"


def sources():
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, f) for f in names]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# Per-source extra flags.  The two-pass decode kernels rotate their MFMA
# accumulators on the VALU every block: keeping those accumulators in VGPRs
# (not AGPRs) avoids a register copy per value and block.
EXTRA = {"decode_two_pass.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def compile_command(src, obj):
    return [hipcc(), *FLAGS, *EXTRA.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
            "-c", src, "-o", obj]


def link_command(objs, out):
    return [hipcc(), "--offload-arch=" + ARCH, "-fPIC", "-shared", *objs, "-o", out,
            "-Wl,-rpath,/opt/rocm/lib"]


def command(out):
    """One hipcc command that builds the whole library (every source, no
    per-source flags): for instrumented copies such as the host-sanitizer test."""
    return [hipcc(), *FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, *sources(), "-o", out,
            "-Wl,-rpath,/opt/rocm/lib"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "packed-fp32-ops"  # host pass does not know the device feature
    msgs = [l for l in res.stdout.splitlines() if noise not in l]
    if verbose and msgs:
        print("\n".join(msgs))
    return res.returncode, msgs


def build(verbose=False):
    """Compile every source to an object (in parallel), then link libfa.so."""
    import concurrent.futures
    import tempfile
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="fa_build_") as d:
        objs = [os.path.join(d, os.path.basename(s) + ".o") for s in sources()]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda so: _run(compile_command(*so), verbose), zip(sources(), objs)))
        for (rc, msgs), src in zip(results, sources()):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, "\n".join(msgs)))
        rc, msgs = _run(link_command(objs, tmp), verbose)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
