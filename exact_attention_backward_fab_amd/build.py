"""Build libfab.so (HIP, gfx950) in-tree: exact_attention_backward_fab_amd/libfab.so.

Each source is compiled to an object of its own (in parallel, with its own extra
flags) and the objects are linked into the shared library."""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libfab.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# source -> extra compile flags
SOURCES = {
    "fab_aux.hip": [],
    "fab_fwd.hip": [],
    "fab_bwd.hip": [],
    # matrix-core accumulators in VGPRs: the online-softmax rescale and the dS
    # arithmetic work on them with plain VALU instructions
    "fab_qouter.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fab_api.cpp": [],
    "fab_noalloc.hip": [],
    "fab_probe.hip": [],
}
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    # no packed-f32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _clean(stderr: str) -> str:
    # host passes do not know the packed-fp32 feature (the flag is for the device pass)
    skip = ("packed-fp32-ops", "warnings generated")
    return "\n".join(l for l in (stderr or "").splitlines() if not any(k in l for k in skip))


def build(verbose: bool = False, extra=None) -> str:
    tmp = tempfile.mkdtemp(prefix="fab_build_")
    try:
        procs = []
        objs = []
        for src, sflags in SOURCES.items():
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC] + FLAGS + sflags + (extra or []) + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            _, err = pr.communicate()
            err = _clean(err)
            if pr.returncode != 0:
                failed.append(f"{src}:\n{err}")
            elif verbose and err.strip():
                print(err)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", OUT + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_clean(r.stderr)}")
        os.replace(OUT + ".tmp", OUT)
        return OUT
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
