"""Compile the HIP sources into the in-tree shared libraries.

libwkv.so        -- the WKV library (csrc/*.hip), C ABI in include/wkv.h
../synth/libwkv_synth.so -- device input generator (synth/philox_fill.hip)

Built for gfx950 only, with packed-fp32 instruction selection disabled and
floating-point contraction off (every fused multiply-add in the kernels is
written out explicitly).
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwkv.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "philox_fill.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libwkv_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
SOURCES = ["wkv_api.hip", "wkv_forward.hip", "wkv_step.hip", "wkv_token_shift.hip", "wkv_session.hip", "wkv_backward.hip", "wkv_mat.hip"]


# Per-source flags: the matrix-state kernels keep their MFMA accumulators in
# ordinary VGPRs (the state is scaled by the vector units between products;
# accumulator registers would add a copy each way every chunk).
EXTRA_FLAGS = {"wkv_mat.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, flush=True)


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> None:
    """Always recompiles both libraries."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append(([HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj],
                     obj))
    synth_obj = os.path.join(objdir, "philox_fill.o")
    jobs.append(([HIPCC, *FLAGS, "-c", SYNTH_SRC, "-o", synth_obj], synth_obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    _link([o for _, o in jobs[:-1]], LIB, verbose)
    _link([synth_obj], SYNTH_LIB, verbose)


if __name__ == "__main__":
    build(verbose=True)
