"""Builds the gfx950 training-step library liblmstep.so in-tree with hipcc.

Every HIP/C++ source under csrc/ is compiled to an object for gfx950, then
linked into one shared library next to this file. Run as a script or call
build().
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblmstep.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(HERE, "..", "include"),
]


# Per-file additions. The attention kernels run their softmax arithmetic on
# the MFMA results: the VGPR form of the MFMA keeps those results out of the
# accumulation registers, which saves a copy per score element.
FILE_FLAGS = {
    "k_attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return src, obj, r.returncode, msg


def build(jobs=None, verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs))
    objs = []
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, msg in ex.map(_compile, srcs):
            if msg.strip() and verbose:
                print(msg, file=sys.stderr)
            if rc:
                raise RuntimeError("hipcc failed on " + src)
            objs.append(obj)
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
