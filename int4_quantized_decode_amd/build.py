"""Build the HIP library (libi4d.so) in-tree for gfx950.

Compiles every source under csrc/ with hipcc (device code for gfx950 only)
and links one shared object next to this file.  Packed fp32 VALU forms are
disabled for all device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libi4d.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api_host.cpp", "api_device.hip", "proj.hip", "attn.hip", "lmhead.hip", "step.hip", "noalloc.hip", "proj_e4m3.hip", "prefill.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-fno-fast-math", "-ffp-contract=fast-honor-pragmas"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-file flags: the prefill GEMM keeps its MFMA results in VGPRs, where the
# group-scale FMAs read them without accumulator-register copies (measured
# faster there; the decode kernels are left to the default)
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC] + COMMON + DEVICE + EXTRA.get(src, []) + ["-c", path, "-o", obj]
        if src.endswith(".cpp"):
            # host-only translation unit: no fp contraction so the packer's
            # products and divisions are single IEEE operations
            cmd = [HIPCC, "-x", "c++"] + [c for c in COMMON if not c.startswith("-ffp-contract")] + \
                  ["-ffp-contract=off", "-c", path, "-o", obj]
        objs.append(obj)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if verbose and text.strip():
            print(text, file=sys.stderr)
        if p.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), text))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
