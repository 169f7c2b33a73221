"""Build libssd.so (HIP, gfx950) in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssd.so")
SOURCES = ["kernels.hip", "attn_group.hip", "decode.hip", "tree.hip", "api.hip", "profile.hip", "noalloc.hip"]
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Kernels that must not use scratch (private) memory: the decode-block
# projections and attention keep every value in registers / LDS.
NO_SCRATCH = {"decode.hip": ("dec_gemm_kernel", "attn_dec_kernel"), "kernels.hip": ("gemm_bf16_tiled",),
              "attn_group.hip": ("attn_group_kernel",)}


def _check_no_scratch(src, remarks):
    """Fail the build when a listed kernel spills to scratch."""
    kernels = NO_SCRATCH[src]
    current = None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            current = line.split("Function Name:")[1].split()[0]
        elif current and any(k in current for k in kernels) and "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size != 0:
                raise RuntimeError("%s uses %d bytes/lane of scratch (register spills)" % (current, size))


def build(verbose=False):
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = ["/opt/rocm/bin/hipcc"] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src in NO_SCRATCH:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for (cmd, p), src in zip(procs, SOURCES):
        out, err = p.communicate()
        if p.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), out, err))
        if src in NO_SCRATCH:
            _check_no_scratch(src, err)
        elif verbose and err:
            print(err)
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
