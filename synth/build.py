"""Compile the seeded input generator: host library (gcc) and device library (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libssd_synth_host.so")
DEV_LIB = os.path.join(HERE, "libssd_synth_dev.so")

HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_host():
    _run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          os.path.join(HERE, "synth_host.c"), "-o", HOST_LIB + ".tmp"])
    os.replace(HOST_LIB + ".tmp", HOST_LIB)


def build_dev():
    _run(["/opt/rocm/bin/hipcc"] + HIP_FLAGS + ["-I", HERE, os.path.join(HERE, "synth_dev.hip"),
                                                "-o", DEV_LIB + ".tmp"])
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


def build():
    build_host()
    build_dev()


if __name__ == "__main__":
    build()
