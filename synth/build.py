"""Build the generator: libsynth.so (host, gcc) and libsynth_gpu.so (device, hipcc gfx950).

Both builds must keep -ffp-contract=off: the two agree bit for bit only if
neither fuses a multiply and an add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build_host():
    out = os.path.join(HERE, "libsynth.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
                    "-Wall", "-Wextra", os.path.join(HERE, "synth.c"), "-o", out], check=True)
    return out


def build_gpu():
    out = os.path.join(HERE, "libsynth_gpu.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fPIC",
                    "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    os.path.join(HERE, "synth_gpu.hip"), "-o", out], check=True,
                   stderr=subprocess.PIPE)
    return out


if __name__ == "__main__":
    print(build_host(), build_gpu())
