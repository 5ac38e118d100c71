"""Build liboracle.so (plain C, host only). Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    out = os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(HERE, "oracle.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
