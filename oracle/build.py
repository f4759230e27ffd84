"""Build the CPU oracle library (plain C, gcc).

TEST INFRASTRUCTURE: the oracle checks the HIP path and is never part of it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gsa_oracle.c")
LIBRARY = os.path.join(HERE, "libgsa_oracle.so")

# No -ffast-math and no FMA contraction: the oracle's arithmetic is exactly
# what its source says, in IEEE double (and float for the fp32 fold).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]


def build(source=SOURCE, output=LIBRARY, extra_flags=()):
    """Compile `source` into the shared library `output`; returns its path."""
    tmp = output + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
