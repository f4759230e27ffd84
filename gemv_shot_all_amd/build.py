"""Build libgsa.so (the HIP library behind include/gsa.h) for gfx950.

Compiled in-tree with hipcc so the shared library travels with the source
tree.  No -ffast-math: the one-shot sum's rank order must not be reassociated.
Packed-fp32 instruction selection is switched off for the device code.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgsa.so")
SOURCES = ["gsa_api.hip", "gemv_allreduce.hip", "moe_a2a.hip", "bias_rmsnorm.hip"]
# The benchmark's achievable-bandwidth reference (include/gsa_probe.h).
PROBE_LIBRARY = os.path.join(PKG, "libgsa_probe.so")
PROBE_SOURCES = ["hbm_read_probe.hip"]
ARCH = os.environ.get("GSA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _compile(srcs, output, extra_flags=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = output + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def build(output=LIBRARY, extra_flags=()):
    """Compile the operator's HIP sources into `output` (and the benchmark's
    read probe into its own library); returns the operator library's path."""
    _compile([os.path.join(CSRC, s) for s in PROBE_SOURCES], PROBE_LIBRARY, extra_flags)
    return _compile(sources(), output, extra_flags)


def needs_build():
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    deps = sources() + [os.path.join(CSRC, "gsa_internal.h"), os.path.join(CSRC, "gsa_device.h"),
                        os.path.join(INCLUDE, "gsa.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build())
