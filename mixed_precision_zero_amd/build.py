"""Build libneox_zero1.so (gfx950) in-tree with hipcc."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SO = os.path.join(PKG, "libneox_zero1.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("zero1_kernels.hip", "zero1_api.hip",
                                                   "zero1_noalloc.hip")]
PROBE_SO = os.path.join(PKG, "libneox_stream_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "stream_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit contraction: every fused multiply-add in the kernels is written out
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


def _hipcc(sources, out, verbose):
    tmp = out + ".tmp"
    res = subprocess.run([HIPCC, *FLAGS, *sources, "-o", tmp], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """The step library, and the bandwidth-probe library the benchmark uses."""
    _hipcc(PROBE_SOURCES, PROBE_SO, verbose)
    return _hipcc(SOURCES, SO, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
