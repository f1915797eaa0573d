"""Build libmxq.so (the HIP kernels and the C ABI) for gfx950, in-tree.

hipcc compiles every source under csrc/ into one shared library next to this
file.  Flags: -O3, no floating-point contraction (each rounding in the
quantizer is the single IEEE operation written), and packed-fp32
instructions disabled.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmxq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile each source to an object (in parallel), then link."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
              "-Wall", "-Wno-unused-function", "-Werror=inline-asm"]
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + common + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    link = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link))
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # the host pass does not know the packed-fp32 target feature; harmless
    lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose=True))
