"""Compile the gfx950 HIP kernels and the C-ABI host code into
attention_backward_fa2_amd/libfa_bwd.so (in-tree, so the built library travels
with the source tree).  Cross-compiles without a GPU."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfa_bwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed-fp32 VALU forms are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Hardware fp32 atomic add for the dQ accumulator (no CAS loop).
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")) +
                  glob.glob(os.path.join(HERE, "csrc", "*.cpp")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 feature;
    # that line is expected and harmless.
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    return res.returncode, msgs


def build(verbose: bool = False, extra=()) -> str:
    """Each source to an object in parallel (the kernel files dominate and
    take similar times), then one link."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(f) + "." + tag + ".o") for f in srcs]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    cmds = [[HIPCC, *compile_flags, *extra, "-c", f, "-o", o] for f, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, msgs), f in zip(results, srcs):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (f, "\n".join(msgs)))
            if verbose and msgs:
                print("\n".join(msgs))
        tmp = LIB + ".tmp" + tag
        rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
