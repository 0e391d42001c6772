"""Build the HIP library ``libpaged_attn.so`` for gfx950, in-tree.

    python -m paged_gqa_attention_02_amd.build

Every kernel is compiled with packed-fp32 VALU instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpaged_attn.so")
SOURCES = ["api.cpp", "decode.hip", "merge.hip", "gather.hip", "extend.hip", "append.hip",
           "mla.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    return res.returncode, err


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object in parallel (one hipcc each), then
    link the shared library; the library is replaced only when all succeed."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC] + flags() + ["-c", "-o", o, s] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
        if err and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([HIPCC] + flags() + ["-shared", "-o", tmp] + objs + ["-ldl"])
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitized variant: the host code (planning, argument checks, the
# scratch lookup) under AddressSanitizer and UndefinedBehaviorSanitizer, every
# finding fatal; device code is built as usual.  A process loading it must
# preload clang's ASan runtime (sanitizer_preload()).
HOST_SOURCES = ["api.cpp", "noalloc.hip"]
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-g"]


def sanitizer_preload() -> str:
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    path = res.stdout.strip()
    if not os.path.isabs(path):
        # older drivers print the bare name: look in the compiler's resource dir
        rd = subprocess.run([HIPCC, "-print-resource-dir"], capture_output=True, text=True,
                            check=True).stdout.strip()
        path = os.path.join(rd, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path


def build_host_sanitized(outdir: str, verbose: bool = False) -> str:
    """Build libpaged_attn.so into outdir with the host sources sanitized and
    the kernels' objects from the last build() (built first if missing)."""
    objdir = os.path.join(PKG, "_build")
    kernels = [s for s in SOURCES if s not in HOST_SOURCES]
    kobjs = [os.path.join(objdir, s + ".o") for s in kernels]
    if not all(os.path.exists(o) for o in kobjs):
        build(verbose=verbose)
    os.makedirs(outdir, exist_ok=True)
    hobjs = []
    for s in HOST_SOURCES:
        o = os.path.join(outdir, s + ".o")
        cmd = [HIPCC] + flags() + ["-O1"] + SANITIZE_HOST + ["-c", "-o", o,
                                                           os.path.join(CSRC, s)]
        rc, err = _run(cmd)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
        hobjs.append(o)
    out = os.path.join(outdir, "libpaged_attn.so")
    rc, err = _run([HIPCC] + flags() + SANITIZE_HOST + ["-Xarch_host", "-shared-libsan",
                                                        "-shared", "-o", out] +
                   hobjs + kobjs + ["-ldl"])
    if rc != 0:
        raise RuntimeError(f"hipcc link failed ({rc}):\n{err}")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
