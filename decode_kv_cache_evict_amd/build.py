"""Build libkvevict.so (HIP for gfx950) in-tree: ``python -m decode_kv_cache_evict_amd.build``."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libkvevict.so")
SOURCES = ["api.cpp", "score.hip", "select.hip", "budgets.hip", "fps.hip", "epikv.hip", "rope.hip", "attention.hip", "skipkv.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         # packed fp32 instructions stay off in every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results in arch VGPRs (no accumulator-register copies in the score loops)
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def _compile(src, extra=(), suffix=""):
    obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False, extra=(), suffix="", lib=LIB):
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, suffix), SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


DEBUG_LIB = os.path.join(LIBDIR, "libkvevict_debug.so")


def build_debug(verbose=False):
    """libkvevict_debug.so: every source built with -DKVE_DEBUG, which checks
    the indices of the select, compact, in-place and gather stages against
    their segment before each access and reports misses through
    kve_debug_flags() instead of touching memory."""
    return build(verbose, extra=("-DKVE_DEBUG",), suffix="_debug", lib=DEBUG_LIB)


STAMPS_LIB = os.path.join(LIBDIR, "libkvevict_stamps.so")


def build_stamps(verbose=False):
    """libkvevict_stamps.so: every source built with -DKVE_STAMPS, whose one-call
    trigger kernels record a memory-clock stamp at each phase boundary of every
    work-group item (read with kve_debug_stamps())."""
    return build(verbose, extra=("-DKVE_STAMPS",), suffix="_stamps", lib=STAMPS_LIB)


SAN_LIB = os.path.join(LIBDIR, "libkvevict_san.so")
# host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C-ABI layer
# (argument checks, workspace carving, launch set-up); device code is built as usual
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_sanitized():
    """libkvevict_san.so: api.cpp built with host ASan/UBSan, linked with the
    kernel objects of the regular build (build() first).  Load it with the
    compiler's ASan runtime preloaded (sanitizer_runtime())."""
    objs = [os.path.join(LIBDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: {missing[0]} is missing")
    obj = os.path.join(LIBDIR, "api_san.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [HIPCC, *flags, *SAN_FLAGS, "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized api.cpp:\n{r.stderr}")
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libasan", *SAN_FLAGS[:4], obj, *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_runtime():
    """The compiler's shared ASan runtime (to preload into the Python process)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to hipcc")
    return hits[-1]


if __name__ == "__main__":
    print(build(verbose=True))
    if "--debug" in sys.argv:
        print(build_debug(verbose=True))
    if "--stamps" in sys.argv:
        print(build_stamps(verbose=True))
    if "--sanitized" in sys.argv:
        print(build_sanitized())
