"""Build libtpshard.so in-tree with hipcc, for gfx950 only.

    python -m megatron_sharded_linears_amd.build                # the library
    python -m megatron_sharded_linears_amd.build --incremental  # recompile changed sources only
    python -m megatron_sharded_linears_amd.build sanitized      # + the host ABI layer under ASan/UBSan

Each source compiles to an object in parallel under _build/ at the repository
root; the objects link into megatron_sharded_linears_amd/libtpshard.so next
to this file. Builds with extra -D flags (tuning) and the sanitized build keep
their objects and libraries under _build/ too, never beside the sources.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtpshard.so")

KERNEL_SOURCES = ["memops.hip", "gemm_skinny.hip", "gemm_tiled.hip", "attention.hip", "noalloc.hip"]
SOURCES = ["abi.cpp"] + KERNEL_SOURCES

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # never emit packed fp32 arithmetic (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def _newest_header():
    paths = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    paths += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return max(os.path.getmtime(p) for p in paths)


def _compile(job):
    src, build_dir, defines, incremental = job
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj) and os.path.getmtime(obj) > max(
            os.path.getmtime(os.path.join(CSRC, src)), _newest_header()):
        return obj
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
    _run(cmd, f"hipcc on {src}")
    return obj


def _objects(build_dir, defines, sources, incremental=False):
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        return list(ex.map(_compile, [(src, build_dir, tuple(defines), incremental) for src in sources]))


def build(verbose=True, lib=None, defines=(), incremental=False):
    """Compile every source and link `lib` (default: the in-tree library).
    `defines` are extra -D flags, for tuning builds (objects in _build/<tag>).
    incremental: reuse objects newer than their source and every header."""
    lib = lib or LIB
    tag = "obj" if not defines else "_".join(d.replace("=", "") for d in defines)
    objs = _objects(os.path.join(BUILD, tag), defines, SOURCES, incremental)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, "link")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_sanitized(verbose=True):
    """The library with its host-side ABI layer (abi.cpp: validation, kernel
    choice, dispatch) compiled by g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the same gfx950 kernel objects as
    the in-tree library (built if missing). GPU code is not instrumented. Load
    it with gcc's libasan preloaded (LD_PRELOAD) and TPSHARD_LIB pointing at
    the returned path."""
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    kdir = os.path.join(BUILD, "obj")
    kobjs = [os.path.join(kdir, s + ".o") for s in KERNEL_SOURCES]
    if not all(os.path.exists(o) for o in kobjs):
        kobjs = _objects(kdir, (), KERNEL_SOURCES)
    abi_obj = os.path.join(out_dir, "abi.cpp.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-I", CSRC] + san +
         ["-c", os.path.join(CSRC, "abi.cpp"), "-o", abi_obj], "g++ (sanitized abi.cpp)")
    lib = os.path.join(out_dir, "libtpshard_asan.so")
    _run(["g++", "-shared", "-o", lib + ".tmp", abi_obj] + kobjs + san +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], "sanitized link")
    os.replace(lib + ".tmp", lib)
    if verbose:
        print(f"built {lib}")
    return lib


def asan_runtime():
    """Path of gcc's AddressSanitizer runtime, to preload."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
    if "sanitized" in sys.argv:
        build_sanitized()
