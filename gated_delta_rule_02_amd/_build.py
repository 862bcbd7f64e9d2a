"""Build libgdn.so (the gfx950 HIP kernels and the C ABI of include/gdn.h) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

# Packed fp32 instructions are disabled: ordinary float code is compiled to
# scalar fp32 instructions only.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source for gfx950 and link libgdn.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp%d" % os.getpid()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


BUILD_INFO = os.path.join(HERE, "build_info.json")


def _write_build_info() -> None:
    """Record the commit the library was built from next to it (the built
    library travels without the git history)."""
    import json
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        sha = r.stdout.strip() if r.returncode == 0 else None
        r = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--", "gated_delta_rule_02_amd/csrc",
                            "include"], capture_output=True, text=True, timeout=10)
        dirty = bool(r.stdout.strip()) if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        sha, dirty = None, None
    with open(BUILD_INFO, "w") as f:
        json.dump({"git_sha": sha, "sources_modified_since_commit": dirty}, f)


# Host-side sanitizers for the C ABI's validation code: AddressSanitizer and
# UBSan on the host pass only (device code is built as usual), every finding
# fatal.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g", "-O1"]


def build_sanitized(out_dir: str) -> str:
    """libgdn.so with gdn_api.cpp (argument validation, dispatch) compiled with
    host AddressSanitizer and UBSan, linked with the regular kernel objects,
    into out_dir.  Load it with the compiler's ASan runtime preloaded."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in sources():
        if os.path.basename(src) == "gdn_api.cpp":
            obj = os.path.join(out_dir, "gdn_api_san.o")
            cmd = [_hipcc(), "-x", "hip", *HIP_FLAGS, *SAN_FLAGS, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
            objs.append(obj)
        else:
            obj = os.path.join(BUILD, os.path.basename(src) + ".o")
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
                obj = _compile(src)
            objs.append(obj)
    lib = os.path.join(out_dir, "libgdn_san.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", lib, *objs,
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    return lib


def asan_runtime() -> str:
    """The host compiler's shared AddressSanitizer runtime (to preload)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([os.path.join(rocm, "llvm", "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                       "libclang_rt.asan-x86_64.so"))
        if not found:
            raise RuntimeError("no clang AddressSanitizer runtime under %s" % rocm)
        path = found[0]
    return path


if __name__ == "__main__":
    print(build())
