"""Host-sanitized build of libedit_attn.so for the CPU tests of the C ABI.

The C ABI's argument checks, workspace layout and launch sequencing live in
abi.cpp, which runs on the host. This builds a copy of the library whose
abi.cpp is compiled with AddressSanitizer and UndefinedBehaviorSanitizer on
the host side only (the device code is unchanged: GPU sanitizers are not part
of this build), linked with the kernels' objects from the ordinary build.
Loading it needs the clang ASan runtime first in the process
(LD_PRELOAD=asan_runtime()), which tests/test_abi_sanitized.py arranges.

    python linear_compressed_attention_amd/build_sanitized.py OUT_DIR
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
sys.path.insert(0, PKG)
import build as _build  # noqa: E402  (the ordinary build: sources, flags, object directory)

CLANG = "/opt/rocm/llvm/bin/clang++"
# host-side sanitizers: every -fsanitize= follows -Xarch_host, so no device code is instrumented
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm/lib/clang")
    return libs[-1]


def build_sanitized(out_dir: str) -> str:
    """Compile abi.cpp host-sanitized into out_dir and link it with the
    ordinary build's kernel objects (built first if missing). Returns the
    library's path."""
    os.makedirs(out_dir, exist_ok=True)
    obj_dir = os.path.join(ROOT, "_build")
    kernels = [s for s in _build.SOURCES if s != "abi.cpp"]
    objs = []
    for src in kernels:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(_build.CSRC, src)):
            os.makedirs(obj_dir, exist_ok=True)
            obj = _build._compile(src, obj_dir)
        objs.append(obj)
    abi_obj = os.path.join(out_dir, "abi_san.o")
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [_build.HIPCC] + flags + HOST_SAN + ["-x", "hip", "-c", os.path.join(_build.CSRC, "abi.cpp"),
                                               "-o", abi_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile of abi.cpp failed:\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(out_dir, "libedit_attn.so")
    # host link only (the objects already carry their gfx950 code), against the shared sanitizer runtime
    cmd = [CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", "-o", lib, abi_obj] + objs + \
          ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build_sanitized(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "sanitized")))
