"""Builds libmla_decode.so (gfx950 HIP kernels + host library) in-tree.

    python -m latent_attention_decode_amd.build

Every HIP translation unit is compiled with packed fp32 arithmetic disabled
(-packed-fp32-ops); the host compiler pass warns that it does not know the
feature, which is harmless.  MFMA accumulators are kept in ordinary VGPRs
(-amdgpu-mfma-vgpr-form): the stage-1 kernels fit in 256 of them, and the
accumulation registers would otherwise cost a copy in and out of every tile.
"""

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_decode.so")
SOURCES = [os.path.join(CSRC, f) for f in ("mla_kernels.hip", "mla_stage1_fp8.hip", "mla_stage1_mxfp4.hip",
                                           "mla_decode.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def build(verbose: bool = False, sanitize: str = "", out: str = LIB) -> str:
    """Compile the library to `out`.  sanitize = "address" or "undefined"
    instruments the host code only (each -fsanitize= goes after -Xarch_host;
    the device code is built as usual) and links the sanitizer runtime
    dynamically; such a build is for host-side tests of the planner and the
    argument checks, loaded with the runtime preloaded."""
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wall", "-Wno-unused-command-line-argument",
           "-I", INCLUDE, "-I", CSRC, "-o", out + ".tmp"] + SOURCES
    if sanitize:
        if sanitize not in ("address", "undefined"):
            raise ValueError("sanitize must be 'address' or 'undefined'")
        cmd[1:1] = ["-Xarch_host", f"-fsanitize={sanitize}", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan", "-g"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and "unknown target feature" not in l.lower()
            and "reserved registers: m0" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


def sanitizer_runtime(sanitize: str) -> str:
    """Path of the clang sanitizer runtime that a build(sanitize=...) library
    links against (to preload into a process that loads the library)."""
    import glob
    name = {"address": "libclang_rt.asan-x86_64.so", "undefined": "libclang_rt.ubsan_standalone-x86_64.so"}[sanitize]
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))),
                                         "llvm", "lib", "clang", "*", "lib", "linux", name)))
    hits += sorted(glob.glob(os.path.join("/opt/rocm/llvm/lib/clang/*/lib/linux", name)))
    if not hits:
        raise FileNotFoundError(name)
    return hits[0]


if __name__ == "__main__":
    print(build(verbose=True))
