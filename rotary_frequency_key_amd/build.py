"""Build libtri.so in place with hipcc for gfx950.

    python -m rotary_frequency_key_amd.build           (or rotary_frequency_key_amd.build.build())
    python -m rotary_frequency_key_amd.build --stamps  (libtri_stamps.so, the measurement build)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("score.hip", "score_max.hip", "select.hip", "compact.hip",
                                                    "noalloc.hip", "tri_api.cpp")]
OUT = os.path.join(HERE, "libtri.so")
STAMPS_OUT = os.path.join(HERE, "libtri_stamps.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed FP32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = OUT, defines=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_stamps(out: str = STAMPS_OUT, verbose: bool = False) -> str:
    """The library with per-workgroup memory-clock stamps in the pass's kernels (include/tri_stamps.h).
    Load it through TRI_LIBRARY; bench.py --timeline reads the stamps of a stream of passes."""
    return build(verbose=verbose, out=out, defines=("TRI_STAMPS",))


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with its host code built with AddressSanitizer and UndefinedBehaviorSanitizer
    (the device code is unsanitized and unoptimised: this build is for the host-side tests, which
    launch no kernel). Load it through TRI_LIBRARY with the ASan runtime preloaded
    (asan_runtime())."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f != "-O3"]
    cmd = [hipcc, *flags, "-O0", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           *SOURCES, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    return out


def asan_runtime() -> str:
    """Path of the ASan runtime of the compiler hipcc drives."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found: " + (res.stdout + res.stderr))
    return path


if __name__ == "__main__":
    if "--stamps" in sys.argv:
        print(build_stamps(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
