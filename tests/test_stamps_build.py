"""The measurement build (per-workgroup timestamps, include/tri_stamps.h): it compiles, exports
every call of include/tri.h plus the two of include/tri_stamps.h, reports its buffer layout
without a GPU, and the normal libtri.so exports neither stamps call. Builds the library into a
temporary directory (about a minute)."""
import ctypes
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    return set(re.findall(r"\b(tri_[a-z0-9_]+)\s*\(", open(os.path.join(ROOT, "include", header)).read()))


def _exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if " T " in ln}


def test_stamps_build_exports_and_layout(tmp_path):
    from rotary_frequency_key_amd import build as B

    lib = B.build_stamps(str(tmp_path / "libtri_stamps.so"))
    stamps = _declared("tri_stamps.h")
    assert stamps == {"tri_stamps_layout", "tri_stamps_attach"}
    assert (_declared("tri.h") | stamps) <= _exported(lib)
    h = ctypes.CDLL(lib)
    w, p, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert h.tri_stamps_layout(ctypes.byref(w), ctypes.byref(p), ctypes.byref(k)) == 0
    assert (w.value, p.value, k.value) == (4096, 8, 3)


def test_normal_build_has_no_stamps():
    lib = os.path.join(ROOT, "rotary_frequency_key_amd", "libtri.so")
    assert not ({"tri_stamps_layout", "tri_stamps_attach"} & _exported(lib))
