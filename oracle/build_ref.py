"""Build and load the C part of the oracle (test infrastructure).

``oracle/codec_ref.c`` is a second, value-based FP8 encoder used to check the
oracle's bit-level encoder over every fp32 bit pattern.  It is compiled with
gcc into ``oracle/lib/libcodecref.so``; only the tests load it.
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "codec_ref.c")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libcodecref.so")


def build(force: bool = True) -> str:
    """Compile codec_ref.c (always when force, else only when missing or older than the source)."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the oracle's C encoder")
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run([cc, "-O2", "-std=c99", "-shared", "-fPIC", SRC, "-o", tmp], check=True,
                   capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    """ctypes handle of the C encoder, building it first if needed."""
    lib = ctypes.CDLL(build(force=False))
    lib.fp8ref_encode_range.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
    lib.fp8ref_encode_range.restype = ctypes.c_int
    lib.fp8ref_encode_bits.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.fp8ref_encode_bits.restype = ctypes.c_int
    return lib
