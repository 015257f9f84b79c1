"""Seeded synthetic inputs (no attention arithmetic here).

Both sides of every parity check draw their inputs from this module: the GPU library gets
device copies, the fp64 oracle gets the host arrays.  The generator is splitmix64 +
Box-Muller, written in ``gen.c`` (built with gcc on first use or by ``build()``).

Seeds are derived from names: ``seed_of("c5", 0, "q")`` = first 8 bytes of
SHA-256("c5/0/q"), so a tensor of any workload can be regenerated alone.  ``FA_SYNTH_LIB`` in
the environment names another build of ``gen.c`` to load (the sanitizer test's).
"""
import ctypes
import hashlib
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gen.c")
LIB = os.path.join(HERE, "libsynth.so")
_lib = None


def build():
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", SRC,
           "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("FA_SYNTH_LIB") or LIB
        if path == LIB and not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(path)
        lib.synth_uniform_f64.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_void_p]
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_neg_inf_mask_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                               ctypes.c_void_p]
        for f in ("synth_uniform_f64", "synth_normal_f32", "synth_f32_to_bf16", "synth_neg_inf_mask_f32"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def seed_of(*parts):
    """Stable 64-bit seed from a name, e.g. seed_of("c3", layer, "k")."""
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little")


def uniform(seed, shape, start=0):
    out = np.empty(shape, np.float64)
    _load().synth_uniform_f64(seed, start, out.size, out.ctypes.data)
    return out


def normal_f32(seed, shape, mean=0.0, std=1.0, start=0):
    """fp32 N(mean, std^2), element n of the stream at flat index n (C order)."""
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, start, out.size, mean, std, out.ctypes.data)
    return out


def to_bf16_bits(a):
    """fp32 array -> uint16 bf16 bits (round to nearest even)."""
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().synth_f32_to_bf16(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed, shape, dtype="f32", mean=0.0, std=1.0):
    """N(mean, std^2) inputs: fp32 array, or uint16 bf16 bits (fp32 values rounded) for 'bf16'."""
    x = normal_f32(seed, shape, mean, std)
    return to_bf16_bits(x) if dtype == "bf16" else x


def neg_inf_mask(seed, shape, p):
    """fp32 mask whose entries are -inf with probability p, else 0."""
    out = np.empty(shape, np.float32)
    _load().synth_neg_inf_mask_f32(seed, 0, out.size, float(p), out.ctypes.data)
    return out
