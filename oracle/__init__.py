"""TEST INFRASTRUCTURE: the fp64 CPU oracle of the FlashAttention forward pass.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import
this package.  It never touches the GPU library and shares no code with it; the two meet
only through the seeded inputs of ``synth``.

``attention()`` is a thin ctypes wrapper of ``fa_oracle.c`` (plain C, fp64, one query row
at a time: visible scores, softmax, weighted sum of V).  The definition it follows is
"FlashAttention forward in C" (tinyllm L9.3) section 2.1 plus the additive mask of
"Fused attention and softmax: fast and exact" (OneModel), "What is computed", and the softcap
and ALiBi score variants the candle page names; the C source header lists the readings taken
where the pages are silent.

Every function here is pinned by ``tests/test_oracle_pins.py`` (worked example, closed
forms, the 50-digit decimal brute force of ``tests/brute_decimal.py``, torch's fp64 SDPA,
planted mistakes).  ``FA_ORACLE_LIB`` in the environment names another build of the same
source to load instead (the sanitizer test runs the pins against an ASan/UBSan build).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F64, F32, BF16 = 0, 1, 2
_LIBS = {}


def _load(path=None):
    path = path or os.environ.get("FA_ORACLE_LIB") or _build.LIB
    if path not in _LIBS:
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.orc_attention.restype = ctypes.c_int
        lib.orc_attention.argtypes = [
            ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_void_p, i64p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ]
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_visible_pairs.restype = ctypes.c_int64
        lib.orc_visible_pairs.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_int64]
        _LIBS[path] = lib
    return _LIBS[path]


def _strides(a, n):
    st = tuple(s // a.itemsize for s in a.strides)
    assert len(st) == n
    return (ctypes.c_int64 * n)(*st)


def _as_input(a, dtype):
    a = np.asarray(a)
    if dtype == BF16:
        a = a.astype(np.uint16, copy=False)
    elif dtype == F32:
        a = a.astype(np.float32, copy=False)
    else:
        a = a.astype(np.float64, copy=False)
    if a.ndim != 4:
        raise ValueError("q, k, v must be 4-d [B, H, T, d]")
    if a.shape[3] > 1 and a.strides[3] != a.itemsize:
        a = np.ascontiguousarray(a)
    return a


def attention(q, k, v, *, scale, q_offset=0, causal=True, window=0, sinks=None, mask=None,
              softcap=0.0, alibi=None, rows=None, dtype=None, threads=None, lib_path=None):
    """fp64 attention rows.

    q: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d] -- numpy arrays of float64, float32, or uint16
    holding bf16 bits (``dtype=BF16``).  ``scale`` is widened exactly (pass the fp32 value the
    GPU receives).  ``mask``: None or a 4-d float32 array indexable as [b, h, i, j] (size-1 or
    stride-0 axes broadcast).  ``sinks``: None or float32 [Hq].  ``softcap``: c > 0 turns the
    logit into c tanh(logit / c) (0: none).  ``alibi``: None or float32 [Hq] slopes (score
    -slope |p - j|).  ``rows``: None (all rows) or an
    int64 array [n, 3] of (b, h, i).  Returns (o, lse) in fp64: [B, Hq, Tq, d] and [B, Hq, Tq]
    for all rows, else [n, d] and [n].
    """
    if dtype is None:
        dtype = BF16 if np.asarray(q).dtype == np.uint16 else (F32 if np.asarray(q).dtype == np.float32 else F64)
    q, k, v = (_as_input(t, dtype) for t in (q, k, v))
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch")
    sk_ = _strides(k, 4)
    if Tk == 0:
        k = v = np.zeros((1, 1, 1, d), q.dtype)
    sinks_arr = None if sinks is None else np.ascontiguousarray(np.asarray(sinks, np.float32))
    alibi_arr = None if alibi is None else np.ascontiguousarray(np.asarray(alibi, np.float32))
    mask_arr = smask = None
    if mask is not None:
        mask_arr = np.asarray(mask, np.float32)
        if mask_arr.ndim != 4:
            raise ValueError("mask must be 4-d [b, h, i, j] (broadcast views allowed)")
        smask = (ctypes.c_int64 * 4)(*[(s // 4) if n > 1 else 0 for s, n in zip(mask_arr.strides, mask_arr.shape)])
    if rows is None:
        n = B * Hq * Tq
        rows_arr = None
        o_shape, l_shape = (B, Hq, Tq, d), (B, Hq, Tq)
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
        n = rows_arr.shape[0]
        o_shape, l_shape = (n, d), (n,)
    o = np.empty(o_shape, np.float64)
    lse = np.empty(l_shape, np.float64)
    lib = _load(lib_path)
    if threads is not None:
        lib.orc_set_threads(int(threads))
    rc = lib.orc_attention(
        q.ctypes.data, _strides(q, 4), k.ctypes.data, _strides(k, 4) if Tk else sk_, v.ctypes.data,
        _strides(v, 4) if Tk else sk_, dtype, B, Hq, Hkv, Tq, Tk, d, float(np.float64(scale)),
        int(q_offset), int(bool(causal)), int(window),
        None if sinks_arr is None else sinks_arr.ctypes.data,
        None if mask_arr is None else mask_arr.ctypes.data, smask, float(softcap),
        None if alibi_arr is None else alibi_arr.ctypes.data,
        None if rows_arr is None else rows_arr.ctypes.data, n if rows_arr is not None else 0,
        o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, lse


def visible_pairs(Tq, Tk, q_offset=0, causal=True, window=0):
    """sum_i |V_i| for one (b, h): the pairs the FLOP count is taken over."""
    return int(_load().orc_visible_pairs(Tq, Tk, q_offset, int(bool(causal)), window))


def threads():
    """OpenMP threads the oracle's row loop uses."""
    return int(_load().orc_max_threads())
