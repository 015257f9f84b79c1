"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol
include/fa.h declares, and rejects bad arguments before any launch.

Every call here is one that must fail validation (or has no rows, so nothing is launched):
no call may reach a kernel launch with these placeholder pointers.
"""
import ast
import ctypes
import os
import re
import subprocess
import sys

import pytest

import flashattention_forward_flash_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
P = 0x10000  # an aligned placeholder address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(fa.EXPORTED), names
    lib = fa.load_library()
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r" T (\w+)$", nm.stdout, re.M))
    assert set(names) <= exported


def test_one_hip_runtime_whatever_the_import_order():
    """torch carries its own HIP runtime: loading the library before importing torch must still
    leave one runtime in the process, or launches on torch's streams fail."""
    code = ("import re, sys; sys.path.insert(0, %r); import flashattention_forward_flash_amd as fa; "
            "fa.load_library(); import torch; "
            "print(sorted(set(re.findall(r'\\S*libamdhip64\\S*', open('/proc/self/maps').read()))))") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         timeout=300).stdout
    runtimes = ast.literal_eval(out.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes


def test_status_strings():
    for s in range(6):
        assert fa.fa_status_str(s)
    assert fa.fa_status_str(99) == "unknown status"


def _call(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Tq=8, Tk=8, d=64, scale=0.125, q_offset=0,
             causal=1, window=0, sinks=None, mask=None, strides=None, dtype=fa.FA_F32, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Tq"], a["Tk"],
                     a["d"], a["scale"], a["q_offset"], a["causal"], a["window"], a["sinks"], a["mask"],
                     a["strides"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(Hq=6, Hkv=4), fa.FA_ESHAPE),
    (dict(Hq=2, Hkv=4), fa.FA_ESHAPE),
    (dict(Hq=4, Hkv=0), fa.FA_ESHAPE),
    (dict(B=-1), fa.FA_EINVAL),
    (dict(Tq=-1), fa.FA_EINVAL),
    (dict(Tk=-5), fa.FA_EINVAL),
    (dict(q_offset=-1), fa.FA_EINVAL),
    (dict(d=0), fa.FA_EINVAL),
    (dict(scale=float("inf")), fa.FA_EINVAL),
    (dict(scale=float("nan")), fa.FA_EINVAL),
    (dict(q=None), fa.FA_EINVAL),
    (dict(o=None), fa.FA_EINVAL),
    (dict(k=None), fa.FA_EINVAL),
    (dict(d=96), fa.FA_EUNSUPPORTED),
    (dict(d=32), fa.FA_EUNSUPPORTED),
    (dict(dtype=7), fa.FA_EUNSUPPORTED),
    (dict(q=P + 8), fa.FA_EUNSUPPORTED),          # q not 16-byte aligned
    (dict(k=P + 4), fa.FA_EUNSUPPORTED),
    (dict(o=P + 8, dtype=fa.FA_F32), fa.FA_EUNSUPPORTED),
    (dict(Tq=2**31), fa.FA_EUNSUPPORTED),
    (dict(B=2**31), fa.FA_EUNSUPPORTED),
    (dict(Hq=2**31, Hkv=1), fa.FA_EUNSUPPORTED),
    (dict(B=2**30, Hq=2**30, Hkv=2**30, Tq=2**10), fa.FA_EUNSUPPORTED),  # B * Hq * Tq overflows
])
def test_validation_errors(kw, want):
    assert _call(**kw) == want


def test_bad_strides_and_tiling():
    st = fa.fa_strides()
    st.q[:] = [8 * 64 * 4, 8 * 64, 64]
    st.k[:] = st.v[:] = [8 * 64 * 2, 8 * 64, 64]
    st.o[:] = st.q[:]
    st.lse[:] = [4 * 8, 8]
    st.mask[:] = [0, 0, -1, 1]
    assert _call(strides=ctypes.byref(st)) == fa.FA_EINVAL   # negative mask stride
    st.mask[:] = [0, 0, 8, 1]
    st.q[2] = 66                                             # q rows not 16-byte aligned
    assert _call(strides=ctypes.byref(st)) == fa.FA_EUNSUPPORTED
    lib = fa.load_library()
    for til in ((48, 1), (32, 3), (64, 4), (0, 2), (-32, 1)):
        t = fa.fa_tiling(*til)
        assert lib.fa_fwd_tiled(P, P, P, P, None, 1, 4, 2, 8, 8, 64, 0.125, 0, 1, 0, None, None, None,
                                fa.FA_F32, None, ctypes.byref(t)) == fa.FA_EINVAL, til


def test_empty_work_returns_ok_without_launch():
    assert _call(Tq=0) == fa.FA_OK
    assert _call(B=0) == fa.FA_OK
    assert _call(Hq=0, Hkv=0, q=None, o=None) == fa.FA_OK
    assert _call(Tq=0, q=None, o=None, k=None, v=None) == fa.FA_OK


def _split_call(split_keys=256, ws=P, ws_bytes=1 << 30, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Tq=1, Tk=1000, d=64, scale=0.125, q_offset=999,
             causal=1, window=0, sinks=None, mask=None, strides=None, dtype=fa.FA_F32, stream=None)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Tq"],
                             a["Tk"], a["d"], a["scale"], a["q_offset"], a["causal"], a["window"], a["sinks"],
                             a["mask"], a["strides"], a["dtype"], a["stream"], None, split_keys, ws, ws_bytes)


def test_splitkv_workspace_bytes():
    # (d + 2) * 4 bytes per (split, row); splits = max(1, ceil(Tk / split_keys))
    assert fa.fa_splitkv_workspace_bytes(2, 4, 8, 1000, 64, 256) == 4 * (2 * 4 * 8) * 66 * 4
    assert fa.fa_splitkv_workspace_bytes(8, 32, 1, 8192, 128, 1024) == 8 * 256 * 130 * 4
    assert fa.fa_splitkv_workspace_bytes(1, 4, 3, 0, 128, 64) == 1 * 12 * 130 * 4
    assert fa.fa_splitkv_workspace_bytes(1, 4, 0, 100, 128, 64) == 0
    assert fa.fa_splitkv_workspace_bytes(1, 4, 3, 100, 128, 0) == 0
    assert fa.fa_splitkv_workspace_bytes(-1, 4, 3, 100, 128, 64) == 0
    assert fa.fa_splitkv_workspace_bytes(2**40, 2**40, 1, 100, 128, 64) == 0  # B * Hq overflows
    assert fa.fa_splitkv_workspace_bytes(2**30, 2**30, 2**10, 100, 128, 64) == 0  # ... times Tq
    assert fa.fa_splitkv_workspace_bytes(2**20, 2**20, 2**20, 100, 128, 64) == 0  # bytes overflow


def test_splitkv_default_keys():
    # decode at 8 x 32/8 heads x 8192 keys: 64 work items per split -> 8 splits of 1024 keys
    assert fa.fa_splitkv_default_keys(8, 32, 8, 1, 8192, 8191, True, 0, fa.FA_BF16) == 1024
    # 9 work items per split: the 64 visible tiles cut into the minimum split (4 tiles bf16, 2 fp32)
    assert fa.fa_splitkv_default_keys(1, 9, 3, 1, 4096, 4095, True, 0, fa.FA_BF16) == 256
    assert fa.fa_splitkv_default_keys(1, 9, 3, 1, 4096, 4095, True, 0, fa.FA_F32) == 128
    for args in ((1, 9, 3, 1, 4096, 4095, True, 0), (1, 16, 8, 511, 511, 0, True, 0),
                 (1, 32, 8, 1, 100000, 99999, True, 4096), (4, 4, 4, 7, 7, 0, False, 0), (1, 1, 1, 1, 0, 0, True, 0)):
        for dt in (fa.FA_F32, fa.FA_BF16):
            s = fa.fa_splitkv_default_keys(*args, dt)
            assert s >= 64 and s % 64 == 0, (args, s)


@pytest.mark.parametrize("kw,want", [
    (dict(split_keys=100), fa.FA_EINVAL),           # not a multiple of 64
    (dict(split_keys=-64), fa.FA_EINVAL),
    (dict(ws=None), fa.FA_EINVAL),                  # no workspace
    (dict(ws_bytes=1000), fa.FA_EINVAL),            # workspace too small (4 splits x 4 rows x 66 x 4)
    (dict(ws=P + 8), fa.FA_EUNSUPPORTED),           # workspace not 16-byte aligned
    (dict(Hq=6, Hkv=4), fa.FA_ESHAPE),
    (dict(d=96), fa.FA_EUNSUPPORTED),
])
def test_splitkv_validation_errors(kw, want):
    assert _split_call(**kw) == want


@pytest.mark.parametrize("split_keys", [2 ** 32, 2 ** 32 + 64, 2 ** 40])
def test_splitkv_huge_split_is_one_split(split_keys):
    """A split of 2^32 keys or more holds every key: the call needs the workspace of one split
    (one byte less is refused) and goes on to the next checks (here a misaligned q, so that
    nothing is launched)."""
    one = fa.fa_splitkv_workspace_bytes(1, 4, 1, 1000, 64, 1024)
    assert fa.fa_splitkv_workspace_bytes(1, 4, 1, 1000, 64, split_keys) == one
    assert _split_call(split_keys=split_keys, ws_bytes=one - 1) == fa.FA_EINVAL
    assert _split_call(split_keys=split_keys, ws_bytes=one, q=P + 8) == fa.FA_EUNSUPPORTED


def _noalloc_call(split_keys=256, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Tq=1, Tk=1000, d=64, scale=0.125, q_offset=999,
             causal=1, window=0, sinks=None, mask=None, strides=None, dtype=fa.FA_F32, stream=None)
    a.update(kw)
    return fa.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                     a["Tq"], a["Tk"], a["d"], a["scale"], a["q_offset"], a["causal"],
                                     a["window"], a["sinks"], a["mask"], a["strides"], a["dtype"], a["stream"],
                                     None, split_keys)


@pytest.mark.parametrize("kw,want", [
    (dict(B=4096, Hq=64, Hkv=8, Tk=1 << 16, split_keys=1024), fa.FA_ESCRATCH),  # 64 splits x 2^18 rows
    (dict(split_keys=100), fa.FA_EINVAL),
    (dict(split_keys=-64), fa.FA_EINVAL),
    (dict(Hq=6, Hkv=4), fa.FA_ESHAPE),
    (dict(d=96), fa.FA_EUNSUPPORTED),
    (dict(q=P + 8), fa.FA_EUNSUPPORTED),
    (dict(Tq=0), fa.FA_OK),
])
def test_noalloc_errors_before_any_device_call(kw, want):
    """The no-allocation entry point checks its arguments and the scratch size before it asks
    for the scratch array's device address (so these hold without a GPU)."""
    assert _noalloc_call(**kw) == want


def test_splitkv_empty_work_returns_ok_without_launch():
    assert _split_call(Tq=0) == fa.FA_OK
    assert _split_call(B=0, ws=None, ws_bytes=0) == fa.FA_OK


def test_fa_ext_layout_matches_the_header(tmp_path):
    """The binding's fa_ext has the C struct's size and field offsets (compiled with gcc)."""
    fields = [f[0] for f in fa.fa_ext._fields_]
    src = tmp_path / "ext.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "fa.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(fa_ext));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(fa_ext, {n}));\n' for n in fields) + "  return 0;\n}\n")
    exe = tmp_path / "ext"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(fa.fa_ext)] + [getattr(fa.fa_ext, n).offset for n in fields]
    assert got == want


def _ext_call(ext, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=2, Hq=4, Hkv=2, Tq=1, Tk=1000, d=64, scale=0.125, q_offset=0,
             causal=1, window=0, sinks=None, mask=None, strides=None, dtype=fa.FA_F32, stream=None)
    a.update(kw)
    return fa.fa_fwd_ext(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Tq"], a["Tk"],
                         a["d"], a["scale"], a["q_offset"], a["causal"], a["window"], a["sinks"], a["mask"],
                         a["strides"], a["dtype"], a["stream"], ctypes.byref(ext))


def _paged(**kw):
    a = dict(block_table=P, block_table_stride=16, block_size=64, num_blocks=100)
    a.update(kw)
    return fa.fa_ext(**a)


@pytest.mark.parametrize("ext,kw,want", [
    (dict(size=0), {}, fa.FA_EINVAL),                                        # size not set
    (dict(split_keys=-2), {}, fa.FA_EINVAL),
    (dict(split_keys=100, workspace=P, workspace_bytes=1 << 30), {}, fa.FA_EINVAL),
    (dict(split_keys=128, workspace=None), {}, fa.FA_EINVAL),
    (dict(paged=dict(block_size=100)), {}, fa.FA_EINVAL),                    # not a multiple of 64
    (dict(paged=dict(block_size=0)), {}, fa.FA_EINVAL),
    (dict(paged=dict(block_table_stride=15)), {}, fa.FA_EINVAL),             # 15 * 64 < Tk = 1000
    (dict(paged=dict(num_blocks=-1)), {}, fa.FA_EINVAL),
    (dict(paged=dict(block_table=P + 2)), {}, fa.FA_EUNSUPPORTED),           # misaligned block table
    (dict(paged=dict(), seqlens_k=P), dict(q_offset=5), fa.FA_EINVAL),       # positions come from seqlens_k
    (dict(seqlens_k=P + 1), {}, fa.FA_EUNSUPPORTED),
    (dict(rows_per_block=48, heads_per_block=1), {}, fa.FA_EINVAL),
    (dict(paged=dict()), dict(Hq=6, Hkv=4), fa.FA_ESHAPE),
    (dict(cu_seqlens_q=P), dict(q_offset=3), fa.FA_EINVAL),              # positions come from the lengths
    (dict(cu_seqlens_q=P), {}, fa.FA_EINVAL),                            # packed layouts need strides
    (dict(cu_seqlens_k=P, seqlens_k=P), dict(strides="bhsd"), fa.FA_EINVAL),  # two sources of key counts
    (dict(paged=dict(), cu_seqlens_k=P), dict(strides="bhsd"), fa.FA_EINVAL),
    (dict(cu_seqlens_q=P + 2), dict(strides="bhsd"), fa.FA_EUNSUPPORTED),
    (dict(softcap=-1.0), {}, fa.FA_EINVAL),
    (dict(softcap=float("nan")), {}, fa.FA_EINVAL),
    (dict(softcap=float("inf")), {}, fa.FA_EINVAL),
    (dict(alibi_slopes=P + 2), {}, fa.FA_EUNSUPPORTED),
])
def test_ext_validation_errors(ext, kw, want):
    ext = dict(ext)
    paged = ext.pop("paged", None)
    e = _paged(**paged) if paged is not None else fa.fa_ext()
    for n, val in ext.items():
        setattr(e, n, val)
    if kw.get("strides") == "bhsd":
        st = fa.fa_strides()
        st.q[:] = st.o[:] = [4 * 64, 64, 4 * 64]
        st.k[:] = st.v[:] = [2 * 1000 * 64, 1000 * 64, 64]
        st.lse[:] = [4, 1]
        kw = dict(kw, strides=ctypes.byref(st))
    assert _ext_call(e, **kw) == want


def test_ext_empty_work_returns_ok_without_launch():
    assert _ext_call(_paged(), Tq=0) == fa.FA_OK
    assert _ext_call(_paged(seqlens_k=P), B=0) == fa.FA_OK
