"""GPU bitwise invariance: a row's bits depend only on its own data and absolute position.

"FlashAttention forward in C" section 2.4 and its tests chunk_invariant_with_q_offset and
query_tile_and_batch_invariant: one call vs chunks with q_offset, every query-tile geometry,
a sequence alone vs in a batch, and (here) the BHSD vs BSHD layouts.  Outputs are compared
bit for bit (raw bits: the library writes every zero output as +0).
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
from gpu_common import bits, dev, make_inputs, say

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16"]
TILINGS_G4 = [(32, 1), (64, 1), (128, 1), (32, 2), (64, 2), (32, 4), (64, 4), (128, 2), (256, 1)]


def _same(a, b, what):
    ba, bb = bits(a), bits(b)
    n = int(np.count_nonzero(ba != bb))
    assert n == 0, f"{what}: {n} elements differ"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", DTYPES)
def test_query_tile_invariant(dtype, d):
    B, Hq, Hkv, Tq, Tk = 2, 8, 2, 203, 203
    q, k, v, z = make_inputs(f"inv-tile/{dtype}/{d}", B, Hq, Hkv, Tq, Tk, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    for flags in (dict(causal=True), dict(causal=True, window=70, sinks=tz), dict(causal=False, q_offset=9)):
        ref = None
        for tiling in TILINGS_G4:
            say("tile-invariance", dtype, d, tiling, sorted(flags))
            o, lse = fa.forward(tq, tk, tv, tiling=tiling, **flags)
            torch.cuda.synchronize()
            if ref is None:
                ref = (o, lse)
            else:
                _same(o, ref[0], f"O {tiling}")
                _same(lse, ref[1], f"LSE {tiling}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_chunk_invariant_with_q_offset(dtype):
    """37 rows in one call vs chunks of 1, 3, 5, 16 (and the rest) at the matching q_offset."""
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 37, 37, 128
    q, k, v, z = make_inputs(f"inv-chunk/{dtype}", B, Hq, Hkv, Tq, Tk, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    for flags in (dict(causal=True), dict(causal=True, window=6, sinks=tz)):
        say("chunk-invariance", dtype, sorted(flags))
        full_o, full_l = fa.forward(tq, tk, tv, **flags)
        for sizes in ([1] * 37, [3] * 12 + [1], [5] * 7 + [2], [16, 16, 5]):
            start = 0
            for n in sizes:
                o, lse = fa.forward(tq[:, :, start:start + n], tk, tv, q_offset=start, **flags)
                torch.cuda.synchronize()
                _same(o, full_o[:, :, start:start + n], f"O chunk {start}+{n}")
                _same(lse, full_l[:, :, start:start + n], f"LSE chunk {start}+{n}")
                start += n


@pytest.mark.parametrize("dtype", DTYPES)
def test_batch_invariant(dtype):
    """A sequence alone equals the same sequence inside a batch of 3."""
    B, Hq, Hkv, Tq, Tk, d = 3, 4, 4, 90, 150, 64
    q, k, v, _ = make_inputs(f"inv-batch/{dtype}", B, Hq, Hkv, Tq, Tk, d, dtype)
    tq, tk, tv = dev(q), dev(k), dev(v)
    say("batch-invariance", dtype)
    o, lse = fa.forward(tq, tk, tv, causal=True, q_offset=60)
    for b in range(B):
        o1, l1 = fa.forward(tq[b:b + 1], tk[b:b + 1], tv[b:b + 1], causal=True, q_offset=60)
        torch.cuda.synchronize()
        _same(o1, o[b:b + 1], f"O batch {b}")
        _same(l1, lse[b:b + 1], f"LSE batch {b}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_layout_invariant(dtype):
    """BHSD tensors and BSHD tensors ([B, T, H, d], the concatenated-heads layout of "IV.5:
    Flash attention") give the same bits."""
    B, Hq, Hkv, T, d = 2, 16, 8, 150, 128
    q, k, v, _ = make_inputs(f"inv-layout/{dtype}", B, Hq, Hkv, T, T, d, dtype)
    tq, tk, tv = dev(q), dev(k), dev(v)
    sq, sk, sv = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (tq, tk, tv))
    assert sq.stride(2) == Hq * d
    say("layout-invariance", dtype)
    o1, l1 = fa.forward(tq, tk, tv, causal=True)
    out = torch.empty((B, T, Hq, d), dtype=tq.dtype, device="cuda").transpose(1, 2)
    o2, l2 = fa.forward(sq, sk, sv, causal=True, out=out)
    torch.cuda.synchronize()
    _same(o2, o1, "O BSHD")
    _same(l2, l1, "LSE BSHD")


@pytest.mark.parametrize("d", [64, 128])
def test_output_d_parts_equal_one_wave(d):
    """Small fp32 calls whose automatic geometry is one-wave workgroups run on the split-role
    kernel (two waves computing the scores of the two 32-key blocks a tile ahead, two taking the
    softmax step and the PV product for half of d each, one copying the tiles): the same bits as
    the one-wave tiling, and the oracle's values.  Cases: causal, offset rows, decode-like,
    non-causal ragged, window with sinks, a call whose rows see no key, a single partial tile."""
    import oracle
    from gpu_common import compare, host, scale_for
    B, Hq, Hkv = 1, 4, 2
    for Tq, Tk, flags in ((100, 100, dict(causal=True)), (65, 300, dict(causal=True, q_offset=235)),
                          (1, 1000, dict(causal=True, q_offset=999)), (70, 129, dict(causal=False)),
                          (50, 500, dict(causal=True, window=64, q_offset=400, sinks=True)),
                          (40, 64, dict(causal=True, window=50, q_offset=200)), (33, 7, dict(causal=False))):
        q, k, v, z = make_inputs(f"inv-dparts/{d}/{Tq}/{Tk}", B, Hq, Hkv, Tq, Tk, d, "f32", sinks=True)
        tq, tk, tv = dev(q), dev(k), dev(v)
        kw = dict(flags)
        kw["sinks"] = dev(z) if flags.get("sinks") else None
        say("d-parts", d, Tq, Tk, sorted(flags))
        o, lse = fa.forward(tq, tk, tv, scale=scale_for(d), **kw)
        o1, l1 = fa.forward(tq, tk, tv, scale=scale_for(d), tiling=(32, 1), **kw)
        torch.cuda.synchronize()
        _same(o, o1, f"O d-parts {Tq}x{Tk}")
        _same(lse, l1, f"LSE d-parts {Tq}x{Tk}")
        o_ref, l_ref = oracle.attention(q, k, v, scale=scale_for(d), q_offset=flags.get("q_offset", 0),
                                        causal=flags["causal"], window=flags.get("window", 0),
                                        sinks=z if flags.get("sinks") else None)
        compare(host(o), host(lse), o_ref, l_ref, "f32", f"d-parts {d} {Tq}x{Tk}")


def test_long_causal_fp32_geometry_choice_keeps_bits():
    """A 2,044-token causal fp32 call at 16/8 heads, d 128 (one layer of the 2,044-token
    prefill): on a 256-CU device the automatic geometry takes the split-role kernel (32-row
    one-head blocks, whose longest chain of tiles outweighs the total work of the 4-wave
    geometry).  Its bits equal those of the 4-wave tiling (64 rows x 2 heads), of the one-wave
    tiling, and of four chunked calls at the matching q_offset."""
    B, Hq, Hkv, T, d = 1, 16, 8, 2044, 128
    q, k, v, _ = make_inputs("inv-geom-2044/f32", B, Hq, Hkv, T, T, d, "f32")
    tq, tk, tv = dev(q), dev(k), dev(v)
    say("geometry choice 2044 f32")
    o, lse = fa.forward(tq, tk, tv, causal=True)
    for tiling in ((64, 2), (32, 1)):
        o1, l1 = fa.forward(tq, tk, tv, causal=True, tiling=tiling)
        torch.cuda.synchronize()
        _same(o1, o, f"O tiling {tiling}")
        _same(l1, lse, f"LSE tiling {tiling}")
    start = 0
    for n in (511, 511, 511, 511):
        oc, lc = fa.forward(tq[:, :, start:start + n], tk, tv, q_offset=start, causal=True)
        torch.cuda.synchronize()
        _same(oc, o[:, :, start:start + n], f"O chunk {start}+{n}")
        _same(lc, lse[:, :, start:start + n], f"LSE chunk {start}+{n}")
        start += n
