"""GPU tests of the 8-wave geometries (two waves per SIMD, 64 to 256 rows of one to four heads
per workgroup, with 32 KiB of K/V tiles staged for eight waves) against the 4-wave kernel.

A row's result depends on its own data and position only ("FlashAttention forward in C",
section 2.4), so every case is held bit for bit to the 4-wave tiling and to the fp64 oracle
within the bf16 tolerance.  The cases cover workgroups with 1, 2, 3 and 4 tiles and longer,
rows whose visible tiles start late (q_offset, windows) or stop early (causal diagonal, ragged
Tk), sinks, d 64, split-KV, paged keys and packed sequences.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
from gpu_common import bits, compare, dev, host, make_inputs, say, scale_for

pytestmark = pytest.mark.gpu

# (name, B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks)
CASES = [
    ("one_tile", 1, 8, 2, 40, 50, 128, 0, True, 0, False),
    ("two_tiles", 1, 8, 2, 64, 128, 128, 0, True, 0, True),
    ("three_tiles_ragged", 2, 8, 2, 100, 150, 128, 50, True, 0, False),
    ("four_tiles", 1, 4, 1, 64, 256, 128, 192, True, 0, False),
    ("long_causal", 1, 8, 2, 700, 700, 128, 0, True, 0, True),
    ("window", 1, 8, 2, 300, 1000, 128, 700, True, 130, False),
    ("window_sinks_d64", 2, 8, 2, 257, 600, 64, 343, True, 65, True),
    ("noncausal_ragged", 1, 8, 4, 77, 333, 128, 0, False, 0, False),
    ("noncausal_d64", 1, 16, 2, 129, 1025, 64, 0, False, 0, True),
    ("late_offset", 1, 8, 8, 33, 900, 128, 867, True, 0, False),
]
TILINGS = {1: [(256, 1)], 2: [(128, 2)], 4: [(64, 4)], 8: [(32, 8)]}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_eight_waves_equal_four(case):
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks = case
    q, k, v, z = make_inputs(f"alt/{name}", B, Hq, Hkv, Tq, Tk, d, "bf16", sinks=with_sinks)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), q_offset=qo, causal=causal, window=window, sinks=tz)
    group = Hq // Hkv
    ref_tiling = (32, 4) if group % 4 == 0 else (32, 2) if group % 2 == 0 else (32, 1)
    say("8-wave", name, "reference tiling", ref_tiling)
    o4, l4 = fa.forward(tq, tk, tv, tiling=ref_tiling, **kw)
    torch.cuda.synchronize()
    for til in TILINGS[group] + ([(64, 4)] if group == 8 else []) + ([(128, 2)] if group in (4, 8) else []):
        say("8-wave", name, "tiling", til)
        o8, l8 = fa.forward(tq, tk, tv, tiling=til, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o8), bits(o4)), f"O differs from the 4-wave kernel at tiling {til}"
        assert np.array_equal(bits(l8), bits(l4)), f"LSE differs from the 4-wave kernel at tiling {til}"
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=qo, causal=causal, window=window, sinks=z)
    compare(host(o4), host(l4), o_ref, l_ref, "bf16", f"8-wave {name}")


@pytest.mark.parametrize("split", [64, 192])
def test_eight_waves_split_kv(split):
    """Split-KV work items with an 8-wave tiling: the same bits as with the 4-wave one."""
    B, Hq, Hkv, Tq, Tk, d = 1, 8, 2, 130, 1000, 128
    q, k, v, z = make_inputs(f"alt/split/{split}", B, Hq, Hkv, Tq, Tk, d, "bf16", sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), q_offset=Tk - Tq, causal=True, sinks=tz, split_keys=split)
    say("8-wave split", split)
    o4, l4 = fa.forward_splitkv(tq, tk, tv, tiling=(32, 4), **kw)
    o8, l8 = fa.forward_splitkv(tq, tk, tv, tiling=(64, 4), **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o8), bits(o4)) and np.array_equal(bits(l8), bits(l4))
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=Tk - Tq, causal=True, sinks=z)
    compare(host(o8), host(l8), o_ref, l_ref, "bf16", f"8-wave split {split}")


def test_eight_waves_paged():
    """Paged keys (block size 128, shuffled table) with an 8-wave tiling equal the contiguous
    call bit for bit."""
    from test_gpu_paged import _page
    B, Hq, Hkv, Tq, Tk, d = 2, 8, 2, 200, 700, 128
    q, k, v, _ = make_inputs("alt/paged", B, Hq, Hkv, Tq, Tk, d, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    kp, vp, table = _page(tk, tv, 128, seed=4)
    kw = dict(scale=scale_for(d), q_offset=Tk - Tq, causal=True, tiling=(64, 4))
    say("8-wave paged")
    o1, l1 = fa.forward(tq, tk, tv, **kw)
    o2, l2 = fa.forward_paged(tq, kp, vp, table, Tk=Tk, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))


def test_eight_waves_varlen():
    """Packed sequences (lengths 0, 1 and around the tile edges) with an 8-wave tiling: each
    sequence equals its own call bit for bit and the oracle within tolerance."""
    from test_gpu_varlen import _check
    lens = [1, 63, 64, 65, 300, 0, 129, 200]
    _check(lens, lens, 8, 2, 128, "bf16", True, 0, True, 0, "alt/varlen", tiling=(64, 4))


@pytest.mark.parametrize("tiling", [(32, 4), (64, 4)])
def test_one_visible_key_returns_its_value(tiling):
    """bf16: the denominator sums the weights as rounded for the PV product, so a row that sees
    exactly one key (causal row 0, no sink) returns that key's value exactly, and a row that
    sees two returns a convex combination of theirs (each output element between the two)."""
    B, Hq, Hkv, Tq, Tk, d = 2, 8, 2, 64, 64, 128
    q, k, v, _ = make_inputs("alt/one_key", B, Hq, Hkv, Tq, Tk, d, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    say("one visible key", tiling)
    o, _ = fa.forward(tq, tk, tv, scale=scale_for(d), causal=True, tiling=tiling)
    torch.cuda.synchronize()
    group = Hq // Hkv
    for h in range(Hq):
        kv = v[:, h // group].view(np.int16) if v.dtype == np.uint16 else None
        assert np.array_equal(o[:, h, 0].view(torch.int16).cpu().numpy(), kv[:, 0]), f"head {h}"
    vf = host(tv)
    o1 = host(o[:, :, 1])
    for h in range(Hq):
        lo = np.minimum(vf[:, h // group, 0], vf[:, h // group, 1])
        hi = np.maximum(vf[:, h // group, 0], vf[:, h // group, 1])
        assert np.all(o1[:, h] >= lo) and np.all(o1[:, h] <= hi), f"head {h}"


# persistent launches: the 8-wave bf16 d 128 kernel with at least two work items per CU walks
# them in one workgroup per CU; (name, B, Hq, Hkv, Tq, Tk, q_offset, causal, window, sinks)
PERSISTENT = [
    ("causal_ragged_rows", 2, 32, 8, 2047, 2048, 1, True, 0, True),
    ("window_offset", 4, 16, 4, 2000, 2560, 560, True, 200, False),
    ("noncausal", 1, 32, 8, 4096, 1024, 0, False, 0, True),
]


@pytest.mark.parametrize("case", PERSISTENT, ids=[c[0] for c in PERSISTENT])
def test_persistent_launch_equals_one_item_per_workgroup(case):
    """Work-item counts of at least 512 (two rounds on 256 CUs) take the persistent launch of the
    8-wave kernel: each row's bits equal the 4-wave kernel's (one workgroup per item), and a
    sample of rows matches the oracle."""
    name, B, Hq, Hkv, Tq, Tk, qo, causal, window, with_sinks = case
    d = 128
    assert B * Hkv * ((Tq + 63) // 64) >= 512 and Tk % 64 == 0
    q, k, v, z = make_inputs(f"persistent/{name}", B, Hq, Hkv, Tq, Tk, d, "bf16", sinks=with_sinks)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), q_offset=qo, causal=causal, window=window, sinks=tz if with_sinks else None)
    say("persistent", name)
    o8, l8 = fa.forward(tq, tk, tv, **kw)  # automatic geometry: 8 waves, persistent
    o4, l4 = fa.forward(tq, tk, tv, tiling=(32, 4), **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o8), bits(o4)), "O differs from the one-item-per-workgroup launch"
    assert np.array_equal(bits(l8), bits(l4)), "LSE differs from the one-item-per-workgroup launch"
    rng = np.random.default_rng(11)
    rows = np.stack([rng.integers(0, B, 64), rng.integers(0, Hq, 64), rng.integers(0, Tq, 64)], axis=1)
    rows[:3] = [[0, 0, 0], [B - 1, Hq - 1, Tq - 1], [B - 1, 0, Tq // 2]]
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=qo, causal=causal, window=window,
                                    sinks=z if with_sinks else None, rows=rows)
    og, lg = host(o8), host(l8)
    compare(og[rows[:, 0], rows[:, 1], rows[:, 2]], lg[rows[:, 0], rows[:, 1], rows[:, 2]], o_ref, l_ref, "bf16",
            f"persistent {name}")
