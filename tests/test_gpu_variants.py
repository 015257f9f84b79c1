"""GPU tests of the score variants softcap and ALiBi (the candle page's flash attention offers
both; definitions: logit c tanh(logit / c), bias -slope_h |p_i - j| at absolute positions).

Parity with the fp64 oracle over a flag matrix (GQA, causal and not, window, sinks, masks,
decode, both head sizes and dtypes), and the bit-level properties the plain path has: query
chunking and tiling do not change a row's bits, paged keys equal contiguous ones, and split-KV
matches the oracle.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
import synth
from gpu_common import bits, compare, dev, host, make_inputs, say, scale_for

pytestmark = pytest.mark.gpu


def alibi_slopes(H):
    """The geometric slopes 2^(-8 (h + 1) / H) of the ALiBi paper (H a power of two)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32)


# (name, B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks, mask, softcap, alibi)
CASES = [
    ("softcap_causal", 2, 8, 2, 100, 100, 128, 0, True, 0, False, False, 5.0, False),
    ("softcap30_mask", 1, 4, 2, 70, 140, 64, 0, False, 0, False, True, 30.0, False),
    ("alibi_causal_offset", 1, 8, 2, 90, 300, 128, 210, True, 0, False, False, 0.0, True),
    ("alibi_noncausal_window", 2, 4, 4, 65, 130, 64, 40, False, 25, False, False, 0.0, True),
    ("both_sinks_window", 1, 8, 2, 130, 130, 64, 0, True, 50, True, False, 8.0, True),
    ("both_mask_d128", 1, 4, 1, 64, 200, 128, 136, True, 0, True, True, 12.0, True),
    ("decode_both", 3, 16, 8, 1, 700, 128, 699, True, 0, False, False, 20.0, True),
    ("softcap_tiny_logits", 1, 4, 2, 33, 33, 64, 0, True, 0, False, False, 50.0, False),
]


def _setup(case, dtype):
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks, with_mask, cap, with_alibi = case
    tag = f"variants/{name}/{dtype}"
    q, k, v, z = make_inputs(tag, B, Hq, Hkv, Tq, Tk, d, dtype, sinks=with_sinks)
    m = None
    if with_mask:
        m = synth.normal_f32(synth.seed_of(tag, "mask"), (Tq, Tk))
        m[synth.neg_inf_mask(synth.seed_of(tag, "mask-inf"), (Tq, Tk), 0.1) == -np.inf] = -np.inf
        m[3] = -np.inf
    al = alibi_slopes(Hq) if with_alibi else None
    kw = dict(scale=scale_for(d), q_offset=qo, causal=causal, window=window)
    return q, k, v, z, m, al, cap, kw


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_variant_parity(case, dtype):
    q, k, v, z, m, al, cap, kw = _setup(case, dtype)
    say("variants", case[0], dtype, dict(softcap=cap, alibi=al is not None), kw)
    o, lse = fa.forward(dev(q), dev(k), dev(v), sinks=dev(z), mask=None if m is None else dev(m), softcap=cap,
                        alibi_slopes=dev(al), **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, sinks=z, mask=None if m is None else m[None, None], softcap=cap,
                                    alibi=al, **kw)
    compare(host(o), host(lse), o_ref, l_ref, dtype, f"variants {case[0]}")
    # split-KV through the same variants
    o2, l2 = fa.forward_splitkv(dev(q), dev(k), dev(v), split_keys=64, sinks=dev(z),
                                mask=None if m is None else dev(m), softcap=cap, alibi_slopes=dev(al), **kw)
    torch.cuda.synchronize()
    compare(host(o2), host(l2), o_ref, l_ref, dtype, f"variants {case[0]} split-KV")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_variant_chunk_tiling_paged_bitwise(dtype):
    """softcap + ALiBi + window + sinks: chunks at q_offset and every tiling give the bits of
    one whole call; paged keys give the bits of contiguous keys."""
    from test_gpu_paged import _page
    Hq, Hkv, T, d = 8, 2, 500, 128
    q, k, v, z = make_inputs(f"variants/inv/{dtype}", 1, Hq, Hkv, T, T, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), causal=True, window=200, sinks=tz, softcap=10.0, alibi_slopes=dev(alibi_slopes(Hq)))
    say("variants whole", dtype)
    o_full, l_full = fa.forward(tq, tk, tv, **kw)
    start = 0
    for n, tiling in ((37, None), (100, (32, 1)), (163, (64, 2)), (200, (32, 4))):
        say("variants chunk", start, n, tiling)
        o, lse = fa.forward(tq[:, :, start:start + n], tk, tv, q_offset=start, tiling=tiling, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o), bits(o_full[:, :, start:start + n])), f"O chunk at {start}"
        assert np.array_equal(bits(lse), bits(l_full[:, :, start:start + n])), f"LSE chunk at {start}"
        start += n
    kp, vp, table = _page(tk, tv, 128, seed=4)
    o2, l2 = fa.forward_paged(tq, kp, vp, table, Tk=T, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_full), bits(o2)) and np.array_equal(bits(l_full), bits(l2))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mask_free_variant_kernels_match_the_general_one(dtype, d):
    """Without a mask, bf16 softcap calls run a softcap kernel and ALiBi-only calls an ALiBi
    kernel with no mask code; an all-zero mask sends the same call to the general variant
    kernel.  Adding 0 changes no score, so every tiling (4 and 8 waves, and 1 wave, which always
    takes the general kernel) must give the bits of the masked call, which in turn matches the
    oracle."""
    Hq, Hkv, T = 8, 2, 300
    q, k, v, z = make_inputs(f"variants/maskfree/{dtype}/{d}", 1, Hq, Hkv, T, T, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    zero = torch.zeros((T, T), dtype=torch.float32, device="cuda")
    al = alibi_slopes(Hq)
    for cap, with_alibi in ((10.0, False), (0.0, True), (10.0, True)):
        kw = dict(scale=scale_for(d), causal=True, window=220, sinks=tz, softcap=cap,
                  alibi_slopes=dev(al) if with_alibi else None)
        say("mask-free variants", dtype, d, dict(softcap=cap, alibi=with_alibi))
        o_m, l_m = fa.forward(tq, tk, tv, mask=zero, **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], causal=True, window=220, sinks=z, softcap=cap,
                                        alibi=al if with_alibi else None)
        compare(host(o_m), host(l_m), o_ref, l_ref, dtype, f"zero mask softcap {cap} alibi {with_alibi}")
        for tiling in (None, (32, 4), (64, 4), (32, 1)):
            o, lse = fa.forward(tq, tk, tv, tiling=tiling, **kw)
            torch.cuda.synchronize()
            assert np.array_equal(bits(o), bits(o_m)), f"O softcap {cap} alibi {with_alibi} tiling {tiling}"
            assert np.array_equal(bits(lse), bits(l_m)), f"LSE softcap {cap} alibi {with_alibi} tiling {tiling}"
