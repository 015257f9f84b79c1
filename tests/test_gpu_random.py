"""Seeded random sweep of the whole feature space against the fp64 oracle.

Each case draws a shape (GQA ratio, ragged Tq and Tk around tile edges, d 64 or 128), the
flags of "FlashAttention forward in C" section 2.1 (q_offset, causal, window, sinks), an
additive mask ("Fused attention and softmax: fast and exact"), the softcap / ALiBi variants,
and an execution path (plain with a random tiling, split-KV, paged K/V), from a fixed seed list,
so the sweep is the same on every run.  Plain-path cases are also recomputed with another tiling
and must match bit for bit (after the -0 normalisation of the other bitwise tests).
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
import synth
from gpu_common import bits, compare, dev, host, say, scale_for

pytestmark = pytest.mark.gpu

TILINGS = {1: [(32, 1), (64, 1), (128, 1), (256, 1)], 2: [(32, 2), (64, 2), (128, 2), (32, 1)],
           4: [(32, 4), (64, 4), (32, 2), (128, 1)], 8: [(32, 8), (32, 4), (64, 2), (32, 1)]}


def draw(seed):
    rng = np.random.default_rng(seed)
    group = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    Hq = group * Hkv
    B = int(rng.integers(1, 3))
    d = int(rng.choice([64, 128]))
    Tk = int(rng.choice([1, 33, 63, 64, 65, 127, 128, 129, 200, 333]))
    Tq = int(rng.choice([1, 2, 17, 31, 32, 33, 64, 100]))
    causal = bool(rng.random() < 0.7)
    q_offset = int(rng.choice([0, 0, max(0, Tk - Tq), int(rng.integers(0, Tk + 20))]))
    window = int(rng.choice([0, 0, 0, 1, 7, 64, 100]))
    sinks = bool(rng.random() < 0.3)
    mask = str(rng.choice(["none", "none", "bcast", "full"]))
    softcap = float(rng.choice([0.0, 0.0, 0.0, 4.0, 25.0]))
    alibi = bool(rng.random() < 0.2)
    dtype = str(rng.choice(["f32", "bf16"]))
    path = str(rng.choice(["plain", "plain", "split", "paged"]))
    tiling = TILINGS[group][int(rng.integers(0, 4))]
    split = int(rng.choice([64, 128, 192]))
    return dict(B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=causal, q_offset=q_offset, window=window,
                sinks=sinks, mask=mask, softcap=softcap, alibi=alibi, dtype=dtype, path=path, tiling=tiling,
                split=split)


SEEDS = list(range(1000, 1200))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(seed):
    c = draw(seed)
    say("random", seed, c)
    tag = f"random/{seed}"
    B, Hq, Hkv, Tq, Tk, d, dt = c["B"], c["Hq"], c["Hkv"], c["Tq"], c["Tk"], c["d"], c["dtype"]
    q = synth.normal(synth.seed_of(tag, "q"), (B, Hq, Tq, d), dt)
    k = synth.normal(synth.seed_of(tag, "k"), (B, Hkv, Tk, d), dt)
    v = synth.normal(synth.seed_of(tag, "v"), (B, Hkv, Tk, d), dt)
    z = synth.normal_f32(synth.seed_of(tag, "z"), (Hq,)) if c["sinks"] else None
    m = None
    if c["mask"] != "none":
        shape = (Tq, Tk) if c["mask"] == "bcast" else (B, Hq, Tq, Tk)
        m = synth.normal_f32(synth.seed_of(tag, "m"), shape)
        m[synth.neg_inf_mask(synth.seed_of(tag, "mi"), shape, 0.15) == -np.inf] = -np.inf
    al = np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], np.float32) if c["alibi"] else None
    sc = scale_for(d)
    kw = dict(scale=sc, q_offset=c["q_offset"], causal=c["causal"], window=c["window"], sinks=dev(z),
              mask=None if m is None else dev(m), softcap=c["softcap"], alibi_slopes=dev(al))
    tq, tk, tv = dev(q), dev(k), dev(v)
    if c["path"] == "plain":
        o, lse = fa.forward(tq, tk, tv, tiling=c["tiling"], **kw)
    elif c["path"] == "split":
        o, lse = fa.forward_splitkv(tq, tk, tv, split_keys=c["split"], tiling=c["tiling"], **kw)
    else:
        from test_gpu_paged import _page
        kp, vp, table = _page(tk, tv, 64 * (1 + seed % 3), seed=seed)
        o, lse = fa.forward_paged(tq, kp, vp, table, Tk=Tk, tiling=c["tiling"], **kw)
    torch.cuda.synchronize()
    m4 = None if m is None else (m[None, None] if m.ndim == 2 else m)
    o_ref, l_ref = oracle.attention(q, k, v, scale=sc, q_offset=c["q_offset"], causal=c["causal"],
                                    window=c["window"], sinks=z, mask=m4, softcap=c["softcap"], alibi=al)
    compare(host(o), host(lse), o_ref, l_ref, dt, f"random {seed}")
    if c["path"] == "plain":
        other = next(t for t in TILINGS[Hq // Hkv] if t != c["tiling"])
        o2, l2 = fa.forward(tq, tk, tv, tiling=other, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o), bits(o2)) and np.array_equal(bits(lse), bits(l2)), f"tiling {other}"
