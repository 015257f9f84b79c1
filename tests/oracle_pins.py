"""Pins of the fp64 oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``attn`` callable with the signature of ``oracle.attention`` and
raises AssertionError when the oracle disagrees with the pin.  ``test_oracle_pins.py`` runs
them on the oracle, and on builds of the oracle with one planted mistake each, to show every
mistake is caught by at least one pin.
"""
import math
import os

import numpy as np

import synth
from brute_decimal import brute_attention

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = (s.strip() for s in line.split("=", 1))
            vals[key] = [float(t) for t in rhs.split()]
    return vals


def _bhsd(rows):
    return np.asarray(rows, np.float64)[None, None]


def pin_hand_example(attn):
    """"FlashAttention forward in C", section 3: o = [3, 4], lse = 1.8619948; causal at q_offset 1."""
    g = golden("hand_example.txt")
    q = _bhsd([g["q"]])
    k = _bhsd([g["k0"], g["k1"], g["k2"]])
    v = _bhsd([g["v0"], g["v1"], g["v2"]])
    o, lse = attn(q, k, v, scale=g["scale"][0], causal=False)
    assert np.max(np.abs(o[0, 0, 0] - g["o"])) <= 1e-12, o
    assert abs(lse[0, 0, 0] - g["lse"][0]) <= 1e-7, lse  # 7 printed decimals
    o, lse = attn(q, k, v, scale=1.0, causal=True, q_offset=int(g["causal_q_offset"][0]))
    assert np.max(np.abs(o[0, 0, 0] - g["causal_o"])) <= 1e-7, o


def pin_sinks(attn):
    """Sinks join the denominator: all-ones values give 2/3 and lse = ln 3."""
    g = golden("sinks_example.txt")
    d, tk = int(g["d"][0]), int(g["tk"][0])
    q = np.zeros((1, 1, 1, d))
    k = synth.normal_f32(1, (1, 1, tk, d)).astype(np.float64)
    v = np.ones((1, 1, tk, d))
    o, lse = attn(q, k, v, scale=0.5, causal=False, sinks=np.array(g["sink"], np.float32))
    assert np.max(np.abs(o[0, 0, 0] - g["o"])) <= 1e-15, o
    assert abs(lse[0, 0, 0] - g["lse"][0]) <= 1e-15, lse


def pin_no_visible_key(attn):
    """A row that sees nothing: zeros and -inf; with a sink, zeros and lse = the sink."""
    q = synth.normal_f32(2, (1, 2, 3, 4)).astype(np.float64)
    k = synth.normal_f32(3, (1, 1, 4, 4)).astype(np.float64)
    v = synth.normal_f32(4, (1, 1, 4, 4)).astype(np.float64)
    # positions 10..12 with window 3 see keys 8..12, none of which exist (Tk = 4)
    o, lse = attn(q, k, v, scale=0.5, q_offset=10, causal=True, window=3)
    assert np.all(o == 0) and not np.any(np.signbit(o)), o
    assert np.all(lse == -np.inf), lse
    z = np.array([0.7, -1.25], np.float32)
    o, lse = attn(q, k, v, scale=0.5, q_offset=10, causal=True, window=3, sinks=z)
    assert np.all(o == 0), o
    assert np.all(lse == z.astype(np.float64)[None, :, None]), lse
    # empty key range
    o, lse = attn(q, k[:, :, :0], v[:, :, :0], scale=0.5, causal=False)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # fully masked row through the additive mask
    mask = np.zeros((1, 1, 3, 4), np.float32)
    mask[..., 1, :] = -np.inf
    o, lse = attn(q, k, v, scale=0.5, causal=False, mask=mask)
    assert np.all(o[:, :, 1] == 0) and np.all(lse[:, :, 1] == -np.inf)
    assert np.all(np.isfinite(lse[:, :, [0, 2]]))


def _interval(p, tk, causal, window):
    hi = min(tk, p + 1) if causal else tk
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, max(lo, hi)


def pin_closed_form_q_zero(attn, geometries=None):
    """q = 0: all visible scores equal, so o = mean of the visible values, lse = ln |V_i|.

    Run at real workload geometries (sampled rows) to pin causal, window, q_offset, GQA and
    sinks without any other implementation."""
    if geometries is None:
        geometries = [
            # (B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks)
            (1, 1, 1, 128, 128, 64, 0, True, 0, False),
            (1, 16, 8, 511, 511, 128, 0, True, 0, False),
            (1, 32, 8, 4096, 4096, 64, 0, True, 512, True),
            (1, 32, 8, 1096, 4096, 64, 3000, True, 512, True),
            (1, 4, 2, 40, 100, 8, 7, False, 9, False),
            (2, 6, 2, 37, 37, 8, 0, True, 6, True),
        ]
    for gi, (B, Hq, Hkv, Tq, Tk, d, qo, causal, w, has_sink) in enumerate(geometries):
        q = np.zeros((B, Hq, Tq, d), np.float32)
        k = synth.normal_f32(synth.seed_of("pin-q0", gi, "k"), (B, Hkv, Tk, d))
        v = synth.normal_f32(synth.seed_of("pin-q0", gi, "v"), (B, Hkv, Tk, d))
        z = synth.normal_f32(synth.seed_of("pin-q0", gi, "z"), (Hq,)) if has_sink else None
        rng = np.random.default_rng(gi)
        n_rows = min(B * Hq * Tq, 600)
        rows = np.stack([rng.integers(0, B, n_rows), rng.integers(0, Hq, n_rows),
                         rng.integers(0, Tq, n_rows)], 1)
        rows[:4] = [[0, 0, 0], [B - 1, Hq - 1, Tq - 1], [0, Hq - 1, min(63, Tq - 1)],
                    [B - 1, 0, min(64, Tq - 1)]]
        o, lse = attn(q, k, v, scale=0.125, q_offset=qo, causal=causal, window=w, sinks=z, rows=rows)
        for r, (b, h, i) in enumerate(rows):
            lo, hi = _interval(qo + i, Tk, causal, w)
            n = hi - lo
            kvh = h // (Hq // Hkv)
            tot = v[b, kvh, lo:hi].astype(np.float64).sum(0)
            den = n + (math.exp(float(z[h])) if has_sink else 0.0)
            if den == 0:
                assert np.all(o[r] == 0) and lse[r] == -np.inf
                continue
            assert np.max(np.abs(o[r] - tot / den)) <= 1e-12, (gi, b, h, i)
            assert abs(lse[r] - math.log(den)) <= 1e-12, (gi, b, h, i, lse[r], den)


def pin_closed_form_q_zero_mask(attn):
    """q = 0 with a 0/-inf additive mask: o = mean of the values whose entry is 0."""
    B, Hq, Hkv, Tq, Tk, d = 1, 2, 1, 70, 70, 8
    q = np.zeros((B, Hq, Tq, d), np.float32)
    v = synth.normal_f32(synth.seed_of("pin-q0m", "v"), (B, Hkv, Tk, d))
    k = synth.normal_f32(synth.seed_of("pin-q0m", "k"), (B, Hkv, Tk, d))
    mask = synth.neg_inf_mask(synth.seed_of("pin-q0m", "m"), (Tq, Tk), 0.3)
    mask[5] = -np.inf
    o, lse = attn(q, k, v, scale=0.3, causal=False, mask=mask[None, None])
    for i in range(Tq):
        keep = mask[i] == 0
        n = int(keep.sum())
        if n == 0:
            assert np.all(o[0, :, i] == 0) and np.all(lse[0, :, i] == -np.inf)
            continue
        ref = v[0, 0, keep].astype(np.float64).mean(0)
        assert np.max(np.abs(o[0, :, i] - ref)) <= 1e-12
        assert np.max(np.abs(lse[0, :, i] - math.log(n))) <= 1e-12


def pin_closed_form_q_zero_mask_offset(attn):
    """q = 0 with a 0/-inf additive mask on a chunk at q_offset > 0, causal, with and without a
    window: o = mean of the values of keys that are both visible at the row's absolute position
    p_i = q_offset + i and kept by mask row i of the call (the mask is indexed like q, by the
    call's row; "Fused attention and softmax: fast and exact", "What is computed" gives the mask
    as [qLen, kLen] of the call).  The mask array has rows past Tq, so that a reading by absolute
    position stays inside it and gives a different answer."""
    B, Hq, Hkv, Tq, Tk, d, qo = 1, 2, 1, 40, 70, 8, 17
    q = np.zeros((B, Hq, Tq, d), np.float32)
    v = synth.normal_f32(synth.seed_of("pin-q0mo", "v"), (B, Hkv, Tk, d))
    k = synth.normal_f32(synth.seed_of("pin-q0mo", "k"), (B, Hkv, Tk, d))
    big = synth.neg_inf_mask(synth.seed_of("pin-q0mo", "m"), (Tq + qo, Tk), 0.3)
    big[7] = -np.inf  # a row that sees nothing
    for window in (0, 9):
        o, lse = attn(q, k, v, scale=0.3, q_offset=qo, causal=True, window=window, mask=big[:Tq][None, None])
        for i in range(Tq):
            lo, hi = _interval(qo + i, Tk, True, window)
            keep = np.zeros(Tk, bool)
            keep[lo:hi] = big[i, lo:hi] == 0
            n = int(keep.sum())
            if n == 0:
                assert np.all(o[0, :, i] == 0) and np.all(lse[0, :, i] == -np.inf), (window, i)
                continue
            ref = v[0, 0, keep].astype(np.float64).mean(0)
            assert np.max(np.abs(o[0, :, i] - ref)) <= 1e-12, (window, i)
            assert np.max(np.abs(lse[0, :, i] - math.log(n))) <= 1e-12, (window, i)


def pin_const_v(attn):
    """Every value row equal to c: o = c (1 - p_sink) for any scores, p_sink = e^{z - lse}."""
    B, Hq, Hkv, Tq, Tk, d = 2, 4, 2, 50, 90, 16
    q = synth.normal_f32(synth.seed_of("pin-cv", "q"), (B, Hq, Tq, d))
    k = synth.normal_f32(synth.seed_of("pin-cv", "k"), (B, Hkv, Tk, d))
    c = synth.normal_f32(synth.seed_of("pin-cv", "c"), (d,))
    v = np.broadcast_to(c, (B, Hkv, Tk, d)).copy()
    z = synth.normal_f32(synth.seed_of("pin-cv", "z"), (Hq,))
    for sinks in (None, z):
        o, lse = attn(q, k, v, scale=0.25, q_offset=40, causal=True, window=60, sinks=sinks)
        keep = np.ones_like(lse) if sinks is None else 1.0 - np.exp(z.astype(np.float64)[None, :, None] - lse)
        assert np.max(np.abs(o - keep[..., None] * c.astype(np.float64))) <= 1e-12


def pin_single_visible_key(attn):
    """Causal row 0 at q_offset 0 sees only key 0: o = v_0 and lse = s_00."""
    q = synth.normal_f32(synth.seed_of("pin-1k", "q"), (1, 2, 5, 8)).astype(np.float64)
    k = synth.normal_f32(synth.seed_of("pin-1k", "k"), (1, 1, 5, 8)).astype(np.float64)
    v = synth.normal_f32(synth.seed_of("pin-1k", "v"), (1, 1, 5, 8)).astype(np.float64)
    o, lse = attn(q, k, v, scale=0.5, causal=True)
    for h in range(2):
        assert np.all(o[0, h, 0] == v[0, 0, 0])
        s00 = 0.5 * sum(q[0, h, 0, x] * k[0, 0, 0, x] for x in range(8))
        assert abs(lse[0, h, 0] - s00) <= 1e-14


def pin_mask_shift(attn):
    """Adding c to every mask entry of a row leaves o unchanged and adds c to lse."""
    B, Hq, Hkv, Tq, Tk, d = 1, 2, 2, 20, 30, 8
    q = synth.normal_f32(synth.seed_of("pin-ms", "q"), (B, Hq, Tq, d))
    k = synth.normal_f32(synth.seed_of("pin-ms", "k"), (B, Hkv, Tk, d))
    v = synth.normal_f32(synth.seed_of("pin-ms", "v"), (B, Hkv, Tk, d))
    # entries on a 2^-10 grid so that m + 3.25 is exact in fp32
    m = np.round(synth.normal_f32(synth.seed_of("pin-ms", "m"), (B, Hq, Tq, Tk)) * 1024) / 1024
    m[synth.neg_inf_mask(synth.seed_of("pin-ms", "inf"), m.shape, 0.2) == -np.inf] = -np.inf
    shift = np.float32(3.25)
    o0, l0 = attn(q, k, v, scale=0.35, causal=False, mask=m)
    o1, l1 = attn(q, k, v, scale=0.35, causal=False, mask=m + shift)
    fin = np.isfinite(l0)
    assert np.max(np.abs(o0 - o1)) <= 1e-12
    assert np.max(np.abs((l1 - l0)[fin] - float(shift))) <= 1e-12
    assert np.all(l1[~fin] == -np.inf)


def _brute_cases():
    cases = []
    for causal in (False, True):
        for window in (0, 1, 3):
            for q_offset in (0, 2, 5):
                for with_sink in (False, True):
                    for with_mask in (False, True):
                        cases.append((causal, window, q_offset, with_sink, with_mask, 0.0, False))
    # the score variants: softcap, ALiBi, both, with and without the other flags
    for ci, (softcap, alibi) in enumerate(((0.9, False), (0.0, True), (1.7, True))):
        for causal in (False, True):
            for q_offset, window, with_sink, with_mask in ((0, 0, False, False), (5, 3, True, True)):
                cases.append((causal, window, q_offset, with_sink, with_mask, softcap, alibi))
    return cases


def pin_brute_force(attn, cases=None):
    """50-digit decimal evaluation of the definition, every flag combination, tiny shapes."""
    geoms = [(1, 2, 1, 5, 9, 3), (2, 4, 2, 4, 7, 2), (1, 3, 3, 6, 6, 4)]
    for ci, (causal, window, q_offset, with_sink, with_mask, softcap, with_alibi) in enumerate(cases or _brute_cases()):
        B, Hq, Hkv, Tq, Tk, d = geoms[ci % len(geoms)]
        q = synth.normal_f32(synth.seed_of("pin-bf", ci, "q"), (B, Hq, Tq, d))
        k = synth.normal_f32(synth.seed_of("pin-bf", ci, "k"), (B, Hkv, Tk, d))
        v = synth.normal_f32(synth.seed_of("pin-bf", ci, "v"), (B, Hkv, Tk, d))
        z = synth.normal_f32(synth.seed_of("pin-bf", ci, "z"), (Hq,)) if with_sink else None
        mask = None
        if with_mask:
            # the view is a slice of a taller array so that a mistaken row index stays in bounds
            full = synth.normal_f32(synth.seed_of("pin-bf", ci, "m"), (B, Hq, Tq + 8, Tk))
            full[synth.neg_inf_mask(synth.seed_of("pin-bf", ci, "mi"), full.shape, 0.25) == -np.inf] = -np.inf
            mask = full[:, :, :Tq]
        scale = np.float32(0.7)
        al = np.abs(synth.normal_f32(synth.seed_of("pin-bf", ci, "al"), (Hq,))) if with_alibi else None
        extra = {}
        if softcap:
            extra["softcap"] = softcap
        if with_alibi:
            extra["alibi"] = al
        o, lse = attn(q, k, v, scale=scale, q_offset=q_offset, causal=causal, window=window, sinks=z, mask=mask,
                      **extra)
        ob, lb = brute_attention(q, k, v, scale=scale, q_offset=q_offset, causal=causal, window=window,
                                 sinks=z, mask=mask, softcap=softcap, alibi=al)
        assert np.all((lb == -np.inf) == (lse == -np.inf)), ci
        fin = np.isfinite(lb)
        assert np.max(np.abs(lse[fin] - lb[fin]) / np.maximum(1, np.abs(lb[fin])), initial=0) <= 1e-13, ci
        assert np.max(np.abs(o - ob) / np.maximum(1, np.abs(ob)), initial=0) <= 1e-13, ci


def _geo(r, n):
    """sum_{k<n} r^k and sum_{k<n} k r^k in closed form (0 < r < 1)."""
    s0 = (1 - r ** n) / (1 - r)
    s1 = r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / (1 - r) ** 2
    return s0, s1


def pin_alibi_closed_form(attn):
    """q = 0 and ALiBi slope m: every dot product is 0, so the weight of key j is r^|p - j| with
    r = e^{-m}; with v_j = (j, 1, ...) the output is a ratio of geometric sums and the lse their
    log.  Checked at absolute positions (q_offset), with a window, and without causal (keys on
    both sides of p)."""
    Hq, Hkv, d = 3, 1, 2
    slopes = np.array([0.05, 0.5, 1.25], np.float32)
    for Tq, Tk, q_offset, causal, window in ((4, 300, 200, True, 0), (3, 300, 250, True, 40),
                                             (5, 120, 30, False, 0), (2, 64, 0, True, 0)):
        q = np.zeros((1, Hq, Tq, d), np.float32)
        k = synth.normal_f32(synth.seed_of("pin-alibi", Tk, "k"), (1, Hkv, Tk, d))
        v = np.zeros((1, Hkv, Tk, d), np.float32)
        v[0, 0, :, 0] = np.arange(Tk)
        v[0, 0, :, 1] = 1.0
        o, lse = attn(q, k, v, scale=np.float32(0.5), q_offset=q_offset, causal=causal, window=window,
                      alibi=slopes)
        for h in range(Hq):
            r = math.exp(-float(slopes[h]))
            for i in range(Tq):
                p = q_offset + i
                hi = min(Tk - 1, p) if causal else Tk - 1        # last visible key
                lo = max(0, p - window + 1) if window > 0 else 0  # first visible key
                # keys at or left of p: distances 0 .. p - lo (only those <= hi); right of p: 1 .. hi - p
                nl = min(p, hi) - lo + 1
                sl0, sl1 = _geo(r, nl)
                dl = p - min(p, hi)                               # distance of the nearest left key
                nr = max(0, hi - p)
                sr0, sr1 = _geo(r, nr)
                # left keys j = p - dl - t (t = 0 .. nl-1), weight r^(dl + t); right keys j = p + 1 + t, weight r^(1 + t)
                w_l, wj_l = r ** dl * sl0, r ** dl * ((p - dl) * sl0 - sl1)
                w_r, wj_r = r * sr0, r * ((p + 1) * sr0 + sr1)
                den = w_l + w_r
                assert abs(o[0, h, i, 0] - (wj_l + wj_r) / den) <= 1e-9 * max(1.0, p), (h, i, causal)
                assert abs(o[0, h, i, 1] - 1.0) <= 1e-12
                assert abs(lse[0, h, i] - math.log(den)) <= 1e-12, (h, i)


def pin_softcap_saturation(attn):
    """Softcap c: a key whose logit is huge scores exactly c (tanh saturates), a key with a zero
    dot product scores 0 plus its mask entry m; with one-hot values the output is
    sigmoid(c - m) and the lse ln(e^c + e^m).  The same keys without softcap keep the raw logit."""
    c, m = 2.0, 1.5
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    k = np.array([[[[1.0e6, 0.0], [0.0, 1.0]]]], np.float32)
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    mask = np.array([[[[0.0, m]]]], np.float32)
    o, lse = attn(q, k, v, scale=np.float32(1.0), causal=False, mask=mask, softcap=c)
    sig = 1.0 / (1.0 + math.exp(-(c - m)))
    assert abs(o[0, 0, 0, 0] - sig) <= 1e-14 and abs(o[0, 0, 0, 1] - (1 - sig)) <= 1e-14
    assert abs(lse[0, 0, 0] - math.log(math.exp(c) + math.exp(m))) <= 1e-14
    # a logit far below the cap is nearly unchanged: c tanh(x / c) = x - x^3 / (3 c^2) + ...
    x = 0.01
    q2 = np.array([[[[x, 0.0]]]], np.float32)
    k2 = np.array([[[[1.0, 0.0], [0.0, 0.0]]]], np.float32)
    o2, lse2 = attn(q2, k2, v, scale=np.float32(1.0), causal=False, softcap=c)
    xs = float(np.float32(x))
    s0 = c * math.tanh(xs / c)
    assert abs(s0 - (xs - xs ** 3 / (3 * c * c))) <= 1e-10
    assert abs(lse2[0, 0, 0] - math.log(math.exp(s0) + 1.0)) <= 1e-14


def pin_sdpa(attn):
    """Special case with a library routine: torch's fp64 scaled_dot_product_attention (q_offset 0,
    no window or sinks; GQA by repeating KV heads; a float additive mask)."""
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, T, d = 2, 6, 2, 70, 16
    q = synth.normal_f32(synth.seed_of("pin-sdpa", "q"), (B, Hq, T, d))
    k = synth.normal_f32(synth.seed_of("pin-sdpa", "k"), (B, Hkv, T, d))
    v = synth.normal_f32(synth.seed_of("pin-sdpa", "v"), (B, Hkv, T, d))
    m = synth.normal_f32(synth.seed_of("pin-sdpa", "m"), (1, 1, T, T))
    m[synth.neg_inf_mask(synth.seed_of("pin-sdpa", "mi"), m.shape, 0.2) == -np.inf] = -np.inf
    m[..., :, 0] = 0.0  # every row keeps key 0, so SDPA has no all -inf row (it would give NaN)
    tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    tk = tk.repeat_interleave(Hq // Hkv, dim=1)
    tv = tv.repeat_interleave(Hq // Hkv, dim=1)
    scale = float(np.float32(0.3))
    for causal, mask in ((True, None), (False, None), (False, m)):
        ref = F.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=None if mask is None else torch.from_numpy(mask.astype(np.float64)),
            is_causal=causal, scale=scale).numpy()
        o, _ = attn(q, k, v, scale=np.float32(0.3), causal=causal,
                    mask=None if mask is None else np.broadcast_to(mask, (B, Hq, T, T)))
        assert np.max(np.abs(o - ref)) <= 1e-12, (causal, mask is None)


def streamed_reference(q, k, v, *, scale, q_offset, causal, window, sinks, bc):
    """fp64 tiled online softmax ("FlashAttention forward in C", section 2.2) over absolute key
    tiles [t*bc, (t+1)*bc); each row skips tiles it cannot see.  Returns o, lse and, per row,
    the (l, a) state after the first visited tile."""
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    o = np.zeros((B, Hq, Tq, d))
    lse = np.full((B, Hq, Tq), -np.inf)
    first = {}
    for b in range(B):
        for h in range(Hq):
            kvh = h // (Hq // Hkv)
            for i in range(Tq):
                p = q_offset + i
                lo, hi = _interval(p, Tk, causal, window)
                if sinks is not None:
                    m, l, a = float(sinks[h]), 1.0, np.zeros(d)
                else:
                    m, l, a = -np.inf, 0.0, np.zeros(d)
                for t in range(0, (Tk + bc - 1) // bc):
                    j0, j1 = max(t * bc, lo), min((t + 1) * bc, hi)
                    if j0 >= j1:
                        continue
                    s = scale * (k[b, kvh, j0:j1] @ q[b, h, i])
                    m_new = max(m, float(s.max()))
                    alpha = math.exp(m - m_new) if m > -np.inf else 0.0
                    w = np.exp(s - m_new)
                    l = alpha * l + w.sum()
                    a = alpha * a + w @ v[b, kvh, j0:j1]
                    m = m_new
                    first.setdefault((b, h, i), (l, a.copy()))
                if l > 0:
                    o[b, h, i] = a / l
                    lse[b, h, i] = m + math.log(l)
    return o, lse, first


def pin_streamed_equals_materialised(attn):
    """Online softmax over tiles is not an approximation: streamed (Bc = 64, 2, 1) = textbook."""
    g = golden("hand_example.txt")
    q = _bhsd([g["q"]]); k = _bhsd([g["k0"], g["k1"], g["k2"]]); v = _bhsd([g["v0"], g["v1"], g["v2"]])
    _, _, first = streamed_reference(q, k, v, scale=1.0, q_offset=0, causal=False, window=0, sinks=None, bc=2)
    l0, a0 = first[(0, 0, 0)]
    # the page prints 7 decimals, truncated or rounded: one unit of the last digit
    assert abs(l0 - g["tile0_l"][0]) <= 1e-7 and np.max(np.abs(a0 - g["tile0_a"])) <= 1e-7
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 33, 150, 8
    q = synth.normal_f32(synth.seed_of("pin-st", "q"), (B, Hq, Tq, d)).astype(np.float64)
    k = synth.normal_f32(synth.seed_of("pin-st", "k"), (B, Hkv, Tk, d)).astype(np.float64)
    v = synth.normal_f32(synth.seed_of("pin-st", "v"), (B, Hkv, Tk, d)).astype(np.float64)
    z = synth.normal_f32(synth.seed_of("pin-st", "z"), (Hq,))
    for (qo, causal, w, sinks) in ((117, True, 0, None), (100, True, 20, z), (0, False, 0, z), (3, False, 40, None)):
        o, lse = attn(q, k, v, scale=0.4, q_offset=qo, causal=causal, window=w, sinks=sinks)
        for bc in (64, 2, 1):
            os_, ls_, _ = streamed_reference(q, k, v, scale=0.4, q_offset=qo, causal=causal, window=w,
                                             sinks=sinks, bc=bc)
            assert np.max(np.abs(o - os_)) <= 1e-12, (qo, bc)
            fin = np.isfinite(ls_)
            assert np.all(np.isfinite(lse) == fin)
            assert np.max(np.abs(lse[fin] - ls_[fin]), initial=0) <= 1e-12


ALL_PINS = [pin_hand_example, pin_sinks, pin_no_visible_key, pin_closed_form_q_zero, pin_alibi_closed_form,
            pin_softcap_saturation,
            pin_closed_form_q_zero_mask, pin_closed_form_q_zero_mask_offset, pin_const_v, pin_single_visible_key, pin_mask_shift,
            pin_brute_force, pin_sdpa, pin_streamed_equals_materialised]
