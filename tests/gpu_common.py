"""Shared helpers of the GPU tests: seeded inputs, device copies, comparison with the oracle.

Inputs come from ``synth`` (one generator for both sides); expected values come only from
``oracle`` (fp64 CPU).  Nothing here computes attention.
"""
import math

import numpy as np
import torch

import oracle
import synth

# Tolerances on max |O - O_oracle| (and on LSE) stated for this path: fp32 inputs 2e-5,
# bf16 inputs (fp32 accumulate, bf16 output) 1.5e-2.
TOL = {"f32": 2e-5, "bf16": 1.5e-2}


def say(*parts):
    """Names the case on stdout before a GPU step, so a failed run still shows what it was."""
    print("[case]", *parts, flush=True)


def scale_for(d):
    return float(np.float32(1.0 / math.sqrt(d)))


def make_inputs(tag, B, Hq, Hkv, Tq, Tk, d, dtype, sinks=False, q_shape=None):
    """Seeded N(0, 1) q, k, v (fp32 arrays, or uint16 bf16 bits) and optional sinks."""
    q = synth.normal(synth.seed_of(tag, "q"), q_shape or (B, Hq, Tq, d), dtype)
    k = synth.normal(synth.seed_of(tag, "k"), (B, Hkv, Tk, d), dtype)
    v = synth.normal(synth.seed_of(tag, "v"), (B, Hkv, Tk, d), dtype)
    z = synth.normal_f32(synth.seed_of(tag, "z"), (Hq,)) if sinks else None
    return q, k, v, z


def dev(a):
    """Host array -> GPU tensor (uint16 arrays are bf16 bits)."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    """GPU tensor -> float32 (bf16 widened exactly) or float64 numpy array."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def bits(t):
    """Raw bits of a GPU tensor as an integer numpy array (bitwise comparisons: the library
    writes every zero output as +0, so no normalisation is needed)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy()
    return t.contiguous().view(torch.int32).cpu().numpy()


def bf16_round(x):
    """fp64/fp32 values rounded to bf16 (nearest even) and widened back, for ulp comparisons."""
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def bf16_ulps(got, ref):
    """Distance in bf16 ulps between bf16 results `got` and RNE(ref), in units of the ulp at the
    larger magnitude (8 significant bits: ulp(x) = 2^(floor(log2 |x|) - 7))."""
    r = bf16_round(ref)
    mag = np.maximum(np.abs(got), np.abs(r))
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7)
    return np.abs(got - r) / ulp


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Asserts parity with the oracle; returns (max |dO|, max |dLSE|).

    Rows with no visible key (oracle LSE -inf) must be exactly +0 (sign bit clear) with LSE -inf.
    For bf16 outputs, elements with |o| >= 4 are held to 1 bf16 ulp of the rounded oracle value
    instead of the absolute bound (half an ulp there is 2^-6 > 1.5e-2); the largest such
    distance is reported.
    """
    tol = TOL[dtype]
    o_gpu = np.asarray(o_gpu, np.float64)
    lse_gpu = np.asarray(lse_gpu, np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    dead = lse_ref == -np.inf
    assert np.array_equal(lse_gpu == -np.inf, dead), f"{what}: -inf LSE rows differ"
    if dead.any():
        od = o_gpu[dead]
        assert np.all(od == 0) and not np.any(np.signbit(od)), f"{what}: a row with no visible key is not +0"
    err = np.abs(o_gpu - o_ref)
    big = np.zeros(o_ref.shape, bool)
    ulps = 0.0
    if dtype == "bf16":
        big = np.abs(o_ref) >= 4
        if big.any():
            ulps = float(np.max(bf16_ulps(o_gpu[big], o_ref[big])))
            assert ulps <= 1.0, f"{what}: {ulps} bf16 ulps at |o| >= 4"
    do = float(np.max(err[~big])) if (~big).any() else 0.0
    dl = float(np.max(np.abs(lse_gpu[~dead] - lse_ref[~dead]))) if (~dead).any() else 0.0
    extra = f" |o|>=4: {int(big.sum())} elements, max {ulps:.2f} bf16 ulp" if big.any() else ""
    print(f"[parity] {what} dtype={dtype} max|dO|={do:.3e} max|dLSE|={dl:.3e} tol={tol:g}{extra}", flush=True)
    assert do <= tol, f"{what}: max |dO| {do} > {tol}"
    assert dl <= tol, f"{what}: max |dLSE| {dl} > {tol}"
    return do, dl


def oracle_rows(q, k, v, rows, **kw):
    return oracle.attention(q, k, v, rows=rows, **kw)


def sample_rows(B, Hq, Tq, n, seed, extra_i=()):
    """n (b, h, i) triples: tile-boundary rows first, then seeded random rows."""
    rng = np.random.default_rng(seed)
    fixed = [i for i in (0, 1, 31, 32, 63, 64, 65, 127, 128, Tq // 2, Tq - 2, Tq - 1, *extra_i) if 0 <= i < Tq]
    rows = [(int(rng.integers(B)), int(rng.integers(Hq)), i) for i in fixed]
    while len(rows) < n:
        rows.append((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Tq))))
    return np.array(rows, np.int64)
