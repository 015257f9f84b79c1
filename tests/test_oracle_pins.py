"""The fp64 oracle against its pins (CPU only), and the pins against planted mistakes."""
import functools
import math

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention)


# Each planted mistake is one plausible error in the oracle (ORACLE_MUTANT in fa_oracle.c).
MUTANTS = {
    3: "round-robin GQA (h mod Hkv)",
    4: "causal as j < p",
    5: "window of w + 1 keys",
    6: "q_offset ignored",
    7: "sink left out of the denominator",
    8: "lse without the maximum",
    9: "divide by l = 0 on a row that sees nothing",
    10: "a dropped term of the dot product",
    11: "scale dropped",
    12: "mask indexed by absolute position",
    13: "mask subtracted",
    14: "wrong sign in the exponent",
    15: "value operand read transposed",
    16: "softcap without its outer factor",
    17: "ALiBi bias with the wrong sign",
    18: "ALiBi distance from the row index instead of the position",
    19: "softcap applied after the bias and the mask",
}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=lambda n: f"m{n}")
def test_planted_mistake_is_caught(n, tmp_path):
    lib = oracle_build.build_mutant(n, str(tmp_path))
    attn = functools.partial(oracle.attention, lib_path=lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(attn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {n}: {MUTANTS[n]}"


def test_visible_pair_counts():
    """Closed forms of sum_i |V_i| at the workload geometries (the FLOP-count basis)."""
    assert oracle.visible_pairs(128, 128) == 128 * 129 // 2
    assert oracle.visible_pairs(511, 511) == 511 * 512 // 2 == 130816
    assert oracle.visible_pairs(2044, 2044) == 2044 * 2045 // 2 == 2089990
    # causal + window 512 over 4096: the first 512 rows see p + 1 keys, the rest see 512
    assert oracle.visible_pairs(4096, 4096, 0, True, 512) == 512 * 513 // 2 + 3584 * 512 == 1966336
    # a chunk is the sum of its rows: chunks of 1000,1000,1000,1096 add up to the full call
    parts = [oracle.visible_pairs(n, 4096, o, True, 512) for n, o in ((1000, 0), (1000, 1000), (1000, 2000), (1096, 3000))]
    assert sum(parts) == 1966336
    assert oracle.visible_pairs(64, 64, 0, False, 0) == 64 * 64


def test_oracle_bf16_inputs_widen_exactly():
    """bf16 bits are the top half of fp32: a bf16 call equals the fp32 call on the rounded values."""
    import synth
    q = synth.normal(synth.seed_of("bf", "q"), (1, 2, 9, 8), "bf16")
    k = synth.normal(synth.seed_of("bf", "k"), (1, 1, 11, 8), "bf16")
    v = synth.normal(synth.seed_of("bf", "v"), (1, 1, 11, 8), "bf16")
    o1, l1 = oracle.attention(q, k, v, scale=0.3, causal=True, q_offset=2)
    o2, l2 = oracle.attention(*(synth.bf16_bits_to_f32(t) for t in (q, k, v)), scale=0.3, causal=True, q_offset=2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_oracle_strided_and_row_subset():
    """Strided (BSHD) views and a row subset give the same numbers as the contiguous full call."""
    import synth
    qs = synth.normal_f32(synth.seed_of("st", "q"), (2, 13, 4, 8))  # [B, T, H, d]
    ks = synth.normal_f32(synth.seed_of("st", "k"), (2, 17, 2, 8))
    vs = synth.normal_f32(synth.seed_of("st", "v"), (2, 17, 2, 8))
    q, k, v = (t.transpose(0, 2, 1, 3) for t in (qs, ks, vs))
    o1, l1 = oracle.attention(q, k, v, scale=0.3, causal=True, q_offset=4)
    o2, l2 = oracle.attention(*(np.ascontiguousarray(t) for t in (q, k, v)), scale=0.3, causal=True, q_offset=4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    rows = np.array([[1, 3, 12], [0, 0, 0], [1, 2, 5]])
    o3, l3 = oracle.attention(q, k, v, scale=0.3, causal=True, q_offset=4, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(o3[r], o1[b, h, i]) and l3[r] == l1[b, h, i]
