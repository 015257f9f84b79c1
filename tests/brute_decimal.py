"""Brute-force attention in 50-digit decimal arithmetic, for tiny inputs only.

It evaluates the definition of "FlashAttention forward in C" (tinyllm L9.3), section 2.1,
with the additive mask of "Fused attention and softmax: fast and exact" (OneModel), "What is
computed", and the softcap / ALiBi score variants (logit c tanh(logit / c); bias
-slope |p - j|), literally: enumerate the visible set, exponentiate every score as is (no
max-subtraction: decimals do not overflow), sum, divide, take the log.  It is structurally
different from the C oracle (which shifts by the row maximum in fp64) and is used only to
pin it.
"""
from decimal import Decimal, getcontext

import numpy as np


def _tanh(x):
    """tanh of a Decimal from its exponential definition."""
    if x < 0:
        return -_tanh(-x)
    e = (-2 * x).exp()
    return (1 - e) / (1 + e)


def brute_attention(q, k, v, *, scale, q_offset=0, causal=True, window=0, sinks=None, mask=None, softcap=0.0,
                    alibi=None):
    getcontext().prec = 50
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    sc = Decimal(float(np.float32(scale)))
    o = np.zeros((B, Hq, Tq, d), np.float64)
    lse = np.zeros((B, Hq, Tq), np.float64)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            for i in range(Tq):
                pos = q_offset + i
                visible = [j for j in range(Tk)
                           if (not causal or j <= pos) and (window <= 0 or j > pos - window)]
                terms = []
                for j in visible:
                    s = sc * sum(Decimal(float(q[b, h, i, x])) * Decimal(float(k[b, kvh, j, x]))
                                 for x in range(d))
                    if softcap > 0:
                        c = Decimal(float(softcap))
                        s = c * _tanh(s / c)
                    if alibi is not None:
                        s -= Decimal(float(np.float32(alibi[h]))) * abs(pos - j)
                    if mask is not None:
                        mv = float(mask[b, h, i, j])
                        if mv == float("-inf"):
                            continue
                        s += Decimal(mv)
                    terms.append((s.exp(), j))
                den = sum((e for e, _ in terms), Decimal(0))
                if sinks is not None:
                    den += Decimal(float(np.float32(sinks[h]))).exp()
                if den == 0:
                    lse[b, h, i] = float("-inf")
                    continue
                for x in range(d):
                    num = sum((e * Decimal(float(v[b, kvh, j, x])) for e, j in terms), Decimal(0))
                    o[b, h, i, x] = float(num / den)
                lse[b, h, i] = float(den.ln())
    return o, lse
