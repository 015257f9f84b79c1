"""GPU tests at large key counts: the 32-bit byte offsets of the tile copies (a (b, KV head)
slice may span up to 2 GiB), long tile loops and the split-KV merge over many splits.

"FlashAttention forward in C" section 2.1 fixes what a row computes whatever the key count.
With 10^5-10^6 random keys every output is a near-uniform mean close to zero, which a loose
absolute tolerance cannot tell from a wrong one, so the keys carry "needles": a few rows far
apart (tiles 0, 2^10, 2^13, ... and the last) whose scores exceed every other by ≈ 20 (natural
units) for every query row.  Each output is then the mean of the needles' values, of order 1,
and a tile read from a wrong offset shows at once.  Cases: a decode over 2^20 + 37 cached keys
(bf16, d 64: a 128 MiB K slice) through the plain kernel and split-KV (default and 4,096-key
splits), and the last 32 rows of a 300,001-key causal prefill with sinks (bf16, d 128) through
the plain kernel and paged keys, all against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
import synth
from gpu_common import bits, compare, dev, host, say, scale_for

pytestmark = pytest.mark.gpu


def _needle_inputs(tag, B, Hq, Hkv, Tq, Tk, d, needles):
    """q = 0.5 + 0.1 N(0, 1) (so every row points the same way), k ~ N(0, 1) except the needle
    rows, which are all 5.0 (score ≈ 5 · 0.5 · d), v ~ N(0, 1), sinks ~ N(0, 1); bf16 bits."""
    q = synth.to_bf16_bits(np.float32(0.5) + np.float32(0.1) * synth.normal_f32(synth.seed_of(tag, "q"), (B, Hq, Tq, d)))
    k = synth.normal(synth.seed_of(tag, "k"), (B, Hkv, Tk, d), "bf16")
    k[:, :, needles, :] = synth.to_bf16_bits(np.full((1,), 5.0, np.float32))[0]
    v = synth.normal(synth.seed_of(tag, "v"), (B, Hkv, Tk, d), "bf16")
    z = synth.normal_f32(synth.seed_of(tag, "z"), (Hq,))
    return q, k, v, z


def test_decode_million_keys():
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 1, 4, (1 << 20) + 37, 64
    needles = [3, 64 * 1024 + 17, 512 * 1024 + 5, Tk - 6]
    q, k, v, z = _needle_inputs("large/decode", B, Hq, Hkv, Tq, Tk, d, needles)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), q_offset=Tk - Tq, causal=True, sinks=tz)
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=Tk - Tq, causal=True, sinks=z)
    assert np.abs(o_ref).max() > 0.3, "the needles do not dominate"
    say("large decode", Tk, "plain")
    o, l = fa.forward(tq, tk, tv, **kw)
    torch.cuda.synchronize()
    compare(host(o), host(l), o_ref, l_ref, "bf16", "decode 2^20+37 keys")
    for split in (0, 4096):  # 0: the default split size
        say("large decode", Tk, "split", split)
        o2, l2 = fa.forward_splitkv(tq, tk, tv, split_keys=split, **kw)
        torch.cuda.synchronize()
        compare(host(o2), host(l2), o_ref, l_ref, "bf16", f"decode 2^20+37 keys split {split}")


def test_long_prefill_tail():
    """The last 32 rows of a 300,001-key causal prefill: one workgroup walks 4,688 tiles, the
    last one ragged; paged keys (blocks of 512) give the same bits."""
    from test_gpu_paged import _page
    B, Hq, Hkv, Tq, Tk, d = 1, 4, 2, 32, 300_001, 128
    needles = [1, 128 * 1024 + 3, 256 * 1024 + 9, Tk - 40]
    q, k, v, z = _needle_inputs("large/prefill_tail", B, Hq, Hkv, Tq, Tk, d, needles)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), q_offset=Tk - Tq, causal=True, sinks=tz)
    say("long prefill tail", Tk)
    o, l = fa.forward(tq, tk, tv, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=Tk - Tq, causal=True, sinks=z)
    assert np.abs(o_ref).max() > 0.3, "the needles do not dominate"
    compare(host(o), host(l), o_ref, l_ref, "bf16", "prefill tail 300,001 keys")
    kp, vp, table = _page(tk, tv, 512, seed=21, extra_blocks=0)
    say("long prefill tail paged")
    o2, l2 = fa.forward_paged(tq, kp, vp, table, Tk=Tk, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o2)) and np.array_equal(bits(l), bits(l2))
