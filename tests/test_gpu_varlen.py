"""GPU tests of packed variable-length batching: sequences of different lengths packed token by
token into q [total_q, Hq, d], k, v [total_k, Hkv, d] with prefix sums cu_seqlens (candle's
B > 1 path; the batch invariance of "FlashAttention forward in C" section 4: a sequence alone
gives the same bits as in a batch).

Every packed row must equal the single-sequence call on its own tokens bit for bit (query rows
at the end of the sequence's keys, q_offset = keys - rows), and the fp64 oracle within
tolerance; lengths cover 0, 1 and the tile edges 63/64/65.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
import synth
from gpu_common import bits, compare, dev, host, say, scale_for

pytestmark = pytest.mark.gpu


def _packed(tag, qlens, klens, Hq, Hkv, d, dtype, fused=False):
    """Packed q, k, v (host arrays, fp32 or bf16 bits) and their GPU tensors.  fused: q, k, v
    are column slices of one [total, Hq + 2 Hkv, d] tensor (a fused QKV projection's output),
    so their token strides are (Hq + 2 Hkv) d."""
    tq, tk = sum(qlens), sum(klens)
    q = synth.normal(synth.seed_of(tag, "q"), (tq, Hq, d), dtype)
    k = synth.normal(synth.seed_of(tag, "k"), (tk, Hkv, d), dtype)
    v = synth.normal(synth.seed_of(tag, "v"), (tk, Hkv, d), dtype)
    if fused:
        assert tq == tk
        qkv = dev(np.concatenate([q, k, v], axis=1))
        gq, gk, gv = qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]
    else:
        gq, gk, gv = dev(q), dev(k), dev(v)
    return q, k, v, gq, gk, gv


def _cu(lens):
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")


def _check(qlens, klens, Hq, Hkv, d, dtype, causal, window, with_sinks, split, tag, fused=False, tiling=None):
    q, k, v, gq, gk, gv = _packed(tag, qlens, klens, Hq, Hkv, d, dtype, fused)
    z = synth.normal_f32(synth.seed_of(tag, "z"), (Hq,)) if with_sinks else None
    tz = dev(z)
    sc = scale_for(d)
    say("varlen", tag, dtype, qlens, klens, dict(causal=causal, window=window, split=split))
    out = torch.full((sum(qlens), Hq, d), float("nan"), dtype=gq.dtype, device="cuda")
    lse = torch.full((Hq, sum(qlens)), float("nan"), device="cuda")
    o, l = fa.forward_varlen(gq, gk, gv, _cu(qlens), _cu(klens), max(qlens), max(klens), scale=sc, causal=causal,
                             window=window, sinks=tz, split_keys=split, out=out, lse=lse, tiling=tiling)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(l).any(), "a packed row was not written"
    q0 = k0 = 0
    for b, (m, n) in enumerate(zip(qlens, klens)):
        if m == 0:
            k0 += n
            continue
        qs = gq[q0:q0 + m].transpose(0, 1)[None]          # [1, Hq, m, d] view of the packed rows
        ks = gk[k0:k0 + n].transpose(0, 1)[None]
        vs = gv[k0:k0 + n].transpose(0, 1)[None]
        qo = n - m
        ob, lb = o[q0:q0 + m].transpose(0, 1)[None], l[:, q0:q0 + m][None]
        if qo >= 0:
            if split:
                o1, l1 = fa.forward_splitkv(qs, ks, vs, split_keys=split, scale=sc, q_offset=qo, causal=causal,
                                            window=window, sinks=tz)
            else:
                o1, l1 = fa.forward(qs, ks, vs, scale=sc, q_offset=qo, causal=causal, window=window, sinks=tz)
            torch.cuda.synchronize()
            assert np.array_equal(bits(o1), bits(ob)), f"O of sequence {b} differs from its own call"
            assert np.array_equal(bits(l1), bits(lb)), f"LSE of sequence {b} differs from its own call"
            o_ref, l_ref = oracle.attention(q[q0:q0 + m].transpose(1, 0, 2)[None], k[k0:k0 + n].transpose(1, 0, 2)[None],
                                            v[k0:k0 + n].transpose(1, 0, 2)[None], scale=sc, q_offset=qo,
                                            causal=causal, window=window, sinks=z)
            compare(host(ob), host(lb), o_ref, l_ref, dtype, f"varlen {tag} b={b}")
        q0 += m
        k0 += n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal,window,sinks", [(True, 0, False), (True, 50, True), (False, 0, False)])
def test_varlen_prefill(dtype, causal, window, sinks):
    """Self-attention prefill of 7 packed sequences (rows = keys per sequence), 16/8 heads, d 128."""
    lens = [1, 63, 64, 65, 300, 0, 129]
    _check(lens, lens, 16, 8, 128, dtype, causal, window, sinks, 0, f"prefill/{causal}/{window}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_fused_qkv_layout_d64(dtype):
    """q, k, v as column slices of one fused [total, Hq + 2 Hkv, d] projection output, d 64,
    GQA 4:1, several query tilings."""
    lens = [200, 17, 64, 1, 90]
    for tiling in (None, (32, 1), (64, 2), (32, 4)):
        _check(lens, lens, 8, 2, 64, dtype, True, 0, False, 0, f"fused/{tiling}", fused=True, tiling=tiling)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("split", [0, 128])
def test_varlen_rows_at_the_end(dtype, split):
    """Fewer rows than keys per sequence (chunked prefill / decode of packed requests): rows are
    each sequence's last positions; also through split-KV."""
    qlens = [5, 1, 30, 0, 1, 64]
    klens = [100, 1, 700, 10, 2000, 64]
    _check(qlens, klens, 8, 2, 128, dtype, True, 0, True, split, f"tail/{split}")
    _check(qlens, klens, 8, 2, 128, dtype, True, 256, False, split, f"tail-window/{split}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("split", [0, 192])
def test_varlen_queries_over_paged_keys(dtype, split):
    """Packed query rows over a paged KV cache (per-sequence key counts from seqlens_k): equal to
    the same call with the keys packed contiguously, bit for bit."""
    from test_gpu_paged import _page
    qlens, klens = [5, 1, 30, 1, 64], [100, 1, 700, 2000, 64]
    Hq, Hkv, d, bs = 8, 2, 128, 128
    q, k, v, gq, gk, gv = _packed(f"vpaged/{dtype}", qlens, klens, Hq, Hkv, d, dtype)
    Tk = max(klens)
    # the same keys per sequence, padded to Tk and paged
    kpad = torch.zeros((len(klens), Hkv, Tk, d), dtype=gk.dtype, device="cuda")
    vpad = torch.zeros_like(kpad)
    k0 = 0
    for b, n in enumerate(klens):
        kpad[b, :, :n] = gk[k0:k0 + n].transpose(0, 1)
        vpad[b, :, :n] = gv[k0:k0 + n].transpose(0, 1)
        k0 += n
    kp, vp, table = _page(kpad, vpad, bs, seed=9)
    seqlens = torch.tensor(klens, dtype=torch.int32, device="cuda")
    sc = scale_for(d)
    say("varlen over paged keys", dtype, split)
    o1, l1 = fa.forward_varlen(gq, gk, gv, _cu(qlens), _cu(klens), max(qlens), Tk, scale=sc, causal=True,
                               split_keys=split)
    o2, l2 = fa.forward_varlen(gq, kp, vp, _cu(qlens), None, max(qlens), Tk, scale=sc, causal=True,
                               split_keys=split, block_table=table, seqlens_k=seqlens)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))
