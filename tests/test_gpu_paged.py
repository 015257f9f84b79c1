"""GPU tests of paged K/V and per-sequence key counts ("FlashAttention forward in C", "Key
Takeaways": paged attention for decode performs the same tile update on blocks, and its tests
hold it to this kernel bit for bit).

The K/V of each sequence are scattered over a pool of blocks through a shuffled block table
(unused pool space holds NaN, so a stray read would show); the paged call must give the same
bits as the contiguous call on the same keys, for every flag, both dtypes, block sizes of 64 to
512 keys, both pool layouts and with split-KV.  Per-sequence key counts (decode batches of
ragged lengths) are held bit for bit to one contiguous call per sequence and checked against the
fp64 oracle.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
from gpu_common import bits, compare, dev, host, make_inputs, say, scale_for

pytestmark = pytest.mark.gpu


def _page(k, v, block_size, seed, layout="hnd", extra_blocks=3):
    """Scatters contiguous k, v [B, Hkv, Tk, d] (GPU) into NaN-filled pools through a shuffled
    block table.  Returns (k_pool, v_pool, block_table) with pools viewed [nb, Hkv, bs, d]."""
    B, Hkv, Tk, d = k.shape
    nbs = -(-Tk // block_size)
    nb = B * nbs + extra_blocks
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)[:B * nbs].reshape(B, nbs)
    table = torch.from_numpy(perm.astype(np.int32)).cuda()
    shape = (nb, Hkv, block_size, d) if layout == "hnd" else (nb, block_size, Hkv, d)
    pools = []
    for t in (k, v):
        pool = torch.full(shape, float("nan"), dtype=t.dtype, device="cuda")
        view = pool if layout == "hnd" else pool.transpose(1, 2)
        for b in range(B):
            for j in range(nbs):
                n = min(block_size, Tk - j * block_size)
                view[perm[b, j], :, :n] = t[b, :, j * block_size:j * block_size + n]
        pools.append(view)
    return pools[0], pools[1], table


# (name, B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks, mask, block_size, layout)
CASES = [
    ("prefill_causal", 2, 8, 2, 300, 300, 128, 0, True, 0, False, False, 64, "hnd"),
    ("chunk_window_sinks", 1, 8, 2, 100, 700, 64, 600, True, 200, True, False, 128, "nhd"),
    ("decode", 3, 16, 8, 1, 1000, 128, 999, True, 0, False, False, 256, "hnd"),
    ("decode_nhd_512", 2, 4, 1, 1, 1500, 64, 1499, True, 0, True, False, 512, "nhd"),
    ("mask_noncausal", 2, 4, 2, 40, 333, 128, 0, False, 0, False, True, 64, "hnd"),
    ("ragged_tail", 1, 4, 2, 65, 65, 64, 0, True, 0, False, False, 128, "hnd"),
]


def _setup(case, dtype):
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks, with_mask, bs, layout = case
    q, k, v, z = make_inputs(f"paged/{name}/{dtype}", B, Hq, Hkv, Tq, Tk, d, dtype, sinks=with_sinks)
    m = None
    if with_mask:
        m = np.where(np.random.default_rng(7).random((Tq, Tk)) < 0.1, -np.inf, 0.0).astype(np.float32)
        m[3] = -np.inf
    kw = dict(scale=scale_for(d), q_offset=qo, causal=causal, window=window, sinks=dev(z),
              mask=None if m is None else dev(m))
    return q, k, v, z, m, kw, bs, layout


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_equals_contiguous(case, dtype):
    q, k, v, z, m, kw, bs, layout = _setup(case, dtype)
    tq, tk, tv = dev(q), dev(k), dev(v)
    kp, vp, table = _page(tk, tv, bs, seed=len(case[0]), layout=layout)
    say("paged", case[0], dtype, "block", bs, layout)
    o1, l1 = fa.forward(tq, tk, tv, **kw)
    o2, l2 = fa.forward_paged(tq, kp, vp, table, Tk=case[5], **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)), "O differs from the contiguous call"
    assert np.array_equal(bits(l1), bits(l2)), "LSE differs from the contiguous call"
    # and with split-KV: equal to the contiguous split-KV call at the same split size
    o3, l3 = fa.forward_splitkv(tq, tk, tv, split_keys=128, **kw)
    o4, l4 = fa.forward_paged(tq, kp, vp, table, Tk=case[5], split_keys=128, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o3), bits(o4)) and np.array_equal(bits(l3), bits(l4)), "split-KV differs"
    m4 = None if m is None else m[None, None]
    o_ref, l_ref = oracle.attention(q, k, v, scale=kw["scale"], q_offset=kw["q_offset"], causal=kw["causal"],
                                    window=kw["window"], sinks=z, mask=m4)
    compare(host(o2), host(l2), o_ref, l_ref, dtype, f"paged {case[0]}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Tq,split", [(1, 0), (1, -1), (1, 192), (4, 0), (4, 256)])
def test_per_sequence_key_counts(dtype, Tq, split):
    """Decode batch of ragged lengths (0, 1, 63, 64, 65, 700, 1000 keys): sequence b's rows are
    its last Tq positions; each equals a contiguous call on its own keys (q_offset = n_b - Tq)
    bit for bit when unsplit, and the oracle within tolerance."""
    lens = [1000, 0, 1, 63, 64, 65, 700]
    B, Hq, Hkv, Tk, d, bs = len(lens), 8, 2, 1000, 128, 128
    q, k, v, z = make_inputs(f"paged/seqlens/{dtype}/{Tq}", B, Hq, Hkv, Tq, Tk, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kp, vp, table = _page(tk, tv, bs, seed=11)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = scale_for(d)
    say("paged seqlens", dtype, "Tq", Tq, "split", split)
    o, lse = fa.forward_paged(tq, kp, vp, table, seqlens_k=seqlens, split_keys=split, scale=sc, causal=True,
                              window=500, sinks=tz)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        qo = n - Tq
        if split == 0 and qo >= 0:
            o1, l1 = fa.forward(tq[b:b + 1], tk[b:b + 1, :, :n], tv[b:b + 1, :, :n], scale=sc, q_offset=qo,
                                causal=True, window=500, sinks=tz)
            torch.cuda.synchronize()
            assert np.array_equal(bits(o1), bits(o[b:b + 1])), f"O of sequence {b}"
            assert np.array_equal(bits(l1), bits(lse[b:b + 1])), f"LSE of sequence {b}"
        # oracle: positions n - Tq + i; rows before position 0 see no key (sink only)
        for i in range(Tq):
            p = n - Tq + i
            if p < 0:
                assert torch.all(o[b, :, i] == 0) and not torch.any(torch.signbit(o[b, :, i])), (b, i)
                np.testing.assert_allclose(host(lse[b, :, i]), z, rtol=0, atol=2e-6)
                continue
            o_ref, l_ref = oracle.attention(q[b:b + 1, :, i:i + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=sc,
                                            q_offset=p, causal=True, window=500, sinks=z)
            compare(host(o[b:b + 1, :, i:i + 1]), host(lse[b:b + 1, :, i:i + 1]), o_ref, l_ref, dtype,
                    f"seqlens b={b} n={n} i={i}")


def test_out_of_range_block_reads_zeros():
    """A block index outside [0, num_blocks) reads zero keys and values: the same as a contiguous
    call whose keys and values in that block are zero."""
    B, Hq, Hkv, Tq, Tk, d, bs = 1, 4, 2, 1, 512, 64, 128
    q, k, v, _ = make_inputs("paged/oob", B, Hq, Hkv, Tq, Tk, d, "f32")
    tq, tk, tv = dev(q), dev(k), dev(v)
    kp, vp, table = _page(tk, tv, bs, seed=3)
    table[0, 1] = -1
    table[0, 2] = kp.shape[0] + 5
    kz, vz = tk.clone(), tv.clone()
    kz[:, :, bs:3 * bs] = 0
    vz[:, :, bs:3 * bs] = 0
    say("paged out-of-range blocks")
    o1, l1 = fa.forward(tq, kz, vz, q_offset=Tk - 1)
    o2, l2 = fa.forward_paged(tq, kp, vp, table, Tk=Tk, q_offset=Tk - 1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))


def test_paged_decode_model_shape_bf16():
    """Decode at the large model shape through pages of 256 keys: B=8, 32/8 heads, d 128, bf16,
    key counts from 1 to 8,192, default split: every row against the oracle."""
    lens = [8192, 1, 4000, 8191, 257, 6000, 64, 5000]
    B, Hq, Hkv, Tk, d, bs = 8, 32, 8, 8192, 128, 256
    q, k, v, _ = make_inputs("paged/decode8192", B, Hq, Hkv, 1, Tk, d, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    kp, vp, table = _page(tk, tv, bs, seed=5, extra_blocks=0)
    seqlens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = scale_for(d)
    say("paged decode 8x32x8192 bf16")
    o, lse = fa.forward_paged(tq, kp, vp, table, seqlens_k=seqlens, split_keys=-1, scale=sc, causal=True)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        o_ref, l_ref = oracle.attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=sc, q_offset=n - 1,
                                        causal=True)
        compare(host(o[b:b + 1]), host(lse[b:b + 1]), o_ref, l_ref, "bf16", f"paged decode b={b} n={n}")
