"""GPU tests of split-KV (decoding): the keys cut into absolute splits that run in parallel
and are merged per row ("FlashAttention forward in C", "Going further": split-KV /
Flash-Decoding, partial (m, l, a) merged with the tile rescale).

Parity against the fp64 oracle (the merged result is the same attention), the decode shapes
of the pages (one query row at q_offset = Tk - 1; 9 query / 3 KV heads, d 64, 1,024 and
4,096 keys from the candle flash-attention page; the 32/8-head d 128 bf16 model at 8,192
keys), ragged key counts around the tile and split edges, and the bit-level promises: one
split equals the unsplit call, and a fixed split size gives results independent of query
chunking, tiling and the workspace's prior contents.
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
import synth
from gpu_common import bits, compare, dev, host, make_inputs, say, scale_for

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16"]

# (name, B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks, mask, split_keys)
#   mask: None, "bcast" ([Tq, Tk] broadcast over b, h), "full" ([B, Hq, Tq, Tk]);
#   split_keys 0: the library's default
CASES = [
    ("decode_tk1", 1, 4, 2, 1, 1, 64, 0, True, 0, False, None, 64),
    ("decode_tk63", 1, 4, 2, 1, 63, 64, 62, True, 0, False, None, 64),
    ("decode_tk64", 1, 4, 2, 1, 64, 128, 63, True, 0, False, None, 64),
    ("decode_tk65_sinks", 1, 4, 2, 1, 65, 128, 64, True, 0, True, None, 64),
    ("decode_gqa4", 2, 8, 2, 1, 1000, 128, 999, True, 0, False, None, 128),
    ("decode_mha", 3, 4, 4, 1, 900, 128, 899, True, 0, False, None, 0),
    ("decode_candle_1024", 1, 9, 3, 1, 1024, 64, 1023, True, 0, False, None, 0),
    ("decode_candle_4096", 1, 9, 3, 1, 4096, 64, 4095, True, 0, False, None, 0),
    ("decode_window_sinks", 1, 32, 8, 1, 5000, 64, 4999, True, 512, True, None, 256),
    ("decode_mask", 1, 4, 2, 1, 700, 128, 699, False, 0, False, "bcast", 192),
    ("decode_past_end", 1, 4, 2, 3, 500, 64, 700, True, 0, False, None, 128),
    ("spec_rows4", 2, 16, 8, 4, 2000, 128, 1996, True, 0, True, None, 320),
    ("multi_row", 1, 8, 2, 200, 1000, 128, 800, True, 0, True, None, 192),
    ("prefill_split", 1, 4, 2, 300, 300, 64, 0, True, 0, False, None, 128),
    ("mask_full_noncausal", 2, 2, 1, 40, 333, 64, 0, False, 0, False, "full", 64),
    ("window_noncausal", 1, 2, 2, 90, 530, 128, 5, False, 20, False, None, 64),
    ("no_visible_rows", 1, 2, 1, 50, 40, 64, 30, False, 10, False, None, 64),
    ("one_split", 1, 8, 2, 70, 700, 128, 630, True, 100, True, None, 704),
]


def _mask(kind, tag, B, Hq, Tq, Tk):
    if kind is None:
        return None
    shape = (Tq, Tk) if kind == "bcast" else (B, Hq, Tq, Tk)
    m = synth.normal_f32(synth.seed_of(tag, "mask"), shape)
    m[synth.neg_inf_mask(synth.seed_of(tag, "mask-inf"), shape, 0.1) == -np.inf] = -np.inf
    if Tq > 3:
        m[..., 3, :] = -np.inf  # one fully masked row
    return m


def _setup(case, dtype):
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks, mkind, split = case
    tag = f"splitkv/{name}/{dtype}"
    q, k, v, z = make_inputs(tag, B, Hq, Hkv, Tq, Tk, d, dtype, sinks=with_sinks)
    m = _mask(mkind, tag, B, Hq, Tq, Tk)
    kw = dict(scale=scale_for(d), q_offset=qo, causal=causal, window=window)
    return q, k, v, z, m, kw, split


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_splitkv_parity(case, dtype):
    q, k, v, z, m, kw, split = _setup(case, dtype)
    say("splitkv", case[0], dtype, case[1:7], kw, "split_keys", split)
    o, lse = fa.forward_splitkv(dev(q), dev(k), dev(v), split_keys=split, sinks=dev(z),
                                mask=None if m is None else dev(m), **kw)
    torch.cuda.synchronize()
    m4 = None if m is None else (m[None, None] if m.ndim == 2 else m)
    o_ref, l_ref = oracle.attention(q, k, v, sinks=z, mask=m4, **kw)
    compare(host(o), host(lse), o_ref, l_ref, dtype, f"splitkv {case[0]}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("name", ["decode_tk65_sinks", "decode_window_sinks", "multi_row", "mask_full_noncausal"])
def test_one_split_equals_unsplit(name, dtype):
    """split_keys >= Tk: one split, merged with weight 2^0 = 1, equals fa_fwd bit for bit."""
    case = next(c for c in CASES if c[0] == name)
    q, k, v, z, m, kw, _ = _setup(case, dtype)
    Tk = case[5]
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    tm = None if m is None else dev(m)
    say("one split", name, dtype)
    o1, l1 = fa.forward(tq, tk, tv, sinks=tz, mask=tm, **kw)
    # (2^32 and 2^32 + 64 keys per split: one split as well; the library caps a split at the keys)
    for split in (64 * ((Tk + 63) // 64), 64 * ((Tk + 63) // 64) + 256, 2 ** 32, 2 ** 32 + 64):
        o2, l2 = fa.forward_splitkv(tq, tk, tv, split_keys=split, sinks=tz, mask=tm, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o1), bits(o2)), f"O differs at split_keys {split}"
        assert np.array_equal(bits(l1), bits(l2)), f"LSE differs at split_keys {split}"


@pytest.mark.parametrize("dtype", DTYPES)
def test_fixed_split_chunk_and_tiling_invariance(dtype):
    """With split_keys fixed, rows computed in query chunks (q_offset), with any tiling, or as
    decode rows one at a time carry the same bits as one whole call."""
    B, Hq, Hkv, T, d, split = 1, 8, 2, 700, 128, 192
    q, k, v, z = make_inputs(f"splitkv/chunks/{dtype}", B, Hq, Hkv, T, T, d, dtype, sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(d), causal=True, window=300, sinks=tz, split_keys=split)
    say("splitkv chunks whole", dtype)
    o_full, l_full = fa.forward_splitkv(tq, tk, tv, **kw)
    start = 0
    for n, tiling in ((100, None), (250, (32, 1)), (300, (64, 2)), (50, (128, 2))):
        say("splitkv chunk", start, n, tiling)
        o, lse = fa.forward_splitkv(tq[:, :, start:start + n], tk, tv, q_offset=start, tiling=tiling, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o), bits(o_full[:, :, start:start + n])), f"O chunk at {start}"
        assert np.array_equal(bits(lse), bits(l_full[:, :, start:start + n])), f"LSE chunk at {start}"
        start += n
    for i in (0, 63, 64, 191, 192, 383, 699):  # decode rows: keys [0, i] only
        say("splitkv decode row", i)
        o, lse = fa.forward_splitkv(tq[:, :, i:i + 1], tk[:, :, :i + 1], tv[:, :, :i + 1], q_offset=i, **kw)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o), bits(o_full[:, :, i:i + 1])), f"O decode row {i}"
        assert np.array_equal(bits(lse), bits(l_full[:, :, i:i + 1])), f"LSE decode row {i}"


def test_workspace_contents_do_not_matter():
    """A workspace full of NaN bit patterns, reused across calls of other sizes, gives the same
    bits as a fresh one."""
    q, k, v, z = make_inputs("splitkv/ws", 2, 8, 2, 1, 3000, 128, "bf16", sinks=True)
    tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
    kw = dict(scale=scale_for(128), q_offset=2999, causal=True, sinks=tz, split_keys=256)
    nbytes = fa.fa_splitkv_workspace_bytes(2, 8, 1, 3000, 128, 256)
    assert nbytes == 12 * 2 * 8 * 130 * 4
    say("splitkv workspace")
    o1, l1 = fa.forward_splitkv(tq, tk, tv, **kw)
    ws = torch.full((nbytes + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    fa.forward_splitkv(tq[:, :, :, :], tk[:, :, :1000], tv[:, :, :1000], workspace=ws,
                       **{**kw, "q_offset": 999})
    o2, l2 = fa.forward_splitkv(tq, tk, tv, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))


def test_errors_leave_outputs_untouched():
    q, k, v, _ = make_inputs("splitkv/err", 1, 4, 2, 1, 500, 64, "f32")
    tq, tk, tv = dev(q), dev(k), dev(v)
    out = torch.full((1, 4, 1, 64), 7.0, device="cuda")
    lse = torch.full((1, 4, 1), 7.0, device="cuda")
    small = torch.empty(100, dtype=torch.uint8, device="cuda")
    say("splitkv errors")
    for kw, want in ((dict(split_keys=100), fa.FA_EINVAL), (dict(split_keys=-64), fa.FA_EINVAL),
                     (dict(split_keys=64, workspace=small), fa.FA_EINVAL)):
        with pytest.raises(fa.FaError) as e:
            fa.forward_splitkv(tq, tk, tv, q_offset=499, out=out, lse=lse, **kw)
        assert e.value.status == want, kw
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


@pytest.mark.parametrize("with_sinks", [False, True])
def test_no_keys(with_sinks):
    """Tk = 0: one empty split; o = 0 and lse = -inf, or the sink logit."""
    q, _, _, z = make_inputs("splitkv/tk0", 1, 4, 2, 5, 0, 64, "f32", sinks=with_sinks)
    k = torch.empty((1, 2, 0, 64), device="cuda")
    say("splitkv Tk=0", with_sinks)
    o, lse = fa.forward_splitkv(dev(q), k, k, split_keys=64, sinks=dev(z), causal=False)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    if with_sinks:
        np.testing.assert_allclose(host(lse), np.broadcast_to(z[None, :, None], (1, 4, 5)), rtol=0, atol=2e-6)
    else:
        assert torch.all(lse == -float("inf"))


def test_decode_model_shape_bf16():
    """Decode at the large model shape: B=8, 32 query / 8 KV heads, d 128, 8,192 cached keys,
    bf16, one query row per sequence at q_offset 8191, default split: every row against the
    oracle; also against the unsplit call."""
    B, Hq, Hkv, Tk, d = 8, 32, 8, 8192, 128
    q, k, v, _ = make_inputs("splitkv/decode8192", B, Hq, Hkv, 1, Tk, d, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    kw = dict(scale=scale_for(d), q_offset=Tk - 1, causal=True)
    say("splitkv decode 8x32x8192 bf16", fa.fa_splitkv_default_keys(B, Hq, Hkv, 1, Tk, Tk - 1, True, 0, fa.FA_BF16))
    o, lse = fa.forward_splitkv(tq, tk, tv, **kw)
    o1, l1 = fa.forward(tq, tk, tv, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, **kw)
    compare(host(o), host(lse), o_ref, l_ref, "bf16", "decode 8x32x8192 split")
    compare(host(o1), host(l1), o_ref, l_ref, "bf16", "decode 8x32x8192 unsplit")
