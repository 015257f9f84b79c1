"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Cases follow the test catalogue of "FlashAttention forward in C" section 4
(gqa_causal_window_match_naive, sinks_join_the_denominator, no_visible_key_...), the
sequence lengths of "IV.5: Flash attention" (1, 17, 100 at 16/8 heads, d 128) and the
additive mask of "Fused attention and softmax: fast and exact".
"""
import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import synth
from gpu_common import compare, dev, host, make_inputs, oracle_rows, say, scale_for
import oracle

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16"]

# (name, B, Hq, Hkv, Tq, Tk, d, q_offset, causal, window, sinks, mask)
#   mask: None, "bcast" ([Tq, Tk] broadcast over b, h), "full" ([B, Hq, Tq, Tk])
CASES = [
    ("gqa62_causal", 2, 6, 2, 100, 100, 64, 0, True, 0, False, None),
    ("mqa_causal_d128", 1, 4, 1, 77, 77, 128, 0, True, 0, False, None),
    ("chunk_q24", 1, 4, 2, 40, 64, 64, 24, True, 0, False, None),
    ("window6", 1, 2, 1, 150, 150, 64, 0, True, 6, False, None),
    ("window_noncausal", 1, 2, 2, 90, 130, 128, 5, False, 20, False, None),
    ("plain", 2, 2, 2, 33, 200, 64, 0, False, 0, False, None),
    ("sinks_window", 1, 8, 2, 130, 130, 64, 0, True, 50, True, None),
    ("sinks_d128", 1, 4, 4, 70, 70, 128, 0, True, 0, True, None),
    ("mask_bcast", 1, 4, 2, 96, 140, 128, 0, False, 0, False, "bcast"),
    ("mask_full_causal", 2, 2, 1, 70, 70, 64, 0, True, 0, False, "full"),
    ("mask_sinks_window", 1, 4, 2, 65, 129, 64, 64, True, 30, True, "bcast"),
    ("decode", 2, 8, 2, 1, 300, 128, 299, True, 0, False, None),
    ("tq_gt_tk", 1, 2, 1, 150, 70, 64, 0, True, 0, False, None),
    ("no_visible_rows", 1, 2, 1, 50, 40, 64, 30, False, 10, False, None),
    ("p1_seq1", 1, 16, 8, 1, 1, 128, 0, True, 0, False, None),
    ("p1_seq17", 1, 16, 8, 17, 17, 128, 0, True, 0, False, None),
    ("p1_seq100", 1, 16, 8, 100, 100, 128, 0, True, 0, False, None),
]


def _mask(kind, tag, B, Hq, Tq, Tk):
    if kind is None:
        return None
    shape = (Tq, Tk) if kind == "bcast" else (B, Hq, Tq, Tk)
    m = synth.normal_f32(synth.seed_of(tag, "mask"), shape)
    m[synth.neg_inf_mask(synth.seed_of(tag, "mask-inf"), shape, 0.1) == -np.inf] = -np.inf
    m[..., 3, :] = -np.inf  # one fully masked row
    return m


def run_case(case, dtype, tiling=None):
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks, mkind = case
    tag = f"parity/{name}/{dtype}"
    q, k, v, z = make_inputs(tag, B, Hq, Hkv, Tq, Tk, d, dtype, sinks=with_sinks)
    m = _mask(mkind, tag, B, Hq, Tq, Tk)
    m4 = None if m is None else (m[None, None] if m.ndim == 2 else m)
    sc = scale_for(d)
    say(name, dtype, (B, Hq, Hkv, Tq, Tk, d), dict(q_offset=qo, causal=causal, window=window))
    o, lse = fa.forward(dev(q), dev(k), dev(v), scale=sc, q_offset=qo, causal=causal, window=window,
                        sinks=dev(z), mask=None if m is None else dev(m), tiling=tiling)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=sc, q_offset=qo, causal=causal, window=window,
                                    sinks=z, mask=m4)
    return compare(host(o), host(lse), o_ref, l_ref, dtype, name)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_flag_matrix(case, dtype):
    run_case(case, dtype)


def test_c1_single_head():
    """B=1, H=1, Tq=Tk=128, d=64, fp32, causal, scale 1/8: full parity."""
    run_case(("c1", 1, 1, 1, 128, 128, 64, 0, True, 0, False, None), "f32")


@pytest.mark.parametrize("dtype", DTYPES)
def test_tk_zero(dtype):
    """Tk = 0: o = 0 and lse = -inf, or lse = the sink ("shape_and_argument_errors")."""
    B, Hq, Hkv, Tq, d = 1, 4, 2, 40, 64
    q, _, _, z = make_inputs(f"tk0/{dtype}", B, Hq, Hkv, Tq, 0, d, dtype, sinks=True)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    empty = torch.empty((B, Hkv, 0, d), dtype=tdt, device="cuda")
    say("tk_zero", dtype)
    o, lse = fa.forward(dev(q), empty, empty, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -float("inf"))
    o, lse = fa.forward(dev(q), empty, empty, causal=True, sinks=dev(z))
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    np.testing.assert_allclose(host(lse), np.broadcast_to(z[None, :, None], (B, Hq, Tq)), rtol=0, atol=2e-6)


@pytest.mark.parametrize("dtype", DTYPES)
def test_sentinel_every_output_written(dtype):
    """O and LSE pre-filled with NaN: after the call every element is finite or -inf (a row
    that sees nothing), i.e. every work item ran and wrote its rows."""
    B, Hq, Hkv, Tq, Tk, d = 3, 8, 2, 333, 333, 128
    q, k, v, _ = make_inputs(f"sentinel/{dtype}", B, Hq, Hkv, Tq, Tk, d, dtype)
    tq = dev(q)
    for tiling in (None, (32, 4), (64, 2), (128, 1), (32, 1), (64, 4), (256, 1)):
        o = torch.full_like(tq, float("nan"))
        lse = torch.full((B, Hq, Tq), float("nan"), device="cuda")
        say("sentinel", dtype, tiling)
        fa.forward(tq, dev(k), dev(v), causal=True, window=100, out=o, lse=lse, tiling=tiling)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(lse).any(), tiling


def test_errors_leave_outputs_untouched():
    """Argument errors are returned before any launch; o and lse keep their contents."""
    B, Hq, Hkv, Tq, Tk, d = 1, 6, 4, 16, 16, 64
    q = torch.randn(B, Hq, Tq, d, device="cuda")
    k = torch.randn(B, Hkv, Tk, d, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, Tq), 7.0, device="cuda")
    st = fa.fa_strides()
    for (args, want) in [
        (dict(Hq=6, Hkv=4), fa.FA_ESHAPE),    # 6 heads on 4 KV heads
        (dict(Hq=4, Hkv=6), fa.FA_ESHAPE),    # Hkv > Hq
        (dict(Tq=-1), fa.FA_EINVAL),
        (dict(q_offset=-3), fa.FA_EINVAL),
        (dict(d=96), fa.FA_EUNSUPPORTED),
        (dict(scale=float("nan")), fa.FA_EINVAL),
    ]:
        kw = dict(Hq=4, Hkv=2, Tq=Tq, d=d, q_offset=0, scale=0.125)
        kw.update(args)
        st.q[:] = [Hq * Tq * d, Tq * d, d]
        st.k[:] = st.v[:] = [Hkv * Tk * d, Tk * d, d]
        st.o[:] = st.q[:]
        st.lse[:] = [Hq * Tq, Tq]
        status = fa.fa_fwd(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), B,
                           kw["Hq"], kw["Hkv"], kw["Tq"], Tk, kw["d"], kw["scale"], kw["q_offset"], 1, 0,
                           None, None, st, fa.FA_F32, None)
        assert status == want, (args, status)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)


@pytest.mark.parametrize("case", [
    ("gqa_causal", 2, 8, 2, 130, 130, 128, 0, True, 0, False),
    ("chunk_sinks_window", 1, 4, 2, 70, 200, 64, 130, True, 40, True),
    ("decode_window3", 3, 8, 4, 1, 300, 128, 299, True, 3, False),
], ids=lambda c: c[0])
def test_bf16_outputs_beyond_4_within_one_ulp(case):
    """bf16 inputs with V ~ N(0, 3^2), so that many outputs reach |o| >= 4 (causal row 0 returns
    v_0 itself): those are held to one bf16 ulp of the rounded oracle value, the others to 1.5e-2
    (the bound of the tolerance table does not fit |o| >= 4, where half a bf16 ulp is 2^-6)."""
    name, B, Hq, Hkv, Tq, Tk, d, qo, causal, window, with_sinks = case
    tag = f"parity-big-o/{name}"
    q, k, _, z = make_inputs(tag, B, Hq, Hkv, Tq, Tk, d, "bf16", sinks=with_sinks)
    v = synth.to_bf16_bits(np.float32(3.0) * synth.normal_f32(synth.seed_of(tag, "v3"), (B, Hkv, Tk, d)))
    sc = scale_for(d)
    say("bf16 |o| >= 4", name)
    o, lse = fa.forward(dev(q), dev(k), dev(v), scale=sc, q_offset=qo, causal=causal, window=window, sinks=dev(z))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=sc, q_offset=qo, causal=causal, window=window, sinks=z)
    assert np.sum(np.abs(o_ref) >= 4) > 0, "the case must reach |o| >= 4"
    compare(host(o), host(lse), o_ref, l_ref, "bf16", f"bf16 |o|>=4 {name}")


def test_library_is_the_hip_path():
    """The binding loads the in-tree libfa.so; there is no other path."""
    lib = fa.load_library()
    assert lib._name == fa.LIB_PATH
