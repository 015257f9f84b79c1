"""fa_fwd_splitkv_noalloc (the split-KV call whose workspace is the library's static scratch)
against fa_fwd_splitkv with a caller-owned workspace, through the C ABI: bit for bit on two
calls in a row (the second smaller, so it runs on scratch left by the first), and against the
fp64 oracle; a call that needs more than the scratch holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import flashattention_forward_flash_amd as fa
import oracle
from gpu_common import bits, compare, dev, host, make_inputs, say, scale_for

pytestmark = pytest.mark.gpu


def _strides(q, k, o, lse):
    st = fa.fa_strides()
    st.q[:] = list(q.stride()[:3])
    st.k[:] = st.v[:] = list(k.stride()[:3])
    st.o[:] = list(o.stride()[:3])
    st.lse[:] = [lse.stride(0), lse.stride(1)]
    st.mask[:] = [0, 0, 0, 0]
    return st


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(dtype):
    dt = fa.FA_BF16 if dtype == "bf16" else fa.FA_F32
    # (B, Hq, Hkv, Tq, Tk, d, q_offset, window, sinks, split_keys): a decode over 10 splits with
    # sinks and a window, then a smaller multi-row call with rows in one split and in several
    cases = [(4, 16, 4, 1, 5000, 128, 4999, 3000, True, 512), (1, 4, 2, 70, 600, 64, 530, 0, False, 128)]
    for n, (B, Hq, Hkv, Tq, Tk, d, qo, window, with_sinks, split) in enumerate(cases):
        q, k, v, z = make_inputs(f"noalloc/{dtype}/{n}", B, Hq, Hkv, Tq, Tk, d, dtype, sinks=with_sinks)
        tq, tk, tv, tz = dev(q), dev(k), dev(v), dev(z)
        sc = scale_for(d)
        o1 = torch.full_like(tq, float("nan"))
        l1 = torch.full((B, Hq, Tq), float("nan"), device="cuda")
        o2 = torch.full_like(tq, float("nan"))
        l2 = torch.full((B, Hq, Tq), float("nan"), device="cuda")
        st = _strides(tq, tk, o1, l1)
        nbytes = fa.fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split)
        assert 0 < nbytes <= fa.FA_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        zp = tz.data_ptr() if tz is not None else None
        say("noalloc", dtype, n, (B, Hq, Hkv, Tq, Tk, d), "split", split)
        s1 = fa.fa_fwd_splitkv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o1.data_ptr(), l1.data_ptr(), B, Hq, Hkv,
                               Tq, Tk, d, sc, qo, 1, window, zp, None, ctypes.byref(st), dt, stream, None, split,
                               ws.data_ptr(), nbytes)
        s2 = fa.fa_fwd_splitkv_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o2.data_ptr(), l2.data_ptr(), B,
                                       Hq, Hkv, Tq, Tk, d, sc, qo, 1, window, zp, None, ctypes.byref(st), dt, stream,
                                       None, split)
        torch.cuda.synchronize()
        assert s1 == fa.FA_OK and s2 == fa.FA_OK, (s1, s2)
        assert np.array_equal(bits(o1), bits(o2)), f"O differs (call {n})"
        assert np.array_equal(bits(l1), bits(l2)), f"LSE differs (call {n})"
        o_ref, l_ref = oracle.attention(q, k, v, scale=sc, q_offset=qo, causal=True, window=window, sinks=z)
        compare(host(o2), host(l2), o_ref, l_ref, dtype, f"noalloc {dtype} call {n}")


def test_noalloc_refuses_more_than_the_scratch():
    B, Hq, Hkv, Tq, Tk, d = 8, 32, 8, 64, 8192, 128
    q = torch.zeros(B, Hq, Tq, d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Hkv, Tk, d, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, Tq), 7.0, device="cuda")
    st = _strides(q, k, o, lse)
    split = 256
    assert fa.fa_splitkv_workspace_bytes(B, Hq, Tq, Tk, d, split) > fa.FA_NOALLOC_SCRATCH_BYTES
    say("noalloc oversize")
    s = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                  Tq, Tk, d, 0.0884, Tk - Tq, 1, 0, None, None, ctypes.byref(st), fa.FA_BF16,
                                  torch.cuda.current_stream().cuda_stream, None, split)
    torch.cuda.synchronize()
    assert s == fa.FA_ESCRATCH
    assert torch.all(o == 7.0) and torch.all(lse == 7.0)
