"""The Python binding rejects, before any launch, tensors that the kernels could not use:
host tensors for sinks, mask, out, lse or the workspace (their pointers would reach a kernel),
and an out buffer whose dtype or shape does not match the output (the kernels would write
outside it).  The outputs passed in keep their contents."""
import pytest
import torch

import flashattention_forward_flash_amd as fa
from gpu_common import say

pytestmark = pytest.mark.gpu


def _inputs(dtype=torch.float32, B=1, Hq=4, Hkv=2, T=40, d=64):
    g = torch.Generator(device="cpu").manual_seed(7)
    q = torch.randn(B, Hq, T, d, generator=g).to(dtype).cuda()
    k = torch.randn(B, Hkv, T, d, generator=g).to(dtype).cuda()
    v = torch.randn(B, Hkv, T, d, generator=g).to(dtype).cuda()
    return q, k, v


@pytest.mark.parametrize("what", ["sinks", "mask", "out", "lse", "out_dtype", "out_shape"])
def test_forward_rejects_unusable_tensors(what):
    q, k, v = _inputs()
    B, Hq, T, d = q.shape
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, T), 7.0, device="cuda")
    kw = dict(out=out, lse=lse)
    if what == "sinks":
        kw["sinks"] = torch.zeros(Hq)
    elif what == "mask":
        kw["mask"] = torch.zeros(T, T)
    elif what == "out":
        kw["out"] = torch.zeros(B, Hq, T, d)
    elif what == "lse":
        kw["lse"] = torch.zeros(B, Hq, T)
    elif what == "out_dtype":
        kw["out"] = torch.zeros(B, Hq, T, d, dtype=torch.bfloat16, device="cuda")
    else:
        kw["out"] = torch.zeros(B, Hq, T - 1, d, device="cuda")
    say("binding rejects", what)
    with pytest.raises(fa.FaError):
        fa.forward(q, k, v, causal=True, **kw)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_splitkv_rejects_a_host_workspace():
    q, k, v = _inputs()
    out = torch.full_like(q, 7.0)
    say("binding rejects host workspace")
    with pytest.raises(fa.FaError):
        fa.forward_splitkv(q, k, v, split_keys=64, workspace=torch.zeros(1 << 20, dtype=torch.uint8), out=out)
    with pytest.raises(fa.FaError):
        fa.forward_splitkv(q, k, v, split_keys=64, workspace=torch.zeros(1 << 20, dtype=torch.uint8), out=out,
                           softcap=5.0)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("what", ["sinks", "out", "out_shape", "workspace"])
def test_varlen_rejects_unusable_tensors(what):
    Hq, Hkv, d, tot = 4, 2, 64, 50
    g = torch.Generator(device="cpu").manual_seed(3)
    q = torch.randn(tot, Hq, d, generator=g).cuda()
    k = torch.randn(tot, Hkv, d, generator=g).cuda()
    v = torch.randn(tot, Hkv, d, generator=g).cuda()
    cu = torch.tensor([0, 20, 50], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    kw = dict(out=out)
    if what == "sinks":
        kw["sinks"] = torch.zeros(Hq)
    elif what == "out":
        kw["out"] = torch.zeros(tot, Hq, d)
    elif what == "out_shape":
        kw["out"] = torch.zeros(tot, Hq, d + 64, device="cuda")
    else:
        kw.update(split_keys=64, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    say("varlen binding rejects", what)
    with pytest.raises(fa.FaError):
        fa.forward_varlen(q, k, v, cu, cu, 30, 30, causal=True, **kw)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
