"""moe_forward_noalloc (the forward pass on the library's own per-GPU
scratch, for callers that cannot allocate) through the C ABI, against
moe_forward on a caller workspace: the same kernels on the same inputs, so
the outputs agree bit for bit. Two calls in a row, the second smaller (the
scratch keeps the first call's contents), a 4-bit decode call, and a call
too large for the scratch refused before any launch."""

import pytest
import torch

import mixture_experts_routed_route_amd as moe
import workloads as W
from helpers import gpu_plan, say, to_dev

pytestmark = pytest.mark.gpu


def _both(wl):
    p = gpu_plan(wl)
    x = wl["x"].cuda()
    w = [to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down")]
    ref = moe.moe_forward(p, x, *w)
    got = moe.moe_forward_noalloc(p, x, *w)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_forward_twice_then_smaller():
    for wl in (W.config(5, T=128), W.config(6, T=4)):
        nbytes = moe.moe_forward_workspace_bytes(
            gpu_plan(wl), wl["D"], wl["F"], moe.MOE_BF16, moe.MOE_BF16)
        assert 0 < nbytes <= moe.MOE_NOALLOC_SCRATCH_BYTES
        say(f"no-alloc forward {wl['name']} ({nbytes} workspace bytes)")
        ref, got = _both(wl)
        assert torch.equal(ref, got)


def test_noalloc_q4_decode_and_repeat():
    wl = W.config(7, T=8)
    say(f"no-alloc forward {wl['name']}")
    ref, got = _both(wl)
    assert torch.equal(ref, got)
    ref2, got2 = _both(wl)
    assert torch.equal(got2, got)


def test_noalloc_refuses_a_call_beyond_the_scratch():
    wl = W.config(3)
    p = gpu_plan(wl)
    nbytes = moe.moe_forward_workspace_bytes(p, wl["D"], wl["F"], moe.MOE_BF16,
                                             moe.MOE_BF16)
    assert nbytes > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = wl["x"].cuda()
    w = [to_dev(wl[n]) for n in ("w_gate", "w_up", "w_down")]
    y = torch.full((wl["T"], wl["D"]), 7.0, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(p, x, *w, out=y)
    assert e.value.status == moe.MOE_EWORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)           # nothing was launched
