"""kda_prefill_noalloc (the prefill on the library's fixed scratch
workspace, for callers that cannot allocate) through the C ABI against
kda_prefill on a caller workspace: two calls in a row, the second smaller
than the first, each equal to kda_prefill bit for bit (same kernels, same
arithmetic) and within the parity bar of the oracle; plus the rejection of
a request larger than the scratch."""
import pytest
import torch

import kda_inputs as ki
from gpu_common import TOL, check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_74_amd as m
    return m


def _pair(kda, x, chunk, s0):
    B, T, H, Dk = x["q"].shape
    Dv = x["v"].shape[-1]
    o1 = torch.full((B, T, H, Dv), float("nan"), dtype=x["q"].dtype,
                    device="cuda")
    s1 = torch.full((B, H, Dk, Dv), float("nan"), device="cuda")
    kda.kda_prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=s0,
                            chunk=chunk, scale=0.9, o=o1, s_out=s1)
    o2, s2 = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                             s0=s0, chunk=chunk, scale=0.9)
    torch.cuda.synchronize()
    return o1, s1, o2, s2


@pytest.mark.parametrize("qkv,D,C,shapes", [
    ("bf16", 128, 64, [(1, 1000, 32), (2, 77, 3)]),
    ("f32", 32, 32, [(3, 300, 4), (1, 41, 2)])])
def test_noalloc_matches_prefill_twice(orc, kda, qkv, D, C, shapes):
    for i, (B, T, H) in enumerate(shapes):
        say(f"noalloc call {i}: qkv={qkv} B{B} T{T} H{H} D{D} C{C}")
        x = ki.prefill_inputs(B, T, H, D, D, qkv=qkv, seed=300 + i + D,
                              device="cuda", with_s0=True)
        assert kda.kda_prefill_workspace_size(
            B, T, H, D, D, C, x["q"].dtype) <= kda.KDA_NOALLOC_SCRATCH_BYTES
        o1, s1, o2, s2 = _pair(kda, x, C, x["s0"])
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
        ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                x["s0"], 0.9)
        check("o", o1, ro, TOL[qkv], (0, 2))
        check("S", s1, rs, TOL[qkv], (0, 1))


def test_noalloc_rejects_oversize(kda):
    x = ki.prefill_inputs(1, 2048, 32, 128, 128, device="cuda")
    need = kda.kda_prefill_workspace_size(1, 2048, 32, 128, 128, 64,
                                          torch.bfloat16)
    assert need > kda.KDA_NOALLOC_SCRATCH_BYTES
    o = torch.full((1, 2048, 32, 128), 7.0, dtype=torch.bfloat16,
                   device="cuda")
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                o=o)
    assert ei.value.status == kda.KDA_ENOSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing launched
