"""GPU parity of the chunked backward (kda_prefill_backward through the C
ABI) against the oracle's fp64 token-loop gradient: every head size and
chunk size, several chunks with a ragged tail, a start state and an
end-state gradient, per-channel and per-head gates, beta up to 2 and -inf
gates; all six gradients (q, k, v, g, beta, S0) within the path's
tolerance."""
import pytest
import torch

import kda_inputs as ki
from gpu_common import TOL, check, rel_err, say, to_cpu64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "ds0")


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_74_amd as m
    return m


def _check(orc, kda, x, qkv, C, scale=0.9, head_gate=False, tol=None):
    B, T, H, Dk = x["q"].shape
    Dv = x["v"].shape[-1]
    gen = torch.Generator(device="cuda").manual_seed(1234 + T + C)
    do = torch.randn((B, T, H, Dv), generator=gen, device="cuda").to(x["q"].dtype)
    dsT = torch.randn((B, H, Dk, Dv), generator=gen, device="cuda")
    got = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                   do, s0=x["s0"], dsT=dsT, chunk=C,
                                   scale=scale)
    torch.cuda.synchronize()
    ref = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["s0"],
                       scale, do, dsT)
    tol = TOL[qkv] if tol is None else tol
    errs = {n: rel_err(a, r) for n, a, r in zip(NAMES, got, ref)}
    say("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol, (n, e)


CASES = []
for D in (16, 32, 64, 128):
    for C in (16, 32, 64):
        CASES.append(("f32", "f32", D, D, C))
        CASES.append(("bf16", "f32", D, D, C))
CASES += [("bf16", "bf16", 128, 128, 64), ("bf16", "f32", 64, 128, 64),
          ("f32", "f32", 32, 64, 32)]


@pytest.mark.parametrize("qkv,gate,Dk,Dv,C", CASES)
def test_backward_small(orc, kda, qkv, gate, Dk, Dv, C):
    say(f"backward qkv={qkv} gate={gate} Dk={Dk} Dv={Dv} C={C}")
    x = ki.prefill_inputs(2, 3 * C + 7, 2, Dk, Dv, qkv=qkv, gate=gate,
                          seed=81 + Dk + C, device="cuda", with_s0=True)
    _check(orc, kda, x, qkv, C)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_backward_per_head_gate(orc, kda, qkv):
    say(f"backward per-head gate qkv={qkv}")
    x = ki.prefill_inputs(1, 100, 3, 64, 64, qkv=qkv, seed=91, device="cuda",
                          with_s0=True, gate_per_head=True)
    _check(orc, kda, x, qkv, 32)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_backward_beta_to_two_and_forgetting(orc, kda, qkv):
    say(f"backward beta in (0,2), -inf gates qkv={qkv}")
    x = ki.prefill_inputs(1, 90, 2, 32, 32, qkv=qkv, seed=92, device="cuda",
                          with_s0=True, beta_max=2.0)
    x["g"][:, 10] = -float("inf")
    x["g"][:, 40, :, 5] = -float("inf")
    _check(orc, kda, x, qkv, 32)


def test_backward_model_shaped_t8192(orc, kda):
    """The headline shape (B1 T8192 H32 D128 C64, bf16 q/k/v, fp32 g/beta)
    in one launch; the oracle's gradient on every head."""
    c = ki.workload(ki.PREFILL)
    say("backward B1 T8192 H32 D128, all heads")
    x = ki.workload_prefill_inputs(ki.PREFILL, device="cuda")
    B, T, H, D = c["B"], c["T"], c["H"], c["Dk"]
    gen = torch.Generator(device="cuda").manual_seed(99)
    do = torch.randn((B, T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    got = kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                   do, chunk=c["chunk"])
    torch.cuda.synchronize()
    ref = orc.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], None, 1.0,
                       do)
    for n, a, r in zip(NAMES, got, ref):
        check(n, a, r, TOL["bf16"], (0, 1) if n == "ds0" else (0, 2))
