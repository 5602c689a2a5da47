"""GPU parity of the two variants of the forward against the fp64 oracle:
the per-head (scalar) gate of Gated DeltaNet, passed as g [B,T,H] with the
KDA_GATE_HEAD flag, and beta in (0,2) ("negative eigenvalues").  For the
per-head gate the result is also compared with the per-channel path fed
the same gate repeated over the key channels: bit for bit where both run
the same kernels, within the bar where the per-head gate takes its own
chunk prep (bf16 q/k/v, d_k = 128, chunk 64, no conv), whose algebra
applies the scalar decay to the Gram products instead of the operands."""
import pytest
import torch

import kda_inputs as ki
from gpu_common import TOL, check, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_74_amd as m
    return m


def _rep(g, Dk):
    return g[..., None].expand(*g.shape, Dk).contiguous()


def _own_prep(qkv, Dk, C, conv=False):
    """whether the per-head gate runs the scalar-gate chunk prep"""
    return qkv == "bf16" and Dk == 128 and C == 64 and not conv


def _same(qkv, Dk, C, o, o2, s, s2):
    if _own_prep(qkv, Dk, C):
        assert rel_err(o, o2.double().cpu().numpy()) <= TOL[qkv]
        assert rel_err(s, s2.double().cpu().numpy()) <= TOL[qkv]
    else:
        assert torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("qkv,gate,Dk,Dv,C,T", [
    ("f32", "f32", 16, 16, 16, 70), ("bf16", "f32", 128, 128, 64, 300),
    ("bf16", "bf16", 64, 32, 32, 129), ("f32", "f32", 128, 64, 32, 100),
    ("bf16", "f32", 32, 128, 16, 47), ("bf16", "bf16", 128, 128, 64, 200),
    ("bf16", "f32", 128, 64, 64, 129), ("bf16", "bf16", 128, 32, 64, 1),
    ("bf16", "f32", 128, 16, 64, 64)])
def test_prefill_per_head_gate(orc, kda, qkv, gate, Dk, Dv, C, T):
    say(f"prefill per-head gate qkv={qkv} gate={gate} Dk={Dk} Dv={Dv} C={C} "
        f"T={T}")
    x = ki.prefill_inputs(2, T, 3, Dk, Dv, qkv=qkv, gate=gate, seed=61 + C,
                          device="cuda", with_s0=True, gate_per_head=True)
    assert x["g"].shape == (2, T, 3)
    o, s = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                           s0=x["s0"], chunk=C, scale=0.8)
    o2, s2 = kda.kda_prefill(x["q"], x["k"], x["v"], _rep(x["g"], Dk),
                             x["beta"], s0=x["s0"], chunk=C, scale=0.8)
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"],
                            x["s0"], 0.8)
    check("o", o, ro, TOL[qkv], (0, 2))
    check("S", s, rs, TOL[qkv], (0, 1))
    _same(qkv, Dk, C, o, o2, s, s2)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_prefill_per_head_gate_forget(orc, kda, qkv):
    """g = -inf and very negative per-head gates: the diagonal blocks take
    the exact running-product path, which reads the per-head gate too."""
    say(f"prefill per-head gate, forgetting extremes qkv={qkv}")
    x = ki.prefill_inputs(1, 150, 2, 32, 32, qkv=qkv, gate="f32", seed=66,
                          device="cuda", with_s0=True, gate_per_head=True)
    g = x["g"]
    g[:, 5] = -float("inf")
    g[:, 31] = -float("inf")
    g[:, 100:108] = -60.0
    o, s = kda.kda_prefill(x["q"], x["k"], x["v"], g, x["beta"], s0=x["s0"],
                           chunk=64)
    o2, s2 = kda.kda_prefill(x["q"], x["k"], x["v"], _rep(g, 32), x["beta"],
                             s0=x["s0"], chunk=64)
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], g, x["beta"], x["s0"])
    eo, es = rel_err(o, ro), rel_err(s, rs)
    say(f"  err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]
    assert torch.equal(o, o2) and torch.equal(s, s2)


@pytest.mark.parametrize("gate", ["f32", "bf16"])
def test_prefill_per_head_gate_forget_d128(orc, kda, gate):
    """The scalar-gate chunk prep with -inf and -60 gates at B = 2, d = 128,
    chunk 64 and a ragged tail: its decay products have no ratio and no
    fallback, so a forget anywhere (on a sub-chunk boundary, in the tail,
    in one batch row only) must come out exact."""
    say(f"prefill per-head gate d128, forgetting extremes gate={gate}")
    x = ki.prefill_inputs(2, 200, 3, 128, 128, qkv="bf16", gate=gate,
                          seed=69, device="cuda", with_s0=True,
                          gate_per_head=True)
    g = x["g"]
    g[1, 5] = -float("inf")
    g[0, 15] = -float("inf")      # last token of a sub-chunk
    g[:, 16] = -float("inf")      # first token of the next
    g[0, 63] = -float("inf")      # last token of a chunk
    g[:, 100:108] = -60.0
    g[1, 193:] = -float("inf")    # in the ragged tail
    o, s = kda.kda_prefill(x["q"], x["k"], x["v"], g, x["beta"], s0=x["s0"],
                           chunk=64, scale=0.8)
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], g, x["beta"], x["s0"],
                            0.8)
    check("o", o, ro, TOL["bf16"], (0, 2))
    check("S", s, rs, TOL["bf16"], (0, 1))
    # every gate -inf: o_t = scale beta_t (q_t . k_t) v_t
    g.fill_(-float("inf"))
    o, _ = kda.kda_prefill(x["q"], x["k"], x["v"], g, x["beta"], s0=x["s0"],
                           chunk=64, scale=0.8)
    torch.cuda.synchronize()
    ro, _ = orc.recurrence(x["q"], x["k"], x["v"], g, x["beta"], x["s0"], 0.8)
    check("o (all forget)", o, ro, TOL["bf16"], (0, 2))


def test_prefill_per_head_gate_t8192(orc, kda):
    """The headline shape with one gate per token-head, every head."""
    c = ki.workload(ki.PREFILL)
    say("prefill per-head gate B1 T8192 H32 D128 C64, all heads")
    x = ki.prefill_inputs(c["B"], c["T"], c["H"], c["Dk"], c["Dv"],
                          qkv=c["qkv"], gate=c["gate"],
                          seed=ki.SEED_BASE + 11, device="cuda",
                          gate_per_head=True)
    o, s = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                           chunk=c["chunk"])
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check("o", o, ro, TOL["bf16"], (0, 2))
    check("S", s, rs, TOL["bf16"], (0, 1))


def test_prefill_per_head_gate_conv(orc, kda):
    say("prefill per-head gate with the fused conv")
    B, T, H, D = 2, 200, 3, 64
    x = ki.prefill_inputs(B, T, H, D, D, conv_width=4, seed=67, device="cuda",
                          gate_per_head=True)
    conv = dict(xq=x["xq"], xk=x["xk"], xv=x["xv"], wq=x["wq"], wk=x["wk"],
                wv=x["wv"], width=4, l2norm_qk=True, eps=1e-6)
    o, s = kda.kda_prefill(None, None, None, x["g"], x["beta"], chunk=64,
                           conv=conv)
    torch.cuda.synchronize()
    rq, rk, rv, _ = orc.conv_prologue(x["xq"], x["xk"], x["xv"], x["wq"],
                                      x["wk"], x["wv"], H, D, D, 1e-6, True)
    ro, rs = orc.recurrence(rq, rk, rv, x["g"], x["beta"])
    assert rel_err(o, ro) <= TOL["bf16"] and rel_err(s, rs) <= TOL["bf16"]


@pytest.mark.parametrize("qkv,gate", [("bf16", "bf16"), ("f32", "f32")])
def test_decode_per_head_gate(orc, kda, qkv, gate):
    say(f"decode per-head gate qkv={qkv}")
    N, H, Dk, Dv = 5, 3, 128, 64
    st = ki.decode_state(N, H, Dk, Dv, device="cuda")
    st2 = st.clone()
    ref = st.detach().cpu().double().numpy()
    for step in range(4):
        x = ki.decode_step_inputs(N, H, Dk, Dv, step, qkv=qkv, gate=gate,
                                  device="cuda", gate_per_head=True)
        o = kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], st)
        o2 = kda.kda_decode_step(x["q"], x["k"], x["v"], _rep(x["g"], Dk),
                                 x["beta"], st2)
        ro, ref = orc.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                  ref)
        torch.cuda.synchronize()
        assert rel_err(o, ro) <= TOL[qkv] and rel_err(st, ref) <= TOL[qkv]
        assert torch.equal(o, o2) and torch.equal(st, st2)
    # several tokens per call
    L = 3
    xt = ki.prefill_inputs(N, L, H, Dk, Dv, qkv=qkv, gate=gate, seed=68,
                           device="cuda", with_s0=True, gate_per_head=True)
    o, s, _ = kda.kda_decode_tokens(xt["q"], xt["k"], xt["v"], xt["g"],
                                    xt["beta"], xt["s0"])
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(xt["q"], xt["k"], xt["v"], xt["g"], xt["beta"],
                            xt["s0"])
    assert rel_err(o, ro) <= TOL[qkv] and rel_err(s, rs) <= TOL[qkv]


@pytest.mark.parametrize("qkv,gate,Dk,Dv,C", [
    ("f32", "f32", 32, 32, 16), ("bf16", "f32", 128, 128, 64),
    ("bf16", "bf16", 64, 64, 32)])
def test_prefill_beta_to_two(orc, kda, qkv, gate, Dk, Dv, C):
    """beta = 2 sigmoid(z) in (0,2): the WY/UT algebra holds for any beta,
    the kernels must not assume beta < 1."""
    say(f"prefill beta in (0,2) qkv={qkv} Dk={Dk} C={C}")
    x = ki.prefill_inputs(2, 3 * C + 5, 3, Dk, Dv, qkv=qkv, gate=gate,
                          seed=71 + C, device="cuda", with_s0=True,
                          beta_max=2.0)
    assert float(x["beta"].max()) > 1.0
    o, s = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                           s0=x["s0"], chunk=C)
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"],
                            x["s0"])
    eo, es = rel_err(o, ro), rel_err(s, rs)
    say(f"  err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]


def test_decode_beta_to_two(orc, kda):
    say("decode beta in (0,2)")
    N, H, D = 6, 4, 128
    st = ki.decode_state(N, H, D, D, device="cuda")
    ref = st.detach().cpu().double().numpy()
    for step in range(5):
        x = ki.decode_step_inputs(N, H, D, D, step, device="cuda",
                                  beta_max=2.0)
        o = kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], st)
        ro, ref = orc.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                  ref)
        torch.cuda.synchronize()
        assert rel_err(o, ro) <= TOL["bf16"] and rel_err(st, ref) <= TOL["bf16"]
