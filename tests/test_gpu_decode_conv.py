"""GPU parity of the decode step and the standalone conv prologue (through
the C ABI) against the fp64 oracle, including the full decode workload
(256 sequences x 32 heads, 1000 steps in place) on every (sequence, head)
and every step, the conv
cache round trip, and fused prologue == standalone prologue + prefill."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from gpu_common import TOL, check, rel_err, say, to_cpu64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_74_amd as m
    return m


@pytest.mark.parametrize("qkv,gate,Dk,Dv", [
    ("bf16", "bf16", 128, 128), ("bf16", "f32", 64, 32), ("f32", "f32", 16, 16),
    ("f32", "f32", 128, 128), ("bf16", "bf16", 32, 128), ("bf16", "f32", 128, 16),
    ("bf16", "bf16", 64, 128), ("f32", "f32", 128, 64)])
def test_decode_steps(orc, kda, qkv, gate, Dk, Dv):
    say(f"decode qkv={qkv} gate={gate} Dk={Dk} Dv={Dv}")
    N, H = 5, 3
    st = ki.decode_state(N, H, Dk, Dv, device="cuda")
    ref = to_cpu64(st)
    for step in range(6):
        x = ki.decode_step_inputs(N, H, Dk, Dv, step, qkv=qkv, gate=gate,
                                  device="cuda")
        o = kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], st,
                                scale=0.8)
        ro, ref = orc.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                  ref, 0.8)
        torch.cuda.synchronize()
        eo, es = rel_err(o, ro), rel_err(st, ref)
        assert eo <= TOL[qkv] and es <= TOL[qkv], (step, eo, es)
    say(f"  err o={eo:.2e} S={es:.2e}")


def test_decode_workload_1000_steps(orc, kda):
    """The whole decode workload: 1000 in-place steps over 256 sequences x
    32 heads, then o of every (sequence, head) at every step and the final
    state of every (sequence, head) against the oracle, which runs the 1000
    steps as one token sequence per (sequence, head) (32 sequences at a
    time to bound its fp64 copies)."""
    c = ki.workload(ki.DECODE)
    N, H, Dk, Dv, steps = c["N"], c["H"], c["Dk"], c["Dv"], c["steps"]
    say(f"decode workload N{N} H{H} D{Dk} x{steps} steps, all (n, h)")
    st = ki.decode_state(N, H, Dk, Dv, std=c["state_std"], device="cuda")
    s0 = st.detach().cpu()
    outs, inps = [], []
    for step in range(steps):
        x = ki.decode_step_inputs(N, H, Dk, Dv, step, device="cuda")
        outs.append(kda.kda_decode_step(x["q"], x["k"], x["v"], x["g"],
                                        x["beta"], st))
        inps.append(x)
    torch.cuda.synchronize()
    o_all = torch.stack(outs, 1)           # [N, steps, H, Dv]
    del outs
    worst_o = worst_s = 0.0
    for n0 in range(0, N, 32):
        ns = slice(n0, n0 + 32)
        seq = {name: torch.stack([x[name][ns] for x in inps], 1).cpu()
               for name in ("q", "k", "v", "g", "beta")}
        ro, rs = orc.recurrence(seq["q"], seq["k"], seq["v"], seq["g"],
                                seq["beta"], s0[ns])
        worst_o = max(worst_o, check(f"o n{n0}-{n0 + 31}", o_all[ns], ro,
                                     2e-2, (0, 2))[1])
        worst_s = max(worst_s, check(f"S n{n0}-{n0 + 31}", st[ns], rs, 2e-2,
                                     (0, 1))[1])
        del seq, ro, rs
    say(f"  worst (n, h) slab over all steps: o {worst_o:.2e}, "
        f"S {worst_s:.2e}")


@pytest.mark.parametrize("qkv,gate,Dk,Dv,L", [
    ("bf16", "bf16", 128, 128, 2), ("bf16", "f32", 64, 128, 5),
    ("f32", "f32", 32, 16, 3), ("f32", "f32", 128, 128, 1),
    ("bf16", "bf16", 16, 64, 8)])
def test_decode_tokens(orc, kda, qkv, gate, Dk, Dv, L):
    """L tokens per sequence in one call against the oracle's token loop:
    outputs, final state, and the state after every token; the input state
    is left alone out of place, and in place gives the same bits."""
    say(f"decode tokens qkv={qkv} gate={gate} Dk={Dk} Dv={Dv} L={L}")
    N, H = 6, 3
    x = ki.prefill_inputs(N, L, H, Dk, Dv, qkv=qkv, gate=gate, seed=31 + L,
                          device="cuda", with_s0=True)
    s_in = x["s0"].clone()
    o, s_out, ts = kda.kda_decode_tokens(x["q"], x["k"], x["v"], x["g"],
                                         x["beta"], s_in, token_states=True,
                                         scale=0.7)
    torch.cuda.synchronize()
    ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"],
                            x["s0"], 0.7)
    eo, es = rel_err(o, ro), rel_err(s_out, rs)
    say(f"  err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]
    for t in range(L):
        cut = {n: x[n][:, :t + 1] for n in ("q", "k", "v", "g", "beta")}
        _, rst = orc.recurrence(cut["q"], cut["k"], cut["v"], cut["g"],
                                cut["beta"], x["s0"], 0.7)
        assert rel_err(ts[:, t], rst) <= TOL[qkv], t
    assert torch.equal(s_in, x["s0"])
    st2 = x["s0"].clone()
    o2, s2, _ = kda.kda_decode_tokens(x["q"], x["k"], x["v"], x["g"],
                                      x["beta"], st2, state_out=st2,
                                      scale=0.7)
    torch.cuda.synchronize()
    assert s2 is st2 and torch.equal(o2, o) and torch.equal(st2, s_out)


@pytest.mark.parametrize("dt,Dk,Dv,W,T,hist", [
    ("bf16", 128, 128, 4, 300, False), ("bf16", 128, 128, 4, 300, True),
    ("f32", 16, 16, 2, 70, True), ("f32", 64, 64, 3, 1, True),
    ("bf16", 32, 32, 4, 65, False),
    # d_k != d_v: the streams' lane groups differ in size and run length
    ("bf16", 128, 64, 4, 700, True), ("f32", 32, 128, 3, 200, False),
    ("bf16", 16, 128, 2, 1100, True)])
def test_conv_prologue(orc, kda, dt, Dk, Dv, W, T, hist):
    say(f"conv prologue dt={dt} Dk={Dk} Dv={Dv} W={W} T={T} hist={hist}")
    B, H = 2, 3
    Dm = max(Dk, Dv)
    x = ki.prefill_inputs(B, T, H, Dk, Dv, qkv=dt, conv_width=W, seed=21,
                          device="cuda")
    state = None
    old = None
    if hist:
        state = torch.randn((B, 3, H * Dm, W - 1), device="cuda")
        old = to_cpu64(state)
    q, k, v = kda.kda_conv_prologue(x["xq"], x["xk"], x["xv"], x["wq"],
                                    x["wk"], x["wv"], H=H, Dk=Dk, Dv=Dv,
                                    conv_state=state, eps=1e-6)
    torch.cuda.synchronize()
    Ds = (Dk, Dk, Dv)
    hist_in = None if old is None else tuple(
        old[:, i, :H * Ds[i]] for i in range(3))
    rq, rk, rv, rh = orc.conv_prologue(x["xq"], x["xk"], x["xv"], x["wq"],
                                       x["wk"], x["wv"], H, Dk, Dv, 1e-6, True,
                                       hist_in)
    for name, a, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        e = rel_err(a, r)
        assert e <= TOL[dt], (name, e)
    if hist:
        for i in range(3):
            assert rel_err(state[:, i, :H * Ds[i]], rh[i]) <= 1e-6


def test_fused_prologue_matches_standalone(kda):
    x = ki.prefill_inputs(2, 250, 4, 128, 128, conv_width=4, seed=33,
                          device="cuda")
    conv = dict(xq=x["xq"], xk=x["xk"], xv=x["xv"], wq=x["wq"], wk=x["wk"],
                wv=x["wv"], width=4, l2norm_qk=True, eps=1e-6)
    of, sf = kda.kda_prefill(None, None, None, x["g"], x["beta"], chunk=64,
                             conv=conv)
    q, k, v = kda.kda_conv_prologue(x["xq"], x["xk"], x["xv"], x["wq"],
                                    x["wk"], x["wv"], H=4, Dk=128, Dv=128)
    ou, su = kda.kda_prefill(q, k, v, x["g"], x["beta"], chunk=64)
    torch.cuda.synchronize()
    assert rel_err(of, to_cpu64(ou)) < 2e-2
    assert rel_err(sf, to_cpu64(su)) < 2e-2


def _cut(x, a, b):
    return {n: x[n][:, a:b] for n in ("xq", "xk", "xv", "g", "beta")}


@pytest.mark.parametrize("qkv,gate,Dk,Dv,W,splits,hist,pingpong", [
    ("bf16", "bf16", 128, 128, 4, (1, 1, 1), True, False),
    ("bf16", "f32", 64, 128, 3, (3, 1), True, False),
    ("f32", "f32", 32, 16, 2, (5,), False, False),
    ("f32", "f32", 128, 64, 4, (1, 2), False, False),
    ("bf16", "bf16", 128, 32, 4, (2, 1, 4), True, False),
    ("f32", "f32", 16, 16, 3, (1, 1), True, False),
    ("bf16", "bf16", 128, 128, 4, (1, 1, 1), True, True),
    ("bf16", "f32", 64, 128, 3, (3, 1, 1), False, True),
    ("bf16", "bf16", 128, 64, 2, (1, 2, 1), True, True),
    ("f32", "f32", 32, 128, 4, (2, 1), False, True),
    ("f32", "f32", 16, 16, 3, (1, 1, 1), True, True)])
def test_decode_tokens_conv(orc, kda, qkv, gate, Dk, Dv, W, splits, hist,
                            pingpong):
    """Decode calls with the conv prologue fused (raw projections in), the
    conv history and the recurrent state carried from call to call, against
    the oracle's conv + recurrence over the whole token run: outputs, final
    state and the rolled conv history.  pingpong: each call writes the
    rolled history into the other of two buffers (conv_state_out) instead
    of rolling it in place; without a starting history the first call reads
    zeros and still writes one."""
    say(f"decode tokens + conv qkv={qkv} gate={gate} Dk={Dk} Dv={Dv} W={W} "
        f"splits={splits} hist={hist} pingpong={pingpong}")
    N, H, T = 4, 3, sum(splits)
    Dm = max(Dk, Dv)
    x = ki.prefill_inputs(N, T, H, Dk, Dv, qkv=qkv, gate=gate, conv_width=W,
                          seed=41 + T, device="cuda", with_s0=True)
    cache = None
    hist_in = None
    if hist:
        cache = torch.randn((N, 3, H * Dm, W - 1), device="cuda")
        old = to_cpu64(cache)
        hist_in = tuple(old[:, i, :H * D] for i, D in enumerate((Dk, Dk, Dv)))
    spare = (torch.full((N, 3, H * Dm, W - 1), float("nan"), device="cuda")
             if pingpong else None)
    st = x["s0"].clone()
    outs, t0 = [], 0
    for L in splits:
        c = _cut(x, t0, t0 + L)
        conv = dict(xq=c["xq"].contiguous(), xk=c["xk"].contiguous(),
                    xv=c["xv"].contiguous(), wq=x["wq"], wk=x["wk"],
                    wv=x["wv"], width=W, l2norm_qk=True, eps=1e-6)
        o, _, _ = kda.kda_decode_tokens(None, None, None,
                                        c["g"].contiguous(),
                                        c["beta"].contiguous(), st,
                                        state_out=st, scale=0.6, conv=conv,
                                        conv_state=cache,
                                        conv_state_out=spare)
        outs.append(o)
        t0 += L
        if pingpong:
            cache, spare = spare, cache
            if spare is None:
                spare = torch.full_like(cache, float("nan"))
            else:
                spare.fill_(float("nan"))
        if cache is None:
            break   # without a history only one call continues correctly
    torch.cuda.synchronize()
    T = t0
    rq, rk, rv, rh = orc.conv_prologue(x["xq"][:, :T], x["xk"][:, :T],
                                       x["xv"][:, :T], x["wq"], x["wk"],
                                       x["wv"], H, Dk, Dv, 1e-6, True, hist_in)
    ro, rs = orc.recurrence(rq, rk, rv, x["g"][:, :T], x["beta"][:, :T],
                            x["s0"], 0.6)
    eo, es = rel_err(torch.cat(outs, 1), ro), rel_err(st, rs)
    say(f"  err o={eo:.2e} S={es:.2e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]
    if cache is not None:
        for i, D in enumerate((Dk, Dk, Dv)):
            assert rel_err(cache[:, i, :H * D], rh[i]) <= 1e-6, i


def test_conv_state_out_same_buffer_is_in_place(kda):
    """conv_state_out naming the conv_state buffer itself means in place:
    the same outputs, state and rolled history as leaving it out."""
    N, H, L, D, W = 3, 2, 2, 64, 4
    x = ki.prefill_inputs(N, L, H, D, D, qkv="bf16", gate="bf16",
                          conv_width=W, seed=77, device="cuda", with_s0=True)
    conv = dict(xq=x["xq"], xk=x["xk"], xv=x["xv"], wq=x["wq"], wk=x["wk"],
                wv=x["wv"], width=W, l2norm_qk=True, eps=1e-6)
    h0 = torch.randn((N, 3, H * D, W - 1), device="cuda")
    ha, hb = h0.clone(), h0.clone()
    oa, sa, _ = kda.kda_decode_tokens(None, None, None, x["g"], x["beta"],
                                      x["s0"], conv=conv, conv_state=ha)
    ob, sb, _ = kda.kda_decode_tokens(None, None, None, x["g"], x["beta"],
                                      x["s0"], conv=conv, conv_state=hb,
                                      conv_state_out=hb)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(sa, sb)
    assert torch.equal(ha, hb) and not torch.equal(ha, h0)
