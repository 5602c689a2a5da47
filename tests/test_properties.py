"""Property tests over drawn shapes, seeds and chunkings (hypothesis, CPU):
invariances the oracle and the chunked algebra must hold for any input, the
input recipe's own guarantees, and the Python binding's refusal of
mismatched tensors.  Small sizes and a bounded number of examples keep the
suite within seconds."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import kda_inputs as ki
from chunk_form import chunked_forward, chunked_forward_scalar_gate
from oracle_pins import _rand

SET = settings(max_examples=25, deadline=None,
               suppress_health_check=[HealthCheck.function_scoped_fixture])


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@SET
@given(T=st.integers(2, 40), H=st.integers(1, 3), Dk=st.integers(1, 6),
       Dv=st.integers(1, 5), seed=st.integers(0, 2 ** 16),
       frac=st.floats(0.05, 0.95), scale=st.floats(0.25, 2.0))
def test_oracle_split_sequence(orc, T, H, Dk, Dv, seed, frac, scale):
    """Running the token loop over [0, t) and then over [t, T) from the
    carried state equals one run over [0, T): the recurrence has no
    hidden state beyond S."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, s0 = _rand(rng, 1, T, H, Dk, Dv)
    t = max(1, min(T - 1, int(frac * T)))
    o, s = orc.recurrence(q, k, v, g, beta, s0, scale)
    cut = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    o1, s1 = orc.recurrence(cut(q, 0, t), cut(k, 0, t), cut(v, 0, t),
                            cut(g, 0, t), cut(beta, 0, t), s0, scale)
    o2, s2 = orc.recurrence(cut(q, t, T), cut(k, t, T), cut(v, t, T),
                            cut(g, t, T), cut(beta, t, T), s1, scale)
    assert np.array_equal(np.concatenate([o1, o2], 1), o)
    assert np.array_equal(s2, s)


@SET
@given(T=st.integers(1, 70), Dk=st.integers(1, 8), Dv=st.integers(1, 6),
       C=st.sampled_from([1, 2, 4, 8, 16, 32, 64]),
       bsd=st.sampled_from([1, 2, 4]), seed=st.integers(0, 2 ** 16),
       forget=st.booleans())
def test_chunk_form_any_chunking(orc, T, Dk, Dv, C, bsd, seed, forget):
    """The chunked WY/UT form equals the token loop for any chunk and
    sub-chunk length, ragged tails and (optionally) -inf gates."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, s0 = _rand(rng, 1, T, 1, Dk, Dv)
    if forget:
        g[0, rng.integers(0, T), 0, :] = -np.inf
    bs = max(1, C // bsd)
    o, s = orc.recurrence(q, k, v, g, beta, s0, 0.9)
    oc, sc = chunked_forward(q, k, v, g, beta, s0, 0.9, C=C, bs=bs)
    assert _rel(oc, o) < 1e-10 and _rel(sc, s) < 1e-10


@SET
@given(T=st.integers(1, 70), Dk=st.integers(1, 8), Dv=st.integers(1, 6),
       C=st.sampled_from([1, 4, 16, 64]), seed=st.integers(0, 2 ** 16),
       forget=st.booleans())
def test_scalar_gate_chunk_form(orc, T, Dk, Dv, C, seed, forget):
    """The per-head-gate arrangement equals the token loop with g [B,T,H]."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, s0 = _rand(rng, 1, T, 1, Dk, Dv)
    gh = g[..., 0].copy()
    if forget:
        gh[0, rng.integers(0, T), 0] = -np.inf
    o, s = orc.recurrence(q, k, v, gh, beta, s0, 1.1)
    oc, sc = chunked_forward_scalar_gate(q, k, v, gh, beta, s0, 1.1, C=C)
    assert _rel(oc, o) < 1e-10 and _rel(sc, s) < 1e-10


@SET
@given(B=st.integers(1, 2), T=st.integers(1, 9), H=st.integers(1, 3),
       D=st.sampled_from([16, 32]), seed=st.integers(0, 2 ** 16),
       head=st.booleans(), beta_max=st.sampled_from([1.0, 2.0]))
def test_input_recipe(B, T, H, D, seed, head, beta_max):
    """The drawn inputs keep the recipe's guarantees: q and k of unit length
    per head, g <= 0, beta in (0, beta_max), the stored dtypes."""
    x = ki.prefill_inputs(B, T, H, D, D, qkv="f32", gate="f32", seed=seed,
                          gate_per_head=head, beta_max=beta_max)
    for n in ("q", "k"):
        norms = x[n].double().norm(dim=-1)
        assert torch.allclose(norms, torch.ones_like(norms), atol=1e-5)
    assert bool((x["g"] <= 0).all())
    assert x["g"].shape == ((B, T, H) if head else (B, T, H, D))
    assert bool((x["beta"] > 0).all()) and bool((x["beta"] < beta_max).all())


@SET
@given(B=st.integers(1, 2), T=st.integers(1, 5), H=st.integers(1, 3),
       Dk=st.sampled_from([16, 32]), Dv=st.sampled_from([16, 32]),
       which=st.sampled_from(["k", "v", "g", "beta"]),
       bump=st.sampled_from([(-1, 1), (1, 1), (-1, 2)]))
def test_binding_refuses_mismatched_shapes(B, T, H, Dk, Dv, which, bump):
    """A tensor whose extent along any axis differs from what q and g imply
    is refused with ValueError before any pointer reaches the library."""
    import gated_delta_rule_74_amd as kda
    shapes = dict(q=(B, T, H, Dk), k=(B, T, H, Dk), v=(B, T, H, Dv),
                  g=(B, T, H, Dk), beta=(B, T, H))
    axis = (bump[1] - 1) % len(shapes[which])
    bad = list(shapes[which])
    bad[axis] = max(1, bad[axis] + bump[0]) if bad[axis] + bump[0] >= 1 \
        else bad[axis] + 1
    if tuple(bad) == shapes[which]:
        bad[axis] += 1
    f32, b16 = torch.float32, torch.bfloat16
    dt = dict(q=b16, k=b16, v=b16, g=f32, beta=f32)
    t = {n: torch.zeros(shapes[n], dtype=dt[n]) for n in shapes}
    # a wrong g disagrees with q and beta, so it is refused as well
    t[which] = torch.zeros(tuple(bad), dtype=dt[which])
    with pytest.raises(ValueError):
        kda.kda_prefill(t["q"], t["k"], t["v"], t["g"], t["beta"])
