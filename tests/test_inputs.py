"""The seeded input generator: determinism, block re-draws, and the
distribution facts the workload recipe states."""
import numpy as np
import torch

import kda_inputs as ki


def test_deterministic_and_seed_sensitive():
    a = ki.prefill_inputs(1, 100, 2, 8, 8, seed=1)
    b = ki.prefill_inputs(1, 100, 2, 8, 8, seed=1)
    c = ki.prefill_inputs(1, 100, 2, 8, 8, seed=2)
    for n in a:
        assert torch.equal(a[n], b[n])
        assert not torch.equal(a[n], c[n])


def test_blocks_redraw_independently():
    full = ki.prefill_inputs(1, ki.BLOCK + 50, 1, 4, 4, qkv="f32", seed=3)
    tail = ki.prefill_inputs(1, ki.BLOCK, 1, 4, 4, qkv="f32", seed=3)
    for n in ("q", "k", "v", "g", "beta"):
        assert torch.equal(full[n][:, :ki.BLOCK], tail[n])


def test_distribution_facts():
    x = ki.prefill_inputs(1, 8192, 4, 32, 32, qkv="bf16", gate="f32", seed=5)
    n = x["q"].float().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=2e-2)
    assert torch.all(x["g"] <= 0)
    # E[exp(-softplus z)] = E[sigmoid(-z)] = 1/2 and E[sigmoid z] = 1/2
    assert abs(x["g"].double().exp().mean().item() - 0.5) < 5e-3
    assert abs(x["beta"].double().mean().item() - 0.5) < 5e-3
    assert torch.all((x["beta"] > 0) & (x["beta"] < 1))
    assert abs(x["v"].float().std().item() - 1.0) < 1e-2


def test_slow_gate_mean():
    x = ki.prefill_inputs(1, 4096, 8, 128, 8, gate_kind="slow", seed=6)
    m = x["g"].double().exp().mean().item()
    assert abs(m - 0.999) < 2e-5


def test_conv_workload_shapes():
    x = ki.prefill_inputs(2, 40, 3, 8, 16, conv_width=4, seed=7)
    assert x["xq"].shape == (2, 40, 24) and x["xv"].shape == (2, 40, 48)
    assert x["wq"].shape == (24, 4) and x["wq"].dtype == torch.float32
    assert abs(x["wq"].std().item() - 0.5) < 0.2
    assert "q" not in x


def test_decode_inputs():
    s = ki.decode_state(4, 2, 16, 16)
    assert s.dtype == torch.float32 and abs(s.std().item() - 0.1) < 1e-2
    a = ki.decode_step_inputs(4, 2, 16, 16, step=3)
    b = ki.decode_step_inputs(4, 2, 16, 16, step=4)
    assert a["q"].shape == (4, 2, 16) and a["beta"].shape == (4, 2)
    assert a["g"].dtype == torch.bfloat16
    assert not torch.equal(a["v"], b["v"])
