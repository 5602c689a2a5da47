"""GPU tests of the concurrent prefill: at bf16 q/k/v, d_k = d_v = 128,
chunk 64, per-channel gate, no conv, B*H a multiple of 8 or not, and at most
one state-pass workgroup per CU, kda_prefill can run the chunk prep and the
state pass at the same time (ready flag per chunk task in the workspace's
sync array).  By default it does so for sequences of 1024 chunks or more;
these tests force it with KDA_CONCURRENT=1 (read by the library at every
call).  Both kernels do the same arithmetic in the same order as the
two-kernel path (kda_prefill_chunk_prep then kda_prefill_state_pass), so
the outputs must be equal bit for bit, with the mode on and off; the sync
array must show every task published and no timed-out wait, also on a
second call over the same workspace, and stay untouched with the mode off.
The small cases are also checked against the oracle here; at full size the
long-context test of test_gpu_prefill.py (4096 chunks per head) runs this
path by default."""
import pytest
import torch

import kda_inputs as ki
from gpu_common import TOL, check, say

pytestmark = pytest.mark.gpu

SYNC_NEXT, SYNC_TIMEOUT, SYNC_FLAGS = 0, 1, 64  # the library's sync layout


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_74_amd as m
    return m


def _sync_view(ws, B, H, NC):
    """The int array after the factor blocks (the last sync_bytes of the
    workspace that kda_prefill_workspace_size sizes)."""
    n = ((SYNC_FLAGS + B * H * NC) * 4 + 255) & ~255
    return ws[ws.numel() - n:].view(torch.int32)


@pytest.mark.parametrize("B,T,H,gate,s0", [
    (1, 8192, 32, "f32", False),   # the model-shaped workload
    (2, 300, 4, "f32", True),      # ragged tail, batch > 1, initial state
    (1, 64, 1, "bf16", True),      # one chunk, bf16 gates
    (3, 1000, 5, "bf16", False)])  # B*H not a multiple of 8
def test_concurrent_equals_two_kernel_path(orc, kda, monkeypatch, B, T, H,
                                           gate, s0):
    say(f"concurrent prefill B{B} T{T} H{H} gate={gate} s0={s0}")
    monkeypatch.setenv("KDA_CONCURRENT", "1")
    D, C = 128, 64
    NC = (T + C - 1) // C
    x = ki.prefill_inputs(B, T, H, D, D, qkv="bf16", gate=gate,
                          seed=700 + T + H, device="cuda", with_s0=s0)
    st0 = x.get("s0")
    ws = kda.alloc_workspace(B, T, H, D, D, C, torch.bfloat16)
    sync = _sync_view(ws, B, H, NC)
    outs = []
    for call in range(2):
        ws[ws.numel() - sync.numel() * 4:].fill_(0x5a)  # stale sync bytes
        o, s = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                               s0=st0, chunk=C, scale=0.9, workspace=ws)
        torch.cuda.synchronize()
        sv = sync.cpu()
        say(f"  call {call}: next={int(sv[SYNC_NEXT])} "
            f"timeout={int(sv[SYNC_TIMEOUT])}")
        assert int(sv[SYNC_TIMEOUT]) == 0, "a state-pass wave timed out"
        assert int(sv[SYNC_NEXT]) >= B * H * NC
        assert bool((sv[SYNC_FLAGS:SYNC_FLAGS + B * H * NC] == 1).all())
        outs.append((o, s))
    # the two-kernel path on its own workspace, and kda_prefill with the
    # mode turned off (untouched sync array)
    monkeypatch.setenv("KDA_CONCURRENT", "0")
    sync.fill_(-7)
    o3, s3 = kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                             s0=st0, chunk=C, scale=0.9, workspace=ws)
    torch.cuda.synchronize()
    assert bool((sync == -7).all())
    outs.append((o3, s3))
    ws2 = kda.alloc_workspace(B, T, H, D, D, C, torch.bfloat16)
    kda.kda_prefill_chunk_prep(x["q"], x["k"], x["v"], x["g"], x["beta"],
                               ws2, chunk=C, scale=0.9)
    o2 = torch.empty_like(outs[0][0])
    s2 = torch.empty_like(outs[0][1])
    kda.kda_prefill_state_pass(ws2, o2, s0=st0, s_out=s2, B=B, T=T, H=H,
                               Dk=D, Dv=D, chunk=C)
    torch.cuda.synchronize()
    for o, s in outs:
        assert torch.equal(o, o2)
        assert torch.equal(s, s2)
    if B * T * H <= 4000:
        ro, rs = orc.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                st0, 0.9)
        check("o", outs[0][0], ro, TOL["bf16"], (0, 2))
        check("S", outs[0][1], rs, TOL["bf16"], (0, 1))
