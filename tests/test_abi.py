"""CPU checks of the C ABI: the library loads, exports every entry point
include/kda.h declares, and rejects invalid arguments before any launch
(no compute call is made here, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_74_amd as kda

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "include", "kda.h")
A = 0x100000  # a 16-byte aligned fake device address (never dereferenced)


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"kda_prefill", "kda_decode_step", "kda_decode_tokens",
            "kda_conv_prologue",
            "kda_prefill_chunk_prep", "kda_prefill_state_pass",
            "kda_prefill_workspace_size", "kda_status_string",
            "kda_abi_version"} <= set(names)
    lib = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    ver = int(re.search(r"#define KDA_ABI_VERSION (\d+)", open(HDR).read())[1])
    assert kda.kda_abi_version() == ver
    for s in range(5):
        assert kda.kda_status_string(s).startswith("KDA_")
    assert "unknown" in kda.kda_status_string(99)


def test_workspace_size():
    ws = kda.kda_prefill_workspace_size
    assert ws(1, 8192, 32, 128, 128, 64, kda.KDA_BF16) > 0
    # grows by one factor block per chunk; a ragged tail costs a whole
    # chunk (the small sync array of the concurrent mode aside)
    step = ws(1, 32, 1, 16, 16, 16, kda.KDA_F32) - \
        ws(1, 16, 1, 16, 16, 16, kda.KDA_F32)
    assert step > 0
    assert ws(1, 65, 1, 16, 16, 16, kda.KDA_F32) - \
        ws(1, 64, 1, 16, 16, 16, kda.KDA_F32) == step
    for bad in [(0, 8, 1, 16, 16, 16), (1, 8, 1, 48, 16, 16),
                (1, 8, 1, 16, 16, 8), (1, 8, 1, 16, 256, 16)]:
        assert ws(*bad, kda.KDA_BF16) == 0
    # fp32 at d_k = 128 runs 64-token requests as 32-token chunks
    assert ws(1, 64, 1, 128, 128, 64, kda.KDA_F32) == \
        ws(1, 64, 1, 128, 128, 32, kda.KDA_F32) > 0


def _prefill(**kw):
    a = dict(q=A, k=A, v=A, io=kda.KDA_BF16, g=A, beta=A, gt=kda.KDA_F32,
             s0=None, s_out=None, o=A + 4096, B=1, T=64, H=2, Dk=16, Dv=16,
             chunk=16, scale=1.0, conv=None, ws=A + 8192, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return kda._prefill(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(B=0), kda.KDA_EINVAL),
    (dict(T=-1), kda.KDA_EINVAL),
    (dict(chunk=0), kda.KDA_EINVAL),
    (dict(q=None), kda.KDA_EINVAL),
    (dict(g=None), kda.KDA_EINVAL),
    (dict(o=None), kda.KDA_EINVAL),
    (dict(ws=None), kda.KDA_EINVAL),
    (dict(k=A + 8), kda.KDA_EINVAL),          # misaligned
    (dict(wsb=16), kda.KDA_EINVAL),            # workspace too small
    (dict(io=7), kda.KDA_EINVAL),
    (dict(o=A), kda.KDA_EINVAL),               # output aliases an input
    (dict(scale=float("nan")), kda.KDA_EINVAL),
    (dict(chunk=48), kda.KDA_EUNSUPPORTED),
    (dict(Dk=48), kda.KDA_EUNSUPPORTED),
    (dict(Dv=256), kda.KDA_EUNSUPPORTED),
    (dict(io=kda.KDA_F32, gt=kda.KDA_BF16), kda.KDA_EUNSUPPORTED),
    # fp32 at d_k = 128 runs chunk 64 as 32-token chunks: accepted, and the
    # workspace it needs is the 32-token chunks' (too small here)
    (dict(io=kda.KDA_F32, Dk=128, Dv=128, chunk=64, wsb=1024), kda.KDA_EINVAL),
    # the per-head gate flag belongs to the gate dtype only
    (dict(io=kda.KDA_BF16 | kda.KDA_GATE_HEAD), kda.KDA_EINVAL),
    (dict(gt=2 | kda.KDA_GATE_HEAD), kda.KDA_EINVAL),
    (dict(io=kda.KDA_F32, gt=kda.KDA_BF16 | kda.KDA_GATE_HEAD),
     kda.KDA_EUNSUPPORTED),
    (dict(gt=kda.KDA_F32 | kda.KDA_GATE_HEAD, B=0), kda.KDA_EINVAL),
])
def test_prefill_rejects(kw, want):
    assert _prefill(**kw) == want


@pytest.mark.parametrize("width,l2,want", [(1, 1, kda.KDA_EINVAL),
                                          (5, 1, kda.KDA_EUNSUPPORTED),
                                          (4, 2, kda.KDA_EINVAL)])
def test_prefill_conv_rejects(width, l2, want):
    d = kda.KdaConvDesc(A, A, A, A, A, A, width, l2, 1e-6)
    assert _prefill(q=None, k=None, v=None, conv=ctypes.byref(d)) == want


def _decode(**kw):
    a = dict(q=A, k=A, v=A, io=kda.KDA_BF16, g=A, beta=A, gt=kda.KDA_BF16,
             state=A + 4096, o=A + 8192, N=4, H=2, Dk=16, Dv=16, scale=1.0,
             stream=None)
    a.update(kw)
    return kda._decode(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(N=0), kda.KDA_EINVAL), (dict(state=None), kda.KDA_EINVAL),
    (dict(v=A + 4), kda.KDA_EINVAL), (dict(o=A + 4096), kda.KDA_EINVAL),
    (dict(Dk=24), kda.KDA_EUNSUPPORTED),
    (dict(io=kda.KDA_F32), kda.KDA_EUNSUPPORTED),
    (dict(io=kda.KDA_F32 | kda.KDA_GATE_HEAD), kda.KDA_EINVAL),
    (dict(gt=3 | kda.KDA_GATE_HEAD), kda.KDA_EINVAL),
    (dict(gt=kda.KDA_BF16 | kda.KDA_GATE_HEAD, state=None), kda.KDA_EINVAL),
])
def test_decode_rejects(kw, want):
    assert _decode(**kw) == want


def _decode_tokens(**kw):
    a = dict(q=A, k=A, v=A, io=kda.KDA_BF16, g=A, beta=A, gt=kda.KDA_BF16,
             s_in=A + 4096, s_out=A + 4096, ts=None, o=A + 8192, N=2, L=2,
             H=2, Dk=16, Dv=16, scale=1.0, conv=None, cstate=None,
             cstate_out=None, stream=None)
    a.update(kw)
    return kda._decode_tokens(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(L=0), kda.KDA_EINVAL), (dict(N=-1), kda.KDA_EINVAL),
    (dict(s_in=None), kda.KDA_EINVAL), (dict(s_out=None), kda.KDA_EINVAL),
    (dict(o=A), kda.KDA_EINVAL), (dict(o=A + 4096), kda.KDA_EINVAL),
    (dict(ts=A + 4096), kda.KDA_EINVAL), (dict(ts=A + 12290), kda.KDA_EINVAL),
    (dict(scale=float("inf")), kda.KDA_EINVAL),
    (dict(Dk=48), kda.KDA_EUNSUPPORTED),
    (dict(io=kda.KDA_F32, gt=kda.KDA_BF16), kda.KDA_EUNSUPPORTED),
    (dict(cstate=A + 16384), kda.KDA_EINVAL),  # a history without a conv
    (dict(cstate_out=A + 16384), kda.KDA_EINVAL),
    (dict(io=kda.KDA_BF16 | kda.KDA_GATE_HEAD), kda.KDA_EINVAL),
    (dict(gt=kda.KDA_GATE_HEAD | 5), kda.KDA_EINVAL),
])
def test_decode_tokens_rejects(kw, want):
    assert _decode_tokens(**kw) == want


def _cdesc(**kw):
    d = dict(xq=A, xk=A, xv=A, wq=A, wk=A, wv=A, width=4, l2norm_qk=1,
             eps=1e-6)
    d.update(kw)
    return ctypes.byref(kda.KdaConvDesc(*d.values()))


@pytest.mark.parametrize("ckw,kw,want", [
    (dict(width=1), {}, kda.KDA_EINVAL), (dict(width=5), {},
                                          kda.KDA_EUNSUPPORTED),
    (dict(xv=None), {}, kda.KDA_EINVAL), (dict(eps=-1.0), {}, kda.KDA_EINVAL),
    (dict(l2norm_qk=2), {}, kda.KDA_EINVAL),
    ({}, dict(cstate=A + 8192), kda.KDA_EINVAL),    # history aliases o
    ({}, dict(cstate=A + 16386), kda.KDA_EINVAL),   # misaligned history
    ({}, dict(cstate_out=A + 8192), kda.KDA_EINVAL),   # rolled history = o
    ({}, dict(cstate_out=A + 4096), kda.KDA_EINVAL),   # ... = the state
    ({}, dict(cstate_out=A + 16392), kda.KDA_EINVAL),  # misaligned
    (dict(xk=A + 16384), dict(cstate_out=A + 16384),
     kda.KDA_EINVAL),                                  # ... = a raw input
    (dict(xq=A + 8192), {}, kda.KDA_EINVAL),        # o aliases a raw input
])
def test_decode_tokens_conv_rejects(ckw, kw, want):
    args = dict(conv=_cdesc(**ckw), q=None, k=None, v=None)
    args.update(kw)
    assert _decode_tokens(**args) == want


def _conv(**kw):
    a = dict(xq=A, xk=A, xv=A, dt=kda.KDA_BF16, wq=A, wk=A, wv=A, width=4,
             state=None, q=A + 4096, k=A + 8192, v=A + 12288, B=1, T=8, H=2,
             Dk=16, Dv=16, l2=1, eps=1e-6, stream=None)
    a.update(kw)
    return kda._conv(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(width=1), kda.KDA_EINVAL), (dict(width=5), kda.KDA_EUNSUPPORTED),
    (dict(xq=None), kda.KDA_EINVAL), (dict(eps=-1.0), kda.KDA_EINVAL),
    (dict(q=A), kda.KDA_EINVAL), (dict(Dv=20), kda.KDA_EUNSUPPORTED),
    (dict(state=A + 2), kda.KDA_EINVAL),
])
def test_conv_rejects(kw, want):
    assert _conv(**kw) == want


# ---------------------------------------------------------------------------
# The Python binding checks shapes and dtypes before it passes any pointer:
# these raise on the CPU (with CPU tensors) before any launch is attempted,
# with the mismatch named rather than the device complaint.

def _t(*shape, dt=None):
    import torch
    return torch.zeros(shape, dtype=dt or torch.bfloat16)


def test_binding_rejects_mismatched_prefill_inputs():
    import torch
    B, T, H, D = 1, 8, 2, 16
    f32 = torch.float32
    q, k, v = _t(B, T, H, D), _t(B, T, H, D), _t(B, T, H, D)
    g, beta = _t(B, T, H, D, dt=f32), _t(B, T, H, dt=f32)
    cases = [
        (dict(beta=_t(B, T, H)), "beta"),                # bf16 beta, fp32 g
        (dict(k=_t(B, T, H, D, dt=f32)), "k"),           # k not in q's dtype
        (dict(v=_t(B, T, H, 2 * D, dt=f32)), "v"),
        (dict(k=_t(B, T, H, 2 * D)), "k"),               # wrong size
        (dict(beta=_t(B, T + 1, H, dt=f32)), "beta"),
        (dict(g=_t(B, T, H, 2 * D, dt=f32)), "q"),       # g says Dk = 32
        (dict(g=_t(B, T, dt=f32)), "g"),                 # 2-d gate
    ]
    for over, what in cases:
        a = dict(q=q, k=k, v=v, g=g, beta=beta)
        a.update(over)
        with pytest.raises(ValueError, match=what):
            kda.kda_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"])
    with pytest.raises(ValueError, match="s0"):
        kda.kda_prefill(q, k, v, g, beta, s0=_t(B, H, D, D))  # bf16 state
    with pytest.raises(ValueError, match="o"):
        kda.kda_prefill(q, k, v, g, beta, o=_t(B, T, H, 2 * D))
    with pytest.raises(ValueError, match="do"):
        kda.kda_prefill_backward(q, k, v, g, beta, _t(B, T, H, D, dt=f32))


def test_binding_rejects_mismatched_decode_and_conv_inputs():
    import torch
    N, H, D, W = 3, 2, 16, 4
    f32 = torch.float32
    q = _t(N, H, D)
    st = _t(N, H, D, D, dt=f32)
    with pytest.raises(ValueError, match="beta"):
        kda.kda_decode_step(q, q, q, _t(N, H, D, dt=f32), _t(N, H), st)
    with pytest.raises(ValueError, match="state"):
        kda.kda_decode_step(q, q, q, _t(N, H, D), _t(N, H), _t(N, H, D, D))
    x = _t(1, 5, H * D)
    w = _t(H * D, W, dt=f32)
    with pytest.raises(ValueError, match="wk"):
        kda.kda_conv_prologue(x, x, x, w, _t(H * D, W), w, H=H, Dk=D, Dv=D)
    with pytest.raises(ValueError, match="xv"):
        kda.kda_conv_prologue(x, x, _t(1, 5, 2 * H * D), w, w, w, H=H, Dk=D,
                              Dv=D)
    with pytest.raises(ValueError, match="conv_state"):
        kda.kda_conv_prologue(x, x, x, w, w, w, H=H, Dk=D, Dv=D,
                              conv_state=_t(1, 3, H * D, W, dt=f32))
    xt = _t(N, 2, H * D)
    conv = dict(xq=xt, xk=xt, xv=xt, wq=w, wk=w, wv=w, width=W)
    with pytest.raises(ValueError, match="conv_state"):
        kda.kda_decode_tokens(None, None, None, _t(N, 2, H), _t(N, 2, H), st,
                              conv=conv, conv_state=_t(N, 3, H * D, W - 2,
                                                       dt=f32))


def test_noalloc_rejects_before_any_launch():
    """kda_prefill_noalloc validates like kda_prefill and refuses a request
    larger than its fixed scratch with KDA_ENOSPACE, all before it looks up
    the scratch or launches (so no GPU is touched here)."""
    f = kda._prefill_noalloc
    base = [A, A, A, kda.KDA_BF16, A, A, kda.KDA_F32, None, None, A + 4096]
    # B=1, T=2048, H=32, d=128, chunk 64: 93 MiB of workspace > 64 MiB
    assert kda.kda_prefill_workspace_size(1, 2048, 32, 128, 128, 64,
                                          kda.KDA_BF16) > \
        kda.KDA_NOALLOC_SCRATCH_BYTES
    assert f(*base, 1, 2048, 32, 128, 128, 64, 1.0, None, None) == \
        kda.KDA_ENOSPACE
    assert f(*base, 1, 2048, 32, 128, 128, 48, 1.0, None, None) == \
        kda.KDA_EUNSUPPORTED
    bad = list(base)
    bad[9] = A  # o aliases q
    assert f(*bad, 1, 64, 2, 16, 16, 16, 1.0, None, None) == kda.KDA_EINVAL
    assert f(*base, 0, 64, 2, 16, 16, 16, 1.0, None, None) == kda.KDA_EINVAL
