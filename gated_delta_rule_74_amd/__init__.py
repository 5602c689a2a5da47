"""Python binding of libkda.so, the MI355X (gfx950) KDA layer forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/kda.h``.  PyTorch supplies
device memory and the current stream.  There is no fallback of any kind: if
the library has not been built, importing this package raises.

Functions mirror the C entry points by name:
  kda_prefill, kda_prefill_noalloc, kda_prefill_chunk_prep,
  kda_prefill_state_pass,
  kda_decode_step, kda_conv_prologue, kda_prefill_workspace_size,
  kda_status_string, kda_abi_version
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python gated_delta_rule_74_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

KDA_OK, KDA_EINVAL, KDA_EUNSUPPORTED, KDA_EHIP, KDA_ENOSPACE = 0, 1, 2, 3, 4
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed workspace of kda_prefill_noalloc
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_HEAD = 16  # gate-dtype flag: g holds one log-decay per token-head

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class KdaConvDesc(ctypes.Structure):
    _fields_ = [("xq", _vp), ("xk", _vp), ("xv", _vp), ("wq", _vp),
                ("wk", _vp), ("wv", _vp), ("width", _i), ("l2norm_qk", _i),
                ("eps", _f)]


def _sig(name, res, args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = args
    return fn


_abi_version = _sig("kda_abi_version", _i, [])
_status_string = _sig("kda_status_string", ctypes.c_char_p, [_i])
_ws_size = _sig("kda_prefill_workspace_size", _sz, [_i] * 6 + [_i])
_prefill = _sig("kda_prefill", _i,
                [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp] + [_i] * 6 +
                [_f, ctypes.POINTER(KdaConvDesc), _vp, _sz, _vp])
_prefill_noalloc = _sig("kda_prefill_noalloc", _i,
                        [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp] +
                        [_i] * 6 + [_f, ctypes.POINTER(KdaConvDesc), _vp])
_prep = _sig("kda_prefill_chunk_prep", _i,
             [_vp, _vp, _vp, _i, _vp, _vp, _i] + [_i] * 6 +
             [_f, ctypes.POINTER(KdaConvDesc), _vp, _sz, _vp])
_state = _sig("kda_prefill_state_pass", _i,
              [_i, _vp, _vp, _vp] + [_i] * 6 + [_vp, _sz, _vp])
_decode = _sig("kda_decode_step", _i,
               [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp] + [_i] * 4 +
               [_f, _vp])
_decode_tokens = _sig("kda_decode_tokens", _i,
                      [_vp, _vp, _vp, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp] +
                      [_i] * 5 + [_f, ctypes.POINTER(KdaConvDesc), _vp, _vp,
                                  _vp])
_bwd = _sig("kda_prefill_backward", _i,
            [_vp, _vp, _vp, _i, _vp, _vp, _i] + [_vp] * 9 + [_i] * 6 +
            [_f, _vp, _sz, _vp])
_bwd_ws_size = _sig("kda_prefill_backward_workspace_size", _sz, [_i] * 7)
_conv = _sig("kda_conv_prologue", _i,
             [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp] +
             [_i] * 5 + [_i, _f, _vp])


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kda_status_string(status)}")


def kda_abi_version() -> int:
    return _abi_version()


def kda_status_string(status: int) -> str:
    return _status_string(status).decode()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gate_dt(g, per_channel_ndim: int) -> int:
    """Gate dtype code; a g with one dimension fewer than the per-channel
    layout is the per-head (scalar) gate."""
    if g.dim() == per_channel_ndim:
        return _dt(g)
    if g.dim() == per_channel_ndim - 1:
        return _dt(g) | KDA_GATE_HEAD
    raise ValueError(f"g has {g.dim()} dimensions")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _need(t, shape, dtype, name):
    """Raise ValueError unless tensor t (skipped when None) has exactly this
    shape and dtype: the C ABI takes bare pointers and derives every extent
    from the sizes passed with them, so a mismatch would read or write past
    a buffer."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected "
                         f"{tuple(int(d) for d in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _io_dtype(t, name):
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"{name}: dtype {t.dtype}, expected float32 or "
                         "bfloat16")
    return t.dtype


def _check_gates(g, beta, lead, Dk):
    """g [*lead, Dk] (per channel) or [*lead] (per head); beta [*lead] in
    g's dtype."""
    gd = _io_dtype(g, "g")
    if g.dim() == len(lead) + 1:
        _need(g, (*lead, Dk), gd, "g")
    else:
        _need(g, lead, gd, "g (per-head gate)")
    _need(beta, lead, gd, "beta (must have g's dtype)")


def _check_conv(conv, B, T, H, Dk, Dv, io):
    W = int(conv.get("width", conv["wq"].shape[-1]))
    for n, D in (("xq", Dk), ("xk", Dk), ("xv", Dv)):
        _need(conv[n], (B, T, H * D), io, n)
    for n, D in (("wq", Dk), ("wk", Dk), ("wv", Dv)):
        _need(conv[n], (H * D, W), torch.float32, n)
    return W


def _check_prefill(q, k, v, g, beta, conv, B, T, H, Dk, Dv, io):
    if conv is None:
        _need(q, (B, T, H, Dk), io, "q")
        _need(k, (B, T, H, Dk), io, "k (must have q's dtype)")
        _need(v, (B, T, H, Dv), io, "v (must have q's dtype)")
    else:
        _check_conv(conv, B, T, H, Dk, Dv, io)
    _check_gates(g, beta, (B, T, H), Dk)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != KDA_OK:
        raise KdaError(st, where)


def kda_prefill_workspace_size(B, T, H, Dk, Dv, chunk, qkv_dtype) -> int:
    dt = qkv_dtype if isinstance(qkv_dtype, int) else (
        KDA_BF16 if qkv_dtype == torch.bfloat16 else KDA_F32)
    return int(_ws_size(B, T, H, Dk, Dv, chunk, dt))


def _conv_desc(conv):
    if conv is None:
        return None, None
    keep = [conv[n] for n in ("xq", "xk", "xv", "wq", "wk", "wv")]
    d = KdaConvDesc(*[_ptr(x) for x in keep],
                    int(conv.get("width", conv["wq"].shape[-1])),
                    int(bool(conv.get("l2norm_qk", True))),
                    float(conv.get("eps", 1e-6)))
    return ctypes.byref(d), (d, keep)


def _prefill_shapes(q, v, g, conv):
    if g.dim() not in (3, 4):
        raise ValueError(f"g has {g.dim()} dimensions (expected 4, or 3 "
                         "for a per-head gate)")
    if g.dim() == 4:
        B, T, H, Dk = g.shape
    else:  # per-head gate [B,T,H]
        B, T, H = g.shape
        Dk = q.shape[-1] if conv is None else conv["xq"].shape[-1] // H
    if conv is not None:
        Dv = conv["xv"].shape[-1] // H
        io = conv["xq"]
    else:
        if q is None or v is None:
            raise ValueError("q, k and v are required without a conv")
        Dv = v.shape[-1]
        io = q
    _io_dtype(io, "q" if conv is None else "xq")
    return B, T, H, Dk, Dv, io


def alloc_workspace(B, T, H, Dk, Dv, chunk, dtype, device="cuda"):
    n = kda_prefill_workspace_size(B, T, H, Dk, Dv, chunk, dtype)
    if n == 0:
        raise KdaError(KDA_EUNSUPPORTED, "kda_prefill_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def kda_prefill(q, k, v, g, beta, *, s0=None, chunk=64, scale=1.0,
                conv=None, o=None, s_out=None, want_state=True,
                workspace=None, stream=None):
    """Chunked prefill.  q,k,g [B,T,H,Dk], v [B,T,H,Dv], beta [B,T,H]
    (q,k,v may be None when `conv` gives raw projections and taps; g may
    be [B,T,H], one log-decay per token-head shared by the key channels).
    Returns (o [B,T,H,Dv], final state [B,H,Dk,Dv] fp32 or None)."""
    B, T, H, Dk, Dv, io = _prefill_shapes(q, v, g, conv)
    _check_prefill(q, k, v, g, beta, conv, B, T, H, Dk, Dv, io.dtype)
    _need(s0, (B, H, Dk, Dv), torch.float32, "s0")
    _need(s_out, (B, H, Dk, Dv), torch.float32, "s_out")
    _need(o, (B, T, H, Dv), io.dtype, "o")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=io.dtype, device=g.device)
    if s_out is None and want_state:
        s_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                            device=g.device)
    if workspace is None:
        workspace = alloc_workspace(B, T, H, Dk, Dv, chunk, io.dtype,
                                    g.device)
    cd, _keep = _conv_desc(conv)
    st = _prefill(_ptr(q), _ptr(k), _ptr(v), _dt(io), _ptr(g), _ptr(beta),
                  _gate_dt(g, 4), _ptr(s0), _ptr(s_out), _ptr(o), B, T, H, Dk, Dv,
                  chunk, scale, cd, _ptr(workspace), workspace.numel(),
                  _stream(stream))
    _check(st, "kda_prefill")
    return o, s_out


def kda_prefill_noalloc(q, k, v, g, beta, *, s0=None, chunk=64, scale=1.0,
                        conv=None, o=None, s_out=None, want_state=True,
                        stream=None):
    """kda_prefill on the library's fixed scratch workspace: the C call
    allocates nothing (pass o and s_out to keep this wrapper from
    allocating them).  Raises KdaError(KDA_ENOSPACE) when the sizes need
    more than KDA_NOALLOC_SCRATCH_BYTES of workspace.  Calls that overlap
    in time on one GPU share the scratch and race."""
    B, T, H, Dk, Dv, io = _prefill_shapes(q, v, g, conv)
    _check_prefill(q, k, v, g, beta, conv, B, T, H, Dk, Dv, io.dtype)
    _need(s0, (B, H, Dk, Dv), torch.float32, "s0")
    _need(s_out, (B, H, Dk, Dv), torch.float32, "s_out")
    _need(o, (B, T, H, Dv), io.dtype, "o")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=io.dtype, device=g.device)
    if s_out is None and want_state:
        s_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                            device=g.device)
    cd, _keep = _conv_desc(conv)
    st = _prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _dt(io), _ptr(g),
                          _ptr(beta), _gate_dt(g, 4), _ptr(s0), _ptr(s_out),
                          _ptr(o), B, T, H, Dk, Dv, chunk, scale, cd,
                          _stream(stream))
    _check(st, "kda_prefill_noalloc")
    return o, s_out


def kda_prefill_chunk_prep(q, k, v, g, beta, workspace, *, chunk=64,
                           scale=1.0, conv=None, Dv=None, stream=None):
    """First prefill phase alone (chunk-local factors -> workspace)."""
    B, T, H, Dk, Dv_, io = _prefill_shapes(q, v, g, conv)
    if Dv is not None and conv is None and int(Dv) != Dv_:
        raise ValueError(f"Dv={Dv} but v has {Dv_} columns")
    Dv_ = Dv_ if Dv is None else int(Dv)
    _check_prefill(q, k, v, g, beta, conv, B, T, H, Dk, Dv_, io.dtype)
    cd, _keep = _conv_desc(conv)
    st = _prep(_ptr(q), _ptr(k), _ptr(v), _dt(io), _ptr(g), _ptr(beta),
               _gate_dt(g, 4), B, T, H, Dk, Dv_, chunk, scale,
               cd, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "kda_prefill_chunk_prep")


def kda_prefill_state_pass(workspace, o, *, s0=None, s_out=None, B, T, H,
                           Dk, Dv, chunk=64, stream=None):
    """Second prefill phase alone (sequential state pass -> o, s_out)."""
    io = _io_dtype(o, "o")
    _need(o, (B, T, H, Dv), io, "o")
    _need(s0, (B, H, Dk, Dv), torch.float32, "s0")
    _need(s_out, (B, H, Dk, Dv), torch.float32, "s_out")
    st = _state(_dt(o), _ptr(s0), _ptr(s_out), _ptr(o), B, T, H, Dk, Dv,
                chunk, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "kda_prefill_state_pass")


def kda_prefill_backward_workspace_size(B, T, H, Dk, Dv, chunk,
                                        qkv_dtype) -> int:
    dt = qkv_dtype if isinstance(qkv_dtype, int) else (
        KDA_BF16 if qkv_dtype == torch.bfloat16 else KDA_F32)
    return int(_bwd_ws_size(B, T, H, Dk, Dv, chunk, dt))


def kda_prefill_backward(q, k, v, g, beta, do, *, s0=None, dsT=None,
                         chunk=64, scale=1.0, workspace=None, want_ds0=True,
                         stream=None):
    """Gradient of kda_prefill (no conv) for the loss sum(o*do) +
    sum(S_T*dsT).  q,k,g [B,T,H,Dk] (g may be [B,T,H]), v, do [B,T,H,Dv],
    beta [B,T,H].  Returns (dq, dk, dv, dg, dbeta, ds0 or None) with dg
    shaped like g."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_dtype(q, "q")
    _check_prefill(q, k, v, g, beta, None, B, T, H, Dk, Dv, io)
    _need(do, (B, T, H, Dv), io, "do (must have q's dtype)")
    _need(s0, (B, H, Dk, Dv), torch.float32, "s0")
    _need(dsT, (B, H, Dk, Dv), torch.float32, "dsT")
    dev = q.device
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv = torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    ds0 = (torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
           if want_ds0 else None)
    need = kda_prefill_backward_workspace_size(B, T, H, Dk, Dv, chunk,
                                               _dt(q))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = _bwd(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(g), _ptr(beta),
              _gate_dt(g, 4), _ptr(s0), _ptr(do), _ptr(dsT), _ptr(dq),
              _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0), B, T, H,
              Dk, Dv, chunk, scale, _ptr(workspace), workspace.numel(),
              _stream(stream))
    _check(st, "kda_prefill_backward")
    return dq, dk, dv, dg, dbeta, ds0


def kda_decode_step(q, k, v, g, beta, state, *, scale=1.0, o=None,
                    stream=None):
    """One decode step; `state` [N,H,Dk,Dv] fp32 is updated in place.
    Returns o [N,H,Dv]."""
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    io = _io_dtype(q, "q")
    _need(k, (N, H, Dk), io, "k (must have q's dtype)")
    _need(v, (N, H, Dv), io, "v (must have q's dtype)")
    _check_gates(g, beta, (N, H), Dk)
    _need(state, (N, H, Dk, Dv), torch.float32, "state")
    _need(o, (N, H, Dv), io, "o")
    if o is None:
        o = torch.empty((N, H, Dv), dtype=q.dtype, device=q.device)
    st = _decode(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(g), _ptr(beta),
                 _gate_dt(g, 3), _ptr(state), _ptr(o), N, H, Dk, Dv, scale,
                 _stream(stream))
    _check(st, "kda_decode_step")
    return o


def kda_decode_tokens(q, k, v, g, beta, state_in, *, state_out=None,
                      token_states=False, scale=1.0, o=None, conv=None,
                      conv_state=None, conv_state_out=None, stream=None):
    """L tokens per sequence in one call (the speculative-decoding verify
    step, or with L = 1 the generation step).  q,k,g [N,L,H,Dk],
    v [N,L,H,Dv], beta [N,L,H]; state_in [N,H,Dk,Dv] fp32.  state_out: a
    tensor to write the final state into (pass state_in itself for in
    place; default: a new tensor).  token_states: True for a new
    [N,L,H,Dk,Dv] tensor of the state after each token, a tensor to fill,
    or False.  conv: dict(xq, xk, xv [N,L,H*D], wq, wk, wv, width,
    l2norm_qk, eps) to make q, k, v from raw projections (q, k, v may then
    be None), with conv_state the fp32 history [N,3,H*max(Dk,Dv),W-1]
    or None (zeros), rolled forward in place unless conv_state_out (a
    second history tensor, written by the decode kernel itself) is given.
    Returns (o, state_out, token_states or None)."""
    if g.dim() == 4:
        N, L, H, Dk = g.shape
    else:  # per-head gate [N,L,H]
        N, L, H = g.shape
        Dk = q.shape[-1] if conv is None else conv["xq"].shape[-1] // H
    if conv is not None:
        Dv = conv["xv"].shape[-1] // H
        io = conv["xq"]
    else:
        Dv = v.shape[-1]
        io = q
    iod = _io_dtype(io, "q" if conv is None else "xq")
    _check_prefill(q, k, v, g, beta, conv, N, L, H, Dk, Dv, iod)
    _need(state_in, (N, H, Dk, Dv), torch.float32, "state_in")
    _need(state_out, (N, H, Dk, Dv), torch.float32, "state_out")
    _need(o, (N, L, H, Dv), iod, "o")
    if conv is not None:
        W = _check_conv(conv, N, L, H, Dk, Dv, iod)
        for n, c in (("conv_state", conv_state),
                     ("conv_state_out", conv_state_out)):
            _need(c, (N, 3, H * max(Dk, Dv), W - 1), torch.float32, n)
    elif conv_state is not None or conv_state_out is not None:
        raise ValueError("conv_state without conv")
    if o is None:
        o = torch.empty((N, L, H, Dv), dtype=io.dtype, device=g.device)
    if state_out is None:
        state_out = torch.empty_like(state_in)
    ts = None
    if token_states is True:
        ts = torch.empty((N, L, H, Dk, Dv), dtype=torch.float32,
                         device=g.device)
    elif token_states is not False and token_states is not None:
        ts = token_states
        _need(ts, (N, L, H, Dk, Dv), torch.float32, "token_states")
    cd, _keep = _conv_desc(conv)
    st = _decode_tokens(_ptr(q), _ptr(k), _ptr(v), _dt(io), _ptr(g),
                        _ptr(beta), _gate_dt(g, 4), _ptr(state_in), _ptr(state_out),
                        _ptr(ts), _ptr(o), N, L, H, Dk, Dv, scale, cd,
                        _ptr(conv_state), _ptr(conv_state_out),
                        _stream(stream))
    _check(st, "kda_decode_tokens")
    return o, state_out, ts


def kda_conv_prologue(xq, xk, xv, wq, wk, wv, *, H, Dk, Dv, conv_state=None,
                      l2norm_qk=True, eps=1e-6, q=None, k=None, v=None,
                      stream=None):
    """Standalone conv (+ L2 on q, k) prologue.  x* [B,T,H*D] -> q,k
    [B,T,H,Dk], v [B,T,H,Dv] (the raw inputs' dtype).  conv_state, if given,
    is fp32 [B,3,H*max(Dk,Dv),W-1], read then updated in place."""
    B, T, _ = xq.shape
    W = wq.shape[-1]
    io = _io_dtype(xq, "xq")
    _check_conv(dict(xq=xq, xk=xk, xv=xv, wq=wq, wk=wk, wv=wv), B, T, H, Dk,
                Dv, io)
    _need(conv_state, (B, 3, H * max(Dk, Dv), W - 1), torch.float32,
          "conv_state")
    for n, t, D in (("q", q, Dk), ("k", k, Dk), ("v", v, Dv)):
        _need(t, (B, T, H, D), io, n)
    if q is None:
        q = torch.empty((B, T, H, Dk), dtype=xq.dtype, device=xq.device)
    if k is None:
        k = torch.empty((B, T, H, Dk), dtype=xq.dtype, device=xq.device)
    if v is None:
        v = torch.empty((B, T, H, Dv), dtype=xq.dtype, device=xq.device)
    st = _conv(_ptr(xq), _ptr(xk), _ptr(xv), _dt(xq), _ptr(wq), _ptr(wk),
               _ptr(wv), W, _ptr(conv_state), _ptr(q), _ptr(k), _ptr(v), B, T,
               H, Dk, Dv, int(bool(l2norm_qk)), eps, _stream(stream))
    _check(st, "kda_conv_prologue")
    return q, k, v
