"""Benchmark of the KDA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                    [--no-cpu] [--only prefill,decode,tokens,conv,long,gdn,bwd,copy]
                    [--decode-steps N]

Headline (`value`): chunked prefill tokens/s on the model-shaped workload
B=1, T=8192, H=32, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 g/beta/state
(synthetic seeded inputs, resident in HBM before timing).  One step = one
kda_prefill call (chunk-prep kernel + state-pass kernel).  The decode
workload (256 sequences x 32 heads, 1000 in-place steps), the fused-conv
prefill (B=8, T=4096) and the long-context prefill (T=262,144) are timed too
and reported in `decode` / `extra`.

Kernel durations are measured with HIP events recorded on the stream the
kernels are launched on.  Rooflines use algorithmic bytes (each input read
once, each output written once) and MI355X peaks (HBM 8 TB/s, dense bf16
MFMA 2.5 PFLOP/s).  `traffic` comes from committed rocprofv3 counter runs
(profiles/traffic.json) and is null when the kernel sources changed since.

The CPU baseline times the fp64 oracle (test infrastructure) on the host
cores over the whole prefill workload, repeated for about 10 s (median pass).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "KDA prefill tokens/s (T=8192,H=32,d=128) + decode-step state GB/s"


def prefill_bytes(B, T, H, Dk, Dv, io=2, gate=4, state=4):
    """Algorithmic HBM bytes of one prefill: q,k,v,g,beta read once, o and
    the final state written once (S0 = 0 is not read)."""
    tok = B * T * H
    return tok * (2 * Dk * io + Dv * io + Dk * gate + gate + Dv * io) + \
        B * H * Dk * Dv * state


def prefill_flops(B, T, H, Dk, Dv, C):
    """Algorithmic flops per token-head: 6 Dk Dv (three chunk x state
    products) + C (3 Dk + 2 Dv) (causal halves of A, P, W, U and P Delta)
    + C^2 / 3 (triangular inverse)."""
    return B * T * H * (6 * Dk * Dv + C * (3 * Dk + 2 * Dv) + C * C / 3)


def decode_bytes(N, H, Dk, Dv, io=2):
    """State read + written once, q,k,v,g,beta read, o written."""
    return N * H * (2 * Dk * Dv * 4 + (3 * Dk + Dv + 1 + Dv) * io)


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_74_amd", "csrc", n),
                  "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, sources):
    """Measured HBM bytes per launch from profiles/traffic.json, or None if
    missing or taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    rec = d.get("kernels", {}).get(kernel)
    if not rec or rec.get("src_hash") != src_hash(sources):
        return None
    return rec.get("bytes_per_launch")


def mfma_busy_for(key, sources):
    """MFMA busy fractions measured by rocprofv3 counters
    (profiles/mfma_busy.json), or None if missing or taken on other kernel
    sources."""
    p = os.path.join(ROOT, "profiles", "mfma_busy.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("src_hash", {}).get(key) != src_hash(sources):
        return None
    return d


def state_loads_alone(ws, BH, NC, Dk, Dv, C):
    """Time the probe that pulls the state pass's per-chunk factor bytes into
    registers with nothing else to do (libkda_probe.so, built beside
    libkda.so), scaled to the bytes the state pass itself loads: what its
    loads cost on their own.  None if the probe library is absent or refuses
    the shape."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "gated_delta_rule_74_amd", "libkda_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.kda_probe_state_reads
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_int] * 6 + \
        [ctypes.POINTER(ctypes.c_double)] * 2
    import torch
    torch.cuda.synchronize()
    us, pb = ctypes.c_double(), ctypes.c_double()
    if fn(ws.data_ptr(), ws.numel(), BH, NC, Dk, Dv, C, 20, ctypes.byref(us),
          ctypes.byref(pb)) != 0:
        return None
    # what one state-pass workgroup loads per chunk: its 1 KiB units of -W,
    # Qtil and Ktil^T, the lower units of P, its slab's U tiles, gamma_C
    nb, nku, ntu = C // 16, Dk // 32, (C // 16 + 1) // 2
    units = 2 * nb * nku + (Dk // 16) * ntu + sum(rt // 2 + 1 for rt in range(nb))
    sb = units * 1024 + nb * 64 * 4 * 2 + Dk * 4
    return dict(probe_us=us.value, probe_bytes_per_wg_chunk=pb.value,
                state_bytes_per_wg_chunk=sb,
                loads_alone_us=us.value * sb / pb.value,
                bytes_per_cu_per_us=pb.value * NC / us.value,
                source="gated_delta_rule_74_amd/csrc/probe_read_rate.hip")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma list of: prefill, decode, tokens, conv, long, "
                         "gdn, copy (tokens = the verify step and the "
                         "generation step with the fused conv; gdn = the "
                         "headline prefill with one gate per token-head; "
                         "bwd = the gradient of the headline prefill; "
                         "copy = a plain 1 GiB device copy, the reference "
                         "for scaling HBM byte counters, and a 512 MiB "
                         "in-place scale, the practical streaming ceiling "
                         "for the decode step; every part runs by default)")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="time fewer decode steps than the workload's 1000 "
                         "(profiling runs)")
    args = ap.parse_args()
    only = None if args.only is None else set(args.only.split(","))
    bad = (only or set()) - {"prefill", "decode", "tokens", "conv", "long",
                           "gdn", "bwd", "copy"}
    if bad:
        ap.error(f"unknown --only part(s): {sorted(bad)}")
    sel = lambda part: only is None or \
        (only is not None and part in only)
    if args.gpus != 1:
        print(f"bench.py: the KDA library runs on one GPU (asked for "
              f"--gpus {args.gpus}); a head-split multi-GPU path is not "
              "implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_74_amd as kda
    import kda_inputs as ki

    torch.cuda.set_device(0)
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    out = {}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def settle(fn, seconds=0.25):
        # untimed, before a part's own warm-up steps: the GPU's clocks ramp
        # over the first ~10-20 ms of sustained work, and a timed region that
        # starts cold reports part of that ramp instead of the steady rate
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()

    # per-kernel durations: K back-to-back launches of each kernel alone
    # (HIP events on the launch stream), so launch gaps are not counted
    def t_back_to_back(fn, reps=None):
        reps = reps or K
        fn()
        torch.cuda.synchronize()
        a, b_ = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / reps

    # ---------------- prefill, model-shaped (headline) ----------------------
    c1 = ki.workload(ki.PREFILL)
    B, T, H, Dk, Dv, C = (c1[n] for n in ("B", "T", "H", "Dk", "Dv", "chunk"))
    run_prefill = sel("prefill")
    if run_prefill:
        log("prefill: generating inputs")
        x = ki.workload_prefill_inputs(ki.PREFILL, device=dev)
        ws = kda.alloc_workspace(B, T, H, Dk, Dv, C, torch.bfloat16, dev)
        o = torch.empty((B, T, H, Dv), dtype=torch.bfloat16, device=dev)
        s = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)

        def step():
            kda.kda_prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],
                            chunk=C, o=o, s_out=s, workspace=ws)

        settle(step)
        for _ in range(W):
            step()
        torch.cuda.synchronize()
        log("prefill: timing")
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        tp = t_back_to_back(lambda: kda.kda_prefill_chunk_prep(
            x["q"], x["k"], x["v"], x["g"], x["beta"], ws, chunk=C))
        ts = t_back_to_back(lambda: kda.kda_prefill_state_pass(
            ws, o, s_out=s, B=B, T=T, H=H, Dk=Dk, Dv=Dv, chunk=C))
        byts = prefill_bytes(B, T, H, Dk, Dv)
        flops = prefill_flops(B, T, H, Dk, Dv, C)
        # one kda_prefill call = chunk prep + state pass, back to back
        t_k = ms * 1e-3
        gbs = byts / t_k / 1e9
        srcs = ["kda_prep_d128.hip", "kda_prep_impl.h", "kda_state.hip",
                "kda_device.h"]
        tr_p = traffic_for("kda_chunk_prep", srcs)
        tr_s = traffic_for("kda_state_pass", srcs)
        out["prefill"] = dict(
            ms_per_step=ms, tokens_per_s=B * T / (ms * 1e-3),
            kernel_ms={"kda_chunk_prep": tp, "kda_state_pass": ts},
            algo_bytes=byts, algo_flops=flops,
            roofline=dict(
                kernel="kda_prefill call (kda_chunk_prep then "
                       "kda_state_pass)",
                bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=gbs / HBM_PEAK_GBS,
                traffic=(None if tr_p is None or tr_s is None
                         else tr_p + tr_s)),
            mfma=dict(achieved=flops / t_k / 1e12,
                      peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=flops / t_k / 1e12 / MFMA_BF16_PEAK_TFLOPS))
        mb = mfma_busy_for("prefill", srcs)
        if mb is not None:
            # rocprofv3: SQ_VALU_MFMA_BUSY_CYCLES over all SIMD cycles
            out["prefill"]["mfma"]["busy_frac_rocprof"] = {
                "kda_chunk_prep": mb["kernels"]["kda_chunk_prep"]["mfma_busy_frac"],
                "kda_state_pass": mb["kernels"]["kda_state_pass"]["mfma_busy_frac"],
                "call": mb["prefill_call_busy_frac"],
                "source": "profiles/mfma_busy.md"}
        log(f"prefill: {ms*1e3:.1f} us/step (prep {tp*1e3:.1f} us, state "
            f"{ts*1e3:.1f} us), {gbs:.0f} GB/s algorithmic")
        rf = state_loads_alone(ws, B * H, (T + C - 1) // C, Dk, Dv, C)
        if rf is not None:
            rf["state_pass_over_loads_alone"] = (ts * 1e3) / rf["loads_alone_us"]
            out["prefill"]["state_pass_loads_alone"] = rf
            log(f"prefill: the state pass's loads alone take "
                f"{rf['loads_alone_us']:.1f} us (probe {rf['probe_us']:.1f} "
                f"us, {rf['bytes_per_cu_per_us']:.0f} B per workgroup per "
                f"us); state pass / loads alone = "
                f"{rf['state_pass_over_loads_alone']:.2f}")
        if not args.no_cpu:
            import oracle
            orc = oracle.get()
            log("prefill: oracle CPU baseline (whole workload, repeated)")
            xc = {n: t.detach().cpu() for n, t in x.items()}
            # whole-workload passes until about 10 s of host time: one pass
            # takes well under a second on the host's cores, so the median of
            # several is the reported rate
            passes = []
            while sum(passes) < 10.0 and len(passes) < 50:
                t0 = time.perf_counter()
                orc.recurrence(xc["q"], xc["k"], xc["v"], xc["g"],
                               xc["beta"])
                passes.append(time.perf_counter() - t0)
            dt = statistics.median(passes)
            out["cpu_baseline"] = dict(
                value=B * T / dt, unit="tokens/s", cores=orc.last_threads,
                kind="oracle",
                sample=f"whole prefill workload B{B} T{T} H{H} D{Dk} (fp64 "
                       f"token loop incl. exact upcast), median of "
                       f"{len(passes)} passes, {dt:.2f} s each, "
                       f"{sum(passes):.1f} s in all")
            del xc
        del x, ws, o, s
        torch.cuda.empty_cache()

    # ---------------- decode workload ---------------------------------------
    c3 = ki.workload(ki.DECODE)
    N, H3, D3, steps = c3["N"], c3["H"], c3["Dk"], c3["steps"]
    if args.decode_steps:
        steps = max(1, min(steps, args.decode_steps))
    if sel("decode") and not args.no_extra:
        log(f"decode: generating {steps} steps of inputs")
        st = ki.decode_state(N, H3, D3, D3, std=c3["state_std"], device=dev)
        xs = [ki.decode_step_inputs(N, H3, D3, D3, i, device=dev)
              for i in range(steps)]
        od = torch.empty((N, H3, D3), dtype=torch.bfloat16, device=dev)
        d0 = xs[0]
        settle(lambda: kda.kda_decode_step(d0["q"], d0["k"], d0["v"], d0["g"],
                                           d0["beta"], st, o=od))
        for i in range(10):
            d = xs[i]
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st,
                                o=od)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for d in xs:
            kda.kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st,
                                o=od)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        byts = decode_bytes(N, H3, D3, D3)
        state_b = N * H3 * D3 * D3 * 4 * 2
        gbs = byts / (ms * 1e-3) / 1e9
        tr = traffic_for("kda_decode", ["kda_decode.hip", "kda_device.h"])
        out["decode"] = dict(
            workload=c3["name"], steps=steps, us_per_step=ms * 1e3,
            tokens_per_s=N / (ms * 1e-3),
            state_gbs=state_b / (ms * 1e-3) / 1e9,
            roofline=dict(kernel="kda_decode", bound="hbm", achieved=gbs,
                          peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=gbs / HBM_PEAK_GBS, traffic=tr))
        log(f"decode: {ms*1e3:.1f} us/step, {gbs:.0f} GB/s")
        del xs, st
        torch.cuda.empty_cache()

    # ---------------- multi-token and conv decode calls ---------------------
    if sel("tokens") and not args.no_extra:
        st = ki.decode_state(N, H3, D3, D3, std=c3["state_std"], device=dev)
        dtok = out["decode_tokens"] = {}
        # the speculative-decoding verify step: 2 tokens per sequence (one
        # guessed token), state read and written once per call
        L = 2
        xt = ki.prefill_inputs(N, L, H3, D3, D3, qkv="bf16", gate="bf16",
                               seed=5, device=dev)
        ot = torch.empty((N, L, H3, D3), dtype=torch.bfloat16, device=dev)
        reps = max(10, steps // 5)
        callt = lambda: kda.kda_decode_tokens(xt["q"], xt["k"], xt["v"],
                                              xt["g"], xt["beta"], st,
                                              state_out=st, o=ot)
        settle(callt)
        for _ in range(5):
            callt()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            callt()
        e1.record(stream)
        torch.cuda.synchronize()
        mt = e0.elapsed_time(e1) / reps
        byt = N * H3 * (2 * D3 * D3 * 4 + L * (3 * D3 + 2 * D3 + 1) * 2)
        dtok["verify_step"] = dict(
            tokens_per_sequence=L, calls=reps, us_per_call=mt * 1e3,
            tokens_per_s=N * L / (mt * 1e-3),
            achieved_gbs=byt / (mt * 1e-3) / 1e9,
            hbm_frac=byt / (mt * 1e-3) / 1e9 / HBM_PEAK_GBS)
        log(f"decode verify (L={L}): {mt*1e3:.1f} us/call, "
            f"{N * L / (mt * 1e-3) / 1e6:.2f} M tokens/s")
        # the generation step with the conv prologue fused: raw projections
        # in, width-4 conv over the rolling history, history rolled forward
        CW = 4
        xc = ki.prefill_inputs(N, 1, H3, D3, D3, qkv="bf16", gate="bf16",
                               conv_width=CW, seed=6, device=dev)
        cache = torch.zeros((N, 3, H3 * D3, CW - 1), device=dev)
        oc = torch.empty((N, 1, H3, D3), dtype=torch.bfloat16, device=dev)
        conv = dict(xq=xc["xq"], xk=xc["xk"], xv=xc["xv"], wq=xc["wq"],
                    wk=xc["wk"], wv=xc["wv"], width=CW, l2norm_qk=True,
                    eps=1e-6)
        callc = lambda: kda.kda_decode_tokens(None, None, None, xc["g"],
                                              xc["beta"], st, state_out=st,
                                              o=oc, conv=conv,
                                              conv_state=cache)
        settle(callc)
        for _ in range(5):
            callc()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            callc()
        e1.record(stream)
        torch.cuda.synchronize()
        mc = e0.elapsed_time(e1) / reps
        # state in + out, raw x, g, beta, o, conv history read + written
        byc = (N * H3 * (2 * D3 * D3 * 4 + (3 * D3 + 2 * D3 + 1) * 2)
               + 2 * cache.numel() * 4)
        dtok["conv_step"] = dict(
            conv_width=CW, calls=reps, us_per_call=mc * 1e3,
            tokens_per_s=N / (mc * 1e-3),
            achieved_gbs=byc / (mc * 1e-3) / 1e9,
            hbm_frac=byc / (mc * 1e-3) / 1e9 / HBM_PEAK_GBS)
        log(f"decode step with fused conv: {mc*1e3:.1f} us/call")
        # the same step with two history buffers used in turn: the decode
        # kernel writes the rolled history into the other buffer itself
        cache2 = torch.zeros_like(cache)
        bufs = [cache, cache2]
        turn = [0]

        def callp():
            a = turn[0]
            turn[0] ^= 1
            kda.kda_decode_tokens(None, None, None, xc["g"], xc["beta"], st,
                                  state_out=st, o=oc, conv=conv,
                                  conv_state=bufs[a],
                                  conv_state_out=bufs[a ^ 1])
        settle(callp)
        for _ in range(6):
            callp()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            callp()
        e1.record(stream)
        torch.cuda.synchronize()
        mp = e0.elapsed_time(e1) / reps
        dtok["conv_step_two_buffers"] = dict(
            conv_width=CW, calls=reps, us_per_call=mp * 1e3,
            tokens_per_s=N / (mp * 1e-3),
            achieved_gbs=byc / (mp * 1e-3) / 1e9,
            hbm_frac=byc / (mp * 1e-3) / 1e9 / HBM_PEAK_GBS)
        log(f"decode step with fused conv, two history buffers: "
            f"{mp*1e3:.1f} us/call")
        del st, xt, xc, cache, cache2, bufs
        torch.cuda.empty_cache()

    # ---------------- fused-conv prefill and long context -------------------
    extra = {}
    for wl, tag in ((ki.CONV_PREFILL, "conv"), (ki.LONG, "long"),
                    (ki.PREFILL, "gdn")):
        if args.no_extra or not sel(tag):
            continue
        c = ki.workload(wl)
        log(f"{tag}: generating inputs")
        if tag == "gdn":
            # the headline shape with one gate per token-head (the Gated
            # DeltaNet special case): g shrinks from [B,T,H,Dk] to [B,T,H]
            x = ki.prefill_inputs(c["B"], c["T"], c["H"], c["Dk"], c["Dv"],
                                  qkv=c["qkv"], gate=c["gate"],
                                  seed=ki.SEED_BASE + 11, device=dev,
                                  gate_per_head=True)
        else:
            x = ki.workload_prefill_inputs(wl, device=dev)
        Bc, Tc, Hc, Dc, Cc = c["B"], c["T"], c["H"], c["Dk"], c["chunk"]
        conv = None
        if c["conv_width"]:
            conv = dict(xq=x["xq"], xk=x["xk"], xv=x["xv"], wq=x["wq"],
                        wk=x["wk"], wv=x["wv"], width=c["conv_width"],
                        l2norm_qk=True, eps=1e-6)
        ws = kda.alloc_workspace(Bc, Tc, Hc, Dc, Dc, Cc, torch.bfloat16, dev)
        o = torch.empty((Bc, Tc, Hc, Dc), dtype=torch.bfloat16, device=dev)
        s = torch.empty((Bc, Hc, Dc, Dc), dtype=torch.float32, device=dev)
        f = lambda: kda.kda_prefill(x.get("q"), x.get("k"), x.get("v"),
                                    x["g"], x["beta"], chunk=Cc, conv=conv,
                                    o=o, s_out=s, workspace=ws)
        settle(f)
        f()
        torch.cuda.synchronize()
        reps = 5 if wl == ki.CONV_PREFILL else 3
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        if conv:
            byts = Bc * Tc * Hc * (3 * Dc * 2 + Dc * 4 + 4 + Dc * 2) + \
                3 * Hc * Dc * 4 * 4 + Bc * Hc * Dc * Dc * 4
        elif tag == "gdn":
            byts = prefill_bytes(Bc, Tc, Hc, Dc, Dc) - Bc * Tc * Hc * (Dc - 1) * 4
        else:
            byts = prefill_bytes(Bc, Tc, Hc, Dc, Dc)
        gbs = byts / (ms * 1e-3) / 1e9
        name = c["name"] + ("_head_gate" if tag == "gdn" else "")
        extra[name] = dict(ms_per_call=ms,
                                tokens_per_s=Bc * Tc / (ms * 1e-3),
                                algo_gbs=gbs, hbm_frac=gbs / HBM_PEAK_GBS)
        kinfo = ""
        if conv:
            # the conv + L2 prologue on its own (the unfused prologue):
            # the raw projections read once, q, k, v written once
            qc, kc, vc = (torch.empty_like(o) for _ in range(3))
            tcv = t_back_to_back(lambda: kda.kda_conv_prologue(
                x["xq"], x["xk"], x["xv"], x["wq"], x["wk"], x["wv"], H=Hc,
                Dk=Dc, Dv=Dc, q=qc, k=kc, v=vc), reps)
            cb = 6 * Bc * Tc * Hc * Dc * 2 + 3 * Hc * Dc * c["conv_width"] * 4
            extra[name]["conv_prologue_alone"] = dict(
                ms=tcv, algo_bytes=cb, algo_gbs=cb / (tcv * 1e-3) / 1e9,
                hbm_frac=cb / (tcv * 1e-3) / 1e9 / HBM_PEAK_GBS)
            kinfo = (f" (the conv prologue alone {tcv*1e3:.1f} us, "
                     f"{cb / (tcv * 1e-3) / 1e9:.0f} GB/s)")
            del qc, kc, vc
        if not conv:
            # the two kernels alone, back to back
            tp = t_back_to_back(lambda: kda.kda_prefill_chunk_prep(
                x["q"], x["k"], x["v"], x["g"], x["beta"], ws, chunk=Cc),
                reps)
            ts = t_back_to_back(lambda: kda.kda_prefill_state_pass(
                ws, o, s_out=s, B=Bc, T=Tc, H=Hc, Dk=Dc, Dv=Dc, chunk=Cc),
                reps)
            extra[name]["kernel_ms"] = {"kda_chunk_prep": tp,
                                        "kda_state_pass": ts}
            if tag == "gdn" and "prefill" in out:
                # the scalar-gate prep against the per-channel prep of the
                # same shape (headline workload)
                extra[name]["prep_vs_per_channel_prep"] = \
                    tp / out["prefill"]["kernel_ms"]["kda_chunk_prep"]
            kinfo = f" (prep {tp*1e3:.1f} us, state {ts*1e3:.1f} us)"
        log(f"{tag}: {ms:.3f} ms/call{kinfo}, {gbs:.0f} GB/s algorithmic")
        del x, ws, o, s
        torch.cuda.empty_cache()

    # ---------------- the oracle on the other workloads (CPU) ---------------
    # bounded samples of each workload (a few seconds of host time each),
    # the same fp64 token loop as cpu_baseline, on the host's cores
    if not args.no_cpu and not args.no_extra and only is None:
        import oracle
        orc = oracle.get()
        ocpu = extra["oracle_cpu"] = {}

        def t_oracle(fn):
            t0 = time.perf_counter()
            fn()
            return time.perf_counter() - t0

        c = ki.workload(ki.CONV_PREFILL)
        log("oracle: conv prefill sample")
        Bs = 2  # two of the eight sequences, every token and head
        xc = ki.prefill_inputs(Bs, c["T"], c["H"], c["Dk"], c["Dv"],
                               qkv=c["qkv"], gate=c["gate"],
                               conv_width=c["conv_width"], seed=c["seed"],
                               device=dev)
        xc = {n: t.detach().cpu() for n, t in xc.items()}
        conv = dict(xq=xc["xq"], xk=xc["xk"], xv=xc["xv"], wq=xc["wq"],
                    wk=xc["wk"], wv=xc["wv"], eps=1e-6, l2norm_qk=True)
        dt = t_oracle(lambda: orc.prefill(None, None, None, xc["g"],
                                          xc["beta"], conv=conv))
        ocpu[c["name"]] = dict(
            value=Bs * c["T"] / dt, unit="tokens/s", cores=orc.last_threads,
            kind="oracle", seconds=dt,
            sample=f"batch rows 0-{Bs - 1} of B{c['B']} (T{c['T']}, all "
                   f"{c['H']} heads): fp64 conv, L2 and token loop")
        del xc, conv
        c = ki.workload(ki.DECODE)
        nst = 50
        log(f"oracle: decode sample ({nst} steps)")
        st0 = ki.decode_state(c["N"], c["H"], c["Dk"], c["Dv"],
                              std=c["state_std"], device=dev).cpu()
        xs = [ki.decode_step_inputs(c["N"], c["H"], c["Dk"], c["Dv"], i,
                                    device=dev) for i in range(nst)]
        seq = {n: torch.stack([x[n] for x in xs], 1).cpu()
               for n in ("q", "k", "v", "g", "beta")}
        del xs
        dt = t_oracle(lambda: orc.recurrence(seq["q"], seq["k"], seq["v"],
                                             seq["g"], seq["beta"], st0))
        ocpu[c["name"]] = dict(
            value=c["N"] * nst / dt, unit="tokens/s", cores=orc.last_threads,
            kind="oracle", seconds=dt,
            sample=f"the first {nst} of {c['steps']} steps, all {c['N']} "
                   f"sequences x {c['H']} heads (fp64 state per head kept "
                   "across the steps)")
        del seq, st0
        c = ki.workload(ki.LONG)
        Ts = 16384
        log(f"oracle: long-context sample ({Ts} tokens)")
        xl = ki.prefill_inputs(c["B"], Ts, c["H"], c["Dk"], c["Dv"],
                               qkv=c["qkv"], gate=c["gate"],
                               gate_kind=c["gate_kind"], seed=c["seed"],
                               device=dev)
        xl = {n: t.detach().cpu() for n, t in xl.items()}
        dt = t_oracle(lambda: orc.recurrence(xl["q"], xl["k"], xl["v"],
                                             xl["g"], xl["beta"]))
        ocpu[c["name"]] = dict(
            value=Ts / dt, unit="tokens/s", cores=orc.last_threads,
            kind="oracle", seconds=dt,
            sample=f"the first {Ts} of {c['T']} tokens, all {c['H']} heads "
                   "(the token loop's cost per token does not depend on "
                   "the position)")
        del xl
        for name, r in ocpu.items():
            log(f"oracle {name}: {r['value']:.0f} {r['unit']} on "
                f"{r['cores']} threads ({r['seconds']:.1f} s)")

    # ---------------- backward of the headline prefill ---------------------
    if sel("bwd") and not args.no_extra:
        c = ki.workload(ki.PREFILL)
        Bc, Tc, Hc, Dc, Cc = c["B"], c["T"], c["H"], c["Dk"], c["chunk"]
        log("bwd: generating inputs")
        x = ki.workload_prefill_inputs(ki.PREFILL, device=dev)
        gen = torch.Generator(device=dev).manual_seed(7)
        do = torch.randn((Bc, Tc, Hc, Dc), generator=gen,
                         device=dev).to(torch.bfloat16)
        ws = torch.empty(kda.kda_prefill_backward_workspace_size(
            Bc, Tc, Hc, Dc, Dc, Cc, torch.bfloat16), dtype=torch.uint8,
            device=dev)
        fb = lambda: kda.kda_prefill_backward(x["q"], x["k"], x["v"], x["g"],
                                              x["beta"], do, chunk=Cc,
                                              workspace=ws)
        settle(fb)
        fb()
        torch.cuda.synchronize()
        reps = 5
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(reps):
            fb()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tok = Bc * Tc * Hc
        # inputs q,k,v,dO (bf16), g (fp32), beta read once; dq,dk,dv (bf16),
        # dg (fp32), dbeta written once; ds0 written
        byts = tok * (4 * Dc * 2 + Dc * 4 + 4 + 3 * Dc * 2 + Dc * 4 + 4) + \
            Bc * Hc * Dc * Dc * 4
        gbs = byts / (ms * 1e-3) / 1e9
        extra[c["name"] + "_backward"] = dict(
            ms_per_call=ms, tokens_per_s=Bc * Tc / (ms * 1e-3), algo_gbs=gbs,
            hbm_frac=gbs / HBM_PEAK_GBS,
            vs_forward=ms / out["prefill"]["ms_per_step"]
            if "prefill" in out else None)
        log(f"bwd: {ms:.3f} ms/call, {gbs:.0f} GB/s algorithmic")
        del x, do, ws
        torch.cuda.empty_cache()

    # ---------------- copy reference for the byte counters -----------------
    # (and the practical streaming ceiling the decode step is compared with)
    if sel("copy"):
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b2 = torch.empty_like(a)
        for _ in range(3):
            b2.copy_(a)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        b2.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out["copy"] = dict(bytes_read=n, bytes_written=n, ms=ms,
                           gbs=2 * n / (ms * 1e-3) / 1e9)
        log(f"copy: 1 GiB in {ms:.3f} ms, {2 * n / (ms * 1e-3) / 1e9:.0f} "
            "GB/s read+write")
        del a, b2
        # the decode state's traffic shape with next to no arithmetic: 512 MiB
        # fp32 scaled in place by torch's elementwise kernel (a practical
        # ceiling for a streaming read-modify-write on this part)
        sref = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        settle(lambda: sref.mul_(0.999))
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(20):
            sref.mul_(0.999)
        e1.record(stream)
        torch.cuda.synchronize()
        ms2 = e0.elapsed_time(e1) / 20
        out["copy"]["inplace_scale_512mib"] = dict(
            ms=ms2, gbs=2 * sref.numel() * 4 / (ms2 * 1e-3) / 1e9)
        log(f"in-place scale of 512 MiB fp32: {ms2:.3f} ms, "
            f"{2 * sref.numel() * 4 / (ms2 * 1e-3) / 1e9:.0f} GB/s read+write")
        del sref
        dec = out.get("decode")
        if dec is not None:
            # the decode step's state traffic against the same read-modify-
            # write pattern with next to no arithmetic
            dec["vs_inplace_scale"] = dec["state_gbs"] / (
                2 * (1 << 27) * 4 / (ms2 * 1e-3) / 1e9)

    pf = out.get("prefill")
    line = {
        "metric": METRIC,
        "value": pf["tokens_per_s"] if pf else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": pf["ms_per_step"] if pf else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the "
                "KDA workloads)",
        "config": {"workload": ki.PREFILL, "B": B, "T": T, "H": H,
                   "d_k": Dk, "d_v": Dv, "chunk": C, "qkv": "bf16",
                   "gate": "f32", "state": "f32"},
        "roofline": pf["roofline"] if pf else None,
        "cpu_baseline": out.get("cpu_baseline"),
        "prefill": ({k: v for k, v in pf.items() if k != "roofline"}
                    if pf else None),
        "decode": out.get("decode"),
        "decode_tokens": out.get("decode_tokens"),
        "extra": extra,
    }
    if "copy" in out:
        line["copy"] = out["copy"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
