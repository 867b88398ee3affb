#!/usr/bin/env python3
"""Benchmark of the Jamba Mamba-1 mixer library on one MI355X.

One step = one jm_mixer_prefill call, i.e. every step of the mixer: conv1d + SiLU, x_proj, the dt/B/C
RMSNorms, dt_proj + softplus, the selective scan, the D skip and the SiLU(z) gate.  The headline workload is
the largest single-GPU one, the 256K-token context (B=1, L=262144, d_inner=8192, d_state=16, dt_rank=256,
bf16 I/O, fp32 state); the 4K prefill (B=1), the batched prefill (B=8, L=4096) and the B=256 decode step are
timed the same way and reported alongside.  Inputs are seeded synthetic tensors already resident in HBM.
W untimed warmup steps, then K timed steps between device synchronisations (events on the stream the
library launches on); value = tokens / second.  A second timed pass records HIP events between the
library's kernels (jm_mixer_prefill_profiled) for the per-kernel roofline: the scan + gate step (its local,
carry and full passes) against HBM with its fixed algorithmic bytes, its vector-ALU rate alongside.  The
decode workload rotates its fp32 state over 4 sets so that it streams from HBM.  The whole Mamba layer
around the mixer, the serving-style calls (a packed batch of prompts of mixed lengths, decode over a state
pool), the exact-ZOH and fp32 I/O variants and the gated scan's training forward and backward are timed at the
4K shapes, and the decode step as one cooperative kernel beside the default decode step.
The fp64 CPU oracle is timed first, on the host's cores, on a prefix of the headline workload as a
baseline.

Prints one JSON line.  Only one GPU is supported: --gpus N with N > 1 exits with a message.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
# fp32 vector ALU without packed math: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz = 39.3 T
# lane-operations/s (a SIMD completes one wave64 fp32 instruction every 4 clocks; AMD's 157.3 TFLOP/s fp32
# vector peak counts an FMA as two flops and a packed pair as two lanes: 39.3 x 2 x 2).  Transcendentals
# (exp, rcp) issue at half that rate: a throughput probe on the box (32 independent chains per lane, 8 waves
# per SIMD) took 4.6 nominal clocks per wave64 v_fma_f32 and 8.6 per v_exp_f32, so each counts as
# TRANS_SLOTS full-rate operations.
VALU_PEAK_TOPS = 39.3
TRANS_SLOTS = 1.9
N_STATE_SETS = 4               # decode state sets rotated per step (4 x 140 MB > the 256 MB last-level cache)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Hip:
    """hipEvent_t handles through the HIP runtime the process already uses (torch's)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def algorithmic_bytes(B, L, C, N, R, esize):
    """Fixed per-stage byte counts (what each step must move at minimum, in the I/O precision):
    conv: x in, xc out; x_proj: xc in, dbc out (fp32), W_x once (conv + x_proj as one kernel: x in, xc and dbc
    out, the weights once); norm + dt_proj: dbc in, delta out,
    B/C out (fp32), W_dt once; scan + gate: xc, delta, z in, B/C in, out, SSM state in and out (fp32)."""
    T = B * L
    W = R + 2 * N
    return {
        "conv_silu": T * C * 2 * esize + C * 5 * esize,
        "x_proj": T * C * esize + T * W * 4 + W * C * esize,
        # the two as one kernel (long inputs): x in, xc out, dbc out, the weights once
        "conv_silu_x_proj": T * C * 2 * esize + C * 5 * esize + T * W * 4 + W * C * esize,
        "norm_dt_proj": T * W * 4 + T * C * esize + T * 2 * N * 4 + C * R * esize + C * esize,
        "scan_gate": T * C * 4 * esize + T * 2 * N * 4 + 2 * B * C * N * 4 + C * (N + 1) * esize,
    }


def scan_alu_ops(B, L, C, N):
    """fp32 VALU work of the scan + gate as the recurrence defines it, one sequential pass over the tokens, in
    full-rate issue slots.  Per (token, channel, state): delta*A, its exponential, (delta*x)*B, the state FMA
    and the C.h FMA = 4 operations + 1 transcendental.  Per (token, channel): delta*x, the D*x FMA, y*SiLU(z)
    and SiLU's multiply, add and multiply = 6 operations + 2 transcendentals (exp, reciprocal)."""
    tc = B * L * C
    ops = tc * N * 4 + tc * 6
    trans = tc * N + tc * 2
    return ops + TRANS_SLOTS * trans


def scan_bwd_alu_ops(B, L, C, N):
    """fp32 VALU work of the scan's backward as the chain rule defines it, in full-rate issue slots, with the
    forward states recomputed (they are not kept between the two calls).  Per (token, channel, state): the
    state's recurrence again (delta*A, its exponential, (delta*x)*B, the FMA: 3 operations + 1 transcendental)
    and the reverse step (g = u + C*dy, g*h*a, the d delta terms, g*delta, d B, d x, d A, d C, C.h for y and
    u = a*g: 13 operations, reusing the exponential).  Per (token, channel): sigmoid(z) (exp, reciprocal),
    SiLU and its derivative, dy, dz, the D terms and d D: 11 operations + 2 transcendentals."""
    tc = B * L * C
    ops = tc * N * 16 + tc * 11
    trans = tc * N + tc * 2
    return ops + TRANS_SLOTS * trans


def decode_bytes(B, C, N, R, K, esize):
    """One decode step: per (sequence, channel) the fp32 state in and out, the conv state in and out, x and z
    in, out; plus every weight once."""
    W = R + 2 * N
    per = 2 * N * 4 + 2 * (K - 1) * esize + 3 * esize
    weights = (C * K + C + W * C + R + 2 * N + C * R + C + C * N + C) * esize
    return B * C * per + weights


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary under
    profiles/, or None when there is none for this workload or the kernel sources changed since it was taken
    (the summary records the sha256 of the sources it measured)."""
    import hashlib

    short = workload.split("_", 2)[-1] if workload.startswith("jamba_prefill_") else workload
    path = os.path.join(ROOT, "profiles", f"{kernel}_{short}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    meta = json.load(open(path))
    if meta.get("workload") != workload or meta.get("kernel") != kernel:
        return None
    src = b"".join(open(os.path.join(ROOT, p), "rb").read() for p in meta["sources"])
    if hashlib.sha256(src).hexdigest() != meta["source_sha256"]:
        return None
    return int(meta["bytes_per_launch"])


def percentiles(vals_ms):
    """p10 / p50 / p90 of per-step times, in microseconds (nearest rank)."""
    v = sorted(vals_ms)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"p10": round(pick(0.1) * 1e3, 2), "p50": round(pick(0.5) * 1e3, 2), "p90": round(pick(0.9) * 1e3, 2)}


def stage_groups(stage_ms, conv_in_xproj=False):
    if conv_in_xproj:   # one kernel: its time is the x_proj stage's, the conv stage is empty
        front = {"conv_silu_x_proj": stage_ms["conv_silu"] + stage_ms["x_proj"]}
    else:
        front = {"conv_silu": stage_ms["conv_silu"], "x_proj": stage_ms["x_proj"]}
    return {
        **front,
        "norm_dt_proj": stage_ms["norm"] + stage_ms["dt_proj"],
        "scan_gate": stage_ms["scan_local"] + stage_ms["scan_carry"] + stage_ms["scan_full"],
    }


def time_prefill(jm, cfg, steps, warmup, hip, zoh=False):
    import torch
    from jm_inputs import make_activations, make_weights

    dev = "cuda"
    w = make_weights(cfg, dev)
    a = make_activations(cfg, dev)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps, zoh=zoh)
    B, L, C = cfg.batch, cfg.seqlen, cfg.d_inner
    out = torch.empty((B, L, C), dtype=cfg.torch_dtype, device=dev)
    cs = torch.empty((B, C, cfg.d_conv - 1), dtype=cfg.torch_dtype, device=dev)
    hs = torch.empty((B, C, cfg.d_state), dtype=torch.float32, device=dev)
    dims = m.dims(B, L)
    ws = m.workspace(jm.prefill_workspace_size(dims))
    stream = torch.cuda.current_stream().cuda_stream
    x, z = a["x"], a["z"]

    def step():
        s = jm.call_prefill(dims, m.packed, x.data_ptr(), z.data_ptr(), out.data_ptr(), None, cs.data_ptr(), None,
                            hs.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_mixer_prefill")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps

    # per-stage pass
    nst = 7
    names = [jm.lib().jm_stage_name(i).decode() for i in range(nst)]
    evs = hip.events(steps * (nst + 1))
    arr_t = ctypes.c_void_p * (nst + 1)
    L_ = jm.lib()
    L_.jm_mixer_prefill_profiled.restype = ctypes.c_int
    for k in range(steps):
        arr = arr_t(*[e.value for e in evs[k * (nst + 1):(k + 1) * (nst + 1)]])
        s = L_.jm_mixer_prefill_profiled(ctypes.byref(dims), ctypes.byref(m.packed), ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(z.data_ptr()), ctypes.c_void_p(out.data_ptr()), None,
                                         ctypes.c_void_p(cs.data_ptr()), None, ctypes.c_void_p(hs.data_ptr()),
                                         ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                         ctypes.c_void_p(stream), arr, ctypes.c_int(nst + 1))
        if s != 0:
            raise jm.JMError(s, "jm_mixer_prefill_profiled")
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in names}
    per_step = []
    for k in range(steps):
        base = k * (nst + 1)
        for i, n in enumerate(names):
            stage_ms[n] += hip.elapsed_ms(evs[base + i], evs[base + i + 1]) / steps
        per_step.append(hip.elapsed_ms(evs[base], evs[base + nst]))
    hip.destroy(evs)
    lay = jm.workspace_layout(dims)
    return {"ms": ms, "wall_s": wall, "stage_ms": stage_ms, "splits": lay.dbc_splits, "pieces": lay.scan_chunks,
            "step_pct": percentiles(per_step), "conv_in_xproj": lay.xproj_path == 4}


def time_decode(jm, cfg, steps, warmup, hip, single=False):
    import torch
    from jm_inputs import make_state, make_weights

    dev = "cuda"
    w = make_weights(cfg, dev)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    B, C = cfg.batch, cfg.d_inner
    st = make_state(cfg, dev)
    sets = [(st["conv_state"].clone(), st["ssm_state"].clone()) for _ in range(N_STATE_SETS)]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    xs = torch.randn((8, B, C), generator=g, device=dev).to(cfg.torch_dtype)
    zs = torch.randn((8, B, C), generator=g, device=dev).to(cfg.torch_dtype)
    out = torch.empty((B, C), dtype=cfg.torch_dtype, device=dev)
    dims = m.dims(B, 1)
    ws = m.workspace(jm.decode_workspace_size(dims))
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        c, h = sets[i % N_STATE_SETS]
        if single:
            s = jm.call_decode_step_single_kernel(dims, m.packed, xs[i % 8].data_ptr(), zs[i % 8].data_ptr(),
                                                  out.data_ptr(), c.data_ptr(), c.data_ptr(), h.data_ptr(),
                                                  h.data_ptr(), 0, None, ws.data_ptr(), ws.numel(), stream)
        else:
            s = jm.call_decode_step(dims, m.packed, xs[i % 8].data_ptr(), zs[i % 8].data_ptr(), out.data_ptr(),
                                    c.data_ptr(), c.data_ptr(), h.data_ptr(), h.data_ptr(), ws.data_ptr(),
                                    ws.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_mixer_decode_step_single_kernel" if single else "jm_mixer_decode_step")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if single:
        return {"ms": ms}

    nst = 7
    names = [jm.lib().jm_stage_name(i).decode() for i in range(nst)]
    evs = hip.events(steps * (nst + 1))
    arr_t = ctypes.c_void_p * (nst + 1)
    L_ = jm.lib()
    for k in range(steps):
        c, h = sets[k % N_STATE_SETS]
        arr = arr_t(*[e.value for e in evs[k * (nst + 1):(k + 1) * (nst + 1)]])
        s = L_.jm_mixer_decode_step_profiled(
            ctypes.byref(dims), ctypes.byref(m.packed), ctypes.c_void_p(xs[k % 8].data_ptr()),
            ctypes.c_void_p(zs[k % 8].data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(c.data_ptr()),
            ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(h.data_ptr()),
            ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream), arr,
            ctypes.c_int(nst + 1))
        if s != 0:
            raise jm.JMError(s, "jm_mixer_decode_step_profiled")
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in names}
    per_step = []
    for k in range(steps):
        base = k * (nst + 1)
        for i, n in enumerate(names):
            stage_ms[n] += hip.elapsed_ms(evs[base + i], evs[base + i + 1]) / steps
        per_step.append(hip.elapsed_ms(evs[base], evs[base + nst]))
    hip.destroy(evs)
    return {"ms": ms, "stage_ms": stage_ms, "step_pct": percentiles(per_step)}


# The CPU baseline's scan runs over channel blocks in forked workers (the recurrence is independent per
# channel once delta, B and C are known); the parent sets this before forking and the workers write their
# block of the output into a shared array.
_CPU_JOB = {}


def _cpu_scan_block(c0c1):
    import numpy as np

    import oracle
    j = _CPU_JOB
    c0, c1 = c0c1
    y, _ = oracle.selective_scan(j["xc"][..., c0:c1], j["delta"][..., c0:c1], j["A_log"][c0:c1], j["bn"], j["cn"],
                                 j["D"][c0:c1], None)
    out = np.frombuffer(j["out"], dtype=np.float64).reshape(j["shape"])
    out[..., c0:c1] = y * oracle.silu(j["z"][..., c0:c1])
    return c1 - c0


def cpu_baseline(cfg, max_tokens):
    """The fp64 oracle (as it stands) on the host's cores, on the first max_tokens tokens of the workload (the
    oracle's cost is linear in the tokens, so tokens/s on a prefix is its rate on the whole sequence).  The
    conv, the projections and the norms run as the oracle's numpy calls, the matmuls on the BLAS threads;
    the scan and the gate run as the oracle's own functions over channel blocks in one forked worker per
    core.  Runs before anything touches the GPU."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from jm_inputs import make_activations, make_weights, to_f64

    cores = len(os.sched_getaffinity(0))
    w = {k: to_f64(v) for k, v in make_weights(cfg).items()}
    L = min(cfg.seqlen, max_tokens)
    a = make_activations(cfg, "cpu", seqlen=L)
    x, z = to_f64(a["x"]), to_f64(a["z"])
    del a
    B, C = cfg.batch, cfg.d_inner
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t0 = time.perf_counter()
    xc, _ = oracle.causal_conv1d_silu(x, w["conv_w"], w["conv_b"], None)
    dl, bv, cv = oracle.split_dbc(oracle.x_proj(xc, w["x_proj_w"]), cfg.dt_rank, cfg.d_state)
    dln = oracle.rms_norm(dl, w["dt_norm_w"], cfg.norm_eps)
    bn = oracle.rms_norm(bv, w["b_norm_w"], cfg.norm_eps)
    cn = oracle.rms_norm(cv, w["c_norm_w"], cfg.norm_eps)
    delta = oracle.dt_proj_softplus(dln, w["dt_proj_w"], w["dt_proj_b"])
    t_front = time.perf_counter() - t0
    shared = mp.RawArray("d", B * L * C)
    _CPU_JOB.update(xc=xc, delta=delta, bn=bn, cn=cn, A_log=w["A_log"], D=w["D"], z=z, out=shared,
                    shape=(B, L, C))
    nblk = max(1, min(cores, C // 64))
    edges = [C * i // nblk for i in range(nblk + 1)]
    with mp.get_context("fork").Pool(nblk) as pool:
        done = sum(pool.map(_cpu_scan_block, list(zip(edges[:-1], edges[1:]))))
    dt = time.perf_counter() - t0
    out = np.frombuffer(shared, dtype=np.float64).reshape(B, L, C)
    assert done == C and np.isfinite(out).all()
    _CPU_JOB.clear()
    return {"value": B * L / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle, prefill of the first {L} of the {cfg.seqlen} tokens of {cfg.name} "
                      f"(B={B}, C={C}; the oracle is linear in the tokens), {dt:.1f} s: conv, projections and "
                      f"norms {t_front:.1f} s with matmuls on {blas} BLAS threads, then the scan and gate over "
                      f"{nblk} channel blocks in {nblk} forked workers; cores = the host cores this process may "
                      f"use (sched_getaffinity)"}


def time_layer(jm, cfg, steps, warmup, decode):
    """The whole Mamba layer (pre-norm, in_proj, mixer, out_proj, residual) on the same synthetic workload;
    decode rotates the states like the mixer's decode timing."""
    import torch
    from jm_inputs import make_layer_input, make_layer_weights, make_state, make_weights

    dev = "cuda"
    layer = jm.Layer(make_layer_weights(cfg, dev), make_weights(cfg, dev), cfg.dt_rank, cfg.d_state, cfg.d_conv,
                     cfg.norm_eps, 1e-6)
    B, C = cfg.batch, cfg.d_inner
    L = 1 if decode else cfg.seqlen
    dims = layer.dims(B, L)
    ws = layer.workspace(jm.layer_workspace_size(dims, decode))
    stream = torch.cuda.current_stream().cuda_stream
    if decode:
        st = make_state(cfg, dev)
        sets = [(st["conv_state"].clone(), st["ssm_state"].clone()) for _ in range(N_STATE_SETS)]
        xs = make_layer_input(cfg, dev, steps=8)
        xin = [xs[:, i].contiguous() for i in range(8)]
    else:
        xin = [make_layer_input(cfg, dev)]
        cs = torch.empty((B, C, cfg.d_conv - 1), dtype=cfg.torch_dtype, device=dev)
        hs = torch.empty((B, C, cfg.d_state), dtype=torch.float32, device=dev)
    out = torch.empty_like(xin[0])

    def step(i):
        if decode:
            c, h = sets[i % N_STATE_SETS]
            ptrs = (c.data_ptr(), c.data_ptr(), h.data_ptr(), h.data_ptr())
        else:
            ptrs = (None, cs.data_ptr(), None, hs.data_ptr())
        s = jm.call_layer(dims, layer.packed, xin[i % len(xin)].data_ptr(), out.data_ptr(), *ptrs, ws.data_ptr(),
                          ws.numel(), stream, decode)
        if s != 0:
            raise jm.JMError(s, "jm_layer_decode_step" if decode else "jm_layer_prefill")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    Dm = cfg.d_model
    gemm_flops = 2.0 * B * L * Dm * (2 * C) + 2.0 * B * L * C * Dm
    return {"workload": f"{cfg.name}: whole Mamba layer (RMSNorm, in_proj, mixer, out_proj, residual)",
            "batch": B, "seq_len": L, "d_model": Dm, "us_per_step": round(ms * 1e3, 2),
            "tokens_per_s": round(B * L / (ms * 1e-3), 1), "gemm_flops_per_step": gemm_flops}


def time_serving(jm, steps, warmup):
    """The serving-style calls at Jamba v0.1's widths: a packed batch of 8 prompts of mixed lengths (4096
    tokens) prefilled in place into rows of a 64-row state pool, and a B=256 decode step over a 1024-row pool
    (four disjoint slot sets rotated, so the states stream from HBM as in the plain decode timing)."""
    import torch
    from jm_inputs import SERVING_CONFIGS, SERVING_POOL_ROWS, make_activations, make_state, make_weights, \
        packed_lengths, pool_slots

    dev = "cuda"
    stream = torch.cuda.current_stream().cuda_stream
    res = {}

    def timed(step):
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # packed variable-length prefill
    cfg, rows = SERVING_CONFIGS[0], SERVING_POOL_ROWS[0]
    w = make_weights(cfg, dev)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    T, C = cfg.seqlen, cfg.d_inner
    a = make_activations(cfg.replace(batch=1), dev)
    x, z = a["x"][0].contiguous(), a["z"][0].contiguous()
    lens = packed_lengths(T, cfg.batch, cfg.seed)
    cu = torch.tensor([0] + [sum(lens[:k + 1]) for k in range(len(lens))], dtype=torch.int32, device=dev)
    slots = torch.tensor(pool_slots(cfg.batch, rows, cfg.seed), dtype=torch.int32, device=dev)
    st = make_state(cfg.replace(batch=rows), dev)
    cp, hp = st["conv_state"], st["ssm_state"]
    out = torch.empty((T, C), dtype=cfg.torch_dtype, device=dev)
    dims = m.dims(cfg.batch, T)
    ws = m.workspace(jm.varlen_workspace_size(dims))

    def pre_step(i):
        s = jm.call_prefill_varlen(dims, m.packed, x.data_ptr(), z.data_ptr(), out.data_ptr(), cu.data_ptr(),
                                   cp.data_ptr(), cp.data_ptr(), hp.data_ptr(), hp.data_ptr(), slots.data_ptr(),
                                   rows, ws.data_ptr(), ws.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_mixer_prefill_varlen")

    log(f"serving {cfg.name}: lengths {lens}")
    ms = timed(pre_step)
    res["varlen_prefill"] = {"workload": f"{cfg.name}: {cfg.batch} prompts of mixed lengths packed into {T} "
                                         f"tokens, states in place in a {rows}-row pool",
                             "lengths": lens, "us_per_step": round(ms * 1e3, 2),
                             "tokens_per_s": round(T / (ms * 1e-3), 1)}
    del m, w, x, z, a, st, cp, hp, out
    # decode over a state pool
    cfg, rows = SERVING_CONFIGS[1], SERVING_POOL_ROWS[1]
    w = make_weights(cfg, dev)
    m = jm.Mixer(w, cfg.dt_rank, cfg.d_state, cfg.d_conv, cfg.norm_eps)
    B, C = cfg.batch, cfg.d_inner
    st = make_state(cfg.replace(batch=rows), dev)
    cp, hp = st["conv_state"], st["ssm_state"]
    perm = pool_slots(rows, rows, cfg.seed)
    sets = [torch.tensor(perm[k * B:(k + 1) * B], dtype=torch.int32, device=dev) for k in range(rows // B)]
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    xs = torch.randn((8, B, C), generator=g, device=dev).to(cfg.torch_dtype)
    zs = torch.randn((8, B, C), generator=g, device=dev).to(cfg.torch_dtype)
    out = torch.empty((B, C), dtype=cfg.torch_dtype, device=dev)
    dims = m.dims(B, 1)
    ws = m.workspace(jm.decode_workspace_size(dims))

    def dec_step(i):
        s = jm.call_decode_step_slots(dims, m.packed, xs[i % 8].data_ptr(), zs[i % 8].data_ptr(), out.data_ptr(),
                                      cp.data_ptr(), hp.data_ptr(), rows, sets[i % len(sets)].data_ptr(),
                                      ws.data_ptr(), ws.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_mixer_decode_step_slots")

    log(f"serving {cfg.name}")
    ms = timed(dec_step)
    db = decode_bytes(B, C, cfg.d_state, cfg.dt_rank, cfg.d_conv, 2)
    gbs = db / (ms * 1e-3) / 1e9
    res["decode_slots"] = {"workload": f"{cfg.name}: B={B} decode, states in a {rows}-row pool, "
                                       f"{len(sets)} disjoint slot sets rotated",
                           "batch": B, "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(B / (ms * 1e-3), 1),
                           "alg_bytes": db, "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def time_training(jm, steps, warmup):
    """The gated scan alone at the 4K prefill's shape (B=1, L=4096, d_inner 8192, bf16): its forward
    (jm_scan_forward) and backward (jm_scan_backward, recomputing the piece states), timed separately, the
    saving forward (jm_scan_forward_train) and the backward given its saved states, alone and as the training
    pair."""
    import torch
    from jm_inputs import CONFIGS, make_scan_problem

    cfg = CONFIGS[1].replace(name="jamba_scan_train_B1_L4096", seed=1301)
    p = make_scan_problem(cfg, "cuda")
    B, L, C, N = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state
    dims = jm.scan_dims(B, L, C, jm.JM_BF16)
    L_ = jm.lib()
    wsf = torch.empty(jm.scan_workspace_size(dims), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(jm.scan_workspace_size(dims, True), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(p["x"])
    h_out = torch.empty((B, C, N), dtype=torch.float32, device="cuda")
    g = {k: torch.empty_like(p["x"]) for k in ("dx", "ddelta", "dz")}
    dbc = torch.empty((B * L, 2 * N), dtype=torch.float32, device="cuda")
    dA = torch.empty((C, N), dtype=torch.float32, device="cuda")
    dD = torch.empty((C,), dtype=torch.float32, device="cuda")
    dh0 = torch.empty((B, C, N), dtype=torch.float32, device="cuda")
    saved = torch.empty(jm.scan_saved_states_size(dims) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()

    def fwd(i):
        s = L_.jm_scan_forward(ctypes.byref(dims), ptr(p["x"]), ptr(p["delta"]), ptr(p["z"]), ptr(p["bc"]),
                               ptr(p["A_log"]), ptr(p["D"]), ptr(p["h0"]), ptr(out), ptr(h_out), ptr(wsf), wsf.numel(),
                               stream)
        if s != 0:
            raise jm.JMError(s, "jm_scan_forward")

    def fwd_train(i):
        s = L_.jm_scan_forward_train(ctypes.byref(dims), ptr(p["x"]), ptr(p["delta"]), ptr(p["z"]), ptr(p["bc"]),
                                     ptr(p["A_log"]), ptr(p["D"]), ptr(p["h0"]), ptr(out), ptr(h_out), ptr(saved),
                                     ptr(wsf), wsf.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_scan_forward_train")

    def bwd(i, states=None):
        s = L_.jm_scan_backward(ctypes.byref(dims), ptr(p["x"]), ptr(p["delta"]), ptr(p["z"]), ptr(p["bc"]),
                                ptr(p["A_log"]), ptr(p["D"]), ptr(p["h0"]), ptr(p["dout"]), ptr(p["dh_final"]),
                                ptr(states), ptr(g["dx"]), ptr(g["ddelta"]), ptr(g["dz"]), ptr(dbc), ptr(dA), ptr(dD),
                                ptr(dh0), ptr(wsb), wsb.numel(), stream)
        if s != 0:
            raise jm.JMError(s, "jm_scan_backward")

    def train_pair(i):
        fwd_train(i)
        bwd(i, saved)

    res = {"workload": f"{cfg.name}: the gated scan alone, B={B} L={L} d_inner={C}, bf16 I/O, fp32 state"}
    bwd_saved = lambda i: bwd(i, saved)   # the states forward_train left in `saved` (timed after it)
    for name, step in (("forward", fwd), ("backward", bwd), ("forward_train", fwd_train),
                       ("backward_from_saved", bwd_saved), ("forward_train_plus_backward", train_pair)):
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"us": round(ms * 1e3, 2), "tokens_per_s": round(B * L / (ms * 1e-3), 1)}
        if name in ("forward", "backward"):
            ops = scan_alu_ops(B, L, C, N) if name == "forward" else scan_bwd_alu_ops(B, L, C, N)
            ach = ops / (ms * 1e-3) / 1e12
            res[name].update({"alg_ops": ops, "T_lane_ops_s": round(ach, 2),
                              "frac_alu": round(ach / VALU_PEAK_TOPS, 4)})
        log(f"  scan {name}: {ms * 1e3:.1f} us")
    # the backward that recomputes the piece states, and the one a training step runs after
    # jm_scan_forward_train, each against the plain forward
    res["backward_over_forward"] = round(res["backward"]["us"] / res["forward"]["us"], 2)
    res["backward_from_saved_over_forward"] = round(res["backward_from_saved"]["us"] / res["forward"]["us"], 2)
    res["saved_states_bytes"] = saved.numel() * 4
    return res


def run_decode(jm, dcfg, args, hip):
    log(f"decode {dcfg.name}: warmup {args.warmup}, steps {args.steps}")
    dec = time_decode(jm, dcfg, args.steps, args.warmup, hip)
    db = decode_bytes(dcfg.batch, dcfg.d_inner, dcfg.d_state, dcfg.dt_rank, dcfg.d_conv, 2)
    gbs = db / (dec["ms"] * 1e-3) / 1e9
    stages = dec["stage_ms"]
    # the single-kernel step records every stage event after its one kernel: report it as one stage
    if sum(v for k, v in stages.items() if k != "conv_silu") < 0.01 * dec["ms"]:
        stages = {"decode_step_kernel": sum(stages.values())}
    for k, t in stages.items():
        log(f"  {k:12s} {t * 1e3:9.2f} us")
    return {"workload": f"{dcfg.name}: one token per sequence, state rotated over {N_STATE_SETS} sets",
            "batch": dcfg.batch, "us_per_step": round(dec["ms"] * 1e3, 2),
            "tokens_per_s": round(dcfg.batch / (dec["ms"] * 1e-3), 1), "alg_bytes": db,
            "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "step_us_events": dec["step_pct"],
            "stage_us": {k: round(v * 1e3, 2) for k, v in stages.items()}}


def run_prefill(jm, cfg, args, hip):
    """One prefill workload: tokens/s, per-stage times against their algorithmic bytes, and the scan + gate
    step against HBM (its roofline) with its vector-ALU rate alongside."""
    import torch

    log(f"prefill {cfg.name}: warmup {args.warmup}, steps {args.steps}")
    pre = time_prefill(jm, cfg, args.steps, args.warmup, hip)
    torch.cuda.empty_cache()
    B, L, C, N, R = cfg.batch, cfg.seqlen, cfg.d_inner, cfg.d_state, cfg.dt_rank
    tokens = B * L
    alg = algorithmic_bytes(B, L, C, N, R, 2)
    groups = stage_groups(pre["stage_ms"], pre["conv_in_xproj"])
    xp = "conv_silu_x_proj" if pre["conv_in_xproj"] else "x_proj"
    stages = {}
    for k, t in groups.items():
        gbs = alg[k] / (t * 1e-3) / 1e9 if t > 0 else 0.0
        stages[k] = {"us": round(t * 1e3, 2), "alg_bytes": alg[k], "GB_s": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    for k, t in pre["stage_ms"].items():
        log(f"  {k:12s} {t * 1e3:9.2f} us")
    xflops = 2.0 * tokens * (R + 2 * N) * C
    stages[xp]["mfma_tflops"] = round(xflops / (groups[xp] * 1e-3) / 1e12, 2)
    stages[xp]["frac_mfma_bf16"] = round(stages[xp]["mfma_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)
    dflops = 2.0 * tokens * R * C
    stages["norm_dt_proj"]["dt_proj_mfma_tflops"] = round(dflops / (pre["stage_ms"]["dt_proj"] * 1e-3) / 1e12, 2)
    # the dominant step: scan + gate (the local, carry and full passes of one launch of the scan), against
    # HBM with its fixed algorithmic bytes; its vector-ALU rate as a second figure
    dom = max(groups, key=lambda k: groups[k])
    ops = scan_alu_ops(B, L, C, N)
    sg = groups["scan_gate"]
    ach_alu = ops / (sg * 1e-3) / 1e12
    roofline = {"bound": "hbm", "kernel": dom, "achieved": stages[dom]["GB_s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": stages[dom]["frac_hbm"], "traffic": measured_traffic(cfg.name, dom),
                "alg_bytes_per_launch": alg[dom], "us_per_launch": stages[dom]["us"]}
    if dom == "scan_gate":
        roofline["launch"] = "scan_local + scan_carry + scan_full (one scan of the step)"
        roofline["alu"] = {"achieved": round(ach_alu, 2), "peak": VALU_PEAK_TOPS,
                           "unit": f"T fp32 lane-ops/s (transcendental = {TRANS_SLOTS})",
                           "frac": round(ach_alu / VALU_PEAK_TOPS, 4), "alg_ops_per_launch": int(ops)}
    return {
        "value": tokens / (pre["ms"] * 1e-3), "ms": pre["ms"],
        "config": {"workload": f"{cfg.name}: Jamba-v0.1 Mamba mixer prefill", "batch": B, "seq_len": L,
                   "d_inner": C, "d_state": N, "dt_rank": R, "d_conv": cfg.d_conv, "io": "bf16", "state": "fp32",
                   "x_proj_splits": pre["splits"], "scan_pieces": pre["pieces"]},
        "roofline": roofline, "stages": stages, "step_us_events": pre["step_pct"],
        "mixer_GB_s": round(sum(alg[k] for k in groups) / (pre["ms"] * 1e-3) / 1e9, 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the headline workload the CPU oracle runs (a prefix; default 65536)")
    ap.add_argument("--config", type=int, default=3, choices=(1, 2, 3),
                    help="headline prefill workload: 3 = B1 L262144 (default), 1 = B1 L4096, 2 = B8 L4096")
    ap.add_argument("--no-other-prefills", action="store_true",
                    help="skip the prefill workloads other than the headline one")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole-layer timing")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the variant timings (ZOH and fp32 prefill, single-kernel decode)")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the gated scan's training forward / backward timing")
    ap.add_argument("--training-only", action="store_true",
                    help="time only the scan's training forward / backward (for per-kernel profiles)")
    ap.add_argument("--no-serving", action="store_true",
                    help="skip the serving-style timings (packed prefill, pooled-state decode)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode workload and print its figures (for per-workload profiles)")
    ap.add_argument("--single-kernel-decode", action="store_true",
                    help="with --decode-only: also time jm_mixer_decode_step_single_kernel")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the headline prefill workload (for per-workload profiles)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three device copies of 256 MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported",
              file=sys.stderr)
        sys.exit(2)
    from jm_inputs import CONFIGS

    only = args.decode_only or args.training_only or args.prefill_only
    cfg = CONFIGS[args.config]
    cpu = None
    if not args.no_cpu_baseline and not only:
        # before anything touches the GPU: the baseline forks its scan workers
        log(f"cpu baseline: oracle on the first {min(args.cpu_tokens, cfg.seqlen)} tokens of {cfg.name} ...")
        cpu = cpu_baseline(cfg, args.cpu_tokens)
        log(f"  {cpu['value']:.1f} tokens/s on {cpu['cores']} cores")

    import torch

    import mamba_selective_scan_05_amd as jm

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    jm.lib()
    hip = Hip()
    if args.copy_calibration:
        src = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.decode_only:
        out = {"decode": run_decode(jm, CONFIGS[4], args, hip)}
        if args.single_kernel_decode:
            sk = time_decode(jm, CONFIGS[4], args.steps, args.warmup, hip, single=True)
            out["decode_single_kernel_us_per_step"] = round(sk["ms"] * 1e3, 2)
        print(json.dumps(out), flush=True)
        return
    if args.training_only:
        print(json.dumps({"training": time_training(jm, args.steps, args.warmup)}), flush=True)
        return
    head = run_prefill(jm, cfg, args, hip)
    result = {
        "metric": "mixer tokens/sec at d_inner=8192 (prefill & decode); achieved HBM GB/s % peak",
        "value": round(head["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "stages": head["stages"],
        # per-step times of the second (event-instrumented) pass: the events between kernels add a little
        "step_us_events": head["step_us_events"],
        "mixer_GB_s": head["mixer_GB_s"],
    }
    if args.prefill_only:
        print(json.dumps(result), flush=True)
        return
    if not args.no_other_prefills:
        others = {}
        for k in (1, 2, 3):
            if k == args.config:
                continue
            r = run_prefill(jm, CONFIGS[k], args, hip)
            others[CONFIGS[k].name] = {"tokens_per_s": round(r["value"], 1), "ms_per_step": round(r["ms"], 4),
                                       "config": r["config"], "scan_gate": r["roofline"] if r["roofline"]["kernel"]
                                       == "scan_gate" else None, "stages": r["stages"],
                                       "mixer_GB_s": r["mixer_GB_s"]}
        result["prefill_workloads"] = others
    if not args.no_decode:
        result["decode"] = run_decode(jm, CONFIGS[4], args, hip)
    one = CONFIGS[1]
    pre1 = result.get("prefill_workloads", {}).get(one.name)
    if not args.no_layer:
        from jm_inputs import LAYER_CONFIGS
        lay = {}
        for name, lcfg, dec in (("prefill", LAYER_CONFIGS[0], False), ("decode", LAYER_CONFIGS[1], True)):
            log(f"layer {lcfg.name}: warmup {args.warmup}, steps {args.steps}")
            lay[name] = time_layer(jm, lcfg, args.steps, args.warmup, dec)
            # the mixer's share of the step, from the mixer-only timings (4K prefill, decode)
            mix_us = (pre1["ms_per_step"] * 1e3 if pre1 else (head["ms"] * 1e3 if args.config == 1 else None)) \
                if name == "prefill" else result.get("decode", {}).get("us_per_step")
            if mix_us:
                rest = lay[name]["us_per_step"] - mix_us
                lay[name]["mixer_us"] = round(mix_us, 2)
                if rest > 0:
                    lay[name]["gemm_norm_us"] = round(rest, 2)
                    tflops = lay[name]["gemm_flops_per_step"] / (rest * 1e-6) / 1e12
                    lay[name]["gemm_tflops_estimate"] = round(tflops, 1)
            log(f"  {name}: {lay[name]['us_per_step']:.1f} us per step")
        result["layer"] = lay
    if not args.no_serving:
        result["serving"] = time_serving(jm, args.steps, args.warmup)
        # the packed batch holds the same 4096 tokens as the B=1 4K prefill
        v1 = pre1["tokens_per_s"] if pre1 else (head["value"] if args.config == 1 else None)
        if v1:
            result["serving"]["varlen_prefill"]["vs_B1_L4096_prefill"] = round(
                result["serving"]["varlen_prefill"]["tokens_per_s"] / v1, 3)
        if "decode" in result:
            result["serving"]["decode_slots"]["vs_plain_decode"] = round(
                result["decode"]["us_per_step"] / result["serving"]["decode_slots"]["us_per_step"], 3)
    if not args.no_variants:
        # the exact zero-order-hold input matrix instead of dt * B, on the 4K prefill
        log(f"prefill {one.name} with the exact ZOH input matrix: warmup {args.warmup}, steps {args.steps}")
        zp = time_prefill(jm, one, args.steps, args.warmup, hip, zoh=True)
        zg = stage_groups(zp["stage_ms"])
        ztok = one.batch * one.seqlen
        result["variants"] = {"zoh_prefill": {
            "workload": f"{one.name} with the exact zero-order-hold input matrix (exp(dt A) - 1) / A * B",
            "us_per_step": round(zp["ms"] * 1e3, 2), "tokens_per_s": round(ztok / (zp["ms"] * 1e-3), 1),
            "scan_gate_us": round(zg["scan_gate"] * 1e3, 2)}}
        if pre1:
            result["variants"]["zoh_prefill"]["vs_default"] = round(pre1["ms_per_step"] / zp["ms"], 3)
        # fp32 I/O (projections on the fp32 matrix cores, nothing rounded to bf16), on the 4K prefill
        f32 = one.replace(io_dtype="f32")
        log(f"prefill {one.name} with fp32 I/O: warmup {args.warmup}, steps {args.steps}")
        fp = time_prefill(jm, f32, args.steps, args.warmup, hip)
        result["variants"]["f32_prefill"] = {
            "workload": f"{one.name} with fp32 x, z, weights and outputs",
            "us_per_step": round(fp["ms"] * 1e3, 2), "tokens_per_s": round(ztok / (fp["ms"] * 1e-3), 1),
            "stage_us": {k: round(v * 1e3, 2) for k, v in fp["stage_ms"].items()}}
        # the decode step as one cooperative kernel (jm_mixer_decode_step_single_kernel), beside the default
        dcfg = CONFIGS[4]
        log(f"decode {dcfg.name} as one kernel: warmup {args.warmup}, steps {args.steps}")
        sk = time_decode(jm, dcfg, args.steps, args.warmup, hip, single=True)
        db = decode_bytes(dcfg.batch, dcfg.d_inner, dcfg.d_state, dcfg.dt_rank, dcfg.d_conv, 2)
        result["variants"]["decode_single_kernel"] = {
            "workload": f"{dcfg.name}: jm_mixer_decode_step_single_kernel, state rotated over {N_STATE_SETS} sets",
            "us_per_step": round(sk["ms"] * 1e3, 2), "tokens_per_s": round(dcfg.batch / (sk["ms"] * 1e-3), 1),
            "frac_hbm": round(db / (sk["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if "decode" in result:
            result["variants"]["decode_single_kernel"]["vs_default"] = round(
                result["decode"]["us_per_step"] / (sk["ms"] * 1e3), 3)
    if not args.no_training:
        log(f"training (scan forward / backward): warmup {args.warmup}, steps {args.steps}")
        result["training"] = time_training(jm, args.steps, args.warmup)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
