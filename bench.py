"""Benchmark: one speculative-decoding verify step on one MI355X.

Workload (the verify step at M = 16, K = 15):
  36 synthetic 4B-class layers x 4 W4A16 group-128 linears
  (2560->6144, 4096->2560, 2560->19456, 9728->2560) at M = 16 rows,
  an int8 lm_head 2560 -> 151,936 with fused per-row argmax, and greedy
  verification of 15 drafts whose accepted length is min(15, Geometric(0.25)).
A step = all 144 linears + the fused lm_head/argmax/verify launch, replayed
from a HIP graph; new drafts are copied in before every step.  All inputs
are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line (rank 0).  ``value`` is the step's algorithmic HBM
throughput in GB/s (bytes the step must read and write, divided by the
measured step time); verified tokens/s and the linears' own GB/s ride along.
``roofline`` covers the dominant kernel (the W4A16 linear): its algorithmic
bytes per launch over its average launch duration, timed with HIP events
on the stream it runs on.  ``cpu_baseline`` times the numpy oracle on a
bounded sample of the same workload on the host cores.  ``prefill`` (the
M = 2048 / 8192 linears), ``drafter`` (prompt-lookup drafting over
8192-token histories, the step before the verify) and ``drafter_int4_step``
(a 4-bit drafter's 21 linears at M = 16), ``g32_target_step`` (a target
quantised with group size 32, fp16 first and last layers and lm_head, K = 23)
and ``gdn_state_commit`` (recurrent states advanced by the accepted prefix,
the step after the verify) are timed after the step, outside its timed
region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
METRIC = "W4A16 verify GEMM HBM GB/s (% of peak) at M=16; verified tokens/s"


def linear_bytes(m, k, n):
    """Algorithmic HBM bytes of one W4A16 linear: weights, scales, zeros, x read, y written."""
    g = k // 128
    return k * n // 2 + g * n * 2 + g * n // 2 + m * k * 2 + m * n * 2


def lmhead_bytes(m, h, v, k_draft):
    return v * h + v * 2 + m * h * 2 + m * 4 + m * 4 + k_draft * 4 + 4 + m * 4


def cpu_baseline(wl, plan, drafts, min_seconds: float = 10.0):
    """Time the oracle on whole verify steps of the same workload (36 layers at
    M = 16, the full lm_head, greedy verify) until ``min_seconds`` have passed,
    with numpy's BLAS on every core the process may use (``cores`` reports the
    BLAS threads actually in use, ``affinity_cores`` the cores available); plus
    the small block-linear step (one 2560 -> 2560 linear, a 4096-word head,
    greedy verify) on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import step as ostep

    affinity = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=affinity, user_api="blas"):
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] + [1])
        steps = 0
        t0 = time.perf_counter()
        while True:
            ostep.verify_step(wl.x, wl.linears, plan, wl.lm_w, wl.lm_s, drafts, 1, drafts.shape[-1])
            steps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        dt = time.perf_counter() - t0
    step_b = sum(linear_bytes(16, k, n) for k, n, _ in plan) + lmhead_bytes(16, 2560, 151936, 15)
    gbs = step_b * steps / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "affinity_cores": affinity,
            "kind": "oracle", "seconds": round(dt, 2), "ms_per_step": round(1e3 * dt / steps, 1),
            "sample": f"{steps} whole verify steps of the same workload (36 layers x 4 linears "
                      f"at M=16, lm_head 2560->151936, greedy verify) through the numpy fp64 "
                      f"oracle, {dt:.1f} s on {threads} BLAS threads ({affinity} cores available)",
            "c1_one_thread": c1_cpu(),
            "drafter": drafter_cpu()}


def c1_cpu(min_seconds: float = 2.0):
    """The oracle's block-linear verify step (one 2560 -> 2560 linear at M = 16,
    a 4096-word int8 head with argmax, greedy verify of 15 drafts) on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import gen
    from oracle import step as ostep

    wl = gen.make_workload(1)
    plan = gen.chain_plan(wl.cfg)
    drafts = np.full((1, wl.cfg.k_draft), -1, dtype=np.int32)
    with threadpool_limits(limits=1, user_api="blas"):
        reps = 0
        t0 = time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < min_seconds:
            ostep.verify_step(wl.x, wl.linears, plan, wl.lm_w, wl.lm_s, drafts, 1, wl.cfg.k_draft)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    return {"ms_per_step": round(1e3 * dt, 2), "cores": 1,
            "sample": f"{reps} block-linear verify steps (one 2560->2560 W4A16 linear at M=16, "
                      f"lm_head 2560->4096, greedy verify) through the numpy fp64 oracle"}


def drafter_cpu():
    """The oracle's prompt-lookup drafting on the drafter leg's B = 8 histories
    (8192 tokens, K = 23, n 4..1), one thread: microseconds per batch."""
    import numpy as np

    import gen
    from oracle import ngram

    hist = gen.token_histories(np.random.default_rng(1008), [8192] * 8, 8192 + 64, 151936)
    rows = [list(r[:8192]) for r in hist]
    reps = 0
    t0 = time.perf_counter()
    while reps < 3 or time.perf_counter() - t0 < 1.0:
        ngram.prompt_lookup_batch(rows, 4, 1, 23)
        reps += 1
    us = (time.perf_counter() - t0) / reps * 1e6
    return {"b8_us": round(us, 1), "cores": 1,
            "sample": f"{reps} calls on 8 histories of 8192 tokens (plain-Python oracle)"}


def counter_traffic():
    """HBM bytes per W4A16 launch from the committed counter summary, or None
    when the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "w4a16_skinny_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        digest = source_digest(rec["sources"])
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if digest == rec["sha256"] else None


def source_digest(sources):
    """sha256 over the given sources with comments removed and whitespace
    collapsed, so that a change of wording does not mark the counters stale
    (code changes do)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def device_info(dev):
    """Name, compute units and clocks of the device the numbers come from (torch's
    properties, and the HIP runtime's attributes for the clocks)."""
    import ctypes
    import torch
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1)}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMemoryClockRate = 60 (kHz)
        for key, attr in (("clock_mhz", 5), ("mem_clock_mhz", 60)):
            if hip.hipDeviceGetAttribute(ctypes.byref(val), attr, dev.index or 0) == 0:
                info[key] = val.value // 1000
    except OSError:
        pass
    return info


def read_probe(dev, mib: int = 1024, reps: int = 10):
    """The HBM read rate the device reaches: w4v_read_probe over a buffer four
    times the last-level cache, averaged over ``reps`` back-to-back calls."""
    import torch

    import w4a16_speculative_verify_amd as w4v
    src = torch.ones(mib << 18, dtype=torch.int32, device=dev)
    out = w4v.read_probe(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        w4v.read_probe(src, out=out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = src.numel() * 4
    del src, out
    return {"bytes": nbytes, "us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def prefill(dev, reps: int = 10):
    """The prefill-shaped linears (gate+up 2560->19456, down 9728->2560) at
    M = 2048 and 8192 through w4a16_gemm (from 33 rows on: the LDS-tiled MFMA
    kernel, each 256 x 256 block tile dequantising its packed weights once into
    LDS, split-K partials and their reduce where the plan splits): TFLOP/s per
    shape, 2*M*K*N flops over the average of ``reps`` back-to-back calls."""
    import numpy as np
    import torch

    import gen
    import w4a16_speculative_verify_amd as w4v

    wl = gen.make_workload(5)
    out = {}
    for m in (2048, 8192):
        for (k, n), lin, xa in zip(wl.cfg.single, wl.linears, wl.extra_x):
            x = torch.from_numpy(np.ascontiguousarray(xa[:m])).to(dev)
            qw, sc, qz = (torch.from_numpy(np.ascontiguousarray(t)).to(dev)
                          for t in (lin.qweight, lin.scales, lin.qzeros))
            y = torch.empty((m, n), dtype=torch.float16, device=dev)
            w4v.w4a16_gemm(x, qw, sc, qz, out=y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                w4v.w4a16_gemm(x, qw, sc, qz, out=y)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            tf = 2.0 * m * k * n / (us * 1e-6) / 1e12
            # yardstick only: the vendor fp16 GEMM on fp16 weights of the same shape
            w16 = torch.randn((k, n), dtype=torch.float16, device=dev) * 0.02
            torch.matmul(x, w16)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                torch.matmul(x, w16)
            e1.record()
            torch.cuda.synchronize()
            us_ref = e0.elapsed_time(e1) * 1e3 / reps
            out[f"m{m}_{k}x{n}"] = {"us": round(us, 2), "tflops": round(tf, 1),
                                    "frac_of_fp16_mfma_peak": round(tf / MFMA_FP16_PEAK_TFLOPS, 4),
                                    "torch_matmul_fp16_us": round(us_ref, 2),
                                    "torch_matmul_fp16_tflops":
                                        round(2.0 * m * k * n / (us_ref * 1e-6) / 1e12, 1)}
            del x, y, w16
    return out


def drafter_gemm(dev, reps: int = 20):
    """The 4-bit drafter's step through the same W4A16 linear: the 12800 -> 2560
    fusion of five tapped hidden states, then five layers of the target's four
    linears, at M = 16 (279.2 MB of weights, scales and zeros), replayed from a
    HIP graph; average of ``reps`` replays."""
    import torch

    import gen
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep

    wl = gen.make_drafter_workload()
    up = lambda a: torch.from_numpy(a).to(dev)
    plan = gen.drafter_plan()
    lins = [DeviceLinear(up(l.qweight), up(l.scales), up(l.qzeros), k, n, a)
            for l, (k, n, a) in zip(wl.linears, plan)]
    step = VerifyStep(lins, None, None, 16, 1, 15, device=dev)
    x = up(wl.x)
    step.linears_only(x)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.linears_only(x)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = sum(linear_bytes(16, k, n) for k, n, _ in plan)
    gbs = nbytes / (us * 1e-6) / 1e9
    del g, step, lins
    return {"linears": len(plan), "m": 16, "us_per_step": round(us, 2), "bytes": nbytes,
            "gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


def g32_target(dev, steps: int = 50, warmup: int = 5):
    """A verify step of team #5's target: 36 layers of the 4B-class linears, W4A16 with
    group size 32 except layers 0, 1, 34 and 35 in fp16 (vendor library GEMM), an fp16
    lm_head 2560 -> 151936 with fused argmax and greedy verify, at K = 23 (24 rows).
    Drafts accept min(23, Geometric(0.25)) tokens against the step's own target ids."""
    import numpy as np
    import torch

    import gen
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep

    tg = gen.make_g32_target()
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    lins, nbytes = [], 0
    m = tg.m
    for l in tg.linears:
        if l.w16 is not None:
            lins.append(DeviceLinear(None, None, None, l.k, l.n, l.alpha, w16=up(l.w16)))
            nbytes += l.n * l.k * 2
        else:
            lins.append(DeviceLinear(up(l.q.qweight), up(l.q.scales), up(l.q.qzeros), l.k, l.n,
                                     l.alpha, group_size=gen.G32_GROUP))
            g = l.k // gen.G32_GROUP
            nbytes += l.k * l.n // 2 + g * l.n * 2 + g * (l.n // 8) * 4
        nbytes += m * l.k * 2 + m * l.n * 2
    v = tg.lm_w16.shape[0]
    nbytes += v * gen.HIDDEN * 2 + m * gen.HIDDEN * 2 + m * 4 + tg.k_draft * 4 + m * 4 + 4
    step = VerifyStep(lins, up(tg.lm_w16), None, m, 1, tg.k_draft, device=dev)
    x = up(tg.x)
    no_drafts = torch.full((1, tg.k_draft), -1, dtype=torch.int32, device=dev)
    t_host = step(x, no_drafts)[0].cpu().numpy()
    rng = np.random.default_rng(2323)
    total = warmup + steps
    drafts = np.stack([gen.drafts_with_prefix(rng, t_host, tg.k_draft, v,
                                              gen.draw_r_geometric(rng, tg.k_draft))
                       for _ in range(total)])[:, None, :]
    drafts_dev = up(drafts.astype(np.int32))
    acc_hist = torch.zeros(total, dtype=torch.int32, device=dev)
    # as the main step: each step reads its own drafts and writes its own
    # accepted length; warm-up eagerly, the timed steps from one HIP graph
    for i in range(warmup):
        step(x, drafts_dev[i], accepted_len=acc_hist[i:i + 1])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(warmup, total):
            step(x, drafts_dev[i], accepted_len=acc_hist[i:i + 1])
    g.replay()
    torch.cuda.synchronize()
    acc_hist[warmup:].zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tokens = int(acc_hist[warmup:].sum().item()) + steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    del g, step, lins
    torch.cuda.empty_cache()
    return {"workload": "36 layers x 4B-class linears, W4A16 g32 with layers 0, 1, 34, 35 in fp16, "
                        "fp16 lm_head 2560->151936 + argmax + greedy verify, K=23 (M=24)",
            "m": m, "k_draft": tg.k_draft, "ms_per_step": round(ms, 4), "step_bytes": nbytes,
            "gbs": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "verified_tokens_per_s": round(tokens / (ms * 1e-3 * steps), 1),
            "mean_accepted_plus_one": round(tokens / steps, 3)}


def gdn_commit(dev, reps: int = 20):
    """Committing Gated DeltaNet states to the accepted prefix after a verify at K = 15:
    27 recurrent layers (three of every four of the 36) x 16 heads of 128 x 128 fp32 state,
    all committed in one launch; B = 1 and 8 sequences with min(15, Geometric(0.25)) accepted
    drafts.  Average of ``reps`` launches replayed from a HIP graph; algorithmic bytes are the
    states read and written plus the accepted positions' keys, values and gates."""
    import numpy as np
    import torch

    import gen
    import w4a16_speculative_verify_amd as w4v

    layers, heads, d, t = 27, 16, gen.GDN_DK, 16
    h = layers * heads
    out = {"layers": layers, "heads_per_layer": heads, "head_dim": d, "positions": t}
    for b in (1, 8):
        rng = np.random.default_rng(4100 + b)
        S, k, v, al, be = gen.gdn_inputs(rng, b, t, h, d, d)
        acc = np.array([gen.draw_r_geometric(rng, t - 1) for _ in range(b)], np.int32)
        up = lambda a: torch.from_numpy(a).to(dev)
        s_d, k_d, v_d, al_d, be_d, acc_d = (up(a) for a in (S, k, v, al, be, acc))
        w4v.gdn_state_commit(s_d, k_d, v_d, al_d, be_d, acc_d)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                w4v.gdn_state_commit(s_d, k_d, v_d, al_d, be_d, acc_d)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = int(b * h * 2 * d * d * 4 + int((acc + 1).sum()) * h * (2 * d + 2) * 4 + b * 4)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[f"b{b}"] = {"us": round(us, 2), "bytes": nbytes, "gbs": round(gbs, 1),
                        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                        "accepted": acc.tolist()}
        del g, s_d, k_d, v_d
    return out


def decode_m1(lins, x16, reps: int = 20):
    """Plain decode (one activation row) through the 144 linears of the verify-step
    workload: 36 copies of one 4B-class layer, so every launch reads fresh weights
    from HBM.  One HIP graph per replay; GB/s per layer over algorithmic bytes."""
    import torch
    from w4a16_speculative_verify_amd.step import VerifyStep
    st = VerifyStep(lins, None, None, 1, 1, 0)
    x1 = x16[:1].contiguous()
    st.linears_only(x1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.linears_only(x1)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    layers = len(lins) // 4
    b = sum(linear_bytes(1, l.k_in, l.n_out) for l in lins)
    return {"layers": layers, "us_per_layer": round(us / layers, 2),
            "bytes_per_layer": b // layers, "gbs": round(b / (us / 1e6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * b / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 2)}


def padded_batch(lins, lm_w, lm_s, steps: int = 50, warmup: int = 5):
    """Padded verify of 8 sequences x 21 rows (K = 20 drafts, -1 padding) through
    one 4B-class layer and the 151,936-word int8 lm_head with fused argmax and
    verify.  Weights: the first layer and the lm_head of the verify-step workload
    (same shapes and distributions); activations and drafts: the padded
    configuration's own seeded streams.  The linears at M = 168 run on the
    LDS-tiled MFMA kernel.  The timed steps run from one HIP graph, each step
    reading its own drafts and writing its own accepted lengths."""
    import numpy as np
    import torch
    import gen
    from w4a16_speculative_verify_amd.step import VerifyStep
    cfg = gen.CONFIGS[4]
    dev = lm_w.device
    r_x = gen.streams(1000 * cfg.cid, 4)[0]
    x = torch.from_numpy(gen.activations(r_x, cfg.m, gen.HIDDEN)).to(dev)
    st = VerifyStep(lins[:4], lm_w, lm_s, cfg.m, cfg.batch, cfg.k_draft)
    none = torch.full((cfg.batch, cfg.k_draft), -1, dtype=torch.int32, device=dev)
    t_ids, _, _, _ = st(x, none)
    t_host = t_ids.cpu().numpy()
    drng = gen.draft_rng(cfg.cid)
    total = warmup + steps
    d_all = np.empty((total, cfg.batch, cfg.k_draft), np.int32)
    planned = np.empty((total, cfg.batch), np.int64)
    for i in range(total):
        d_all[i], planned[i] = gen.make_drafts(drng, cfg, t_host)
    d_dev = torch.from_numpy(d_all).to(dev)
    acc = torch.zeros((total, cfg.batch), dtype=torch.int32, device=dev)
    # step i reads its own drafts (resident in HBM, as a drafter on the device
    # leaves them) and writes its accepted lengths to its own row
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            st(x, d_dev[i], accepted_len=acc[i])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # the timed steps in one graph, so that the host's per-replay cost is not timed
    g_steps, g_lin = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_steps):
        for i in range(warmup, total):
            st(x, d_dev[i], accepted_len=acc[i])
    with torch.cuda.graph(g_lin):
        st.linears_only(x)
    g_steps.replay()
    torch.cuda.synchronize()
    acc[warmup:].zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / steps
    a = acc.cpu().numpy().astype(np.int64)
    if not np.array_equal(a, planned):
        raise RuntimeError("padded batch: accepted lengths differ from the planned ones")
    for _ in range(3):
        g_lin.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        g_lin.replay()
    e1.record()
    torch.cuda.synchronize()
    lin_us = e0.elapsed_time(e1) * 1e3 / steps
    lin_flop = sum(2 * cfg.m * l.k_in * l.n_out for l in lins[:4])
    head_flop = 2 * cfg.m * gen.HIDDEN * cfg.vocab
    head_us = step_us - lin_us
    head_b = lmhead_bytes(cfg.m, gen.HIDDEN, cfg.vocab, cfg.k_draft)
    tokens = int(np.sum(a[warmup:] + 1))
    return {"workload": "8 sequences x 21 rows (K=20, -1 padding): one 4B-class layer + int8 "
                        "lm_head 2560->151936 + argmax + greedy verify", "m": cfg.m,
            "step_us": round(step_us, 2), "linears_us": round(lin_us, 2),
            "linears_tflops": round(lin_flop / (lin_us / 1e6) / 1e12, 1),
            "linears_frac_of_fp16_mfma_peak": round(lin_flop / (lin_us / 1e6) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
            "head_us": round(head_us, 2),
            "head_tflops": round(head_flop / (head_us / 1e6) / 1e12, 1),
            "head_gbs": round(head_b / (head_us / 1e6) / 1e9, 1),
            "verified_tokens_per_s": round(tokens / (step_us * steps / 1e6), 1),
            "mean_accepted_plus_one": round(tokens / (steps * cfg.batch), 3)}


def c1_row(dev, reps: int = 10):
    """The block-linear configuration: one verify step of B = 1, M = 16, K = 15
    through one W4A16 2560 -> 2560 linear, an int8 lm_head 2560 -> 4096 with
    fused argmax, and greedy verify.  Its 3.6 MB linear and 10.6 MB head sit
    below the bandwidth-delay product, so both are latency-bound by design.
    Each kernel's GB/s is taken over >= 1 GB of distinct weight copies launched
    back to back from a HIP graph (every launch reads its weights from HBM: no
    copy is reused within the 256 MB last-level cache); the whole step is timed
    as 200 consecutive steps, each with its own drafts, captured in one HIP graph."""
    import numpy as np
    import torch

    import gen
    import w4a16_speculative_verify_amd as w4v
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep

    cfg = gen.CONFIGS[1]
    wl = gen.make_workload(1)
    lin = wl.linears[0]
    k, n = lin.qweight.shape[0] * 8, lin.qweight.shape[1]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = up(wl.x)
    qw, sc, qz = up(lin.qweight), up(lin.scales), up(lin.qzeros)
    lin_b = linear_bytes(cfg.m, k, n)
    n_lin = -(-(1 << 30) // lin_b)
    copies = [(qw.clone(), sc.clone(), qz.clone()) for _ in range(n_lin)]
    y = torch.empty((cfg.m, n), dtype=torch.float16, device=dev)
    ws = w4v.new_workspace(max(w4v.gemm_workspace_size(cfg.m, n, k), 256), dev)

    def timed_graph(fn, count):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps / count

    def all_linears():
        for c in copies:
            w4v.w4a16_gemm(x, *c, out=y, workspace=ws)

    lin_us = timed_graph(all_linears, n_lin)
    del copies
    lm_w, lm_s = up(wl.lm_w), up(wl.lm_s)
    head_b = lmhead_bytes(cfg.m, gen.HIDDEN, cfg.vocab, cfg.k_draft)
    n_head = -(-(1 << 30) // head_b)
    heads = [(lm_w.clone(), lm_s.clone()) for _ in range(n_head)]
    lws = w4v.new_workspace(w4v.lmhead_workspace_size(cfg.m, gen.HIDDEN, cfg.vocab), dev)
    t_ids = torch.empty(cfg.m, dtype=torch.int32, device=dev)

    def all_heads():
        for w, s8 in heads:
            w4v.w8a16_lmhead_argmax(x[:, :gen.HIDDEN], w, s8, target_ids=t_ids, workspace=lws)

    head_us = timed_graph(all_heads, n_head)
    del heads
    # the whole step, fresh drafts per replay
    st = VerifyStep([DeviceLinear(qw, sc, qz, k, n, 1.0)], lm_w, lm_s, cfg.m, cfg.batch,
                    cfg.k_draft)
    none = torch.full((1, cfg.k_draft), -1, dtype=torch.int32, device=dev)
    t0, _, _, _ = st(x, none)
    t_host = t0.cpu().numpy()
    drng = gen.draft_rng(1)
    steps = 200
    d_all = np.empty((steps, 1, cfg.k_draft), np.int32)
    planned = np.empty(steps, np.int64)
    for i in range(steps):
        d_all[i], r = gen.make_drafts(drng, cfg, t_host)
        planned[i] = r[0]
    d_dev, d_buf = up(d_all), torch.empty((1, cfg.k_draft), dtype=torch.int32, device=dev)
    acc = torch.zeros(steps, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st(x, d_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # all the steps in one graph (each reads its own drafts, resident in HBM as a
    # drafter running on the device would leave them, and writes its accepted
    # length to its own slot), so that the host's per-replay launch cost, larger
    # than this step, does not set the time
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            st(x, d_dev[i], accepted_len=acc[i:i + 1])
    g.replay()
    torch.cuda.synchronize()
    acc.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3 / steps
    a = acc.cpu().numpy().astype(np.int64)
    if not np.array_equal(a, planned):
        raise RuntimeError("block-linear step: accepted lengths differ from the planned ones")
    tokens = int(np.sum(a + 1))
    return {"workload": "block-linear verify step M=16 (K=15): W4A16 g128 2560->2560 + int8 "
                        "lm_head 2560->4096 with fused argmax + greedy verify",
            "gemm_us": round(lin_us, 3), "gemm_bytes": lin_b,
            "gemm_gbs": round(lin_b / (lin_us * 1e-6) / 1e9, 1),
            "gemm_pct_of_hbm_peak": round(100 * lin_b / (lin_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
            "gemm_copies": n_lin,
            "lmhead_us": round(head_us, 3), "lmhead_bytes": head_b,
            "lmhead_gbs": round(head_b / (head_us * 1e-6) / 1e9, 1),
            "lmhead_copies": n_head,
            "step_us": round(step_us, 2),
            "verified_tokens_per_s": round(tokens / (step_us * steps / 1e6), 1),
            "mean_accepted_plus_one": round(tokens / steps, 3)}


def chain_linears(lins, x, reps: int = 20):
    """The same 144 linears in one persistent launch (w4a16_chain): each CU's
    share of every linear streamed into LDS ahead of the math, ready flags
    between the linears.  Average of ``reps`` launches; GB/s over the same
    algorithmic bytes as the per-launch path."""
    import torch
    import w4a16_speculative_verify_amd as w4v

    ch = w4v.Chain([(l.qweight, l.scales, l.qzeros, l.alpha) for l in lins], x.shape[0], x.device)
    y = torch.empty((x.shape[0], lins[-1].n_out), dtype=torch.float16, device=x.device)
    for _ in range(3):
        ch(x, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ch(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    if ch.error() != 0:
        raise RuntimeError(f"chain error word {ch.error()}")
    us = e0.elapsed_time(e1) * 1e3 / reps
    b = sum(linear_bytes(x.shape[0], l.k_in, l.n_out) for l in lins)
    del ch
    return {"us": round(us, 2), "gbs": round(b / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}


def drafter(dev, reps: int = 200):
    """Prompt-lookup drafting ahead of the verify (not part of the timed step):
    ngram_draft over B synthetic histories of 8192 tokens (half copied spans),
    K = 23 drafts, n from 4 down to 1.  Reports the average of ``reps``
    back-to-back calls replayed from a HIP graph and the algorithmic bytes (each
    history read once, the drafts written) over that time."""
    import numpy as np
    import torch

    import gen
    import w4a16_speculative_verify_amd as w4v

    length, k, n_max, n_min = 8192, 23, 4, 1
    out = {"history_tokens": length, "k": k, "n_max": n_max, "n_min": n_min}
    for b in (1, 8, 64):
        rng = np.random.default_rng(1000 + b)
        hist = torch.from_numpy(gen.token_histories(rng, [length] * b, length + 64, 151936)).to(dev)
        lens = torch.full((b,), length, dtype=torch.int32, device=dev)
        drafts = torch.empty((b, k), dtype=torch.int32, device=dev)
        w4v.ngram_draft(hist, lens, n_max, n_min, k, drafts=drafts)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()                # replayed: the host call rate is not timed
        with torch.cuda.graph(g):
            for _ in range(reps):
                w4v.ngram_draft(hist, lens, n_max, n_min, k, drafts=drafts)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        del g
        nbytes = b * (length * 4 + 4 + k * 4)
        out[f"b{b}"] = {"us": round(us, 2), "bytes": nbytes,
                        "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del hist, lens, drafts
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--gemm-reps", type=int, default=50,
                    help="replays of the linears-only graph for the roofline timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-shaped (M = 2048 / 8192) GEMM timing")
    ap.add_argument("--no-drafter", action="store_true",
                    help="skip the timings of the steps around the verify (prompt lookup, "
                         "4-bit drafter step, recurrent-state commit)")
    ap.add_argument("--no-g32", action="store_true",
                    help="skip the group-size-32 target step (fp16 first and last layers)")
    ap.add_argument("--no-other-m", action="store_true",
                    help="skip the plain-decode (M = 1) and padded-batch (M = 168) timings")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="one device-to-device copy of this many MiB before timing (counter calibration)")
    ap.add_argument("--path", choices=["chain", "per-linear"], default="per-linear",
                    help="one persistent launch for all linears, or one launch per linear")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the one-launch chain timing of the same linears")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the verify step has no multi-GPU path "
              "in this build (sharding is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import w4a16_speculative_verify_amd as w4v
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep

    w4v.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = gen.CONFIGS[3]
    print(f"[bench] generating the seeded verify-step workload ({cfg.note})", file=sys.stderr,
          flush=True)
    wl = gen.make_workload(3)
    plan = gen.chain_plan(cfg)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    lins = [DeviceLinear(up(l.qweight), up(l.scales), up(l.qzeros), k, n, a)
            for l, (k, n, a) in zip(wl.linears, plan)]
    step = VerifyStep(lins, up(wl.lm_w), up(wl.lm_s), cfg.m, cfg.batch, cfg.k_draft,
                      chain=args.path == "chain")
    x = up(wl.x)
    torch.cuda.synchronize()

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # target ids of this input (untimed), then one draft block per step
    no_drafts = torch.full((1, cfg.k_draft), -1, dtype=torch.int32, device=dev)
    t_ids, _, _, _ = step(x, no_drafts)
    t_host = t_ids.cpu().numpy()
    drng = gen.draft_rng(3)
    total = args.warmup + args.steps
    drafts_all = np.empty((total, 1, cfg.k_draft), dtype=np.int32)
    planned = np.empty(total, dtype=np.int64)
    for i in range(total):
        drafts_all[i], r = gen.make_drafts(drng, cfg, t_host)
        planned[i] = r[0]
    drafts_dev = up(drafts_all)
    acc_hist = torch.zeros(total, dtype=torch.int32, device=dev)

    # every step reads its own drafts and writes its own accepted length in HBM
    # (as a drafter running on the device leaves them); the warm-up steps run
    # eagerly, the timed ones from HIP graphs of `chunk` consecutive steps, with
    # an event between graphs (per-step times: each graph's time / its steps)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(args.warmup):
            step(x, drafts_dev[i], accepted_len=acc_hist[i:i + 1])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    chunk = 10
    starts = list(range(args.warmup, total, chunk))
    sizes = [min(chunk, total - c0) for c0 in starts]
    graphs = []
    for c0, n_c in zip(starts, sizes):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(c0, c0 + n_c):
                step(x, drafts_dev[i], accepted_len=acc_hist[i:i + 1])
        graphs.append(g)
    # the linears alone (roofline timing)
    g_lin = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_lin):
        step.linears_only(x)
    for g in graphs:                                # first replays: untimed
        g.replay()
    torch.cuda.synchronize()
    acc_hist[args.warmup:].zero_()

    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for j, g in enumerate(graphs):
        g.replay()
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = np.array([evs[j].elapsed_time(evs[j + 1]) / sizes[j] for j in range(len(graphs))])
    p10, p50, p90 = (float(np.percentile(per_step, q)) for q in (10, 50, 90))

    acc = acc_hist.cpu().numpy().astype(np.int64)
    if not np.array_equal(acc, planned):
        print(f"[bench] accepted lengths differ from the planned ones", file=sys.stderr)
        sys.exit(1)
    tokens = int(np.sum(acc[args.warmup:] + 1))
    tok_per_s = tokens / (step_ms * args.steps / 1e3)

    # linears only: average launch duration of the W4A16 kernel
    for _ in range(3):
        g_lin.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.gemm_reps):
        g_lin.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    lin_ms = e0.elapsed_time(e1) / args.gemm_reps
    n_launch = len(plan)
    lin_b = sum(linear_bytes(cfg.m, k, n) for k, n, _ in plan)
    lm_b = lmhead_bytes(cfg.m, gen.HIDDEN, cfg.vocab, cfg.k_draft)
    act_launch_us = lin_ms * 1e3 / n_launch
    gemm_gbs = lin_b / (lin_ms / 1e3) / 1e9
    step_gbs = (lin_b + lm_b) / (step_ms / 1e3) / 1e9

    c1 = None
    if not args.no_other_m:
        print("[bench] timing the block-linear configuration (M = 16, one linear, 4096-word head)",
              file=sys.stderr, flush=True)
        c1 = c1_row(dev)

    chain = None
    if not args.no_chain and args.path != "chain":
        print("[bench] timing the same linears in one persistent launch", file=sys.stderr,
              flush=True)
        chain = chain_linears(lins, x)

    m1 = padded = None
    if not args.no_other_m:
        print("[bench] timing plain decode (M = 1) and the padded batch (M = 168)",
              file=sys.stderr, flush=True)
        m1 = decode_m1(lins, x)
        padded = padded_batch(lins, step.lm_w, step.lm_s)

    pre = None
    if not args.no_prefill:
        print("[bench] timing the prefill-shaped linears", file=sys.stderr, flush=True)
        del graphs, g_lin
        pre = prefill(dev)

    commit = None
    if not args.no_drafter:
        print("[bench] timing the recurrent-state commit", file=sys.stderr, flush=True)
        commit = gdn_commit(dev)

    g32 = None
    if not args.no_g32:
        print("[bench] timing the group-size-32 target step (generating its weights)",
              file=sys.stderr, flush=True)
        g32 = g32_target(dev)

    dgemm = None
    if not args.no_drafter:
        print("[bench] timing the 4-bit drafter step", file=sys.stderr, flush=True)
        dgemm = drafter_gemm(dev)

    draft = None
    if not args.no_drafter:
        print("[bench] timing the prompt-lookup drafter", file=sys.stderr, flush=True)
        draft = drafter(dev)

    print("[bench] probing the HBM read rate", file=sys.stderr, flush=True)
    probe = read_probe(dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, plan, drafts_all[0], args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_p10_p50_p90": [round(p10, 4), round(p50, 4), round(p90, 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "verify step M=16 (K=15): 36 layers x W4A16 g128 "
                               "(2560->6144, 4096->2560, 2560->19456, 9728->2560) + int8 "
                               "lm_head 2560->151936 with fused argmax + greedy verify",
                   "m": cfg.m, "layers": 36, "vocab": cfg.vocab, "k_draft": cfg.k_draft,
                   "global_batch": cfg.batch, "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "verified_tokens_per_s": round(tok_per_s, 1),
        "mean_accepted_plus_one": round(tokens / args.steps, 3),
        "gemm_gbs": round(gemm_gbs, 1),
        "gemm_pct_of_hbm_peak": round(100 * gemm_gbs / HBM_PEAK_GBS, 2),
        "hbm_read_probe": probe,
        "gemm_pct_of_probed_read": round(100 * gemm_gbs / probe["gbs"], 2),
        "linears_us_per_step": round(lin_ms * 1e3, 2),
        "step_bytes": lin_b + lm_b,
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(),
                     "kernel": "w4a16_skinny_kernel (QKV, O, gate+up, down x 36 layers)",
                     "bytes_per_launch": round(lin_b / n_launch),
                     "avg_launch_us": round(act_launch_us, 3)},
        "cpu_baseline": cpu,
        "device": device_info(dev),
        "block_linear_c1": c1,
        "linears_one_launch_chain": chain,
        "prefill": pre,
        "decode_m1": m1,
        "padded_batch_m168": padded,
        "drafter": draft,
        "drafter_int4_step": dgemm,
        "g32_target_step": g32,
        "gdn_state_commit": commit,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
