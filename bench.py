"""Benchmark of the eager latent-attention forward path on one MI355X.

One step = one pass of the whole hot path (the cos/sin tables are built once
per length before the steps, as the pages cache them):
  prefill (Kimi-K2 shape, B=2, T=8192, H=64, Dn/Dr/Dv 128/64/128, YaRN):
    latent RMSNorm with the shared rotary key's rotation -> kv_b_proj
    expansion -> causal attention;
  decode (Kimi-K2 shape, B=32 sequences at position 1000, 1001 cached rows):
    latent RMSNorm -> kv_b_proj expansion appended into the expanded cache ->
    split-K decode attention;
  decode against a compressed-latent cache (same shape, 576 fp16 values per
    cached token): RMSNorm + rotary key into the cache row -> absorbed
    split-K attention (W_uk folded into the query, W_uv after the merge).
Inputs are drawn on the GPU (same seeded recipe as the parity tests) and are
resident in HBM before the timed region starts.

Reported (one JSON line):
  value           prefill attention TFLOP/s (causal-pair flops over the mean
                  event-timed attention launch of a step); the whole prefill
                  path (attention + kv_b_proj flops) is config.prefill_path_*
  roofline        prefill attention kernel: algorithmic flops per launch over
                  its mean launch time (HIP events on the launch stream)
                  against the MI355X dense 16-bit MFMA peak
  decode          decode attention GB/s (algorithmic bytes) and HBM fraction
  decode_latent   step time of the latent-cache decode and its attention
  graphs          both decode steps recorded once as HIP graphs and replayed
  decode_latent_reexpand  the same latent-cache decode by re-expanding every
                  cached row on each call (timed after the steps)
  block           the whole attention block at the 8k prefill shape (hidden
                  7168, q rank 1536): projections, query RMSNorm, the path,
                  o_proj (timed after the steps)
  chunked         prefill against a past cache: the last 1024-token chunk of
                  the 8k sequence attending to its 7168 cached rows (timed
                  after the steps, attention call only)
  other shapes    prefill attention at Kimi-K2 1k (warm, and cold after a
                  512 MB write that evicts the last-level cache, with its
                  attainable rate from the HBM roofline) and GLM-5 4k
  ceilings        what this chip sustains: a streaming HBM read and a dense
                  fp16 MFMA loop on random operands (the library's
                  measurement aids), and the vendor bf16 GEMM on random
                  8192^3 operands; the attention and decode figures are also
                  given as fractions of these
  cpu_baseline    the fp64 CPU oracle on a bounded sample (--cpu-baseline)
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
PREFILL = "kimi_k2_8k"
DECODE = "kimi_k2_decode"
DECODE_LATENT = "kimi_k2_decode_latent"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(w) -> float:
    """Causal attention flops: B*H*T(T+1)/2 key pairs x 2*(Dqk+Dv)."""
    return w.B * w.H * w.T * (w.T + 1) / 2 * 2 * (w.Dqk + w.Dv)


def expand_flops(w) -> float:
    return 2.0 * w.B * w.T * w.R * w.H * (w.Dn + w.Dv)


def decode_bytes(w) -> float:
    """Algorithmic bytes of decode attention: K and V caches, q and out."""
    L = w.cache_len
    return 2.0 * w.B * w.H * (L * (w.Dqk + w.Dv) + w.Dqk + w.Dv)


def measured_traffic(kernel_source: str, key=None):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain device copy),
    or None when the kernel's source has changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if key:
        rec = rec.get(key, {})
    src = os.path.join(ROOT, kernel_source)
    if rec.get("source") != kernel_source or not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return int(round(rec["fetch_bytes"] + rec["write_bytes"]))


def cpu_baseline(budget_s: float) -> dict:
    """The fp64 oracle (as is) on a bounded sample of the prefill workload:
    whole heads of sequence 0 (expansion of that head + causal attention over
    all 8192 rows), as many as fit in `budget_s` seconds (at least one)."""
    import dataclasses

    import numpy as np

    import workloads
    from oracle import mla_oracle as O

    try:
        import threadpoolctl
        threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    w = workloads.WORKLOADS[PREFILL]
    inp = workloads.make_inputs(dataclasses.replace(w, B=1))
    wh = dataclasses.replace(w, B=1, H=1)
    n = w.Dn + w.Dv
    t0 = time.perf_counter()
    heads = 0
    while True:
        sub = {"q": inp["q"][:, heads:heads + 1], "latent": inp["latent"], "k_pe": inp["k_pe"],
               "gain": inp["gain"], "W": inp["W"][heads * n:(heads + 1) * n]}
        parts = O.prefill_parts(wh, sub)
        O.prefill_head(wh, parts, 0, 0)
        heads += 1
        if time.perf_counter() - t0 > budget_s or heads >= w.H:
            break
    dt = time.perf_counter() - t0
    flops = heads * (attn_flops(wh) + expand_flops(wh))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{heads} head(s) of sequence 0 of {PREFILL} (T=8192): fp64 expansion + causal "
                      f"attention over all rows, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0 = automatic)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import head_latent_attention_rmsnorm_amd as mla
    import workloads

    dev = "cuda"
    wp = workloads.WORKLOADS[PREFILL]
    wd = workloads.WORKLOADS[DECODE]
    log(f"[bench] drawing inputs on the GPU: {PREFILL}, {DECODE}")
    ip = workloads.make_inputs(wp, device=dev)
    idc = workloads.make_inputs(wd, device=dev)
    rope_p = mla.api.params_from(wp.rope, wp.Dr)
    rope_d = mla.api.params_from(wd.rope, wd.Dr)
    bufs = mla.pipeline.alloc_prefill(wp.B, wp.T, wp.H, wp.R, wp.Dn, wp.Dr, wp.Dv, dev)
    seq = torch.full((wd.B,), wd.cache_len, dtype=torch.int32, device=dev)
    qpos = torch.full((wd.B,), wd.q_pos, dtype=torch.int32, device=dev)
    c_dec = torch.empty((wd.B, 1, wd.R), dtype=torch.float16, device=dev)
    out_dec = torch.empty((wd.B, wd.H, 1, wd.Dv), dtype=torch.bfloat16, device=dev)
    splits = args.splits or 0
    ws_dec = torch.empty((max(1, 64 << 20),), dtype=torch.uint8, device=dev)
    wl = workloads.WORKLOADS[DECODE_LATENT]
    il = workloads.make_inputs(wl, device=dev)
    rope_l = mla.api.params_from(wl.rope, wl.Dr)
    w_ukt = mla.api.mla_absorb_prepare(il["W"], wl.H, wl.Dn, wl.Dv)  # weight preparation, once
    seq_l = torch.full((wl.B,), wl.cache_len, dtype=torch.int32, device=dev)
    qpos_l = torch.full((wl.B,), wl.q_pos, dtype=torch.int32, device=dev)
    out_lat = torch.empty((wl.B, wl.H, 1, wl.Dv), dtype=torch.bfloat16, device=dev)
    ws_lat = torch.empty((64 << 20,), dtype=torch.uint8, device=dev)

    if args.calib_copy_mib:
        src = torch.empty((args.calib_copy_mib << 20,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
        del src, dst

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    rec = {"prefill": [], "attn": [], "decode": [], "dec_attn": [], "lat": [], "lat_attn": []}

    # cos/sin tables: built once per length, as the pages cache them
    tab = mla.pipeline.build_table(rope_p, wp.T, wp.Dqk, dev)
    tdec = mla.pipeline.build_table(rope_d, wd.cache_len, wd.Dqk, dev)
    tlat = mla.pipeline.build_table(rope_l, wl.cache_len, wl.Dqk, dev)

    def step(timed: bool):
        e = [ev() for _ in range(8)] if timed else None
        if timed:
            e[0].record()
        mla.api.mla_latent_prepare(ip["latent"], ip["gain"], wp.eps, ip["k_pe"], tab.cos, tab.sin, wp.pairing,
                                   c_norm=bufs.c_norm, k_rot=bufs.k_rot)
        mla.api.mla_kv_expand(bufs.c_norm, ip["W"], wp.H, wp.Dn, wp.Dv, k=bufs.k_nope, v=bufs.v, v_layout="cols")
        if timed:
            e[1].record()
        mla.api.mla_prefill_attention_cached(ip["q"], bufs.k_nope, bufs.k_rot, bufs.v, 0, tab.cos, tab.sin,
                                             tab.scale, wp.pairing, out=bufs.out)
        if timed:
            e[2].record()
        mla.api.mla_latent_rmsnorm(idc["latent"], idc["gain"], wd.eps, out=c_dec)
        mla.api.mla_kv_expand(c_dec, idc["W"], wd.H, wd.Dn, wd.Dv, k=idc["k_cache"], v=idc["v_cache"],
                              t_off=wd.q_pos, k_pe=idc["k_pe"], cos=tdec.cos, sin=tdec.sin, pos=qpos.view(-1, 1),
                              pairing=wd.pairing)
        if timed:
            e[3].record()
        mla.api.mla_decode_attention(idc["q"], idc["k_cache"], idc["v_cache"], seq, qpos, tdec.cos, tdec.sin,
                                     tdec.scale, wd.Dn, wd.pairing, splits, out=out_dec, workspace=ws_dec)
        if timed:
            e[4].record()
        mla.api.mla_latent_cache_append(il["latent"].view(wl.B, wl.R), il["gain"], il["k_pe"].view(wl.B, wl.Dr),
                                        tlat.cos, tlat.sin, qpos_l, il["latent_cache"], wl.eps, wl.pairing)
        if timed:
            e[5].record()
        mla.api.mla_decode_absorbed(il["q"], il["W"], w_ukt, il["latent_cache"], seq_l, qpos_l, tlat.cos, tlat.sin,
                                    tlat.scale, wl.Dn, wl.Dv, wl.pairing, 0, out=out_lat, workspace=ws_lat)
        if timed:
            e[6].record()
        return e

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        evs.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in evs:
        rec["prefill"].append(e[0].elapsed_time(e[2]))
        rec["attn"].append(e[1].elapsed_time(e[2]))
        rec["decode"].append(e[2].elapsed_time(e[4]))
        rec["dec_attn"].append(e[3].elapsed_time(e[4]))
        rec["lat"].append(e[4].elapsed_time(e[6]))
        rec["lat_attn"].append(e[5].elapsed_time(e[6]))
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731

    # chunked prefill: fill the expanded cache with the whole sequence (the
    # chunk's own rows included), then time the chunk's attention call
    TQ = 1024
    past = wp.T - TQ
    mla.api.mla_latent_prepare(ip["latent"], ip["gain"], wp.eps, ip["k_pe"], tab.cos, tab.sin, wp.pairing,
                               c_norm=bufs.c_norm, k_rot=bufs.k_rot)
    mla.api.mla_kv_expand(bufs.c_norm, ip["W"], wp.H, wp.Dn, wp.Dv, k=bufs.k_nope, v=bufs.v, v_layout="cols")
    k_rot = bufs.k_rot
    q_chunk = ip["q"][:, :, past:].contiguous()
    out_chunk = torch.empty((wp.B, wp.H, TQ, wp.Dv), dtype=torch.bfloat16, device=dev)

    def chunk():
        mla.api.mla_prefill_attention_cached(q_chunk, bufs.k_nope, k_rot, bufs.v, past, tab.cos, tab.sin, tab.scale,
                                             wp.pairing, out=out_chunk)
    for _ in range(2):
        chunk()
    torch.cuda.synchronize()
    ce = [ev() for _ in range(11)]
    ce[0].record()
    for i in range(10):
        chunk()
        ce[i + 1].record()
    torch.cuda.synchronize()
    t_chunk = mean([ce[i].elapsed_time(ce[i + 1]) for i in range(10)]) * 1e-3
    chunk_flops = 2.0 * wp.B * wp.H * (TQ * past + TQ * (TQ + 1) / 2) * (wp.Dqk + wp.Dv)

    # latent-cache decode by re-expansion of every cached row (the eager
    # alternative to the absorbed form), attention call only
    ws_rx = torch.empty((1400 << 20,), dtype=torch.uint8, device=dev)

    def reexpand():
        mla.api.mla_decode_latent_expanded(il["q"], il["W"], il["latent_cache"], seq_l, qpos_l, tlat.cos, tlat.sin,
                                           tlat.scale, wl.Dn, wl.Dv, wl.pairing, 0, out=out_lat, workspace=ws_rx)
    reexpand()
    torch.cuda.synchronize()
    re = [ev() for _ in range(6)]
    re[0].record()
    for i in range(5):
        reexpand()
        re[i + 1].record()
    torch.cuda.synchronize()
    t_rx = mean([re[i].elapsed_time(re[i + 1]) for i in range(5)]) * 1e-3
    del ws_rx

    # the whole attention block at the 8k prefill shape
    import dataclasses
    wb = dataclasses.replace(workloads.WORKLOADS["kimi_k2_block_1k"], B=wp.B, T=wp.T)
    ib = workloads.make_inputs(wb, device=dev)
    tb = mla.pipeline.build_table(mla.api.params_from(wb.rope, wb.Dr), wb.T, wb.Dqk, dev)

    def block():
        return mla.pipeline.block_forward(ib["hidden"], ib["W_qa"], ib["gain_q"], ib["W_qb"], ib["W_kva"], ib["gain"],
                                          ib["W"], ib["W_o"], tb, wb.H, wb.Dn, wb.Dr, wb.Dv, wb.pairing, wb.eps)
    block()
    torch.cuda.synchronize()
    be = [ev() for _ in range(4)]
    be[0].record()
    for i in range(3):
        block()
        be[i + 1].record()
    torch.cuda.synchronize()
    t_block = mean([be[i].elapsed_time(be[i + 1]) for i in range(3)]) * 1e-3
    mt = wb.B * wb.T
    block_flops = (2.0 * mt * (wb.hidden * wb.q_lora + wb.q_lora * wb.H * wb.Dqk + wb.hidden * (wb.R + wb.Dr) +
                               wb.H * wb.Dv * wb.hidden) + attn_flops(wb) + expand_flops(wb))
    del ib

    def launch_times(fn, n):
        """Per-launch times (ms) of n back-to-back calls, HIP events on the stream."""
        fn()
        torch.cuda.synchronize()
        e = [ev() for _ in range(n + 1)]
        e[0].record()
        for i in range(n):
            fn()
            e[i + 1].record()
        torch.cuda.synchronize()
        return [e[i].elapsed_time(e[i + 1]) for i in range(n)]

    median = lambda xs: sorted(xs)[len(xs) // 2]  # noqa: E731

    # prefill attention at the other two prefill shapes: Kimi-K2 1k (warm,
    # and cold after a 512 MB write that evicts the last-level cache) and
    # GLM-5 4k (Dqk 256, Dv 256, interleaved pairing)
    shapes = {}
    for name in ("kimi_k2_1k", "glm5_4k"):
        w = workloads.WORKLOADS[name]
        inp = workloads.make_inputs(w, device=dev)
        b = mla.pipeline.alloc_prefill(w.B, w.T, w.H, w.R, w.Dn, w.Dr, w.Dv, dev)
        t = mla.pipeline.build_table(mla.api.params_from(w.rope, w.Dr), w.T, w.Dqk, dev)
        mla.api.mla_latent_prepare(inp["latent"], inp["gain"], w.eps, inp["k_pe"], t.cos, t.sin, w.pairing,
                                   c_norm=b.c_norm, k_rot=b.k_rot)
        mla.api.mla_kv_expand(b.c_norm, inp["W"], w.H, w.Dn, w.Dv, k=b.k_nope, v=b.v, v_layout="cols")

        def attn(w=w, inp=inp, b=b, t=t):
            mla.api.mla_prefill_attention_cached(inp["q"], b.k_nope, b.k_rot, b.v, 0, t.cos, t.sin, t.scale,
                                                 w.pairing, out=b.out)
        rec_s = {"warm_ms": median(launch_times(attn, 20))}
        if name == "kimi_k2_1k":
            flush = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
            cold = []
            for i in range(10):
                flush.fill_(i)
                e0, e1 = ev(), ev()
                e0.record()
                attn()
                e1.record()
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1))
            rec_s["cold_ms"] = median(cold)
            del flush
        # algorithmic bytes: q, k_nope, v, out per head and the shared k_pe
        abytes = 2.0 * w.B * w.H * w.T * (w.Dqk + w.Dn + 2 * w.Dv) + 2.0 * w.B * w.T * w.Dr
        rec_s["flops"] = attn_flops(w)
        rec_s["attainable_tflops"] = min(MFMA_PEAK_TFLOPS, attn_flops(w) / abytes * HBM_PEAK_GBS / 1e3)
        shapes[name] = rec_s
        del inp, b

    # the two decode steps recorded once as HIP graphs and replayed (the same
    # calls as in the timed steps, table build included): launch-bound steps
    td, tl = tdec, tlat

    def dec_step():
        mla.api.mla_latent_rmsnorm(idc["latent"], idc["gain"], wd.eps, out=c_dec)
        mla.api.mla_kv_expand(c_dec, idc["W"], wd.H, wd.Dn, wd.Dv, k=idc["k_cache"], v=idc["v_cache"],
                              t_off=wd.q_pos, k_pe=idc["k_pe"], cos=td.cos, sin=td.sin, pos=qpos.view(-1, 1),
                              pairing=wd.pairing)
        return mla.api.mla_decode_attention(idc["q"], idc["k_cache"], idc["v_cache"], seq, qpos, td.cos, td.sin,
                                            td.scale, wd.Dn, wd.pairing, splits, out=out_dec, workspace=ws_dec)

    def lat_step():
        mla.api.mla_latent_cache_append(il["latent"].view(wl.B, wl.R), il["gain"], il["k_pe"].view(wl.B, wl.Dr),
                                        tl.cos, tl.sin, qpos_l, il["latent_cache"], wl.eps, wl.pairing)
        return mla.api.mla_decode_absorbed(il["q"], il["W"], w_ukt, il["latent_cache"], seq_l, qpos_l, tl.cos,
                                           tl.sin, tl.scale, wl.Dn, wl.Dv, wl.pairing, 0, out=out_lat,
                                           workspace=ws_lat)
    g_dec = mla.pipeline.StepGraph(dec_step)
    g_lat = mla.pipeline.StepGraph(lat_step)
    t_dec_graph = median(launch_times(g_dec.replay, 20)) * 1e-3
    t_lat_graph = median(launch_times(g_lat.replay, 20)) * 1e-3
    del g_dec, g_lat

    # sustained ceilings of this chip: a streaming HBM read and a dense fp16
    # MFMA loop on random operands (our own kernels), and the vendor bf16 GEMM
    # (torch.matmul, hipBLASLt) on random 8192^3 operands as a black box
    hbm_buf = torch.empty((2 << 30,), dtype=torch.uint8, device=dev).fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    hbm_gbs = (2 << 30) / median(launch_times(lambda: mla.api.mla_ceiling_hbm_read(hbm_buf, sink), 10)) / 1e6
    del hbm_buf
    gen = torch.Generator(device=dev).manual_seed(11)
    ops = torch.randn(24576, generator=gen, device=dev).to(torch.float16)
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    mfma_ceiling = {}
    for lds in (False, True):
        fl = [0.0]

        def loop(lds=lds, fl=fl):
            fl[0] = mla.api.mla_ceiling_mfma(ops, 1000, lds, fsink)
        t_loop = median(launch_times(loop, 8))  # runs the loop (and sets its flop count) first
        mfma_ceiling[lds] = fl[0] / t_loop / 1e9
    ga = torch.randn((8192, 8192), generator=gen, device=dev).to(torch.bfloat16)
    gb = torch.randn((8192, 8192), generator=gen, device=dev).to(torch.bfloat16)
    gemm_tflops = 2.0 * 8192 ** 3 / median(launch_times(lambda: torch.matmul(ga, gb), 8)) / 1e9
    del ga, gb
    # the chip at hand: compute units and peak clocks as the runtime reports
    # them, and the dense 16-bit MFMA rate they imply (4096 flop/clk per CU)
    device = mla.api.mla_device_info(0)
    device["arch"] = torch.cuda.get_device_properties(0).gcnArchName
    device["mfma_f16_peak_at_peak_sclk_tflops"] = round(
        device["compute_units"] * 4096 * device["peak_sclk_mhz"] * 1e6 / 1e12, 1)
    ms_step = wall * 1e3 / args.steps
    t_prefill = mean(rec["prefill"]) * 1e-3
    t_attn = mean(rec["attn"]) * 1e-3
    t_dec_attn = mean(rec["dec_attn"]) * 1e-3
    t_decode = mean(rec["decode"]) * 1e-3
    t_lat = mean(rec["lat"]) * 1e-3
    t_lat_attn = mean(rec["lat_attn"]) * 1e-3
    lat_bytes = wl.B * wl.cache_len * (wl.R + wl.Dr) * 2  # the latent cache rows read
    fa, fe = attn_flops(wp), expand_flops(wp)
    path_tflops = (fa + fe) / t_prefill / 1e12
    attn_tflops = fa / t_attn / 1e12
    value = attn_tflops  # the metric: prefill attention TFLOP/s
    dec_gbs = decode_bytes(wd) / t_dec_attn / 1e9
    log(f"[bench] prefill path {t_prefill * 1e3:.3f} ms ({path_tflops:.1f} TFLOP/s), attention {t_attn * 1e3:.3f} ms "
        f"({attn_tflops:.1f} TFLOP/s, {attn_tflops / MFMA_PEAK_TFLOPS:.1%} of peak); decode step "
        f"{t_decode * 1e6:.1f} us, decode attention {t_dec_attn * 1e6:.1f} us ({dec_gbs:.0f} GB/s); latent-cache "
        f"decode step {t_lat * 1e6:.1f} us (attention {t_lat_attn * 1e6:.1f} us); chunked prefill (1024 after "
        f"7168) {t_chunk * 1e3:.3f} ms ({chunk_flops / t_chunk / 1e12:.1f} TFLOP/s); latent-cache decode by "
        f"re-expansion {t_rx * 1e6:.0f} us; attention block (8k) {t_block * 1e3:.3f} ms "
        f"({block_flops / t_block / 1e12:.1f} TFLOP/s)")
    log(f"[bench] decode steps replayed as HIP graphs: expanded cache {t_dec_graph * 1e6:.1f} us, latent cache "
        f"{t_lat_graph * 1e6:.1f} us")
    k1, g4 = shapes["kimi_k2_1k"], shapes["glm5_4k"]
    log(f"[bench] prefill attention kimi_k2_1k {k1['flops'] / k1['warm_ms'] / 1e9:.1f} TFLOP/s warm, "
        f"{k1['flops'] / k1['cold_ms'] / 1e9:.1f} cold (attainable {k1['attainable_tflops']:.0f}); glm5_4k "
        f"{g4['flops'] / g4['warm_ms'] / 1e9:.1f} TFLOP/s; ceilings: HBM read {hbm_gbs:.0f} GB/s, fp16 MFMA on "
        f"random operands {mfma_ceiling[False]:.0f} TFLOP/s (A from LDS {mfma_ceiling[True]:.0f}), vendor bf16 "
        f"GEMM 8192^3 {gemm_tflops:.0f} TFLOP/s")

    result = {
        "metric": "MLA prefill attn TFLOP/s + % bf16 MFMA peak; decode GB/s at 1k ctx",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp16 k/v + MFMA, fp32 acc",
        "data": "synthetic",
        "config": {
            "workload": f"{PREFILL} prefill (B=2 T=8192 H=64 R=512 Dn/Dr/Dv=128/64/128 YaRN f=32) + "
                        f"{DECODE} step (B=32 L=1001 pos 1000)",
            "prefill_attention_tflops": round(attn_tflops, 2),
            "prefill_attention_ms": round(t_attn * 1e3, 4),
            "prefill_path_ms": round(t_prefill * 1e3, 4),
            "prefill_path_tflops": round(path_tflops, 2),
            "prefill_tokens_per_s": round(wp.B * wp.T / t_prefill, 1),
            "decode_attention_us": round(t_dec_attn * 1e6, 2),
            "decode_attention_gbs": round(dec_gbs, 1),
            "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "decode_step_us": round(t_decode * 1e6, 2),
            "decode_tokens_per_s": round(wd.B / t_decode, 1),
            "decode_splits": splits,
            "decode_traffic_bytes": measured_traffic("head_latent_attention_rmsnorm_amd/csrc/decode_attn.hip",
                                                     "decode"),
            "decode_algorithmic_bytes": int(decode_bytes(wd)),
            "decode_latent_workload": f"{DECODE_LATENT} (B=32 L=1001 pos 1000, fp16 latent cache 576/token)",
            "decode_latent_step_us": round(t_lat * 1e6, 2),
            "decode_latent_attention_us": round(t_lat_attn * 1e6, 2),
            "decode_latent_tokens_per_s": round(wl.B / t_lat, 1),
            "decode_latent_cache_bytes": int(lat_bytes),
            "decode_latent_cache_gbs": round(lat_bytes / t_lat_attn / 1e9, 1),
            "decode_latent_reexpand_attention_us": round(t_rx * 1e6, 1),
            "decode_step_graph_us": round(t_dec_graph * 1e6, 2),
            "decode_latent_step_graph_us": round(t_lat_graph * 1e6, 2),
            "block_workload": "attention block at the 8k prefill shape (hidden 7168, q rank 1536, no biases)",
            "block_ms": round(t_block * 1e3, 4),
            "block_tflops": round(block_flops / t_block / 1e12, 2),
            "chunked_prefill_workload": f"{PREFILL} last {TQ} tokens after {past} cached rows",
            "chunked_prefill_attention_ms": round(t_chunk * 1e3, 4),
            "chunked_prefill_attention_tflops": round(chunk_flops / t_chunk / 1e12, 2),
            "prefill_kimi_k2_1k_attention_tflops": round(k1["flops"] / k1["warm_ms"] / 1e9, 2),
            "prefill_kimi_k2_1k_attention_tflops_cold": round(k1["flops"] / k1["cold_ms"] / 1e9, 2),
            "prefill_kimi_k2_1k_attainable_tflops": round(k1["attainable_tflops"], 1),
            "prefill_glm5_4k_attention_tflops": round(g4["flops"] / g4["warm_ms"] / 1e9, 2),
            "prefill_glm5_4k_mfma_frac": round(g4["flops"] / g4["warm_ms"] / 1e9 / MFMA_PEAK_TFLOPS, 4),
            "device": device,
            "ceiling_hbm_read_gbs": round(hbm_gbs, 1),
            "ceiling_mfma_f16_random_tflops": round(mfma_ceiling[False], 1),
            "ceiling_mfma_f16_random_lds_operand_tflops": round(mfma_ceiling[True], 1),
            "ceiling_vendor_gemm_bf16_random_8192_tflops": round(gemm_tflops, 1),
            "prefill_attention_frac_of_mfma_ceiling": round(attn_tflops / mfma_ceiling[False], 4),
            "decode_attention_frac_of_hbm_read_ceiling": round(dec_gbs / hbm_gbs, 4),
            "decode_latent_attn_kernel_traffic_bytes": measured_traffic(
                "head_latent_attention_rmsnorm_amd/csrc/decode_latent.hip", "decode_latent"),
        },
        "roofline": {
            "kernel": "prefill_dual_kernel (causal flash attention, Dqk 192, Dv 128, two row blocks per wave)",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("head_latent_attention_rmsnorm_amd/csrc/prefill_dual.hip", "prefill"),
        },
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (fp64 oracle, ~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
