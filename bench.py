#!/usr/bin/env python3
"""Benchmark of the OAL causal-attention hot path on one MI355X.

Prefill (headline): the Qwen2.5-0.5B-shaped layer, B=1, T=4096, 14 query heads over 2 KV
heads, d=64, bf16 inputs (synthetic, seeded). A step is one oal_prefill call over the
batch: chunk-state scan + readout. Successive steps continue the state (each step is
another 4096 tokens of the same sequences), so no extra work enters the timed region.

Decode: 64 sequences whose prefix states were built by oal_prefill from 4096 synthetic
tokens each; then --warmup untimed and --decode-steps timed oal_decode_step calls (one token
per sequence each).

Contribution scores: oal_contribution (the per-dim causal statistic chi and its prompt
mean) over a calibration batch of 8 prompts x 4096 tokens, timed over 50 back-to-back calls.

Decode against HBM: 512 sequences (571 MB of prefix state, more than the 256 MB last-level
cache), each step reading and writing every state once.

Prints one JSON line. `value` is prefill tokens/s; `roofline` is the whole prefill step (its
three kernels together) against the bf16 MFMA peak, with the readout kernel (the dominant
one) as `roofline.readout`; `achievable_peaks` holds the rates of a matrix-core loop and a
streaming copy measured on this device; `decode` holds decode tokens/s and the decode kernel
against HBM peak (`decode.hbm_512seq` for the state that does not fit in the cache);
`contribution` the chi kernel against HBM peak; `backward` the prefill backward (dq, dk, dv)
of the headline workload against the fp32 MFMA peak (its fp32-accurate products run as six
bf16 MFMA products, whose ceiling is also given); `cpu_baseline` is the fp64 CPU oracle on
the full prefill batch, timed on this host, with the other workloads under
`cpu_baseline.other_workloads`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "OAL attention tokens/s at T=4096 (prefill) + decode tok/s; % MFMA/HBM peak"
D, V1, NFEAT = 64, 65, 2145
FLOP_PER_TOKEN_HEAD = 2 * NFEAT * V1          # 278,850: one feature-space contraction
PEAK_BF16_TFLOPS = 2500.0                     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0                         # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3                      # MI355X fp32 MFMA dense (fp64: 78.6)
PHASE_EVERY = 4                               # timed steps with per-kernel events


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=128)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--seq", type=int, default=4096)
    ap.add_argument("--decode-seqs", type=int, default=64)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--hbm-decode-seqs", type=int, default=512,
                    help="sequences of the decode run whose state exceeds the caches (0: skip)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the matrix-core loop and streaming-copy measurements")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-contribution", action="store_true",
                    help="skip the contribution-score (chi) measurement")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the prefill-backward measurement")
    ap.add_argument("--no-scaling", action="store_true",
                    help="skip the B=8 x T=4096 chunk sweep and the T=32768 prefill")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "profiles", "traffic.json"))
    return ap.parse_args()


def measured_traffic(tj, key):
    """HBM bytes per launch from the stored FETCH_SIZE/WRITE_SIZE counters, or None when the
    kernel's source file has changed since they were taken (the stored sha256 differs)."""
    import hashlib
    rec = tj.get(key)
    if not rec or "source" not in rec:
        return None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "grouped_positive_quadratic_amd",
                        "csrc", rec["source"])
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return rec["bytes_per_launch"] if digest == rec.get("source_sha256") else None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU: the OAL hot path here is a "
                                   "single-device kernel library; multi-GPU runs are not supported "
                                   f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})"}))
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 64 << 20                                     # 64 Mi floats = 256 MiB each way
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return
    import grouped_positive_quadratic_amd as gpq
    from oal_synth import qwen_like, cfg5_prefix, cfg5_steps

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ---------------- prefill ----------------
    B, T, C = args.batch, args.seq, args.chunk
    inp = qwen_like(B, T, 2, name="prefill") if B > 1 or T != 4096 else qwen_like(1, 4096, 2, name="cfg2")
    Bq, Hq, Hkv, _, _, _ = inp.dims
    dims = gpq.make_dims(B, Hq, Hkv, "bf16")
    hp = gpq.HeadParamsC.from_params(inp.params)
    params, state, ws, _ = gpq.alloc_buffers(dims, T, C)
    gpq.oal_state_init(dims, hp, params, state)
    q = torch.from_numpy(inp.q).to(torch.bfloat16).to(dev).contiguous()
    k = torch.from_numpy(inp.k).to(torch.bfloat16).to(dev).contiguous()
    v = torch.from_numpy(inp.v).to(torch.bfloat16).to(dev).contiguous()
    y = torch.empty((B, Hq, T, D), dtype=torch.float32, device=dev)
    # Per-kernel times come from events recorded around the kernels on the launch stream, in
    # every PHASE_EVERY-th timed step only: each recorded event costs a few microseconds of
    # device time between two kernels (fence-free timing events, still a marker packet), which
    # would otherwise be counted in ms_per_step.
    timed_steps = [i for i in range(args.steps) if i % PHASE_EVERY == 0]
    marks = {i: [gpq.TimingEvent() for _ in range(3)] for i in timed_steps}
    for mk in marks.values():
        for m in mk:
            m.record(stream)          # create the underlying events
    for _ in range(args.warmup):
        gpq.oal_prefill(dims, T, C, q, k, v, params, state, ws, y)
    torch.cuda.synchronize()
    t_start, t_end = gpq.TimingEvent(), gpq.TimingEvent()
    t_start.record(stream)
    for i in range(args.steps):
        if i in marks:
            gpq.oal_prefill_timed(dims, T, C, q, k, v, params, state, ws, y, marks[i])
        else:
            gpq.oal_prefill(dims, T, C, q, k, v, params, state, ws, y)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    scan_ms = float(np.mean([mk[0].elapsed_time(mk[1]) for mk in marks.values()]))
    read_ms = float(np.mean([mk[1].elapsed_time(mk[2]) for mk in marks.values()]))
    # the same K steps captured into one HIP graph and replayed (no per-launch host work)
    gr = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        gpq.oal_prefill(dims, T, C, q, k, v, params, state, ws, y)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        for _ in range(args.steps):
            gpq.oal_prefill(dims, T, C, q, k, v, params, state, ws, y)
    gr.replay()
    torch.cuda.synchronize()
    g0, g1 = gpq.TimingEvent(), gpq.TimingEvent()
    g0.record(stream)
    gr.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    ms_graph = g0.elapsed_time(g1) / args.steps
    del gr
    tokens = B * T
    readout_flops = FLOP_PER_TOKEN_HEAD * tokens * Hq
    scan_flops = FLOP_PER_TOKEN_HEAD * tokens * Hkv
    achieved = readout_flops / (read_ms * 1e-3) / 1e12
    tj = {}
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
        except (OSError, ValueError):
            tj = {}
    traffic = measured_traffic(tj, f"readout_B{B}_T{T}_C{C}")
    step_flops = readout_flops + scan_flops
    step_tflops = step_flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill B={B} T={T} Hq={Hq} Hkv={Hkv} d=64 (Qwen2.5-0.5B-shaped layer)",
                   "global_batch": B, "seq_len": T, "chunk": C, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "whole prefill step (intra/increments, chunk prefix, readout)",
                     "achieved": step_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": step_tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(tj, f"prefill_step_B{B}_T{T}_C{C}"), "avg_ms": ms_step,
                     "algorithmic_flops_per_launch": step_flops,
                     "readout": {"kernel": "oal_readout", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                                 "traffic": traffic, "avg_ms": read_ms,
                                 "algorithmic_flops_per_launch": readout_flops}},
        "phases_ms": {"intra_and_scan": scan_ms, "readout": read_ms,
                      "sampled_steps": len(marks), "note": "events around the kernels in every "
                      f"{PHASE_EVERY}th timed step"},
        "graph_replay": {"ms_per_step": ms_graph, "value": tokens / (ms_graph * 1e-3),
                         "note": "the timed steps captured into one HIP graph, replayed once"},
    }
    del q, k, v, y, ws, state, params
    torch.cuda.empty_cache()

    # ---------------- achievable peaks on this device ----------------
    if not args.no_peaks:
        props = torch.cuda.get_device_properties(dev)
        nblk = props.multi_processor_count * 8          # 2 wavefronts per SIMD
        mout = torch.empty(nblk * 256, dtype=torch.float32, device=dev)
        gpq.oal_calib_mfma_bf16(nblk, 2048, mout)       # warm-up: code object load, clock ramp
        torch.cuda.synchronize()
        e0, e1 = gpq.TimingEvent(), gpq.TimingEvent()
        e0.record(stream)
        mflops = sum(gpq.oal_calib_mfma_bf16(nblk, 2048, mout) for _ in range(3))
        e1.record(stream)
        mms = e0.elapsed_time(e1)
        mfma_tflops = mflops / (mms * 1e-3) / 1e12
        del mout
        nbytes = 1 << 30                                # 1 GiB each way: 8x the last-level cache
        csrc = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        cdst = torch.empty_like(csrc)
        gpq.oal_calib_copy(csrc, cdst, nbytes)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            gpq.oal_calib_copy(csrc, cdst, nbytes)
        e1.record(stream)
        cms = e0.elapsed_time(e1) / 5
        copy_gbs = 2 * nbytes / (cms * 1e-3) / 1e9
        del csrc, cdst
        torch.cuda.empty_cache()
        out["achievable_peaks"] = {
            "mfma_bf16": {"tflops": mfma_tflops, "frac_of_nominal": mfma_tflops / PEAK_BF16_TFLOPS,
                          "kernel": "oal_calib_mfma_bf16: 8 independent 16x16x32 bf16 MFMA chains per "
                                    f"wavefront, {nblk} workgroups x 4 wavefronts, 3 x 2048 rounds"},
            "hbm_copy": {"gbs": copy_gbs, "frac_of_nominal": copy_gbs / PEAK_HBM_GBS,
                         "kernel": "oal_calib_copy: 1 GiB device-to-device, one 16-byte load and "
                                   "store per thread; bytes read + written"},
            "prefill_step_frac_of_achievable": step_tflops / mfma_tflops,
            "readout_frac_of_achievable": achieved / mfma_tflops}

    cache = {}

    def get_cfg3():
        if "cfg3" not in cache:
            from oal_synth import cfg3
            cache["cfg3"] = cfg3()
        return cache["cfg3"]

    # ---------------- the other prefill workloads (context, not the headline) ----------------
    if not args.no_scaling:
        def prefill_rate(inp, C, reps):
            Bx, Hqx, Hkvx, Tx, _, _ = inp.dims
            dx = gpq.make_dims(Bx, Hqx, Hkvx, "bf16")
            px, sx, wx, _ = gpq.alloc_buffers(dx, Tx, C)
            gpq.oal_state_init(dx, gpq.HeadParamsC.from_params(inp.params), px, sx)
            qx, kx, vx = (torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous() for a in (inp.q, inp.k, inp.v))
            yx = torch.empty((Bx, Hqx, Tx, D), dtype=torch.float32, device=dev)
            gpq.oal_prefill(dx, Tx, C, qx, kx, vx, px, sx, wx, yx)      # warm-up
            torch.cuda.synchronize()
            e0, e1 = gpq.TimingEvent(), gpq.TimingEvent()
            e0.record(stream)
            for _ in range(reps):
                gpq.oal_prefill(dx, Tx, C, qx, kx, vx, px, sx, wx, yx)
            e1.record(stream)
            ms = e0.elapsed_time(e1) / reps
            del px, sx, wx, qx, kx, vx, yx
            torch.cuda.empty_cache()
            return Bx * Tx / (ms * 1e-3), ms
        from oal_synth import cfg4
        c3 = get_cfg3()
        batch8 = {}
        for C in (64, 128, 256):
            r, ms = prefill_rate(c3, C, 5)
            batch8[f"chunk{C}"] = {"tokens_per_s": r, "ms_per_call": ms}
        c4 = cfg4()
        r4, ms4 = prefill_rate(c4, 128, 3)
        del c4
        from oal_synth import per_dim_params
        cg = qwen_like(1, 4096, 64, name="cfg2_g64")
        cg.params = per_dim_params(640, 14)
        rg, msg = prefill_rate(cg, 128, 5)
        del cg
        out["prefill_other_workloads"] = {
            "B8_T4096": {"workload": "prefill B=8 T=4096 14q/2kv bf16, one call per step", **batch8},
            "B1_T32768": {"workload": "prefill B=1 T=32768 14q/2kv bf16, chunk 128", "tokens_per_s": r4,
                          "ms_per_call": ms4,
                          "vs_T4096_tokens_per_s": r4 / out["value"]},
            "B1_T4096_G64": {"workload": "prefill B=1 T=4096 14q/2kv bf16, chunk 128, per-dimension "
                                         "variant (G = 64 on every head: general coefficient blob)",
                             "tokens_per_s": rg, "ms_per_call": msg,
                             "vs_G_small_tokens_per_s": rg / out["value"]},
        }

    # ---------------- contribution scores (chi) on a calibration batch ----------------
    if not args.no_contribution:
        c3 = get_cfg3()
        Bc, Hqc, Hkvc, Tc, _, _ = c3.dims
        cd = gpq.make_dims(Bc, Hqc, Hkvc, "bf16")
        cq, ck = (torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous() for a in (c3.q, c3.k))
        cws = torch.empty(gpq.oal_contribution_workspace_bytes(cd, Tc), dtype=torch.uint8, device=dev)
        chi = torch.empty((Bc, Hqc, D), dtype=torch.float32, device=dev)
        chi_mean = torch.empty((Hqc, D), dtype=torch.float32, device=dev)
        for _ in range(3):
            gpq.oal_contribution(cd, Tc, cq, ck, cws, chi, chi_mean)
        torch.cuda.synchronize()
        reps = 50
        e0, e1 = gpq.TimingEvent(), gpq.TimingEvent()
        e0.record(stream)
        for _ in range(reps):
            gpq.oal_contribution(cd, Tc, cq, ck, cws, chi, chi_mean)
        e1.record(stream)
        cms = e0.elapsed_time(e1) / reps
        cbytes = (Bc * (Hqc + Hkvc) * Tc * D * 2          # q and k read once
                  + (Bc * Hqc + Hqc) * D * 4)              # chi and its prompt mean written
        cach = cbytes / (cms * 1e-3) / 1e9
        out["contribution"] = {
            "workload": f"causal contribution scores chi, B={Bc} prompts x T={Tc}, {Hqc}q/{Hkvc}kv, bf16",
            "value": Bc * Tc / (cms * 1e-3), "unit": "tokens/s", "ms_per_call": cms, "calls": reps,
            "roofline": {"bound": "hbm", "kernel": "oal_chi_kernel (the call's one launch)",
                         "achieved": cach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": cach / PEAK_HBM_GBS,
                         "traffic": measured_traffic(tj, f"contribution_B{Bc}_T{Tc}"),
                         "algorithmic_bytes_per_launch": cbytes}}
        del cq, ck, cws, chi, chi_mean
        torch.cuda.empty_cache()
    cache.clear()

    # ---------------- prefill backward on the headline workload ----------------
    if not args.no_backward:
        bi = qwen_like(1, 4096, 2, name="cfg2")
        Bb, Hqb, Hkvb, Tb, _, _ = bi.dims
        Cb = 64
        bd = gpq.make_dims(Bb, Hqb, Hkvb, "bf16")
        bparams = torch.empty(gpq.oal_params_bytes(bd), dtype=torch.uint8, device=dev)
        gpq.oal_state_init(bd, gpq.HeadParamsC.from_params(bi.params), bparams, None)
        bq, bk, bv = (torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous() for a in (bi.q, bi.k, bi.v))
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        bdy = torch.randn((Bb, Hqb, Tb, D), generator=gen, dtype=torch.float32, device=dev)
        bws = torch.empty(gpq.oal_prefill_backward_workspace_bytes(bd, Tb, Cb), dtype=torch.uint8, device=dev)
        bdq = torch.empty((Bb, Hqb, Tb, D), dtype=torch.float32, device=dev)
        bdk = torch.empty((Bb, Hkvb, Tb, D), dtype=torch.float32, device=dev)
        bdv = torch.empty_like(bdk)
        bdL = torch.empty((Hqb, 65, 65), dtype=torch.float32, device=dev)
        bde = torch.empty((Hqb,), dtype=torch.float32, device=dev)
        for _ in range(2):
            gpq.oal_prefill_backward(bd, Tb, Cb, bq, bk, bv, bdy, bparams, bws, bdq, bdk, bdv, bdL, bde)
        torch.cuda.synchronize()
        reps = 5
        e0, e1 = gpq.TimingEvent(), gpq.TimingEvent()
        e0.record(stream)
        for _ in range(reps):
            gpq.oal_prefill_backward(bd, Tb, Cb, bq, bk, bv, bdy, bparams, bws, bdq, bdk, bdv, bdL, bde)
        e1.record(stream)
        bms = e0.elapsed_time(e1) / reps
        # algorithmic fp32 work: six state-sized contractions of 2 * 2145 * 65 flops per token --
        # per query head: the readout u, S g and the query increment; per KV head: the key
        # increment, R^T psi(k) and R [v; 1]
        bflops = (3 * Bb * Hqb + 3 * Bb * Hkvb) * Tb * 2 * 2145 * 65
        bach = bflops / (bms * 1e-3) / 1e12
        out["backward"] = {
            "workload": f"prefill backward (dq, dk, dv, dL, deps) from an empty prefix, B={Bb} T={Tb} "
                        f"{Hqb}q/{Hkvb}kv, bf16 inputs, fp32-accurate arithmetic, chunk {Cb}",
            "value": Bb * Tb / (bms * 1e-3), "unit": "tokens/s", "ms_per_call": bms, "calls": reps,
            "roofline": {"bound": "mfma",
                         "kernel": "the call's launches together (state contractions and intra-chunk "
                                   "products on bf16 MFMA with three-part split fp32 operands)",
                         "achieved": bach, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                         "frac": bach / PEAK_FP32_TFLOPS, "traffic": None,
                         "algorithmic_flops_per_call": bflops,
                         # six bf16 products per fp32-accurate product: the split ceiling
                         "split_bf16_peak": PEAK_BF16_TFLOPS / 6,
                         "frac_of_split_peak": bach / (PEAK_BF16_TFLOPS / 6)}}
        del bq, bk, bv, bdy, bws, bdq, bdk, bdv, bdL, bde, bparams
        torch.cuda.empty_cache()

    # ---------------- decode ----------------
    if not args.no_decode:
        nseq, nsteps = args.decode_seqs, args.decode_steps
        pre = cfg5_prefix(n_seq=nseq)
        toks = cfg5_steps(n_seq=nseq, steps=nsteps)
        ddims = gpq.make_dims(nseq, 14, 2, "bf16")
        dhp = gpq.HeadParamsC.from_params(pre.params)
        dparams, dstate, dws_pre, dws = gpq.alloc_buffers(ddims, 4096, 128)
        gpq.oal_state_init(ddims, dhp, dparams, dstate)
        pk = torch.from_numpy(pre.k).to(torch.bfloat16).to(dev).contiguous()
        pv = torch.from_numpy(pre.v).to(torch.bfloat16).to(dev).contiguous()
        gpq.oal_prefill(ddims, 4096, 128, None, pk, pv, dparams, dstate, dws_pre, None)  # state only
        torch.cuda.synchronize()
        del pk, pv, dws_pre
        torch.cuda.empty_cache()
        tq = torch.from_numpy(toks.q).to(torch.bfloat16).to(dev).permute(2, 0, 1, 3).contiguous()
        tk = torch.from_numpy(toks.k).to(torch.bfloat16).to(dev).permute(2, 0, 1, 3).contiguous()
        tv = torch.from_numpy(toks.v).to(torch.bfloat16).to(dev).permute(2, 0, 1, 3).contiguous()
        dy = torch.empty((nsteps, nseq, 14, D), dtype=torch.float32, device=dev)
        for i in range(min(args.warmup, nsteps)):   # untimed: first launch loads the code object
            gpq.oal_decode_step(ddims, tq[i], tk[i], tv[i], dparams, dstate, dws, dy[i])
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(nsteps):
            gpq.oal_decode_step(ddims, tq[i], tk[i], tv[i], dparams, dstate, dws, dy[i])
        ev[1].record(stream)
        torch.cuda.synchronize()
        dms = ev[0].elapsed_time(ev[1]) / nsteps
        # the same step loop captured once into a HIP graph and replayed (a serving loop's
        # launch path): same kernels and work, no per-launch host submission
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            gpq.oal_decode_step(ddims, tq[0], tk[0], tv[0], dparams, dstate, dws, dy[0])
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            for i in range(nsteps):
                gpq.oal_decode_step(ddims, tq[i], tk[i], tv[i], dparams, dstate, dws, dy[i])
        gr.replay()                                   # warm-up replay
        torch.cuda.synchronize()
        ev[0].record(stream)
        gr.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        gms = ev[0].elapsed_time(ev[1]) / nsteps
        state_bytes = 2 * nseq * 2 * NFEAT * V1 * 4                   # state read + write
        io_bytes = nseq * (14 * D * 2 + 2 * 2 * D * 2 + 14 * D * 4)   # q, k, v in; y out
        alg = state_bytes + io_bytes
        dach = alg / (dms * 1e-3) / 1e9
        out["decode"] = {"value": nseq / (dms * 1e-3), "unit": "tokens/s", "ms_per_step": dms,
                         "steps": nsteps, "warmup": min(args.warmup, nsteps), "config": {"workload": f"decode {nseq} seqs, 4096-token prefix states, 14q/2kv"},
                         "roofline": {"bound": "hbm", "kernel": "oal_decode_kernel", "achieved": dach,
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dach / PEAK_HBM_GBS,
                                      "traffic": measured_traffic(tj, f"decode_{nseq}seq"),
                                      "algorithmic_bytes_per_launch": alg},
                         "graph_replay": {"ms_per_step": gms, "value": nseq / (gms * 1e-3),
                                          "frac": alg / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                          "note": "the timed step loop captured into one HIP graph, replayed once"}}

        # ---- the same step on 512 sequences: 571 MB of state, more than the last-level cache ----
        if args.hbm_decode_seqs > 0:
            n2 = args.hbm_decode_seqs
            d2 = gpq.make_dims(n2, 14, 2, "bf16")
            p2, s2, _, w2 = gpq.alloc_buffers(d2, 0, 128)
            gpq.oal_state_init(d2, dhp, p2, s2)
            # sequence b starts from the prefix state of sequence b % nseq (same structure and
            # size; the step's traffic does not depend on the values)
            blk = gpq.STATE_STRIDE * 2
            s2.view(n2, blk).copy_(dstate.view(nseq, blk).repeat((n2 + nseq - 1) // nseq, 1)[:n2])
            ns2 = 16
            t2 = cfg5_steps(n_seq=n2, steps=ns2)
            q2, k2, v2 = (torch.from_numpy(a).to(torch.bfloat16).to(dev).permute(2, 0, 1, 3).contiguous()
                          for a in (t2.q, t2.k, t2.v))
            y2 = torch.empty((ns2, n2, 14, D), dtype=torch.float32, device=dev)
            gpq.oal_decode_step(d2, q2[0], k2[0], v2[0], p2, s2, w2, y2[0])     # untimed
            torch.cuda.synchronize()
            ev[0].record(stream)
            for i in range(1, ns2):
                gpq.oal_decode_step(d2, q2[i], k2[i], v2[i], p2, s2, w2, y2[i])
            ev[1].record(stream)
            torch.cuda.synchronize()
            hms = ev[0].elapsed_time(ev[1]) / (ns2 - 1)
            alg2 = 2 * n2 * 2 * NFEAT * V1 * 4 + n2 * (14 * D * 2 + 2 * 2 * D * 2 + 14 * D * 4)
            hach = alg2 / (hms * 1e-3) / 1e9
            out["decode"]["hbm_512seq"] = {
                "workload": f"decode {n2} seqs, 4096-token prefix states ({2 * n2 * NFEAT * V1 * 4 / 1e6:.0f} MB "
                            "of state), 14q/2kv, eager launches",
                "value": n2 / (hms * 1e-3), "unit": "tokens/s", "ms_per_step": hms, "steps": ns2 - 1,
                "roofline": {"bound": "hbm", "kernel": "oal_decode_kernel", "achieved": hach,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": hach / PEAK_HBM_GBS,
                             "traffic": measured_traffic(tj, f"decode_{n2}seq"),
                             "algorithmic_bytes_per_launch": alg2}}
            del p2, s2, w2, q2, k2, v2, y2
            torch.cuda.empty_cache()

    # ---------------- CPU oracle baseline ----------------
    if not args.no_cpu_baseline:
        import oracle
        from oal_synth import cfg2
        ref = cfg2()
        oracle.dense(ref.q[:, :, :64], ref.k[:, :, :64], ref.v[:, :, :64], ref.params)   # load
        t0 = time.perf_counter()
        oracle.dense(ref.q, ref.k, ref.v, ref.params)
        wall = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": 4096 / wall, "unit": "tokens/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": "full prefill batch (B=1, T=4096, 14 q heads), dense O(T^2) fp64, 1 pass",
                               "wall_s": wall}
        other = {}
        from oal_synth import cfg3, cfg4
        c3 = cfg3()
        t0 = time.perf_counter()
        oracle.dense(c3.q, c3.k, c3.v, c3.params)
        w3 = time.perf_counter() - t0
        other["B8_T4096"] = {"value": c3.q.shape[0] * 4096 / w3, "unit": "tokens/s", "wall_s": w3,
                             "sample": "all 8 sequences x 4096 positions, dense O(T^2) fp64, 1 pass"}
        del c3
        c4 = cfg4()
        n4 = 4096
        t0 = time.perf_counter()
        oracle.dense(c4.q[:, :, :n4], c4.k[:, :, :n4], c4.v[:, :, :n4], c4.params)
        w4 = time.perf_counter() - t0
        T4 = c4.q.shape[2]
        scale = (T4 / n4) ** 2                       # the dense definition's cost grows as T^2
        other["B1_T32768"] = {"value": T4 / (w4 * scale), "unit": "tokens/s", "wall_s_sample": w4,
                              "extrapolated": True,
                              "sample": f"first {n4} positions (their outputs are exact: causal), timed, then "
                                        f"x{scale:.0f} for the full {T4} (dense cost ~ T^2): extrapolated"}
        del c4
        # decode: each new token's output by the dense definition over its prefix
        ns, nt = 8, 32
        p5 = cfg5_prefix(n_seq=ns)
        s5 = cfg5_steps(n_seq=ns, steps=args.decode_steps)
        T0 = p5.k.shape[2]
        t0 = time.perf_counter()
        for b in range(ns):
            kk = np.concatenate([p5.k[b:b + 1], s5.k[b:b + 1, :, :nt]], axis=2)
            vv = np.concatenate([p5.v[b:b + 1], s5.v[b:b + 1, :, :nt]], axis=2)
            qq = np.zeros((1, 14, T0 + nt, D))
            qq[:, :, T0:] = s5.q[b:b + 1, :, :nt]
            rows = [(0, h, T0 + t) for t in range(nt) for h in range(14)]
            oracle.dense_rows(qq, kk, vv, p5.params, rows)
        w5 = time.perf_counter() - t0
        other["decode_64seq"] = {"value": ns * nt / w5, "unit": "tokens/s", "wall_s": w5,
                                 "sample": f"{ns} of the 64 sequences x the first {nt} decode steps after "
                                           f"the {T0}-token prefix; each new token's 14 head outputs by the "
                                           "dense definition over its prefix (O(T) per token)"}
        out["cpu_baseline"]["other_workloads"] = other
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
