#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already
resident in HBM:
  * prefill of the layer workload (B=1, T=4096, 16 q/k heads, 48 value
    heads, d=128, bf16 q/k/v, fp32 alpha/beta/state, zero initial state), and
  * one decode step of the batched workload (B=256, same heads, fp32 states
    updated in place).
Shapes follow "The Hybrid Attention in Qwen3.8-27B" (section "Grouped-query
attention multiplies on top of that").

Reported: prefill tokens/s (value) with its fraction of the bf16 MFMA peak,
decode state-update GB/s with its fraction of HBM bandwidth, both from HIP
events on the stream the kernels run on; and the fp64 oracle timed on the
host cores as a CPU baseline. Timed apart from the step: under
"prefill_prefix_states" the same prefill also writing the state after every
1024 tokens; under "prepared_inputs" the prefill and decode step from raw
q, k and gate logits (prepared inside the kernels); under "segmented_prefill"
the per-GPU share of the layer at 8-way head-group sharding (6 value heads,
T = 4096 and 262,144) in one pass and split into segments; and under "decode_multi"
the K-token decode against a slot pool (B=256 sequences verifying K=4 tokens
each), in tokens/s and HBM GB/s.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (% bf16 MFMA peak); decode state-update GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CHUNK = 64


def prefill_flops_per_token(Hk, Hv, dk, dv, C=CHUNK):
    """Algorithmic flops per token of the chunk-64 method (triangular
    products counted as triangular, Gram products once per q/k head):
    Hk*2*C*dk + Hv*(6*dk*dv + (C+1)*(2*dv + dk) + C^2/3)."""
    return Hk * 2 * C * dk + Hv * (6 * dk * dv + (C + 1) * (2 * dv + dk) + C * C / 3.0)


def prefill_bytes_per_token(Hk, Hv, dk, dv, es=2):
    """Required HBM bytes per token: q, k, v in, o out, alpha and beta (fp32)."""
    return 2 * Hk * dk * es + 2 * Hv * dv * es + 2 * Hv * 4


def decode_bytes_per_step(B, Hk, Hv, dk, dv, es=2):
    """Required HBM bytes of one decode step: each fp32 state read and written
    once, q, k, v read, o written, alpha and beta read."""
    return B * (Hv * dv * dk * 4 * 2 + 2 * Hk * dk * es + 2 * Hv * dv * es + 2 * Hv * 4)


def decode_multi_bytes(B, K, Hk, Hv, dk, dv, es=2):
    """Required HBM bytes of one K-token decode against a slot pool: each
    sequence's fp32 state read from its source slot and written to its
    destination slot once, K tokens of q, k, v read and o written, alpha and
    beta read, and the two slot indices per sequence."""
    return (B * Hv * dv * dk * 4 * 2
            + B * K * (2 * Hk * dk * es + 2 * Hv * dv * es + 2 * Hv * 4) + B * 8)


def _src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, digest):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a copy-kernel calibration), if recorded for the
    current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(d, w, budget_s=20.0):
    """Time the fp64 oracle on the prefill workload on the host cores: whole
    passes over all 48 value heads until about budget_s seconds are spent
    (at least one pass)."""
    import oracle
    threads = oracle.default_threads()
    tokens = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, threads=threads)
        passes += 1
        tokens += w.B * w.T
        el = time.perf_counter() - t0
        if el >= budget_s or el * (passes + 1) / passes > 1.5 * budget_s:
            break
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} full pass(es) of the fp64 token-by-token oracle over "
                      f"{w.name} (B={w.B}, T={w.T}, {w.Hv} value heads), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-workload", default="layer_prefill_4k",
                    help="prefill workload name from gdn_synth.WORKLOADS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra prefill calls, each after overwriting a 1 GiB scratch buffer "
                         "(evicts the 256 MiB Infinity Cache), reported as ms_cold")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (library copy and bf16 GEMM)")
    ap.add_argument("--no-prepared", action="store_true",
                    help="skip the prefill / decode from raw inputs (in-kernel preparation)")
    ap.add_argument("--no-prefix", action="store_true",
                    help="skip the prefill with block-aligned prefix states")
    ap.add_argument("--no-segmented", action="store_true",
                    help="skip the few-long-sequence prefill (segmented vs one pass)")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the K-token slot-pool decode measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times (the "
                         "reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the token mixer is sharded by sequence or by "
              "q/k head group with no exchange, so throughput at N GPUs is N x this figure; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_token_amd as gdn
    from gdn_synth import WORKLOADS, generate, to_torch

    gdn.load_library()
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wp = WORKLOADS[args.prefill_workload]
    wd = WORKLOADS["decode_b256"]
    dp = generate(wp)
    dd = generate(wd)

    pt = {n: to_torch(dp[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
    p_s0 = to_torch(dp["S0"], dev) if dp["S0"] is not None else None
    p_out = torch.empty(pt["v"].shape, dtype=pt["q"].dtype, device=dev)
    p_sf = torch.empty((wp.B, wp.Hv, wp.D, wp.D), dtype=torch.float32, device=dev)
    varlen = wp.kind == "varlen"
    p_cu = to_torch(dp["cu_seqlens"], dev) if varlen else None
    # the workspace the library asks for (none: single-pass kernel), allocated once
    ntok = int(pt["v"].shape[0]) if varlen else wp.T
    ws_bytes = gdn.gdn_prefill_workspace_size(wp.B, ntok, wp.Hk, wp.Hv, wp.D, wp.D,
                                              pt["q"].dtype, varlen)
    p_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    dt = {n: to_torch(dd[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
    d_state = to_torch(dd["S0"], dev)
    d_out = torch.empty((wd.B, wd.Hv, wd.D), dtype=dt["q"].dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step_prefill():
        if varlen:
            gdn.gdn_varlen_prefill(pt["q"], pt["k"], pt["v"], pt["alpha"], pt["beta"], p_cu,
                                   p_s0, out=p_out, final_state=p_sf, workspace=p_ws,
                                   stream=stream)
        else:
            gdn.gdn_prefill_chunked(pt["q"], pt["k"], pt["v"], pt["alpha"], pt["beta"], p_s0,
                                    out=p_out, final_state=p_sf, workspace=p_ws, stream=stream)

    def step_decode():
        gdn.gdn_decode_step(dt["q"], dt["k"], dt["v"], dt["alpha"], dt["beta"], d_state,
                            out=d_out, stream=stream)

    for _ in range(args.warmup):
        step_prefill()
        step_decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step_prefill()
        ev[i][1].record(stream)
        step_decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    pre_avg = float(np.mean(pre_ms))
    dec_avg = float(np.mean(dec_ms))

    # cold prefill: the inputs are evicted from the Infinity Cache first
    cold_ms = []
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            scratch.fill_(i & 0xFF)
            evc[i][0].record(stream)
            step_prefill()
            evc[i][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = [e0.elapsed_time(e1) for e0, e1 in evc]
        del scratch

    # the same prefill emitting block-aligned prefix states (one per 1024
    # tokens): what a prefix cache keeps
    prefix = None
    if not varlen and wp.T >= 1024 and not args.no_prefix:
        every = 16
        rows = gdn.prefix_state_rows(wp.B, wp.T, every, False)
        p_pre = torch.empty((rows, wp.Hv, wp.D, wp.D), dtype=torch.float32, device=dev)

        def step_prefill_prefix():
            gdn.gdn_prefill_chunked(pt["q"], pt["k"], pt["v"], pt["alpha"], pt["beta"], p_s0,
                                    out=p_out, final_state=p_sf, prefix_states=p_pre,
                                    prefix_interval=every, workspace=p_ws, stream=stream)
        step_prefill_prefix()
        torch.cuda.synchronize()
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            evp[i][0].record(stream)
            step_prefill_prefix()
            evp[i][1].record(stream)
        torch.cuda.synchronize()
        pp_ms = [e0.elapsed_time(e1) for e0, e1 in evp]
        prefix = {"block_tokens": 64 * every, "states": rows * wp.Hv,
                  "bytes_written": rows * wp.Hv * wp.D * wp.D * 4,
                  "ms": round(float(np.mean(pp_ms)), 5),
                  "ms_median": round(float(np.median(pp_ms)), 5),
                  "overhead_vs_plain": round(float(np.median(pp_ms)) / float(np.median(pre_ms)) - 1,
                                             4)}
        del p_pre

    # the same prefill and decode step from raw inputs (q, k before their L2
    # normalisation, gate logits), prepared inside the kernels; beside them
    # the time of a separate preparation pass (torch ops) over the same inputs
    prepared = None
    if not varlen and not args.no_prepared:
        flags = gdn.GDN_QK_L2NORM | gdn.GDN_GATE_LOGITS
        rp = generate(wp, raw=True)
        rt = {n: to_torch(rp[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
        rd = generate(wd, raw=True)
        rdt = {n: to_torch(rd[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
        r_state = to_torch(rd["S0"], dev)

        def timed_ms(fn, reps):
            fn()
            torch.cuda.synchronize()
            out_ms = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                out_ms.append(e0.elapsed_time(e1))
            return float(np.median(out_ms))

        def torch_prepare(t):
            qf, kf = t["q"].float(), t["k"].float()
            qn = (qf * torch.rsqrt((qf * qf).sum(-1, keepdim=True) + 1e-6)).to(t["q"].dtype)
            kn = (kf * torch.rsqrt((kf * kf).sum(-1, keepdim=True) + 1e-6)).to(t["k"].dtype)
            a = torch.exp(-torch.nn.functional.softplus(t["alpha"]))
            b = torch.sigmoid(t["beta"])
            return qn, kn, a, b
        pre_raw = timed_ms(lambda: gdn.gdn_prefill_chunked(
            rt["q"], rt["k"], rt["v"], rt["alpha"], rt["beta"], None, out=p_out, final_state=p_sf,
            flags=flags, workspace=p_ws, stream=stream), K)
        pre_plain = timed_ms(step_prefill, K)
        pre_torch = timed_ms(lambda: torch_prepare(rt), K)
        dec_raw = timed_ms(lambda: gdn.gdn_decode_step(
            rdt["q"], rdt["k"], rdt["v"], rdt["alpha"], rdt["beta"], r_state, out=d_out,
            flags=flags, stream=stream), K)
        dec_plain = timed_ms(step_decode, K)
        dec_torch = timed_ms(lambda: torch_prepare(rdt), K)
        prepared = {"flags": "GDN_QK_L2NORM | GDN_GATE_LOGITS",
                    "prefill_ms": round(pre_raw, 5), "prefill_plain_ms": round(pre_plain, 5),
                    "prefill_separate_torch_pass_ms": round(pre_torch, 5),
                    "decode_ms": round(dec_raw, 5), "decode_plain_ms": round(dec_plain, 5),
                    "decode_separate_torch_pass_ms": round(dec_torch, 5),
                    "note": "medians of back-to-back calls; the torch pass is what a caller "
                            "without the flags would run first"}
        del rt, rdt, rp, rd, r_state

    # few long sequences: the per-GPU share of the layer at 8-way head-group
    # sharding (6 value heads), whole sequence in one pass vs split into
    # segments that run in parallel
    segmented = None
    if not args.no_segmented:
        segmented = {}
        for wname, reps in (("layer_prefill_4k_tp8", max(K, 5)), ("long_prefill_256k_tp8", 3)):
            ws_ = WORKLOADS[wname]
            dg = generate(ws_)
            gt = {n: to_torch(dg[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
            g_out = torch.empty(gt["v"].shape, dtype=gt["q"].dtype, device=dev)
            g_sf = torch.empty((ws_.B, ws_.Hv, ws_.D, ws_.D), dtype=torch.float32, device=dev)
            row = {}
            for label, env in (("unsegmented", "0"), ("segmented", None)):
                if env is None:
                    os.environ.pop("GDN_PREFILL_SEGMENTS", None)
                else:
                    os.environ["GDN_PREFILL_SEGMENTS"] = env
                nws = gdn.gdn_prefill_workspace_size(ws_.B, ws_.T, ws_.Hk, ws_.Hv, ws_.D, ws_.D,
                                                     gt["q"].dtype, False)
                g_ws = torch.empty(nws, dtype=torch.uint8, device=dev)
                ms = []
                for i in range(reps + 1):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    gdn.gdn_prefill_chunked(gt["q"], gt["k"], gt["v"], gt["alpha"], gt["beta"],
                                            None, out=g_out, final_state=g_sf, workspace=g_ws,
                                            stream=stream)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    if i:
                        ms.append(e0.elapsed_time(e1))
                med = float(np.median(ms))
                tf = ws_.B * ws_.T * prefill_flops_per_token(ws_.Hk, ws_.Hv, ws_.D, ws_.D) / (
                    med * 1e-3) / 1e12
                row[label] = {"ms": round(med, 5), "workspace_bytes": nws,
                              "tokens_per_s": round(ws_.B * ws_.T / (med * 1e-3), 1),
                              "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
                del g_ws
            os.environ.pop("GDN_PREFILL_SEGMENTS", None)
            row["speedup"] = round(row["unsegmented"]["ms"] / row["segmented"]["ms"], 3)
            segmented[wname] = row
            del gt, dg, g_out, g_sf

    # K tokens per sequence against a slot pool (speculative verification):
    # timed on its own, after the step, on the same stream
    multi = None
    if not args.no_multi:
        from gdn_synth import SPEC_DECODE, multi_decode
        wm = SPEC_DECODE
        dm = multi_decode(wm["B"], wm["K"], wm["Hk"], wm["Hv"], wm["D"], wm["dtype"],
                          wm["seed"], plan=wm["plan"])
        mt = {n: to_torch(dm[n], dev) for n in ("q", "k", "v", "alpha", "beta", "pool",
                                                 "src_slot", "dst_slot")}
        m_out = torch.empty(mt["v"].shape, dtype=mt["q"].dtype, device=dev)

        def step_multi():
            gdn.gdn_decode_multi(mt["q"], mt["k"], mt["v"], mt["alpha"], mt["beta"], mt["pool"],
                                 mt["src_slot"], mt["dst_slot"], out=m_out, stream=stream)
        for _ in range(max(args.warmup, 1)):
            step_multi()
        torch.cuda.synchronize()
        evm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for i in range(K):
            evm[i][0].record(stream)
            step_multi()
            evm[i][1].record(stream)
        torch.cuda.synchronize()
        m_ms = [e0.elapsed_time(e1) for e0, e1 in evm]
        m_avg = float(np.mean(m_ms))
        m_bytes = decode_multi_bytes(wm["B"], wm["K"], wm["Hk"], wm["Hv"], wm["D"], wm["D"])
        m_gbs = m_bytes / (m_avg * 1e-3) / 1e9
        multi = {"workload": wm["name"], "B": wm["B"], "K": wm["K"], "Hk": wm["Hk"],
                 "Hv": wm["Hv"], "d": wm["D"],
                 "slots": f"pool of {dm['pool'].shape[0]} fp32 states; sequence b reads slot "
                          f"2b and writes slot 2b+1",
                 "ms": round(m_avg, 5), "ms_median": round(float(np.median(m_ms)), 5),
                 "ms_min": round(float(np.min(m_ms)), 5),
                 "tokens_per_s": round(wm["B"] * wm["K"] / (m_avg * 1e-3), 1),
                 "roofline": {"kernel": "decode_multi_kernel", "bound": "hbm",
                              "achieved": round(m_gbs, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(m_gbs / PEAK_HBM_GBS, 4),
                              "traffic": _traffic("decode_multi_" + wm["name"],
                                                  _src_digest("gdn_decode.hip",
                                                              "gdn_device.hpp"))}}
        del mt, dm

    # measured ceilings beside the spec peaks: a device-to-device copy and a
    # large bf16 GEMM, both through the runtime's own libraries
    ceilings = None
    if not args.no_ceilings:
        def timed(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e-3
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        t_copy = timed(lambda: dst.copy_(src))
        del src, dst
        n = 8192
        a = torch.randn(n, n, device=dev).to(torch.bfloat16)
        b = torch.randn(n, n, device=dev).to(torch.bfloat16)
        t_gemm = timed(lambda: torch.matmul(a, b))
        del a, b
        ceilings = {"copy_GBps": round(2 * (1 << 30) / t_copy / 1e9, 1),
                    "copy": "1 GiB device-to-device copy, bytes read + written",
                    "bf16_gemm_tflops": round(2 * n ** 3 / t_gemm / 1e12, 1),
                    "gemm": "torch.matmul bf16 8192 x 8192 x 8192"}

    tokens = int(pt["v"].shape[0] * (1 if varlen else pt["v"].shape[1]))
    f_tok = prefill_flops_per_token(wp.Hk, wp.Hv, wp.D, wp.D)
    pre_tflops = tokens * f_tok / (pre_avg * 1e-3) / 1e12
    pre_tok_s = tokens / (pre_avg * 1e-3)
    pre_gbs = tokens * prefill_bytes_per_token(wp.Hk, wp.Hv, wp.D, wp.D) / (pre_avg * 1e-3) / 1e9
    dec_bytes = decode_bytes_per_step(wd.B, wd.Hk, wd.Hv, wd.D, wd.D)
    dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9

    pdig = _src_digest("gdn_prefill.hip", "gdn_chunk.hpp", "gdn_device.hpp")
    prefill_kernels = (["prep_kernel", "chain_db_kernel" if wp.D == 128 or wp.D == 64 else
                        "chain_kernel"] if ws_bytes else ["prefill_kernel"])
    ddig = _src_digest("gdn_decode.hip", "gdn_device.hpp")
    res = {
        "metric": METRIC,
        "value": round(pre_tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wp.name} prefill + {wd.name} decode step",
            "prefill": {"B": wp.B, "T": wp.T if not varlen else None, "tokens": tokens,
                        "Hk": wp.Hk, "Hv": wp.Hv, "d": wp.D,
                        "path": "two-pass (workspace %d bytes)" % ws_bytes if ws_bytes
                        else "single-pass",
                        "chunk": CHUNK, "io": "bf16 q/k/v/o, fp32 alpha/beta/state"},
            "decode": {"B": wd.B, "Hk": wd.Hk, "Hv": wd.Hv, "d": wd.D,
                       "state": "fp32, updated in place"},
        },
        "prefill": {"tokens_per_s": round(pre_tok_s, 1), "ms": round(pre_avg, 5),
                    "ms_median": round(float(np.median(pre_ms)), 5),
                    "ms_min": round(float(np.min(pre_ms)), 5),
                    "ms_cold": round(float(np.median(cold_ms)), 5) if cold_ms else None,
                    "algorithmic_tflops": round(pre_tflops, 2),
                    "frac_mfma_peak": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                    "required_io_GBps": round(pre_gbs, 1)},
        "decode": {"GB_per_s": round(dec_gbs, 1), "ms": round(dec_avg, 5),
                   "ms_median": round(float(np.median(dec_ms)), 5),
                   "ms_min": round(float(np.min(dec_ms)), 5),
                   "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "tokens_per_s": round(wd.B / (dec_avg * 1e-3), 1)},
        # the step's dominant kernel by time is the decode step
        "roofline": {"kernel": "decode_kernel", "bound": "hbm",
                     "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": _traffic("decode_" + wd.name, ddig)},
        "roofline_prefill": {"kernels": prefill_kernels, "bound": "mfma",
                             "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                             "traffic": _traffic("prefill_" + wp.name, pdig)},
    }
    if prefix is not None:
        res["prefill_prefix_states"] = prefix
    if prepared is not None:
        res["prepared_inputs"] = prepared
    if segmented is not None:
        res["segmented_prefill"] = segmented
    if multi is not None:
        res["decode_multi"] = multi
    if ceilings is not None:
        ceilings["decode_frac_of_copy"] = round(dec_gbs / ceilings["copy_GBps"], 4)
        ceilings["prefill_frac_of_gemm"] = round(pre_tflops / ceilings["bf16_gemm_tflops"], 4)
        res["measured_ceilings"] = ceilings
    if not args.no_cpu_baseline and not varlen:
        res["cpu_baseline"] = cpu_baseline(dp, wp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
