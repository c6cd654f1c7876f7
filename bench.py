#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already
resident in HBM:
  * prefill of the long-context workload (B=1, T=262,144, 16 q/k heads, 48
    value heads, d=128, bf16 q/k/v, fp32 alpha/beta/state, zero initial
    state), and
  * one decode step of the batched workload (B=256, same heads, fp32 states
    updated in place).
Shapes follow "The Hybrid Attention in Qwen3.8-27B" (section "Grouped-query
attention multiplies on top of that"; the 262,144-token native context from
its section "Why 27B parameters can carry 262K tokens").

Reported: the long prefill's tokens/s (value) with its fraction of the bf16
MFMA peak, the decode step's state-update GB/s with its fraction of HBM
bandwidth, both from HIP events on the stream the kernels run on; beside
them, each with its own roofline object, the layer prefill (T=4096) and the
packed 64-sequence prefill (1,141,939 tokens, nonzero initial states); and
the fp64 oracle timed on the host cores as a CPU baseline. Timed apart from
the step: under "prefill_prefix_states" the layer prefill also writing the
state after every 1024 tokens; under "prepared_inputs" the layer prefill and
the decode step from raw q, k and gate logits (prepared inside the kernels);
under "segmented_prefill" the per-GPU share of the layer at 8-way head-group
sharding (6 value heads, T = 4096 and 262,144) in one pass and split into
segments; and under "decode_multi" the K-token decode against a slot pool
(B=256 sequences verifying K=4 tokens each), in tokens/s and HBM GB/s.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2]
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
    """Time the fp64 oracle on the layer prefill workload on the host cores:
    whole passes over all 48 value heads until about budget_s seconds are
    spent (at least one pass)."""
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
    return {"value": tokens / el, "unit": "tokens/s", "cores": threads,
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{passes} full pass(es) of the fp64 token-by-token oracle over "
                      f"{w.name} (B={w.B}, T={w.T}, {w.Hv} value heads), {el:.1f} s, on "
                      f"{threads} threads of the {os.cpu_count()} host CPUs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--prefill-workload", default="long_prefill_256k",
                    help="workload of the step's prefill (gdn_synth.WORKLOADS)")
    ap.add_argument("--legs", default="layer_prefill_4k,varlen_64seq",
                    help="comma-separated prefill workloads timed beside the step, each with "
                         "its own roofline object ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="extra layer-prefill calls, each after overwriting a 1 GiB scratch "
                         "buffer (evicts the 256 MiB Infinity Cache), reported as ms_cold")
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
    ap.add_argument("--no-decode", action="store_true",
                    help="leave the decode step out of the step (prefill-only profiles)")
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
    stream = torch.cuda.current_stream(dev)
    # a recorded byte count holds while the sources of the kernels it covers
    # (and the headers they include) are unchanged
    heads = ("gdn_chunk.hpp", "gdn_device.hpp", "gdn_seq.hpp", "gdn_launch.hpp")
    pdig = {"two-pass": _src_digest("gdn_prefill.hip", "gdn_chain4.hip", *heads),
            "single-pass": _src_digest("gdn_fused2.hip", *heads)}
    ddig = _src_digest("gdn_decode.hip", "gdn_device.hpp")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    class Prefill:
        """One prefill workload resident on the device, with its call."""

        def __init__(self, name):
            self.w = w = WORKLOADS[name]
            self.d = generate(w)
            self.t = {n: to_torch(self.d[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
            self.s0 = to_torch(self.d["S0"], dev) if self.d["S0"] is not None else None
            self.varlen = w.kind == "varlen"
            self.out = torch.empty(self.t["v"].shape, dtype=self.t["q"].dtype, device=dev)
            self.sf = torch.empty((w.B, w.Hv, w.D, w.D), dtype=torch.float32, device=dev)
            self.cu = to_torch(self.d["cu_seqlens"], dev) if self.varlen else None
            self.tokens = int(self.t["v"].shape[0] if self.varlen else w.B * w.T)
            ntok = self.tokens if self.varlen else w.T
            # the workspace the library asks for (none: single-pass kernel), allocated once
            self.ws_bytes = gdn.gdn_prefill_workspace_size(w.B, ntok, w.Hk, w.Hv, w.D, w.D,
                                                           self.t["q"].dtype, self.varlen)
            self.ws = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
                       if self.ws_bytes else None)

        def __call__(self):
            t = self.t
            if self.varlen:
                gdn.gdn_varlen_prefill(t["q"], t["k"], t["v"], t["alpha"], t["beta"], self.cu,
                                       self.s0, out=self.out, final_state=self.sf,
                                       workspace=self.ws, stream=stream)
            else:
                gdn.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], self.s0,
                                        out=self.out, final_state=self.sf, workspace=self.ws,
                                        stream=stream)

        def kernels(self):
            # the library's choice for these shapes (bf16, d = 128): with few
            # (sequence, value head) chains the two-pass path (per-chunk
            # factors, then the chain at four value-column slices per head);
            # with at least one chain per CU the single-pass kernel, one
            # workgroup per chain
            w = self.w
            if self.ws_bytes:
                return ["prep_kernel", "chain4_kernel" if w.D == 128 else "chain_db_kernel"]
            return ["fused2_kernel" if w.D == 128 else "prefill_kernel"]

        def summary(self, ms_list, extra=None):
            w = self.w
            avg = float(np.mean(ms_list))
            f_tok = prefill_flops_per_token(w.Hk, w.Hv, w.D, w.D)
            tflops = self.tokens * f_tok / (avg * 1e-3) / 1e12
            gbs = self.tokens * prefill_bytes_per_token(w.Hk, w.Hv, w.D, w.D) / (avg * 1e-3) / 1e9
            r = {"workload": w.name, "tokens": self.tokens,
                 "tokens_per_s": round(self.tokens / (avg * 1e-3), 1),
                 "ms": round(avg, 5), "ms_median": round(float(np.median(ms_list)), 5),
                 "ms_min": round(float(np.min(ms_list)), 5), "calls": len(ms_list),
                 "path": ("two-pass (workspace %d bytes)" % self.ws_bytes if self.ws_bytes
                          else "single-pass"),
                 "algorithmic_tflops": round(tflops, 2),
                 "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                 "required_io_GBps": round(gbs, 1),
                 "roofline": {"kernels": self.kernels(), "bound": "mfma",
                              "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                              "traffic": _traffic("prefill_" + w.name,
                                                  pdig["two-pass" if self.ws_bytes
                                                       else "single-pass"])}}
            if extra:
                r.update(extra)
            return r

        def free(self):
            del self.t, self.out, self.sf, self.ws, self.s0, self.cu, self.d

    def timed_calls(fn, reps, warm=1):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    # ------------------------------------------------------------ the step
    K = args.steps
    main_pf = Prefill(args.prefill_workload)
    wd = WORKLOADS["decode_b256"]
    dd = generate(wd)
    dt = {n: to_torch(dd[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
    d_state = to_torch(dd["S0"], dev)
    d_out = torch.empty((wd.B, wd.Hv, wd.D), dtype=dt["q"].dtype, device=dev)

    def step_decode():
        gdn.gdn_decode_step(dt["q"], dt["k"], dt["v"], dt["alpha"], dt["beta"], d_state,
                            out=d_out, stream=stream)

    for _ in range(args.warmup):
        main_pf()
        if not args.no_decode:
            step_decode()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        main_pf()
        ev[i][1].record(stream)
        if not args.no_decode:
            step_decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    main_sum = main_pf.summary(pre_ms)
    main_w = main_pf.w
    main_pf.free()
    del main_pf

    decode = None
    if not args.no_decode:
        dec_avg = float(np.mean(dec_ms))
        dec_bytes = decode_bytes_per_step(wd.B, wd.Hk, wd.Hv, wd.D, wd.D)
        dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
        decode = {"workload": wd.name, "GB_per_s": round(dec_gbs, 1), "ms": round(dec_avg, 5),
                  "ms_median": round(float(np.median(dec_ms)), 5),
                  "ms_min": round(float(np.min(dec_ms)), 5),
                  "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                  "tokens_per_s": round(wd.B / (dec_avg * 1e-3), 1),
                  "roofline": {"kernel": "decode_kernel", "bound": "hbm",
                               "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                               "traffic": _traffic("decode_" + wd.name, ddig)}}

    # ------------------------------------------------ the other prefill legs
    legs = {}
    c1 = None  # the layer prefill stays resident for the extra legs below
    for name in [x for x in args.legs.split(",") if x]:
        pf = Prefill(name)
        reps = max(3, K // 2) if pf.tokens > 100000 else max(K, 10)
        ms = timed_calls(pf, reps)
        extra = None
        if name == "layer_prefill_4k" and args.cold_steps > 0:
            scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.cold_steps)]
            for i in range(args.cold_steps):
                scratch.fill_(i & 0xFF)
                evc[i][0].record(stream)
                pf()
                evc[i][1].record(stream)
            torch.cuda.synchronize()
            extra = {"ms_cold": round(float(np.median([a.elapsed_time(b) for a, b in evc])), 5)}
            del scratch
        legs[name] = pf.summary(ms, extra)
        if name == "layer_prefill_4k":
            c1 = pf
        else:
            pf.free()
            del pf
        torch.cuda.empty_cache()
    if c1 is None and not (args.no_prefix and args.no_prepared and args.no_cpu_baseline):
        c1 = Prefill("layer_prefill_4k")
    wp = WORKLOADS["layer_prefill_4k"]

    # the layer prefill emitting block-aligned prefix states (one per 1024
    # tokens): what a prefix cache keeps
    prefix = None
    if not args.no_prefix:
        every = 16
        rows = gdn.prefix_state_rows(wp.B, wp.T, every, False)
        p_pre = torch.empty((rows, wp.Hv, wp.D, wp.D), dtype=torch.float32, device=dev)
        t = c1.t

        def step_prefill_prefix():
            gdn.gdn_prefill_chunked(t["q"], t["k"], t["v"], t["alpha"], t["beta"], None,
                                    out=c1.out, final_state=c1.sf, prefix_states=p_pre,
                                    prefix_interval=every, workspace=c1.ws, stream=stream)
        pp_ms = timed_calls(step_prefill_prefix, max(K, 10))
        plain_ms = timed_calls(c1, max(K, 10))
        prefix = {"workload": wp.name, "block_tokens": 64 * every, "states": rows * wp.Hv,
                  "bytes_written": rows * wp.Hv * wp.D * wp.D * 4,
                  "ms": round(float(np.mean(pp_ms)), 5),
                  "ms_median": round(float(np.median(pp_ms)), 5),
                  "plain_ms_median": round(float(np.median(plain_ms)), 5),
                  "overhead_vs_plain": round(float(np.median(pp_ms)) /
                                             float(np.median(plain_ms)) - 1, 4)}
        del p_pre

    # the layer prefill and the decode step from raw inputs (q, k before
    # their L2 normalisation, gate logits), prepared inside the kernels;
    # beside them the time of a separate preparation pass (torch ops)
    prepared = None
    if not args.no_prepared:
        flags = gdn.GDN_QK_L2NORM | gdn.GDN_GATE_LOGITS
        rp = generate(wp, raw=True)
        rt = {n: to_torch(rp[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
        rd = generate(wd, raw=True)
        rdt = {n: to_torch(rd[n], dev) for n in ("q", "k", "v", "alpha", "beta")}
        r_state = to_torch(rd["S0"], dev)

        def med(fn):
            return float(np.median(timed_calls(fn, max(K, 10))))

        def torch_prepare(t):
            qf, kf = t["q"].float(), t["k"].float()
            qn = (qf * torch.rsqrt((qf * qf).sum(-1, keepdim=True) + 1e-6)).to(t["q"].dtype)
            kn = (kf * torch.rsqrt((kf * kf).sum(-1, keepdim=True) + 1e-6)).to(t["k"].dtype)
            a = torch.exp(-torch.nn.functional.softplus(t["alpha"]))
            b = torch.sigmoid(t["beta"])
            return qn, kn, a, b
        pre_raw = med(lambda: gdn.gdn_prefill_chunked(
            rt["q"], rt["k"], rt["v"], rt["alpha"], rt["beta"], None, out=c1.out,
            final_state=c1.sf, flags=flags, workspace=c1.ws, stream=stream))
        pre_plain = med(c1)
        pre_torch = med(lambda: torch_prepare(rt))
        dec_raw = med(lambda: gdn.gdn_decode_step(
            rdt["q"], rdt["k"], rdt["v"], rdt["alpha"], rdt["beta"], r_state, out=d_out,
            flags=flags, stream=stream))
        dec_plain = med(step_decode)
        dec_torch = med(lambda: torch_prepare(rdt))
        prepared = {"flags": "GDN_QK_L2NORM | GDN_GATE_LOGITS", "prefill_workload": wp.name,
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
                ms = timed_calls(lambda: gdn.gdn_prefill_chunked(
                    gt["q"], gt["k"], gt["v"], gt["alpha"], gt["beta"], None, out=g_out,
                    final_state=g_sf, workspace=g_ws, stream=stream), reps)
                med_ms = float(np.median(ms))
                tf = ws_.B * ws_.T * prefill_flops_per_token(ws_.Hk, ws_.Hv, ws_.D, ws_.D) / (
                    med_ms * 1e-3) / 1e12
                row[label] = {"ms": round(med_ms, 5), "workspace_bytes": nws,
                              "tokens_per_s": round(ws_.B * ws_.T / (med_ms * 1e-3), 1),
                              "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
                del g_ws
            os.environ.pop("GDN_PREFILL_SEGMENTS", None)
            row["speedup"] = round(row["unsegmented"]["ms"] / row["segmented"]["ms"], 3)
            segmented[wname] = row
            del gt, dg, g_out, g_sf

    # K tokens per sequence against a slot pool (speculative verification)
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
        m_ms = timed_calls(step_multi, K, warm=max(args.warmup, 1))
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
                              "traffic": _traffic("decode_multi_" + wm["name"], ddig)}}
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

    res = {
        "metric": METRIC,
        "value": main_sum["tokens_per_s"],
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
            "workload": f"{main_w.name} prefill" + ("" if args.no_decode else
                                                    f" + {wd.name} decode step"),
            "prefill": {"B": main_w.B, "T": main_w.T if main_w.kind == "prefill" else None,
                        "tokens": main_sum["tokens"], "Hk": main_w.Hk, "Hv": main_w.Hv,
                        "d": main_w.D, "path": main_sum["path"], "chunk": CHUNK,
                        "io": "bf16 q/k/v/o, fp32 alpha/beta/state"},
            "decode": None if args.no_decode else
            {"B": wd.B, "Hk": wd.Hk, "Hv": wd.Hv, "d": wd.D, "state": "fp32, updated in place"},
        },
        "prefill": main_sum,
        # the step's headline: the long prefill (its kernels together)
        "roofline": main_sum["roofline"],
    }
    if decode is not None:
        res["decode"] = decode
        res["roofline_decode"] = decode["roofline"]
    if legs:
        res["prefill_legs"] = legs
    if prefix is not None:
        res["prefill_prefix_states"] = prefix
    if prepared is not None:
        res["prepared_inputs"] = prepared
    if segmented is not None:
        res["segmented_prefill"] = segmented
    if multi is not None:
        res["decode_multi"] = multi
    if ceilings is not None:
        if decode is not None:
            ceilings["decode_frac_of_copy"] = round(decode["GB_per_s"] / ceilings["copy_GBps"], 4)
        ceilings["prefill_frac_of_gemm"] = round(main_sum["algorithmic_tflops"] /
                                                 ceilings["bf16_gemm_tflops"], 4)
        res["measured_ceilings"] = ceilings
    if not args.no_cpu_baseline:
        if c1 is None:
            c1 = Prefill("layer_prefill_4k")
        res["cpu_baseline"] = cpu_baseline(c1.d, c1.w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
