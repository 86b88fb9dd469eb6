"""Throughput of the segment-causal attention path on one MI355X.

One step = one turn of the whole hot path at the full-lifelong-cache shape
(a 12 s segment: 72 latent frames x 880 = 63,360 new tokens, 16 heads x 128,
over 288 cached latent frames = 253,440 INT8 tokens):
    nomas_seg_attn   (63,360 queries x 316,800 keys, RoPE fused, INT8 cache)
    nomas_cam_xattn  (63,360 video queries x 72 camera tokens)
    nomas_rope3d     (the segment's keys, before caching)
    nomas_kv_quant_append (the segment's K/V into the cache at 253,440)
The append writes the same cache slots every step, so every step sees the
same 253,440-token history.  Inputs are seeded synthetic tensors resident in
HBM before timing starts.

value = algorithmic attention FLOPs per step / wall time per step (TFLOP/s),
with algorithmic FLOPs = 4 * 128 * H * (allowed query-key pairs).
The roofline block times nomas_seg_attn alone (its launches: the pack
pre-pass, the attention kernel and, since this shape splits each query
tile's key range in two, the merge) with HIP events on its stream.
The CPU baseline times the oracle on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
       python bench.py --copy-calibration   (plain copy kernel for counter scaling)
       python bench.py --workloads          (the other workloads, one JSON line each; see workloads())
       python bench.py --workloads --only train   (a subset of them, by group)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense BF16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "seg_attn_fullcache_traffic.json")
KERNEL_SOURCES = ["segment_causal_attention_amd/csrc/seg_attn.hip", "segment_causal_attention_amd/csrc/common.hpp"]


def kernel_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for_current_kernel():
    """HBM bytes per nomas_seg_attn call (pack, attention and merge kernels) from the
    committed counter summary, or None when the kernel source changed since
    the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_digest") != kernel_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class ClockSampler:
    """Shader-clock samples of GPU 0 while the timed steps run: the SMU's
    per-XCD current graphics clock (amdsmi gpu metrics), read every ~10 ms on
    a host thread.  The peak of 2516.6 TFLOP/s assumes 2.4 GHz; a kernel held
    below that clock by the power limit cannot reach it, so the bench line
    also states the fraction of the peak at the measured clock.  Everything
    degrades to None when the metrics cannot be read."""

    def __init__(self, period_s=0.01):
        import threading
        self.period = period_s
        self.samples = []
        self.avg_samples = []
        self._stop = threading.Event()
        self._thread = None
        self._h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            self._smi = amdsmi
            self._h = hs[0] if hs else None
        except Exception as e:          # no GPU metrics here: report no clock
            log("clock sampler unavailable: %s" % e)

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        xs = m.get("current_gfxclks")
        vals = [float(x) for x in xs if isinstance(x, (int, float)) and 0 < x < 10000] if isinstance(xs, list) else []
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [float(m["current_gfxclk"])]
        avg = m.get("average_gfxclk_frequency")
        return (sum(vals) / len(vals) if vals else None), (float(avg) if isinstance(avg, (int, float)) else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                cur, avg = self._read()
                if cur:
                    self.samples.append(cur)
                if avg:
                    self.avg_samples.append(avg)
            except Exception:
                pass
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._h is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        try:
            if self._h is not None:
                self._smi.amdsmi_shut_down()
        except Exception:
            pass
        if not self.samples:
            return None
        xs = sorted(self.samples)
        av = sorted(self.avg_samples)
        pick = lambda f: xs[min(len(xs) - 1, int(f * len(xs)))]
        # the median: single readings dip far below the clock the kernel runs
        # at (down to ~160 MHz), which drags a mean down by up to 25%
        return {"median_mhz": pick(0.5), "p10_mhz": pick(0.1), "p90_mhz": pick(0.9), "samples": len(xs),
                "smu_average_mhz": round(sum(av) / len(av), 1) if av else None,
                "source": "amdsmi gpu metrics current_gfxclks (mean over XCDs), sampled every 10 ms during the "
                          "timed steps"}


def clock_fraction(clk, achieved_tflops):
    """Adds the dense BF16 MFMA peak at the sampled clock (256 CUs x 4096 FLOP
    per clock) and the kernel's fraction of it.  A median clock at which the
    kernel would exceed that peak cannot be the clock it ran at (under a
    profiler the SMU readings have stayed at an idle ~95 MHz): then both stay
    None and a note says why."""
    peak = round(256 * 4096 * clk["median_mhz"] * 1e6 / 1e12, 1)
    if peak <= 0 or achieved_tflops > peak:
        clk["peak_at_clock_tflops"] = None
        clk["frac_at_clock"] = None
        clk["note"] = ("median reading %.0f MHz is below the clock needed for the measured %.1f TFLOP/s: "
                       "not the clock the kernel ran at" % (clk["median_mhz"], achieved_tflops))
    else:
        clk["peak_at_clock_tflops"] = peak
        clk["frac_at_clock"] = round(achieved_tflops / peak, 4)
    return clk


def copy_calibration():
    """A plain device copy of a known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--workloads", action="store_true")
    ap.add_argument("--only", default="", help="with --workloads: comma-separated groups (tiny, turn3s, seg4s, "
                    "fiveturns, decoder, w8a16, fullcache, train)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workloads:
        workloads([w for w in args.only.split(",") if w], cpu=not args.no_cpu_baseline)
        return

    import numpy as np
    import torch

    import segment_causal_attention_amd as nomas
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS["fullcache"]
    H, Lq, Lc = cfg.H, cfg.Lq, cfg.Lc
    (seg,) = cfg.new_segs
    (hseg,) = cfg.hist_segs
    cap = Lc + Lq
    sm = float(np.float32(1.0 / math.sqrt(128)))
    Nc = 72

    t0 = time.time()
    inp = synth.layer_inputs("fullcache")
    cam_in = synth.turn_inputs(0, with_cam=True)
    log("inputs generated in %.1f s" % (time.time() - t0))

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    q, k_new, v_new = d16(inp["q"]), d16(inp["k_new"]), d16(inp["v_new"])
    q_cam = d16(cam_in["q_cam"])
    w_k, w_v = d16(cam_in["w_k"]), d16(cam_in["w_v"])
    cam = torch.from_numpy(nomas.cam_tokens(cam_in["c2w"])).to(dev)
    kc = torch.empty((H, cap, 128), dtype=torch.int8, device=dev)
    vc = torch.empty((H, cap, 128), dtype=torch.int8, device=dev)
    ks = torch.empty((H, cap), dtype=torch.float32, device=dev)
    vs = torch.empty((H, cap), dtype=torch.float32, device=dev)
    # build the 288-frame history the way the path does: rotate, then quantise
    kh = d16(inp["k_hist"])
    vh = d16(inp["v_hist"])
    nomas.rope3d(kh, [hseg], out=kh)
    n = nomas.kv_quant_append(kh, vh, kc, vc, ks, vs, 0)
    assert n == Lc
    del kh, vh
    out = torch.empty_like(q)
    out_cam = torch.empty_like(q_cam)
    k_rot = torch.empty_like(k_new)
    ws = torch.empty(nomas.seg_attn_workspace([seg], Lc, H), dtype=torch.uint8, device=dev)
    ws_cam = torch.empty(nomas.cam_xattn_workspace(H, Nc), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i=None):
        if i is not None:
            ev[i][0].record(stream)
        nomas.seg_attn(q, k_new, v_new, [seg], kc, vc, ks, vs, cache_len=Lc, sm_scale=sm, out=out, workspace=ws,
                       stream=stream)
        if i is not None:
            ev[i][1].record(stream)
        nomas.cam_xattn(q_cam, cam, w_k, w_v, sm_scale=sm, out=out_cam, workspace=ws_cam, stream=stream)
        nomas.rope3d(k_new, [seg], out=k_rot, stream=stream)
        nomas.kv_quant_append(k_rot, v_new, kc, vc, ks, vs, Lc, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    clock = ClockSampler()
    clock.start()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    clk = clock.stop()

    pairs = Lq * (Lc + Lq)
    flops = 4.0 * 128 * H * pairs
    ms_step = wall * 1e3 / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log("step %.3f ms, nomas_seg_attn %.3f ms (%.1f TFLOP/s, %.1f%% of peak)"
        % (ms_step, attn_ms, achieved, 100 * achieved / PEAK_BF16_TFLOPS))
    if clk:
        clock_fraction(clk, achieved)
        log("shader clock %.0f MHz (median of %d samples, p10 %.0f, p90 %.0f): %s"
            % (clk["median_mhz"], clk["samples"], clk["p10_mhz"], clk["p90_mhz"],
               "%.1f%% of the peak at that clock" % (100 * clk["frac_at_clock"]) if clk["frac_at_clock"] is not None
               else clk["note"]))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, cfg, sm)

    line = {
        "metric": "seg-causal attention TFLOP/s (BF16 MFMA) + % of peak, 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, INT8 cache quantised on the GPU)",
        "config": {
            "workload": "fullcache: 12 s segment (72 latent frames x 880 = 63,360 queries) over 288 cached "
                        "latent frames (253,440 INT8 keys) + own segment = 316,800 keys, 16 heads x 128; "
                        "step = seg_attn + cam_xattn (72 camera tokens) + rope3d + kv_quant_append",
            "heads": H, "head_dim": 128, "queries": Lq, "cache_tokens": Lc, "keys_per_query": Lc + Lq,
            "algorithmic_flop_per_step": flops,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "nomas_seg_attn (pack_kernel + seg_attn_kernel + merge_kernel)",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(attn_ms, 3),
            "traffic": traffic_for_current_kernel(),
            "clock": clk,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def workloads(only=None, cpu=True):
    """Throughput of the path on the other workloads, one JSON line each, all
    inputs seeded synthetic and resident in HBM before timing, HIP events on
    the launch stream:
      tiny        2 segments of 64 tokens (16 text + 2 x 4 x 6 video), 2 heads:
                  the second over the first as a 64-token INT8 cache (median of 20)
      turn3s      16,096 queries over 15,840 cached + 16,096 own keys (median of 10 calls)
      seg4s       54 distinct layers (outlier channels x20) x 8 steps = 432 calls
                  timed end to end (median of 3 sequences)
      fiveturns   per turn k = 0..4: seg_attn over a cache of 63,360 k tokens,
                  cam_xattn (72 camera tokens), rope3d and kv_quant_append, each
                  the median of 5 calls, the HBM-bound ones in GB/s of
                  algorithmic bytes
      fullcache-sel18  the full-cache shape attending to 18 of the 288 cached
                  latent frames (the last of every 16) through the history
                  selection, plus its own 63,360 tokens (median of 5 calls)
      fullcache-h2  the full-cache shape with 2 heads: one GPU's share when the
                  16 heads are split over 8 GPUs (median of 5 calls)
      decoder-window  gqa_attn over one 10-latent-frame decoder window at
                  1280x704 (35,200 tokens, 32 query / 8 KV heads; median of 5)
      w8a16-qkv, w8a16-ffn-up, w8a16-ffn-down, w8a16-out  INT8-weight linear
                  layers of one 12 s segment (63,360 x 2048 -> 6144, 2048 -> 8192,
                  8192 -> 2048, 2048 -> 2048; median of 10), with the
                  dequantisation pass alone and torch's BF16 matmul on the
                  dequantised weights as context
      train-fwd, train-bwd  segment-forcing training: 22 packed 3 s turns
                  (354,112 tokens, block-causal) with 2 heads (one GPU's share
                  of a head-sharded layer), forward and backward (median of 5)
    History caches are built on the GPU by rope3d + kv_quant_append (bit-exact
    to the oracle's quantiser).  With cpu, the attention lines also carry the
    oracle (numpy float64, as it stands) timed on the host: tiny, turn3s and
    one seg4s call (layer 0) in full, and 4,096 query rows of head 0 on turns 0
    and 4 of fiveturns; the oracle quantises its own caches, untimed."""
    import numpy as np
    import torch

    import segment_causal_attention_amd as nomas
    import synth

    dev = torch.device("cuda:0")
    sm = float(np.float32(1.0 / math.sqrt(128)))
    stream = torch.cuda.current_stream()

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def build_cache(k_hist, v_hist, hist_segs, H, cap):
        kc = torch.empty((H, cap, 128), dtype=torch.int8, device=dev)
        vc = torch.empty((H, cap, 128), dtype=torch.int8, device=dev)
        ks = torch.empty((H, cap), dtype=torch.float32, device=dev)
        vs = torch.empty((H, cap), dtype=torch.float32, device=dev)
        if k_hist is not None:
            kh = d16(k_hist)
            nomas.rope3d(kh, hist_segs, out=kh)
            nomas.kv_quant_append(kh, d16(v_hist), kc, vc, ks, vs, 0)
            del kh
        return kc, vc, ks, vs

    def timed(fn, n, warm=2):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def want(group):
        return not only or group in only

    def emit(name, **kw):
        line = dict(workload=name, **kw)
        print(json.dumps(line), flush=True)

    def attn_line(name, ms, H, Lq, keys, extra=None, cpu_b=None):
        fl = 4.0 * 128 * H * Lq * keys
        tf = fl / (ms * 1e-3) / 1e12
        more = dict(extra or {})
        if cpu_b is not None:
            more["cpu_baseline"] = dict(cpu_b, gpu_over_cpu=round(tf / cpu_b["value"], 1))
        emit(name, metric="attention TFLOP/s", value=round(tf, 3 if tf < 1 else 2), unit="TFLOP/s", ms=round(ms, 4),
             pct_of_peak=round(100 * tf / PEAK_BF16_TFLOPS, 3), heads=H, queries=Lq, keys_per_query=keys,
             algorithmic_flop=fl, **more)

    if cpu:
        import oracle

    if want("tiny"):
        # ---- tiny: segment 1 over segment 0 as a 64-token INT8 cache
        log("workload tiny")
        inp = synth.tiny_inputs()
        segs = [s.astuple() for s in inp["segs"]]
        n = 64
        cache = build_cache(inp["k"][:n], inp["v"][:n], segs[:1], 2, n)
        q, k, v = (d16(inp[x][n:2 * n]) for x in ("q", "k", "v"))
        out = torch.empty_like(q)
        ws = torch.empty(nomas.seg_attn_workspace(segs[1:2], n, 2), dtype=torch.uint8, device=dev)
        ms = timed(lambda: nomas.seg_attn(q, k, v, segs[1:2], *cache, cache_len=n, sm_scale=sm, out=out, workspace=ws,
                                          stream=stream), 20, 3)
        cpu_b = None
        if cpu:
            oc = oracle.build_cache(inp["k"][:n], inp["v"][:n], segs[:1])
            qn, kn, vn = (np.ascontiguousarray(inp[x][n:2 * n]) for x in ("q", "k", "v"))
            cpu_b = oracle_timing(lambda: oracle.seg_attn(qn, kn, vn, segs[1:2], *oc, n, sm), 4.0 * 128 * 2 * n * 2 * n,
                                  "numpy float64 oracle, the whole call (64 queries x 128 keys x 2 heads)")
        attn_line("tiny", ms, 2, n, 2 * n, dict(cache_tokens=n), cpu_b)
        del q, k, v, out, ws, cache

    if want("turn3s"):
        # ---- turn3s
        log("workload turn3s")
        cfg = synth.WORKLOADS["turn3s"]
        inp = synth.layer_inputs("turn3s")
        (seg,) = cfg.new_segs
        cache = build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs, cfg.H, cfg.Lc)
        q, k, v = d16(inp["q"]), d16(inp["k_new"]), d16(inp["v_new"])
        out = torch.empty_like(q)
        ws = torch.empty(nomas.seg_attn_workspace([seg], cfg.Lc, cfg.H), dtype=torch.uint8, device=dev)
        ms = timed(lambda: nomas.seg_attn(q, k, v, [seg], *cache, cache_len=cfg.Lc, sm_scale=sm, out=out, workspace=ws,
                                          stream=stream), 10, 3)
        cpu_b = None
        if cpu:
            oc = oracle.build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs)
            cpu_b = oracle_timing(
                lambda: oracle.seg_attn(inp["q"], inp["k_new"], inp["v_new"], cfg.new_segs, *oc, cfg.Lc, sm),
                4.0 * 128 * cfg.H * cfg.Lq * (cfg.Lc + cfg.Lq),
                "numpy float64 oracle, the whole call (16,096 queries x 31,936 keys x 16 heads)")
            del oc
        attn_line("turn3s", ms, cfg.H, cfg.Lq, cfg.Lc + cfg.Lq, cpu_b=cpu_b)
        del q, k, v, out, ws, cache, inp

    if want("seg4s"):
        # ---- seg4s: 54 layers resident, 8 steps over all of them
        log("workload seg4s: 54 layers resident, 8 steps over all of them")
        cfg = synth.WORKLOADS["seg4s"]
        (seg,) = cfg.new_segs
        layers = []
        t0 = time.time()
        for l in range(cfg.layers):
            inp = synth.layer_inputs("seg4s", l)
            cache = build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs, cfg.H, cfg.Lc)
            layers.append((d16(inp["q"]), d16(inp["k_new"]), d16(inp["v_new"])) + cache)
            del inp
            if l % 6 == 5:
                log("seg4s: %d of %d layers resident (%.0f s)" % (l + 1, cfg.layers, time.time() - t0))
        out = torch.empty_like(layers[0][0])
        ws = torch.empty(nomas.seg_attn_workspace([seg], cfg.Lc, cfg.H), dtype=torch.uint8, device=dev)

        def sequence():
            for _ in range(cfg.steps):
                for (q, k, v, kc, vc, ks, vs) in layers:
                    nomas.seg_attn(q, k, v, [seg], kc, vc, ks, vs, cache_len=cfg.Lc, sm_scale=sm, out=out, workspace=ws,
                                   stream=stream)

        ms = timed(sequence, 3, 1)
        calls = cfg.layers * cfg.steps
        del layers
        cpu_b = None
        if cpu:
            inp = synth.layer_inputs("seg4s", 0)
            oc = oracle.build_cache(inp["k_hist"], inp["v_hist"], cfg.hist_segs)
            cpu_b = oracle_timing(
                lambda: oracle.seg_attn(inp["q"], inp["k_new"], inp["v_new"], cfg.new_segs, *oc, cfg.Lc, sm),
                4.0 * 128 * cfg.H * cfg.Lq * (cfg.Lc + cfg.Lq),
                "numpy float64 oracle, one whole call (layer 0: 21,376 queries x 37,216 keys x 16 heads)")
            del inp, oc
        attn_line("seg4s", ms / calls, cfg.H, cfg.Lq, cfg.Lc + cfg.Lq,
                  dict(calls=calls, sequence_ms=round(ms, 1), outlier_channels=cfg.outliers), cpu_b)
        del out, ws

    if want("fiveturns"):
        # ---- fiveturns
        log("workload fiveturns")
        cfg = synth.WORKLOADS["fiveturns"]
        H = cfg.H
        n = synth.turn_seg(0).ntok
        cache = build_cache(None, None, None, H, 5 * n)
        length = 0
        ohead = []              # the oracle's own INT8 rows of head 0, turn by turn
        for t in range(5):
            inp = synth.turn_inputs(t)
            seg = inp["seg"]
            q, k, v, qc = d16(inp["q"]), d16(inp["k_new"]), d16(inp["v_new"]), d16(inp["q_cam"])
            wk, wv = d16(inp["w_k"]), d16(inp["w_v"])
            cam = torch.from_numpy(nomas.cam_tokens(inp["c2w"])).to(dev)
            out, oc, kr = torch.empty_like(q), torch.empty_like(qc), torch.empty_like(k)
            ws = torch.empty(nomas.seg_attn_workspace([seg], length, H), dtype=torch.uint8, device=dev)
            ms_a = timed(lambda: nomas.seg_attn(q, k, v, [seg], *cache, cache_len=length, sm_scale=sm, out=out,
                                                workspace=ws, stream=stream), 5)
            wsc = torch.empty(nomas.cam_xattn_workspace(H, cam.shape[0]), dtype=torch.uint8, device=dev)
            ms_c = timed(lambda: nomas.cam_xattn(qc, cam, wk, wv, sm_scale=sm, out=oc, workspace=wsc, stream=stream), 5)
            ms_r = timed(lambda: nomas.rope3d(k, [seg], out=kr, stream=stream), 5)
            # appending the same rows at the same offset is idempotent
            ms_q = timed(lambda: nomas.kv_quant_append(kr, v, *cache, length, stream=stream), 5)
            elems = n * H * 128
            gbs = lambda b, m: round(b / (m * 1e-3) / 1e9, 1)
            cpu_b = None
            if cpu and t in (0, 4):
                rows = np.arange(4096)
                oc = [np.zeros((1, max(1, length), 128), np.int8), np.zeros((1, max(1, length), 128), np.int8),
                      np.zeros((1, max(1, length)), np.float32), np.zeros((1, max(1, length)), np.float32)]
                if length:
                    for i in range(4):
                        oc[i][0, :length] = np.concatenate([r[i] for r in ohead])
                q1, k1, v1 = (np.ascontiguousarray(inp[x][:, :1]) for x in ("q", "k_new", "v_new"))
                cpu_b = oracle_timing(
                    lambda: oracle.seg_attn(q1, k1, v1, [seg], *oc, length, sm, rows=rows),
                    4.0 * 128 * len(rows) * (length + n),
                    "numpy float64 oracle, head 0, query rows 0..4095 of %d, each over all %d keys"
                    % (n, length + n))
            attn_line("fiveturns-turn%d" % t, ms_a, H, n, length + n,
                      dict(cache_tokens=length,
                           cam_xattn=dict(ms=round(ms_c, 4), GBps=gbs(4 * elems, ms_c), camera_tokens=cam.shape[0]),
                           rope3d=dict(ms=round(ms_r, 4), GBps=gbs(4 * elems, ms_r)),
                           kv_quant_append=dict(ms=round(ms_q, 4), GBps=gbs(2 * 3 * elems + 2 * 4 * n * H, ms_q)),
                           hbm_peak_GBps=PEAK_HBM_GBS), cpu_b)
            if cpu and t < 4:
                k_rot_o = oracle.bf16_round(oracle.rope3d(oracle.bf16_bits_to_f64(inp["k_new"][:, :1]), [seg]))[:, 0]
                kq, ksc = oracle.quantise(k_rot_o)
                vq, vsc = oracle.quantise(oracle.bf16_bits_to_f64(inp["v_new"][:, 0]))
                ohead.append((kq, vq, ksc, vsc))
            length = nomas.kv_quant_append(kr, v, *cache, length, stream=stream)
            torch.cuda.synchronize()
            del q, k, v, qc, out, oc, kr, ws
        del cache

    if want("decoder"):
        # ---- decoder window: 10 latent frames of 4x16x16 tubelets at 1280x704
        log("workload decoder-window")
        L, Hq, Hkv = 10 * 44 * 80, 32, 8
        q = d16(synth.random_bf16(501, (L, Hq, 128)))
        k = d16(synth.random_bf16(502, (L, Hkv, 128)))
        v = d16(synth.random_bf16(503, (L, Hkv, 128)))
        out = torch.empty_like(q)
        ws = torch.empty(nomas.gqa_attn_workspace(L, Hq, Hkv), dtype=torch.uint8, device=dev)
        ms = timed(lambda: nomas.gqa_attn(q, k, v, sm_scale=sm, out=out, workspace=ws, stream=stream), 5)
        attn_line("decoder-window", ms, Hq, L, L, dict(kv_heads=Hkv, entry="nomas_gqa_attn"))
        del q, k, v, out, ws

    if want("w8a16"):
        # ---- INT8-weight linear layers of one 12 s segment (63,360 tokens, hidden 2048, FFN 8192)
        for name, K, N in (("w8a16-qkv", 2048, 6144), ("w8a16-ffn-up", 2048, 8192), ("w8a16-ffn-down", 8192, 2048),
                           ("w8a16-out", 2048, 2048)):
            log("workload " + name)
            M = 63360
            x = d16(synth.random_bf16(601, (M, K)))
            g = np.random.default_rng(602)
            codes = torch.from_numpy(g.integers(-127, 128, size=(N, K), dtype=np.int8)).to(dev)
            scale = torch.from_numpy((1.0 / (73.0 * math.sqrt(K)) * (0.5 + g.random(N))).astype(np.float32)).to(dev)
            y = torch.empty((M, N), dtype=torch.int16, device=dev)
            ws = torch.empty(nomas.w8a16_linear_workspace(K, N), dtype=torch.uint8, device=dev)
            ms = timed(lambda: nomas.w8a16_linear(x, codes, scale, out=y, workspace=ws, stream=stream), 10, 3)
            # context: the dequantisation pass alone (M = 0), and torch's BF16 matmul on the dequantised weights
            ms_dq = timed(lambda: nomas.w8a16_linear(x[:0], codes, scale, out=y[:0], workspace=ws, stream=stream), 10, 3)
            wb = ws[:N * K * 2].view(torch.bfloat16).view(N, K)
            xb = x.view(torch.bfloat16)
            wt = wb.t().contiguous()
            ms_t = timed(lambda: torch.matmul(xb, wt), 10, 3)
            fl = 2.0 * M * N * K
            tf = fl / (ms * 1e-3) / 1e12
            emit(name, metric="linear TFLOP/s", value=round(tf, 2), unit="TFLOP/s", ms=round(ms, 4),
                 pct_of_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2), M=M, K=K, N=N, algorithmic_flop=fl,
                 dequant_ms=round(ms_dq, 4), context_torch_bf16_matmul_ms=round(ms_t, 4))
            del x, codes, scale, y, ws, wt

    if want("fullcache"):
        # ---- fullcache-sel18 and fullcache-h2 share the full-cache inputs
        log("workload fullcache-sel18 / fullcache-h2: generating the full-cache inputs")
        cfg = synth.WORKLOADS["fullcache"]
        inp = synth.layer_inputs("fullcache")
        (seg,) = cfg.new_segs
        (hseg,) = cfg.hist_segs
        frame = hseg.Hg * hseg.Wg
        # history selection: 18 of the 288 cached latent frames, the last of every 16
        sel = [[(f * frame, (f + 1) * frame) for f in range(15, hseg.T, 16)]]
        nsel = sum(hi - lo for lo, hi in sel[0])
        cache = build_cache(inp["k_hist"], inp["v_hist"], [hseg], cfg.H, cfg.Lc)
        q, k, v = d16(inp["q"]), d16(inp["k_new"]), d16(inp["v_new"])
        out = torch.empty_like(q)
        ws = torch.empty(nomas.seg_attn_workspace([seg], cfg.Lc, cfg.H, sel=sel), dtype=torch.uint8, device=dev)
        ms = timed(lambda: nomas.seg_attn(q, k, v, [seg], *cache, cache_len=cfg.Lc, sm_scale=sm, out=out, workspace=ws,
                                          stream=stream, sel=sel), 5)
        attn_line("fullcache-sel18", ms, cfg.H, cfg.Lq, nsel + cfg.Lq,
                  dict(cache_tokens=cfg.Lc, selected_frames=len(sel[0]), selected_tokens=nsel))
        del q, k, v, out, ws, cache

        # ---- fullcache-h2: one GPU's share of the full-cache shape
        log("workload fullcache-h2: one GPU's share of the full-cache shape")
        H = 2
        sub = lambda a: np.ascontiguousarray(a[:, :H])
        cache = build_cache(sub(inp["k_hist"]), sub(inp["v_hist"]), [hseg], H, cfg.Lc)
        q, k, v = d16(sub(inp["q"])), d16(sub(inp["k_new"])), d16(sub(inp["v_new"]))
        del inp
        out = torch.empty_like(q)
        ws = torch.empty(nomas.seg_attn_workspace([seg], cfg.Lc, H), dtype=torch.uint8, device=dev)
        ms = timed(lambda: nomas.seg_attn(q, k, v, [seg], *cache, cache_len=cfg.Lc, sm_scale=sm, out=out, workspace=ws,
                                          stream=stream), 5)
        attn_line("fullcache-h2", ms, H, cfg.Lq, cfg.Lc + cfg.Lq, dict(note="heads 0-1 of the full-cache inputs"))
        del q, k, v, out, ws, cache

    if want("train"):
        # ---- segment-forcing training: packed forward and backward
        log("workload train-fwd / train-bwd: 22 packed 3 s turns, 2 heads")
        segs = synth.train_segs()
        H = 2
        inp = synth.train_inputs(segs, H)
        q, k, v, do = (d16(inp[x]) for x in ("q", "k", "v", "d_out"))
        del inp
        L = q.shape[0]
        n_a = [s.ntok for s in segs]
        pairs = H * sum(n_a[a] * sum(n_a[:a + 1]) for a in range(len(n_a)))
        out = torch.empty_like(q)
        lse = torch.empty((H, L), dtype=torch.float32, device=dev)
        ws = torch.empty(nomas.seg_attn_workspace(segs, 0, H), dtype=torch.uint8, device=dev)
        ms_f = timed(lambda: nomas.seg_attn(q, k, v, segs, cache_len=0, sm_scale=sm, out=out, lse=lse, workspace=ws,
                                            stream=stream), 5)
        fl_f = 4.0 * 128 * pairs
        tf_f = fl_f / (ms_f * 1e-3) / 1e12
        emit("train-fwd", metric="attention TFLOP/s", value=round(tf_f, 2), unit="TFLOP/s", ms=round(ms_f, 3),
             pct_of_peak=round(100 * tf_f / PEAK_BF16_TFLOPS, 2), heads=H, tokens=L, segments=len(segs),
             allowed_pairs=pairs, algorithmic_flop=fl_f)
        del ws
        wsb = torch.empty(nomas.seg_attn_bwd_workspace(segs, H), dtype=torch.uint8, device=dev)
        g = [torch.empty((L, H, 128), dtype=torch.float32, device=dev) for _ in range(3)]
        ms_b = timed(lambda: nomas.seg_attn_bwd(q, k, v, out, lse, do, segs, sm_scale=sm, dq=g[0], dk=g[1], dv=g[2],
                                                workspace=wsb, stream=stream), 5)
        # algorithmic: five products of 2 x 128 flops per allowed pair (S recomputed once);
        # the kernels execute seven (S and dP in both the dK/dV and the dQ kernel)
        fl_b = 10.0 * 128 * pairs
        tf_b = fl_b / (ms_b * 1e-3) / 1e12
        emit("train-bwd", metric="attention backward TFLOP/s", value=round(tf_b, 2), unit="TFLOP/s",
             ms=round(ms_b, 3), pct_of_peak=round(100 * tf_b / PEAK_BF16_TFLOPS, 2), heads=H, tokens=L,
             segments=len(segs), allowed_pairs=pairs, algorithmic_flop=fl_b,
             executed_mfma_flop=14.0 * 128 * pairs,
             executed_pct_of_peak=round(100 * 1.4 * tf_b / PEAK_BF16_TFLOPS, 2),
             fwd_plus_bwd_ms=round(ms_f + ms_b, 3))


def _cpu_info():
    """Threads the oracle's BLAS uses and the host CPU model."""
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max((i.get("num_threads") or 1) for i in info) if info else int(threads)
    except Exception:
        cores = int(threads)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return int(cores), model


def oracle_timing(run, flops, sample):
    """Time one oracle call (numpy float64, as it stands) and report it as a
    cpu_baseline object in TFLOP/s of algorithmic attention FLOPs."""
    t0 = time.perf_counter()
    run()
    dt = time.perf_counter() - t0
    cores, model = _cpu_info()
    log("cpu baseline: %.2f s for %.3e FLOP (%s)" % (dt, flops, sample))
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 4), "cpu_model": model, "sample": sample}


def cpu_baseline(inp, cfg, sm):
    """The oracle (numpy float64) on a bounded sample: head 0, the first 8192
    of the 63,360 query rows, all 316,800 allowed keys."""
    import numpy as np

    import oracle

    H, Lq, Lc = cfg.H, cfg.Lq, cfg.Lc
    rows = np.arange(8192)
    kc, vc, ks, vs = oracle.build_cache(inp["k_hist"][:, :1], inp["v_hist"][:, :1], cfg.hist_segs)
    q1 = np.ascontiguousarray(inp["q"][:, :1])
    k1 = np.ascontiguousarray(inp["k_new"][:, :1])
    v1 = np.ascontiguousarray(inp["v_new"][:, :1])
    flops = 4.0 * 128 * len(rows) * (Lc + Lq)
    return oracle_timing(
        lambda: oracle.seg_attn(q1, k1, v1, cfg.new_segs, kc, vc, ks, vs, Lc, sm, rows=rows), flops,
        "numpy float64 oracle, head 0 of 16, query rows 0..8191 of 63,360, each over all 316,800 "
        "allowed keys (%.2e algorithmic FLOP), timed including its per-head key dequantisation "
        "and rotation" % flops)


if __name__ == "__main__":
    main()
