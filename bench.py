#!/usr/bin/env python3
"""Benchmark of one MoE FFN layer forward pass on one MI355X.

A step is one pass of the whole layer (route -> permute -> grouped SwiGLU FFN ->
combine, plus the shared expert where the workload has one) over one batch of
synthetic tokens already resident in HBM.

With no --workload the suite runs: the headline line is the DeepSeek-V3-shaped fp8
prefill layer (T=8192, d=7168, E=256, top-8 grouped sigmoid, F=2048 plus a shared
expert; the largest workload that fits one GPU), timed for exactly --steps steps after
--warmup; its "configs" object carries the other workloads measured in the same run,
each with its own roofline, step-time percentiles and CPU baseline: the
Mixtral-8x7B-shaped bf16 prefill, the Qwen1.5-MoE-shaped bf16 decode at 1, 8 and 64
tokens (eager launches queued ahead of the GPU, graph replays beside them), and the
expert-offload decode through a 32-slot LRU pool (256 steps; blocking and device-planned
modes beside it).

Prints one JSON line: tokens/s for the whole job, the dominant kernel's roofline
(algorithmic flops or bytes per launch over its average duration, timed with hipEvents
on its launch stream inside the timed region), and the float64 CPU oracle timed on a
bounded sample of the same workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens T]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; HBM TB/s (decode) & MFMA TFLOP/s (prefill) vs peak"
# dense MFMA peaks; MXFP4 experts run E4M3 x E2M1 block-scaled MFMAs, priced at the fp8 rate
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 5000.0, "f32": 157.3}
PEAK_PCIE_GBS = 63.0   # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 encoding
PEAK_HBM_GBS = 8000.0
WORKLOADS = ["suite", "mixtral_prefill_bf16", "dsv3_prefill_fp8", "mixtral_prefill_mxfp4", "qwen_decode_bf16", "tiny_fp32", "offload_decode_bf16",
             "offload_decode_mxfp4"]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none for this workload or any source file of the kernel changed since the
    counters were taken (the record lists the sha256 of each)."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic-record:"):
                    continue
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("workload") != workload or rec.get("kernel") != kernel:
                    continue
                for rel, sha in rec["sources"].items():
                    src = os.path.join(ROOT, rel)
                    if not os.path.exists(src):
                        return None
                    with open(src, "rb") as g:
                        if hashlib.sha256(g.read()).hexdigest() != sha:
                            return None
                return int(rec["bytes_per_launch"])
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _x_dev(cfg, x_store, torch):
    if cfg.act_dtype == "f32":
        return torch.from_numpy(x_store).to("cuda")
    return torch.from_numpy(x_store.view(np.int16)).view(torch.bfloat16).to("cuda")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, w, sample_tokens, logit_bias=False):
    """The float64 oracle, as it stands, on the first `sample_tokens` tokens of batches 0, 1, ...
    (with logit_bias, batch i takes the Zipf prior of decode step i, as the offload stream does)."""
    from oracle import formats, moe  # CPU baseline leg only

    def dec(a):
        return np.asarray(a, np.float64) if cfg.act_dtype == "f32" else formats.decode_bf16(a)

    def dec_w(m):
        if cfg.dtype == "fp8":
            return formats.dequantize_weight_blocks(*m)
        if cfg.dtype == "mxfp4":
            return formats.dequantize_mxfp4_weight(*m)
        return dec(m)

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p["num_threads"] for p in info)
    except Exception:
        pass
    from expert_offloaded_ffn_amd import synth
    nb = (sample_tokens + cfg.T - 1) // cfg.T
    x_store = np.concatenate([synth.gen_x(cfg, i) for i in range(nb)])[:sample_tokens]
    lb = None
    if logit_bias:
        lb = np.concatenate([np.repeat(synth.zipf_logit_bias(cfg, i)[None], cfg.T, 0) for i in range(nb)])
        lb = lb[:sample_tokens].astype(np.float64)
    t0 = time.perf_counter()
    x = dec(x_store)
    route_kw = dict(k=cfg.k, score_fn=cfg.score_fn, renormalize=bool(cfg.renormalize), route_scale=cfg.route_scale,
                    n_groups=cfg.n_groups, topk_groups=cfg.topk_groups, group_topn=cfg.group_topn,
                    select_bias=w.get("sb"), w_shared_gate=None if w.get("w_sg") is None else dec(w["w_sg"]))
    if lb is None:
        r = moe.route(x, dec(w["router"]), **route_kw)
    else:   # one routing call per batch: the prior differs between steps
        rs = [moe.route(x[i:i + cfg.T], dec(w["router"]), logit_bias=lb[i], **route_kw)
              for i in range(0, sample_tokens, cfg.T)]
        r = moe.Routing(*[None if getattr(rs[0], f) is None else np.concatenate([getattr(q, f) for q in rs])
                          for f in ("logits", "keys", "idx", "gate", "shared_gate")])

    def expert(e):
        return moe.ExpertWeights(*[dec_w(m) for m in w["experts"][e]])

    shared = None if w.get("shared") is None else moe.ExpertWeights(*[dec_w(m) for m in w["shared"]])
    quant = "e4m3" if cfg.dtype == "fp8" else ("mxfp8" if cfg.dtype == "mxfp4" and cfg.T > 64 else None)
    moe.moe_layer(x, r, expert, cfg.E, shared=shared, quant_act=quant)
    dt = time.perf_counter() - t0
    return {"value": round(sample_tokens / dt, 3), "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of batches 0.. of {cfg.name} (T={cfg.T}), float64, "
                      f"expert weights decoded per expert; {dt:.1f} s"}


def percentiles(ms):
    return [round(float(np.percentile(ms, q)), 4) for q in (10, 50, 90)]


OFFLOAD_MODES = ("overlapped", "blocking", "overlapped_freq", "device_plan", "device_plan_graph",
                 "device_plan_freq_graph")


def bench_offload(args, torch, B, synth, MoELayer, modes=OFFLOAD_MODES, cpu_sample=0):
    """Expert-offload decode: T tokens per step through an n_slots HBM slot pool fed from pinned host
    bundles, Zipf-biased routing re-drawn every zipf_epoch steps. The same steps run with every
    expert resident (compute time) and then in each of `modes`: the host-planned LRU pool with
    overlapped copies (the pages' design, and the line's value), the same pool in blocking mode
    (a wave's copies start after all compute before them: the overlap reference), overlapped with
    frequency-aware victims (--freq-decay), and the pool planned on the device (copy kernels, no
    host synchronisation), eager and as one graph replay per step, with LRU and frequency-aware
    victims. Every mode starts from an empty pool. Returns the result dict."""
    from expert_offloaded_ffn_amd.layer import W_CODE
    cfg = synth.get_config(args.workload if args.workload.startswith("offload") else "offload_decode_bf16")
    if args.tokens:
        cfg = cfg.with_T(args.tokens)
    steps = cfg.steps if args.workload == "suite" else args.steps
    log(f"[bench] offload {cfg.name}: generating {cfg.E} experts")
    router, experts = synth.gen_router(cfg), synth.gen_experts(cfg, threads=16)
    xs = [_x_dev(cfg, synth.gen_x(cfg, s), torch) for s in range(steps)]
    lbs = [torch.from_numpy(synth.zipf_logit_bias(cfg, s)).to("cuda") for s in range(steps)]

    def run(layer):
        """Wall time of the steps, and each step's span from hipEvents on the compute stream."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            evs[s][0].record()
            layer.forward(xs[s], logit_bias=lbs[s])
            evs[s][1].record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, np.array([a.elapsed_time(b) for a, b in evs])

    res = MoELayer(cfg, router=router, experts=experts, threads=16)
    for s in range(min(3, steps)):
        res.forward(xs[s], logit_bias=lbs[s])
    t_comp, _ = run(res)
    del res
    torch.cuda.empty_cache()
    out = {}
    host_modes = {"overlapped": (False, 0.0), "blocking": (True, 0.0), "overlapped_freq": (False, args.freq_decay)}
    for mode in [m for m in modes if m in host_modes]:
        blocking, decay = host_modes[mode]
        log(f"[bench] offload mode {mode}")
        lay = MoELayer(cfg, router=router, experts=experts, pool_slots=cfg.n_slots, blocking=blocking, threads=16,
                       freq_decay=decay)
        t_wall, ms = run(lay)
        st = lay.cache.stats()
        t_copy = st["copy_ms"] / 1e3
        acc = st["hits"] + st["misses"]
        out[mode] = {"wall_s": round(t_wall, 4), "tokens_per_s": round(cfg.T * steps / t_wall, 1),
                     "step_ms_p10_p50_p90": percentiles(ms),
                     "hit_rate": round(st["hits"] / max(acc, 1), 4), "hits": st["hits"], "misses": st["misses"],
                     "evictions": st["evictions"], "waves": st["waves"], "h2d_bytes": st["h2d_bytes"],
                     "d2h_bytes": st["d2h_bytes"], "copy_s": round(t_copy, 4), "wait_s": round(st["wait_ms"] / 1e3, 4),
                     "h2d_GBps": round(st["h2d_bytes"] / max(t_copy, 1e-9) / 1e9, 2),
                     "overlap": round(max(0.0, (t_copy + t_comp - t_wall) / max(min(t_copy, t_comp), 1e-9)), 4)}
        lay.cache.close()
        del lay
        torch.cuda.empty_cache()
    dev_modes = [m for m in modes if m.startswith("device_plan")]
    if dev_modes:
        # the device-planned pool: no host synchronisation; eager, then every step one graph replay
        log(f"[bench] offload modes {dev_modes}")
        lay = MoELayer(cfg, router=router, experts=experts, pool_slots=cfg.n_slots, device_plan=True, threads=16)
        timed = []
        t_wall, ms = run(lay)
        if "device_plan" in dev_modes:
            timed.append(("device_plan", t_wall, ms, lay.cache_dev.stats()))
        lay.cache_dev.reset()
        x_static, lb_static = xs[0].clone(), lbs[0].clone()
        graph, _ = lay.capture(x_static, lb_static)
        for mode, decay in (("device_plan_graph", 0.0), ("device_plan_freq_graph", args.freq_decay)):
            if mode not in dev_modes:
                continue
            lay.cache_dev.set_frequency(decay)
            lay.cache_dev.reset()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(steps):
                x_static.copy_(xs[s])
                lb_static.copy_(lbs[s])
                evs[s][0].record()
                graph.replay()
                evs[s][1].record()
            torch.cuda.synchronize()
            timed.append((mode, time.perf_counter() - t0, np.array([a.elapsed_time(b) for a, b in evs]),
                          lay.cache_dev.stats()))
        for mode, t, ms, stt in timed:
            acc = stt["hits"] + stt["misses"]
            out[mode] = {"wall_s": round(t, 4), "tokens_per_s": round(cfg.T * steps / t, 1),
                         "step_ms_p10_p50_p90": percentiles(ms),
                         "hit_rate": round(stt["hits"] / max(acc, 1), 4), "hits": stt["hits"],
                         "misses": stt["misses"], "evictions": stt["evictions"], "waves": stt["waves"],
                         "h2d_bytes": stt["h2d_bytes"], "h2d_GBps_wall": round(stt["h2d_bytes"] / t / 1e9, 2)}
        lay.cache_dev.close()
        del lay, graph
        torch.cuda.empty_cache()
    # the line's value is the pages' design: LRU over the host-planned pool with overlapped
    # copies; the other modes are reported beside it
    main_mode = "overlapped" if "overlapped" in out else next(iter(out))
    o = out[main_mode]
    result = {
        "metric": METRIC, "value": o["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 0,
        "ms_per_step": round(o["wall_s"] / steps * 1e3, 4), "step_ms_p10_p50_p90": o["step_ms_p10_p50_p90"],
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded; Zipf(1.1) log-prior re-drawn every 64 steps)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.F, "n_slots": cfg.n_slots, "weights": cfg.dtype, "policy": "lru", "mode": main_mode,
                   "bundle_bytes": B.bundle_bytes(cfg.d, cfg.F, W_CODE[cfg.dtype])},
        "hit_rate": o["hit_rate"], "h2d_bytes": o["h2d_bytes"], "overlap": o.get("overlap"),
        "resident_compute_s": round(t_comp, 4), "offload": out,
    }
    h2d = o.get("h2d_bytes", 0)
    if h2d:
        a = h2d / o["wall_s"] / 1e9
        result["roofline"] = {"bound": "pcie", "kernel": "host-to-HBM bundle copies of the missed experts",
                              "achieved": round(a, 2), "peak": PEAK_PCIE_GBS, "unit": "GB/s",
                              "frac": round(a / PEAK_PCIE_GBS, 4), "traffic": None,
                              "work_per_launch": "bundle bytes of the step's misses over the whole run's wall time"}
    if cpu_sample:
        log(f"[bench] cpu baseline: oracle on {cpu_sample} tokens")
        result["cpu_baseline"] = cpu_baseline(cfg, dict(router=router, experts=experts), cpu_sample, logit_bias=True)
    return result


def bench_stack(args, torch, B, synth, MoELayer):
    """Expert-offload decode through a synthetic stack of L layers whose experts share one HBM slot
    pool (entry l*E + e), so the layers compete for the same slots. Each layer step may prefetch the
    next layer's predicted experts once its own waves are issued: "prev" predicts the experts that
    layer touched in the previous step, "zipf" the top-N experts of its routing prior for the step
    (the synthetic stand-in for a shadow router). The layers share expert weights (distinct cache
    entries, real copies) and take independent inputs; the same steps also run with every expert
    resident (compute time) and with no prefetch, under plain LRU and under the layer order (victims
    from the layer that runs furthest ahead first)."""
    from expert_offloaded_ffn_amd.layer import W_CODE, SharedSlotPool, pack_bundles
    cfg = synth.get_config(args.workload)
    if args.tokens:
        cfg = cfg.with_T(args.tokens)
    L, steps, E = args.layers, args.steps, cfg.E
    n_slots = args.slots or cfg.n_slots * L
    cfgs = synth.stack_configs(cfg, L)
    log(f"[bench] stack: {L} layers, {n_slots} shared slots, generating {E} experts")
    experts = synth.gen_experts(cfg, threads=16)
    routers = [synth.gen_router(c) for c in cfgs]
    xs = [[_x_dev(c, synth.gen_x(c, s), torch) for s in range(steps)] for c in cfgs]
    priors = [[synth.zipf_logit_bias(c, s) for s in range(steps + 1)] for c in cfgs]
    lbs = [[torch.from_numpy(p).to("cuda") for p in pl[:steps]] for pl in priors]

    def run(layers, pool=None, predictor="none"):
        prev = [[] for _ in range(L)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            for l in range(L):
                nl, ns = (l + 1) % L, s + (l + 1) // L
                pred = None
                if predictor == "prev":
                    pred = [nl * E + e for e in prev[nl]]
                elif predictor == "zipf":
                    pred = [nl * E + int(e) for e in np.argsort(-priors[nl][ns], kind="stable")[:args.prefetch_n]]
                g = layers[l].forward(xs[l][s], logit_bias=lbs[l][s], prefetch=pred)
                if pool is not None and predictor == "prev":
                    prev[l] = sorted({en[0] - l * E for w in range(g["waves"]) for en in pool.cache.wave_plan(w)})
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    res = [MoELayer(c, router=r, experts=experts, threads=16) for c, r in zip(cfgs, routers)]
    for l in range(L):
        res[l].forward(xs[l][0], logit_bias=lbs[l][0])
    t_comp = run(res)
    del res
    torch.cuda.empty_cache()
    bundles = pack_bundles(cfg, experts, cfg.d, cfg.F, pin=True, threads=16)
    out = {}
    predictors = ["none"] + [p for p in args.prefetch.split(",") if p and p != "none"]
    for policy, predictor in [(pol, pr) for pol in args.policies.split(",") for pr in predictors]:
        dev = policy.startswith("dev")   # planned on the device (no prefetch there)
        if dev and predictor != "none":
            continue
        key = f"{policy}/{predictor}"
        pool = SharedSlotPool([bundles] * L, n_slots, cfg.d, cfg.F, W_CODE[cfg.dtype],
                              layer_order=policy.removeprefix("dev").startswith("layer"),
                              freq_decay=args.freq_decay if policy.endswith("freq") else 0.0, device_plan=dev)
        layers = [MoELayer(c, router=r, experts=None, shared_pool=pool, layer_index=l)
                  for l, (c, r) in enumerate(zip(cfgs, routers))]
        t_wall = run(layers, pool, predictor)
        st = (pool.cache_dev if dev else pool.cache).stats()
        acc = st["hits"] + st["misses"]
        out[key] = {"wall_s": round(t_wall, 4), "tokens_per_s": round(cfg.T * steps / t_wall, 1),
                          "ms_per_step": round(t_wall / steps * 1e3, 3),
                          "hit_rate": round(st["hits"] / max(acc, 1), 4), "hits": st["hits"],
                          "misses": st["misses"], "prefetches": st["prefetches"],
                          "prefetch_used": st["prefetch_used"],
                          "prefetch_accuracy": round(st["prefetch_used"] / max(st["prefetches"], 1), 4),
                          "h2d_GB": round(st["h2d_bytes"] / 1e9, 3),
                          "h2d_GBps_wall": round(st["h2d_bytes"] / t_wall / 1e9, 2)}
        log(f"[bench] stack {key}: {out[key]}")
        (pool.cache_dev if dev else pool.cache).close()
        del layers, pool
        torch.cuda.empty_cache()
    best = max(out, key=lambda k: out[k]["tokens_per_s"])
    result = {
        "metric": METRIC, "value": out[best]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": 0, "ms_per_step": out[best]["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; per-layer routers and Zipf(1.1) priors, expert weights shared by the layers)",
        "config": {"workload": cfg.name + "_stack", "layers": L, "T": cfg.T, "d_model": cfg.d, "n_experts": E,
                   "top_k": cfg.k, "d_ff": cfg.F, "n_slots_shared": n_slots, "weights": cfg.dtype,
                   "prefetch_n_zipf": args.prefetch_n, "best": best,
                   "bundle_bytes": B.bundle_bytes(cfg.d, cfg.F, W_CODE[cfg.dtype])},
        "resident_compute_s": round(t_comp, 4), "stack": out,
    }
    b = out[best]
    if b["h2d_GB"] > 0:
        result["roofline"] = {"bound": "pcie", "kernel": "host-to-HBM bundle copies of the missed experts",
                              "achieved": b["h2d_GBps_wall"], "peak": PEAK_PCIE_GBS, "unit": "GB/s",
                              "frac": round(b["h2d_GBps_wall"] / PEAK_PCIE_GBS, 4), "traffic": None,
                              "work_per_launch": "bundle bytes copied (misses and prefetches) over the run's wall time"}
    print(json.dumps(result), flush=True)
    return 0


class TimingEvent:
    """A timing-only hipEvent created with hipEventDisableSystemFence: its record runs no
    system-scope cache write-back and invalidate between the timed work and the event (torch's
    events carry one). Created through the HIP runtime the process already has loaded."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = "libamdhip64.so"
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self, torch):
        import ctypes
        self._torch, self._c = torch, ctypes
        self.e = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.e), 0x20000000)  # hipEventDisableSystemFence
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self):
        rc = self._hip.hipEventRecord(self.e, self._c.c_void_p(self._torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end):
        if self._hip.hipEventSynchronize(end.e) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = self._c.c_float()
        if self._hip.hipEventElapsedTime(self._c.byref(ms), self.e, end.e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self):
        """Frees the event (explicitly, while the runtime is up: not from a finaliser, which can
        run after the runtime has shut down at interpreter exit)."""
        if self.e:
            self._hip.hipEventDestroy(self.e)
            self.e = self._c.c_void_p()


def destroy_events(evs):
    for pair in evs:
        for e in pair:
            e.destroy()


def _sleep_cycles_per_ms(torch):
    """Cycles of torch.cuda._sleep (a bounded spin on the shader clock) per millisecond."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c = 20_000_000
    torch.cuda._sleep(c)
    e0.record()
    torch.cuda._sleep(c)
    e1.record()
    torch.cuda.synchronize()
    return c / max(e0.elapsed_time(e1), 1e-3)


def queued_ahead(torch, n, body, group=25):
    """Runs body(i) for i < n, each group of steps queued by the host behind a bounded GPU sleep
    long enough for the host to issue the whole group, so no step waits on the host's launches:
    event spans inside body then time the GPU's work. body(-1) is an untimed step that sizes the
    sleep. Returns the host's time per body() call in ms."""
    cpm = _sleep_cycles_per_ms(torch)
    t0 = time.perf_counter()
    for i in range(min(3, n)):     # the host's cost of one step, untimed
        body(-1)
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) / min(3, n) * 1e3
    for g0 in range(0, n, group):
        g = min(group, n - g0)
        torch.cuda._sleep(int(min(500.0, 2.0 + 1.5 * g * host_ms) * cpm))
        for i in range(g0, g0 + g):
            body(i)
        torch.cuda.synchronize()
    return host_ms


def bench_decode(args, torch, B, synth, MoELayer, workload=None, T=None, steps=None, warmup=None, graph=None,
                 cpu_sample=0):
    """Decode layer (few tokens): each step's time is measured alone with hipEvents, after a
    512 MiB pass that evicts the 256 MB last-level cache, so weights stream from HBM (a read by
    default, leaving clean lines as other layers' weight reads would; --mall-flush write leaves
    dirty lines that the step's own reads must first write back). The host issues the flush and
    the step faster than a serving loop would need but slower than the GPU runs them (the flush
    alone costs it more host time than the step costs the GPU), so the steps are queued ahead of
    the GPU in groups (queued_ahead) and the events time the GPU's work; the host's own time per
    step is reported beside it. The roofline is HBM bytes: the distinct touched experts' bundles
    + the shared expert + router weights + activations in and out. Returns the result dict."""
    from expert_offloaded_ffn_amd.layer import FUSE_COMBINE_MAX_T, W_CODE
    workload = workload or args.workload
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    use_graph = args.graph if graph is None else graph
    cfg = synth.get_config(workload)
    if T or args.tokens:
        cfg = cfg.with_T(T or args.tokens)
    log(f"[bench] decode {cfg.name} T={cfg.T}: generating inputs")
    w = dict(router=synth.gen_router(cfg), experts=synth.gen_experts(cfg, threads=16),
             shared=synth.gen_shared(cfg) if cfg.F_shared else None,
             w_sg=synth.gen_shared_gate(cfg) if cfg.shared_gate else None)
    layer = MoELayer(cfg, router=w["router"], experts=w["experts"], shared=w["shared"], w_shared_gate=w["w_sg"],
                     threads=16, fuse_combine=not args.no_fuse_combine, fused_step=not args.separate_calls)
    nb = max(args.batches, 64)
    xs = [_x_dev(cfg, synth.gen_x(cfg, 1 + i), torch) for i in range(nb)]
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    flush_words = flush.view(torch.int32)
    bundle = B.bundle_bytes(cfg.d, cfg.F, W_CODE[cfg.dtype])
    shared_bytes = B.bundle_bytes(cfg.d, cfg.F_shared, W_CODE[cfg.dtype]) if cfg.F_shared else 0
    act = 2 * cfg.T * cfg.d * 2 + cfg.E * cfg.d * 2 + (cfg.d * 2 if cfg.shared_gate else 0)
    touched = []
    for x in xs:
        c = B.route(x, layer.w_router_t, **layer.route_args())["counts"].cpu().numpy()
        touched.append(int((c > 0).sum()))
    for i in range(warmup):
        layer.forward(xs[i % nb])
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        # the whole layer as one HIP graph; inputs are refilled in place before each replay
        x_static = torch.empty_like(xs[0])
        x_static.copy_(xs[0])
        graph, _ = layer.capture(x_static)
    evs = [(TimingEvent(torch), TimingEvent(torch)) for _ in range(steps)]

    def flush_cache(i):
        if args.mall_flush == "write":
            flush.fill_(i & 255)      # leaves the last-level cache full of dirty lines
        else:
            flush_words.max()         # reads 512 MiB: clean lines, as other layers' weight reads leave it

    host_s = [0.0]   # the host's time in the layer's launches (replay or forward) over the timed steps

    def step(i):
        flush_cache(max(i, 0))
        x = xs[max(i, 0) % nb]
        if graph is not None:
            x_static.copy_(x)
        if i >= 0:
            evs[i][0].record()
        t = time.perf_counter()
        if graph is not None:
            graph.replay()
        else:
            layer.forward(x)
        if i >= 0:
            host_s[0] += time.perf_counter() - t
            evs[i][1].record()

    def eager_step(i):
        flush_cache(max(i, 0))
        layer.forward(xs[max(i, 0) % nb])

    # the timed steps run without the library's per-launch events (they cost GPU time between
    # the launches); the same steps once more as eager launches with the events, each after the
    # same cache flush, time the kernels for the roofline (events cannot be taken inside a replay)
    B.profile_enable(False)
    queued_ahead(torch, steps, step)
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    destroy_events(evs)
    B.profile_enable(True)
    queued_ahead(torch, steps, eager_step)
    prof = B.profile_read()
    B.profile_enable(False)
    del flush, flush_words
    step_bytes = np.array([touched[i % nb] * bundle + shared_bytes + act for i in range(steps)], np.float64)
    # The launch timed as the roofline kernel streams the touched routed experts' W_gu. In the
    # fused step (moe_decode_step) it also streams the shared expert's W_dn (the shared gate/up
    # ran beside the routing); in the separate calls it carries the shared expert's W_gu when
    # the layer runs the shared expert inside the routed launches.
    fused = layer.fused_decode_step(cfg.T)
    merged = layer.shared_in_decode_launch(cfg.T)
    wbytes = 0.5 + 1 / 32 if cfg.dtype == "mxfp4" else 2.0   # bytes per weight (codes and scales)
    if fused:
        shared_w = cfg.F_shared * cfg.d * wbytes
        who = "routed gate/up + shared down" if cfg.F_shared else "routed gate/up"
        kname = "ffn_decode_down_gateup" if cfg.F_shared else "ffn_decode_bf16<gate/up+SwiGLU>"
        work = ("gate/up weight bytes of the touched routed experts + the shared expert's down weight bytes"
                if cfg.F_shared else "gate/up weight bytes of the touched routed experts")
    else:
        shared_w = 2 * cfg.F_shared * cfg.d * wbytes if merged else 0
        who = "routed experts + shared expert" if merged else "routed experts"
        kname = "ffn_decode_bf16<gate/up+SwiGLU>"
        work = f"gate/up weight bytes of the touched {who}"
    gu_bytes = sum(touched[i % nb] * 2 * cfg.F * cfg.d * wbytes + shared_w for i in range(steps))
    gu_ms, gu_n = prof[B.PROF_DEC_GATEUP]
    hbm = float(step_bytes.sum() / (ms.sum() / 1e3) / 1e9)
    hbm_med = float(np.median(step_bytes) / (np.median(ms) / 1e3) / 1e9)
    result = {
        "metric": METRIC, "value": round(cfg.T * steps / (ms.sum() / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(float(ms.mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "n_experts": cfg.E, "top_k": cfg.k,
                   "d_ff": cfg.F, "d_ff_shared": cfg.F_shared, "mall_flush_MiB": 512, "mall_flush": args.mall_flush,
                   "hip_graph": bool(use_graph), "fused_step": bool(fused),
                   "combine_in_down_launch": bool(cfg.T <= FUSE_COMBINE_MAX_T and
                                                  (fused or (layer.fuse_combine and merged)))},
        "step_ms_p10_p50_p90": percentiles(ms),
        "timing": "GPU time per step: each group of steps queued by the host behind a bounded GPU sleep",
        "host_ms_per_step": round(host_s[0] / steps * 1e3, 4),
        "touched_experts_mean": round(float(np.mean([touched[i % nb] for i in range(steps)])), 2),
        "layer_hbm": {"achieved": round(hbm, 1), "achieved_at_median_step": round(hbm_med, 1), "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": round(hbm / PEAK_HBM_GBS, 4),
                      "bytes_per_step_mean": int(step_bytes.mean())},
    }
    if gu_n:
        a = gu_bytes / (gu_ms / 1e3) / 1e9
        # HBM bytes per launch from the committed counter record of this workload and batch size
        traffic = recorded_traffic(f"{cfg.name}@T{cfg.T}", f"{kname} ({who})")
        result["roofline"] = {"bound": "hbm", "kernel": f"{kname} ({who})",
                              "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(a / PEAK_HBM_GBS, 4), "traffic": traffic,
                              "avg_launch_ms": round(gu_ms / gu_n, 4),
                              "work_per_launch": work,
                              "timed": "eager launches of the same steps, with per-launch events"}
    if graph is not None:
        del graph
    del layer, xs
    torch.cuda.empty_cache()
    if cpu_sample:
        log(f"[bench] cpu baseline: oracle on {cpu_sample} tokens")
        result["cpu_baseline"] = cpu_baseline(cfg, w, cpu_sample)
    return result


def bench_prefill(args, torch, B, synth, MoELayer, workload=None, steps=None, warmup=None, cpu_sample=None):
    """Prefill layer (thousands of tokens, every expert resident): `warmup` untimed steps, then
    exactly `steps` timed steps over rotating input batches, bracketed by synchronisations, with
    an event pair per step for the percentiles (timing-only events, TimingEvent). The dominant
    kernel is the routed experts' gate/up GEMM (real rows only): achieved = its flops per launch
    / its average launch time, from hipEvents on its own stream. Returns the result dict."""
    workload = workload or args.workload
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    cfg = synth.get_config(workload)
    if args.tokens:
        cfg = cfg.with_T(args.tokens)
    log(f"[bench] workload {cfg.name} T={cfg.T}: generating inputs")
    w = dict(router=synth.gen_router(cfg), experts=synth.gen_experts(cfg, threads=16),
             shared=synth.gen_shared(cfg) if cfg.F_shared else None,
             w_sg=synth.gen_shared_gate(cfg) if cfg.shared_gate else None,
             sb=synth.gen_select_bias(cfg) if cfg.select_bias else None)
    layer = MoELayer(cfg, router=w["router"], experts=w["experts"], shared=w["shared"], w_shared_gate=w["w_sg"],
                     select_bias=w["sb"], threads=16)
    xs = [_x_dev(cfg, synth.gen_x(cfg, 1 + i), torch) for i in range(args.batches)]
    # skewed prefill: a Zipf(alpha) log-prior over a seeded permutation of the experts added to
    # every token's logits, so a few experts get several times the average rows
    lb = None
    if args.skew_zipf > 0:
        import dataclasses
        zcfg = dataclasses.replace(cfg, zipf_alpha=args.skew_zipf, zipf_epoch=1)
        lb = torch.from_numpy(synth.zipf_logit_bias(zcfg, 0)).to("cuda")
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup}")
    for i in range(warmup):
        layer.forward(xs[i % len(xs)], logit_bias=lb)
    torch.cuda.synchronize()
    # rows per expert of each batch (real rows only; used for the algorithmic work)
    rows_e = []
    for x in xs:
        rows_e.append(B.route(x, layer.w_router_t, logit_bias=lb, select_bias=layer.select_bias,
                              **layer.route_args())["counts"].cpu().numpy())
    torch.cuda.synchronize()

    log(f"[bench] timing {steps} steps")
    B.profile_enable(True)
    ev0, ev1 = TimingEvent(torch), TimingEvent(torch)
    evs = [(TimingEvent(torch), TimingEvent(torch)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        evs[i][0].record()
        layer.forward(xs[i % len(xs)], logit_bias=lb)
        evs[i][1].record()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = B.profile_read()
    B.profile_enable(False)
    ms_total = ev0.elapsed_time(ev1)
    ms_steps = np.array([a.elapsed_time(b) for a, b in evs])
    destroy_events(evs + [(ev0, ev1)])
    ms_step = ms_total / steps
    tokens_per_s = cfg.T * steps / (ms_total / 1e3)

    d, F, E, T, k = cfg.d, cfg.F, cfg.E, cfg.T, cfg.k
    rows = np.array([rows_e[i % len(xs)].sum() for i in range(steps)], dtype=np.float64)
    gateup_flops = 4.0 * rows * d * F
    down_flops = 2.0 * rows * F * d
    shared_flops = 6.0 * T * d * cfg.F_shared
    router_flops = 2.0 * T * d * E
    layer_flops = float((gateup_flops + down_flops).mean() + shared_flops + router_flops)
    gu_ms, gu_n = prof[B.PROF_GATEUP]
    dn_ms, dn_n = prof[B.PROF_DOWN]
    dtype = cfg.dtype
    peak = PEAK_TFLOPS[dtype]
    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "step_ms_p10_p50_p90": percentiles(ms_steps),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) weights)",
        "config": {"workload": cfg.name, "T": T, "d_model": d, "n_experts": E, "top_k": k, "d_ff": F,
                   "d_ff_shared": cfg.F_shared, "score_fn": cfg.score_fn, "all_experts_resident": True},
    }
    if lb is not None:
        re = np.stack(rows_e)
        result["config"]["zipf_skew_alpha"] = args.skew_zipf
        result["data"] += f"; routing skewed by a Zipf({args.skew_zipf}) log-prior"
        result["rows_per_expert"] = {"max": int(re.max()), "mean": round(float(re.mean()), 1), "min": int(re.min())}
    # a shared expert that runs as one more group of the routed experts' launches is part of
    # those launches' work
    folded = getattr(layer, "shared_in_routed_launch", lambda T: False)(T)
    gu_work = gateup_flops.mean() + (4.0 * T * d * cfg.F_shared if folded else 0.0)
    dn_work = down_flops.mean() + (2.0 * T * d * cfg.F_shared if folded else 0.0)
    if gu_n:
        gu_avg_s = gu_ms / gu_n / 1e3
        achieved = float(gu_work) / gu_avg_s / 1e12
        kname = {"fp8": "ffn_gemm_fp8<gate/up+SwiGLU+requant>", "mxfp4": "ffn_gemm_mx<gate/up+SwiGLU+MXFP8 requant>"}.get(
            dtype, "ffn_gemm_bf16<gate/up+SwiGLU>")
        who = "routed experts and the shared expert" if folded else "routed experts"
        result["roofline"] = {"bound": "mfma", "kernel": kname,
                              "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                              "frac": round(achieved / peak, 4), "traffic": recorded_traffic(cfg.name, kname),
                              "avg_launch_ms": round(gu_ms / gu_n, 4),
                              "work_per_launch": f"4*rows*d*F flops of the {who}, routed rows = T*k = "
                                                 f"{int(rows.mean())}" + (f", shared rows = T = {T}" if folded else "")}
        if dn_n:
            dn_avg_s = dn_ms / dn_n / 1e3
            result["down_gemm"] = {"avg_launch_ms": round(dn_ms / dn_n, 4),
                                   "achieved_tflops": round(float(dn_work) / dn_avg_s / 1e12, 1)}
        sg_ms, sg_n = prof[B.PROF_LABELED + B.PROF_GATEUP]
        sd_ms, sd_n = prof[B.PROF_LABELED + B.PROF_DOWN]
        if sg_n and sd_n:
            result["shared_expert"] = {"gateup_avg_launch_ms": round(sg_ms / sg_n, 4),
                                       "down_avg_launch_ms": round(sd_ms / sd_n, 4),
                                       "note": "side stream, overlapping the routed path"}
    result["layer_tflops"] = round(layer_flops / (ms_step / 1e3) / 1e12, 1)
    result["layer_frac_of_peak"] = round(layer_flops / (ms_step / 1e3) / 1e12 / peak, 4)
    result["host_wall_s"] = round(wall, 3)
    del layer, xs
    torch.cuda.empty_cache()
    if cpu_sample is None and not args.no_cpu_baseline:
        # sized for roughly 10-30 s of oracle work: the fp8 oracle dequantises every touched
        # expert to float64, so its sample is a handful of tokens
        cpu_sample = args.cpu_sample_tokens or {"fp8": 32, "mxfp4": cfg.T}.get(cfg.dtype, 3 * cfg.T)
    if cpu_sample:
        log(f"[bench] cpu baseline: oracle on {cpu_sample} tokens")
        result["cpu_baseline"] = cpu_baseline(cfg, w, cpu_sample)
    return result


def bench_suite(args, torch, B, synth, MoELayer):
    """The headline (DeepSeek-V3-shaped fp8 prefill, the largest workload on one GPU) and every
    other workload in one run; returns the headline dict with a "configs" object."""
    head = bench_prefill(args, torch, B, synth, MoELayer, "dsv3_prefill_fp8",
                         cpu_sample=0 if args.no_cpu_baseline else 32)
    configs = {}
    configs["mixtral_prefill_bf16"] = bench_prefill(args, torch, B, synth, MoELayer, "mixtral_prefill_bf16",
                                                    steps=max(args.steps, 20), warmup=max(args.warmup, 3),
                                                    cpu_sample=0 if args.no_cpu_baseline else 8192)
    for T in (1, 8, 64):
        # eager launches: with the steps queued ahead of the GPU, a graph replay of the same three
        # launches takes about 8 us longer per step on this ROCm stack (measured beside it)
        r = bench_decode(args, torch, B, synth, MoELayer, "qwen_decode_bf16", T=T, steps=200, warmup=10,
                         graph=False, cpu_sample=0 if args.no_cpu_baseline else 256)
        g = bench_decode(args, torch, B, synth, MoELayer, "qwen_decode_bf16", T=T, steps=200, warmup=10, graph=True)
        r["graph_replay"] = {"ms_per_step": g["ms_per_step"], "step_ms_p10_p50_p90": g["step_ms_p10_p50_p90"],
                             "host_ms_per_step": g["host_ms_per_step"]}
        configs[f"qwen_decode_bf16_T{T}"] = r
    configs["offload_decode_bf16"] = bench_offload(args, torch, B, synth, MoELayer,
                                                   modes=("overlapped", "blocking", "device_plan_graph"),
                                                   cpu_sample=0 if args.no_cpu_baseline else 64)
    head["configs"] = configs
    return head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="suite", choices=WORKLOADS,
                    help="suite (default): the DeepSeek-V3-shaped fp8 prefill headline plus every other workload")
    ap.add_argument("--tokens", type=int, default=None, help="override T (decode batch size)")
    ap.add_argument("--batches", type=int, default=4, help="rotating input batches")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="decode: replay the layer as one captured HIP graph")
    ap.add_argument("--resident", action="store_true",
                    help="offload workloads: every expert resident in HBM (the decode bench, weights streamed "
                         "from HBM each step) instead of the slot pool")
    ap.add_argument("--no-fuse-combine", action="store_true",
                    help="decode: run the combine as its own launch instead of inside the down launch")
    ap.add_argument("--separate-calls", action="store_true",
                    help="decode: the separate calls (route_permute, the batched FFN, the combine) instead of "
                         "moe_decode_step")
    ap.add_argument("--skew-zipf", type=float, default=0.0,
                    help="prefill: add a Zipf(alpha) log-prior to the routing logits (0 = unskewed)")
    ap.add_argument("--mall-flush", choices=["read", "write"], default="read",
                    help="decode: evict the last-level cache before each step by reading (default) or writing 512 MiB")
    ap.add_argument("--layers", type=int, default=1,
                    help="offload workloads: a stack of this many layers sharing one slot pool")
    ap.add_argument("--slots", type=int, default=0, help="stack: shared slots (default n_slots per layer x layers)")
    ap.add_argument("--prefetch", default="prev,zipf",
                    help="stack: predictors to run besides none (prev = the layer's previous step, "
                         "zipf = top-N of its routing prior)")
    ap.add_argument("--prefetch-n", type=int, default=16, help="stack: experts the zipf predictor names")
    ap.add_argument("--freq-decay", type=float, default=0.8,
                    help="offload: decay of the routing frequency for the frequency-aware pool modes")
    ap.add_argument("--policies", default="lru,layer,layerfreq,devlayerfreq",
                    help="stack: victim choices to run (lru = plain LRU, layer = the layer that runs furthest "
                         "ahead first, then LRU, layerfreq = the layer order, then decayed routing frequency; "
                         "a dev prefix plans on the device)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only time a plain device-to-device copy of this many MiB (HBM ceiling and the "
                         "reference for the FETCH_SIZE/WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is not sharded across GPUs.",
              file=sys.stderr)
        return 2

    import torch
    from expert_offloaded_ffn_amd import binding as B
    from expert_offloaded_ffn_amd import synth
    from expert_offloaded_ffn_amd.layer import MoELayer

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_probe_bytes": n, "ms_per_copy": round(ms, 4),
                          "hbm_read_plus_write_GBps": round(2 * n / (ms / 1e3) / 1e9, 1)}), flush=True)
        return 0

    if args.workload == "suite":
        result = bench_suite(args, torch, B, synth, MoELayer)
    elif args.workload.startswith("offload_decode") and args.layers > 1:
        return bench_stack(args, torch, B, synth, MoELayer)
    elif args.workload.startswith("offload_decode") and not args.resident:
        result = bench_offload(args, torch, B, synth, MoELayer,
                               cpu_sample=0 if args.no_cpu_baseline else (args.cpu_sample_tokens or 64))
    elif args.workload == "qwen_decode_bf16" or args.workload.startswith("offload_decode"):
        result = bench_decode(args, torch, B, synth, MoELayer,
                              cpu_sample=0 if args.no_cpu_baseline else (args.cpu_sample_tokens or 256))
    else:
        result = bench_prefill(args, torch, B, synth, MoELayer)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
