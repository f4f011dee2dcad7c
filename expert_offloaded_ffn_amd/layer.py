"""One MoE FFN layer on the device: buffers plus the sequence of library calls.

Holds the packed expert bundles (a resident pool with an identity slot table, or
an expert slot pool fed from pinned host bundles), the router weights and the
workspaces, and runs route + permute -> grouped FFN (routed, and the shared expert on a side
stream) -> combine as calls into libmoeffn. No arithmetic of the layer happens here.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import binding as B

W_CODE = {"f32": B.MOE_F32, "bf16": B.MOE_BF16, "fp8": B.MOE_FP8_E4M3, "mxfp4": B.MOE_MXFP4}


def _bits_to_tensor(a: np.ndarray, act: str, device) -> torch.Tensor:
    """Storage-format numpy array -> device tensor (bf16 bits reinterpreted, no rounding)."""
    if act == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def pack_bundles(cfg, expert_weights, d, F, pin=False, threads=8):
    """Packs experts (synth storage tuples) into host bundles; returns a list of uint8 tensors."""
    w = W_CODE[cfg.dtype]
    nb = B.bundle_bytes(d, F, w)

    def one(ws):
        out = torch.empty(nb, dtype=torch.uint8, pin_memory=pin)
        if cfg.dtype == "fp8":
            (gq, gs), (uq, us), (dq, ds) = ws
            return B.pack_expert(d, F, w, gq, uq, dq, gs, us, ds, out=out)
        if cfg.dtype == "mxfp4":   # E8M0 exponents -> the fp32 powers of two the packer takes
            (gq, gs), (uq, us), (dq, ds) = ws
            p2 = lambda e: np.ldexp(np.float32(1.0), e.astype(np.int32) - 127).astype(np.float32)
            return B.pack_expert(d, F, w, gq, uq, dq, p2(gs), p2(us), p2(ds), out=out)
        return B.pack_expert(d, F, w, ws[0], ws[1], ws[2], out=out)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(one, expert_weights))


class ResidentPool:
    """All bundles resident in one device tensor [n, stride] with the identity slot table."""

    def __init__(self, bundles, d, F, w_dtype, device):
        self.n = len(bundles)
        nb = bundles[0].numel()
        self.stride = (nb + 255) // 256 * 256
        self.pool = torch.empty(self.n, self.stride, dtype=torch.uint8, device=device)
        for i, b in enumerate(bundles):
            self.pool[i, :nb].copy_(b, non_blocking=False)
        self.slots = torch.arange(self.n, dtype=torch.int32, device=device)
        self.table = B.expert_table(self.pool, self.stride, self.slots, self.n, d, F, w_dtype)


class SharedSlotPool:
    """One expert slot pool, and one LRU over it, for the layers of a stack: expert e of layer l
    is entry l*E + e of the cache, so the layers compete for the same HBM slots and one layer's
    step can prefetch the next layer's predicted experts (expert_slot_cache_prefetch).
    bundles_per_layer: [L] lists of E pinned host bundles (layers may share bundle tensors).
    layer_order: victims from the layer that runs furthest ahead, then LRU (expert_slot_cache_set_layers);
    else plain LRU. freq_decay: victims by decayed routing frequency before recency (0 = off)."""

    def __init__(self, bundles_per_layer, n_slots, d, F, w_dtype, device="cuda", layer_order=False, freq_decay=0.0,
                 device_plan=False):
        self.L = len(bundles_per_layer)
        self.E = len(bundles_per_layer[0])
        self.d, self.F, self.w_code = d, F, w_dtype
        self.device = torch.device(device)
        flat = [b for layer in bundles_per_layer for b in layer]
        self.bundle_bytes = flat[0].numel()
        self.stride = (self.bundle_bytes + 255) // 256 * 256
        self.slot_pool = torch.empty(n_slots, self.stride, dtype=torch.uint8, device=self.device)
        self.slot_table = torch.full((self.L * self.E,), -1, dtype=torch.int32, device=self.device)
        self.counts = torch.zeros(self.L * self.E, dtype=torch.int32, device=self.device)
        self.cache = self.cache_dev = None
        if device_plan:   # planned on the device: one hit table and one miss table per wave
            self.cache_dev = B.DeviceSlotCache(self.L * self.E, n_slots, self.bundle_bytes, self.stride, flat,
                                               self.slot_pool)
            self.miss_slot_tables = torch.full((self.cache_dev.max_waves, self.L * self.E), -1, dtype=torch.int32,
                                               device=self.device)
            policy = self.cache_dev
        else:
            self.cache = B.SlotCache(self.L * self.E, n_slots, self.bundle_bytes, self.stride, flat, self.slot_pool)
            policy = self.cache
        if layer_order:   # evict from the layer that runs furthest ahead, then LRU
            policy.set_layers(self.L)
        if freq_decay:    # then by decayed routing frequency, then LRU
            policy.set_frequency(freq_decay)

    def table(self, layer: int, slots=None):
        """The expert table of one layer: its E entries of the shared slot table (or of `slots`,
        a per-wave miss table of the device plan)."""
        slots = self.slot_table if slots is None else slots
        view = slots[layer * self.E:(layer + 1) * self.E]
        return B.expert_table(self.slot_pool, self.stride, view, self.E, self.d, self.F, self.w_code)


# Largest decode batch whose combine runs inside the down launch. Each workgroup that finishes
# a unit then waits for its stores and an arrival count before it exits; that pays off only
# while the down launch is about one round of workgroups (1-4 tokens: MI355X, Qwen1.5-MoE
# shape, 0.056 vs 0.058 ms per step at one token, 0.1185 vs 0.1175 ms at eight).
FUSE_COMBINE_MAX_T = 4


class MoELayer:
    def __init__(self, cfg, *, router, experts, shared=None, w_shared_gate=None, select_bias=None, device="cuda",
                 pool_slots=None, blocking=False, threads=8, fuse_combine=True, shared_pool=None, layer_index=0,
                 device_plan=False, freq_decay=0.0, fused_step=True):
        """router: W_r [d, E] storage; experts: list of synth expert tuples; shared: synth tuple or None.
        pool_slots: None = every expert resident; an int = expert slot pool of that many slots.
        shared_pool: a SharedSlotPool this layer's experts live in (entry layer_index*E + e);
        experts is then unused.
        device_plan: with pool_slots, plan residency and copy missed bundles on the device
        (expert_slot_cache_dev): no host synchronisation, and capture() works.
        freq_decay: with pool_slots, victims by decayed routing frequency before recency
        (expert_slot_cache_set_frequency / expert_slot_cache_dev_set_frequency); 0 = plain LRU.
        fuse_combine: a decode step of at most FUSE_COMBINE_MAX_T tokens that runs the shared expert
        in the routed experts' launches combines inside the down launch (moe_grouped_ffn_combine)
        instead of a moe_combine call.
        fused_step: a resident decode step (fused_decode_step) runs as one moe_decode_step call;
        False keeps the separate calls (moe_route_permute, the batched FFN, the combine), which
        give the same bits."""
        self.fuse_combine = fuse_combine
        self.fused_step = fused_step
        self.cfg = cfg
        self.device = torch.device(device)
        self.act = cfg.act_dtype
        self.act_code = W_CODE[self.act]
        self.w_code = W_CODE[cfg.dtype]
        self.E, self.d, self.F, self.k = cfg.E, cfg.d, cfg.F, cfg.k
        self.w_router_t = _bits_to_tensor(np.ascontiguousarray(np.asarray(router).T), self.act, self.device)
        self.w_sg = None if w_shared_gate is None else _bits_to_tensor(w_shared_gate, self.act, self.device)
        self.select_bias = None if select_bias is None else torch.from_numpy(select_bias).to(self.device)
        self.cache = None
        self.cache_dev = None
        self.cache_base = None   # first cache entry of this layer in a shared pool
        if shared_pool is not None:
            self.cache = shared_pool.cache
            self.cache_dev = shared_pool.cache_dev
            self.cache_base = layer_index * self.E
            self.slot_table = shared_pool.slot_table
            self.counts_all = shared_pool.counts
            self.table = shared_pool.table(layer_index)
            self.bundle_bytes = shared_pool.bundle_bytes
            if self.cache_dev is not None:
                self.miss_slot_tables = shared_pool.miss_slot_tables
                self.miss_tables = [shared_pool.table(layer_index, t) for t in shared_pool.miss_slot_tables]
        else:
            bundles = pack_bundles(cfg, experts, self.d, self.F, pin=pool_slots is not None, threads=threads)
            self.bundle_bytes = bundles[0].numel()
        if shared_pool is not None:
            pass   # the stack's pool holds this layer's bundles
        elif pool_slots is None:
            self.pool = ResidentPool(bundles, self.d, self.F, self.w_code, self.device)
            self.table = self.pool.table
        else:
            self.host_bundles = bundles
            stride = (self.bundle_bytes + 255) // 256 * 256
            self.slot_pool = torch.empty(pool_slots, stride, dtype=torch.uint8, device=self.device)
            self.slot_table = torch.full((self.E,), -1, dtype=torch.int32, device=self.device)
            if device_plan:
                self.cache_dev = B.DeviceSlotCache(self.E, pool_slots, self.bundle_bytes, stride, bundles,
                                                   self.slot_pool)
                if freq_decay:
                    self.cache_dev.set_frequency(freq_decay)
                nw = self.cache_dev.max_waves
                self.miss_slot_tables = torch.full((nw, self.E), -1, dtype=torch.int32, device=self.device)
                self.miss_tables = [B.expert_table(self.slot_pool, stride, self.miss_slot_tables[w], self.E, self.d,
                                                   self.F, self.w_code) for w in range(nw)]
            else:
                self.cache = B.SlotCache(self.E, pool_slots, self.bundle_bytes, stride, bundles, self.slot_pool,
                                         blocking=blocking)
                if freq_decay:
                    self.cache.set_frequency(freq_decay)
            self.table = B.expert_table(self.slot_pool, stride, self.slot_table, self.E, self.d, self.F, self.w_code)
        self.shared = None
        if shared is not None:
            Fs = cfg.F_shared
            sb = pack_bundles(cfg, [shared], self.d, Fs, threads=1)
            self.shared = ResidentPool(sb, self.d, Fs, self.w_code, self.device)
        self._ws = {}
        self._side = None

    def _buf(self, name, numel, dtype=torch.uint8):
        t = self._ws.get(name)
        if t is None or t.numel() < numel or t.dtype != dtype:
            t = torch.empty(max(numel, 64), dtype=dtype, device=self.device)
            self._ws[name] = t
        return t[:max(numel, 1)] if numel else t[:1]

    def _zbuf(self, name, numel):
        """A device byte buffer zero-filled when (re)allocated: moe_decode_step's workspace, whose
        arrival counters must be zero before its first call and are left zero by every call."""
        t = self._ws.get(name)
        if t is None or t.numel() < numel:
            t = torch.zeros(max(numel, 256), dtype=torch.uint8, device=self.device)
            self._ws[name] = t
        return t

    def _shared_offsets(self, T):
        """Device [0, T] offsets of the single shared-expert group (cached per T)."""
        key = ("shared_offsets", T)
        t = self._ws.get(key)
        if t is None:
            t = torch.tensor([0, T], dtype=torch.int32).to(self.device)
            self._ws[key] = t
        return t

    def route_args(self):
        c = self.cfg
        return dict(k=c.k, score_fn=B.MOE_SIGMOID if c.score_fn == "sigmoid" else B.MOE_SOFTMAX,
                    renormalize=c.renormalize, route_scale=c.route_scale, n_groups=c.n_groups,
                    topk_groups=c.topk_groups, group_topn=c.group_topn)

    def _side_stream(self):
        """The stream the shared expert runs on (default priority, created once)."""
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
        return self._side

    def shared_in_decode_launch(self, T: int) -> bool:
        """Whether a T-token forward runs the shared expert inside the routed experts' decode
        launches (bf16 or MXFP4, every expert resident, at most 64 rows per expert) instead of on a
        side stream. A slot pool (host- or device-planned) runs its routed experts in waves through
        the pool's tables, so its shared expert always takes the side stream."""
        return (self.shared is not None and self.cache is None and self.cache_dev is None
                and self.w_code in (B.MOE_BF16, B.MOE_MXFP4) and 0 < T <= 64)

    def fused_decode_step(self, T: int) -> bool:
        """Whether a T-token forward is one moe_decode_step call: every expert resident, bf16
        activations, bf16 or MXFP4 weights, 1..64 tokens, at most 256 experts."""
        return (self.fused_step and self.cache is None and self.cache_dev is None and self.act == "bf16"
                and self.w_code in (B.MOE_BF16, B.MOE_MXFP4) and 0 < T <= 64 and self.E <= 256 and self.d % 32 == 0)

    def mx_prefill(self, T: int) -> bool:
        """Whether a T-token forward runs MXFP4 experts on the block-scaled MFMA (more than 64
        tokens: activations and hidden activations in MXFP8) rather than on the decode kernels
        (bf16 activations)."""
        return self.w_code == B.MOE_MXFP4 and T > 64

    def shared_in_routed_launch(self, T: int) -> bool:
        """Whether a T-token forward runs the shared expert as one more group of the routed
        experts' prefill GEMM launches (fp8 weights, or MXFP4 weights past the decode sizes; every
        expert resident): one tile list for both, so neither GEMM competes with the other from a
        second stream."""
        return (self.shared is not None and self.cache is None and self.cache_dev is None and T > 0
                and (self.w_code == B.MOE_FP8_E4M3 or self.mx_prefill(T)))

    def _shared_ffn(self, T, a, a_scale, a_code, ydt, main):
        """Launches the shared expert's FFN on the side stream once `a` is ready on `main`; the
        caller joins the side stream back before the combine."""
        offs = self._shared_offsets(T)
        shared_y = torch.empty(T, self.d, device=self.device, dtype=torch.float32 if ydt == B.MOE_F32 else torch.bfloat16)
        sws = self._buf("shared_ws", B.grouped_ffn_workspace_size(self.shared.table, T, a_code))
        side = self._side_stream()
        side.wait_stream(main)
        B.profile_label(1)   # timed apart from the routed experts when profiling is on
        try:
            B.grouped_ffn(self.shared.table, T, offs, a, a_scale=a_scale, act_dtype=a_code, y=shared_y, y_dtype=ydt,
                          ws=sws, stream=side)
        finally:
            B.profile_label(0)
        return shared_y

    def forward(self, x: torch.Tensor, logit_bias: torch.Tensor | None = None, stream=None, prefetch=None) -> dict:
        """x [T, d] device tensor in the activation dtype. Returns the layer output and routing tensors.
        prefetch (slot pool only): cache entries predicted for a later step, handed to
        expert_slot_cache_prefetch once this step's waves are issued.
        The shared expert (when there is one) runs inside the routed experts' launches for a
        decode step (shared_in_decode_launch), else on a second stream, forked once the routing
        is issued, concurrently with the routed experts, and joined before the combine."""
        T = x.shape[0]
        k, E, d = self.k, self.E, self.d
        if prefetch is not None and self.cache is None:
            raise ValueError("prefetch= needs the host-planned slot pool (expert_slot_cache_prefetch); this layer "
                             "is resident or planned on the device")
        main = torch.cuda.current_stream(self.device) if stream is None else stream
        ydt = B.MOE_F32 if self.act == "f32" else B.MOE_BF16
        if self.fused_decode_step(T):
            # routing beside the shared expert's gate/up, its down beside the routed gate/up, then
            # the routed down with the combine: three launches (four past 4 tokens)
            shared_table = self.shared.table if self.shared is not None else None
            ws = self._zbuf("step_ws", B.decode_step_workspace_size(T, self.d, E, k, self.table, shared_table))
            r = B.decode_step(x, self.w_router_t, self.table, shared_table, logit_bias=logit_bias,
                              select_bias=self.select_bias, w_shared_gate=self.w_sg, out_dtype=ydt, ws=ws,
                              stream=main, **self.route_args())
            return {"out": r["out"], "route": r, "perm": r, "y": None, "shared_y": None, "waves": 0}
        shared_y = None
        merged = self.shared_in_decode_launch(T)
        ws = self._buf("perm_ws", B.route_permute_workspace_size(T, k, E, d))
        rows = T * k
        y = torch.empty(rows, d, device=self.device, dtype=torch.float32 if ydt == B.MOE_F32 else torch.bfloat16)
        a, a_scale, a_code = x, None, self.act_code
        if self.w_code == B.MOE_FP8_E4M3 or self.mx_prefill(T):
            qcode = B.MOE_FP8_E4M3 if self.w_code == B.MOE_FP8_E4M3 else B.MOE_MXFP8
            r = B.route(x, self.w_router_t, logit_bias=logit_bias, select_bias=self.select_bias,
                        w_shared_gate=self.w_sg, stream=main, **self.route_args())
            # grouping plus one quantisation of every token (token order: e4m3 per 128 for fp8
            # weights, MXFP8 for MXFP4 weights); the GEMMs gather rows through perm_src
            p = B.permute(r["idx"], E, x=x, out_dtype=qcode, gather=0, ws=ws, stream=main)
            a, a_scale, a_code = p["x_out"], p["x_out_scale"], qcode
            if self.shared is not None and not self.shared_in_routed_launch(T):
                shared_y = self._shared_ffn(T, a, a_scale, a_code, ydt, main)
        else:
            # routing and grouping in one call; the routed chain is the critical path, so it
            # is issued first and the shared expert forks off behind it
            r = p = B.route_permute(x, self.w_router_t, logit_bias=logit_bias, select_bias=self.select_bias,
                                    w_shared_gate=self.w_sg, ws=ws, stream=main, **self.route_args())
            if self.shared is not None and not merged:
                shared_y = self._shared_ffn(T, x, None, self.act_code, ydt, main)
        if self.shared_in_routed_launch(T):
            # the routed experts and the shared expert (a group of its own, every token) share
            # one launch per GEMM
            shared_y = torch.empty(T, d, device=self.device, dtype=y.dtype)
            probs = [B.ffn_problem(self.table, rows, p["offsets"], a, a_scale=a_scale, act_dtype=a_code,
                                   a_row_src=p["perm_src"], a_row_div=k, y=y, y_dtype=ydt),
                     B.ffn_problem(self.shared.table, T, self._shared_offsets(T), a, a_scale=a_scale,
                                   act_dtype=a_code, y=shared_y, y_dtype=ydt)]
            bws = self._buf("batch_ws", B.grouped_ffn_batch_workspace_size(probs))
            B.grouped_ffn_batch(probs, ws=bws, stream=main)
            out = B.combine(y, p["perm_dst"], r["gate"], shared_y=shared_y, shared_gate=r["shared_gate"],
                            stream=main)
            return {"out": out, "route": r, "perm": p, "y": y, "shared_y": shared_y, "waves": 0}
        if merged:
            # a decode step: the shared expert's blocks (dispatched first, they carry the longer
            # rows of its down projection) and the routed experts' share one launch per GEMM
            shared_y = torch.empty(T, d, device=self.device, dtype=y.dtype)
            probs = [B.ffn_problem(self.shared.table, T, self._shared_offsets(T), x, act_dtype=self.act_code,
                                   y=shared_y, y_dtype=ydt),
                     B.ffn_problem(self.table, rows, p["offsets"], a, act_dtype=a_code, a_row_src=p["perm_src"],
                                   a_row_div=k, y=y, y_dtype=ydt)]
            if self.fuse_combine and T <= FUSE_COMBINE_MAX_T:
                # the down launch also combines: y and shared_y stay in the call's workspace
                cws = self._buf("comb_ws", B.grouped_ffn_combine_workspace_size(probs[1], probs[0]))
                out = B.grouped_ffn_combine(probs[1], probs[0], p["perm_dst"], r["gate"],
                                            shared_gate=r["shared_gate"], out_dtype=ydt, ws=cws, stream=main)
                return {"out": out, "route": r, "perm": p, "y": None, "shared_y": None, "waves": 0}
            bws = self._buf("batch_ws", B.grouped_ffn_batch_workspace_size(probs))
            B.grouped_ffn_batch(probs, ws=bws, stream=main)
            waves = 0
        elif self.cache_dev is not None:
            # plan on the device; the hits run while the misses' copy kernel reads host memory
            fws = self._buf("ffn_ws", B.grouped_ffn_workspace_size(self.table, rows, a_code))
            counts = r["counts"]
            if self.cache_base is not None:   # this layer's histogram into the stack-wide one
                self.counts_all.zero_()
                self.counts_all[self.cache_base:self.cache_base + E].copy_(counts)
                counts = self.counts_all
            self.cache_dev.step(counts, self.slot_table, self.miss_slot_tables, stream=main)
            ffn = lambda table: B.grouped_ffn(table, rows, p["offsets"], a, a_scale=a_scale, act_dtype=a_code,
                                              a_row_src=p["perm_src"], a_row_div=k, y=y, y_dtype=ydt, ws=fws,
                                              stream=main)
            for w, miss_table in enumerate(self.miss_tables):
                self.cache_dev.copy(w, stream=main)
                if w == 0:
                    ffn(self.table)
                self.cache_dev.join(w, stream=main)
                ffn(miss_table)
            waves = len(self.miss_tables)
        elif self.cache is None:
            fws = self._buf("ffn_ws", B.grouped_ffn_workspace_size(self.table, rows, a_code))
            B.grouped_ffn(self.table, rows, p["offsets"], a, a_scale=a_scale, act_dtype=a_code,
                          a_row_src=p["perm_src"], a_row_div=k, y=y, y_dtype=ydt, ws=fws, stream=main)
            waves = 0
        else:
            fws = self._buf("ffn_ws", B.grouped_ffn_workspace_size(self.table, rows, a_code))
            counts = r["counts"]
            if self.cache_base is not None:   # this layer's histogram into the stack-wide one
                self.counts_all.zero_()
                self.counts_all[self.cache_base:self.cache_base + E].copy_(counts)
                counts = self.counts_all
            waves = self.cache.acquire(counts, stream=main)
            for w in range(waves):
                for part in (0, 1):
                    n = self.cache.wave(w, part, self.slot_table, stream=main)
                    if n:
                        B.grouped_ffn(self.table, rows, p["offsets"], a, a_scale=a_scale, act_dtype=a_code,
                                      a_row_src=p["perm_src"], a_row_div=k, y=y, y_dtype=ydt, ws=fws, stream=main)
                self.cache.release(w, stream=main)
            if prefetch is not None:
                self.cache.prefetch(prefetch)
        if shared_y is not None and not merged:
            main.wait_stream(self._side_stream())
        out = B.combine(y, p["perm_dst"], r["gate"], shared_y=shared_y, shared_gate=r["shared_gate"], stream=main)
        return {"out": out, "route": r, "perm": p, "y": y, "shared_y": shared_y, "waves": waves}

    def capture(self, x_static: torch.Tensor, logit_bias_static: torch.Tensor | None = None):
        """Records forward() for fixed input buffers as one HIP graph (resident layers, or a slot
        pool planned on the device; the host-planned pool synchronises with the host every step).
        Returns (graph, outputs); refill x_static (and logit_bias_static) in place, then
        graph.replay() recomputes outputs. The warm-up runs before capture are real steps: a
        device-planned pool's residency and counters include them."""
        if self.cache is not None:
            raise RuntimeError("capture() needs a resident layer or device_plan=True; the host-planned slot pool "
                               "synchronises with the host each step")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                self.forward(x_static, logit_bias_static)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            outputs = self.forward(x_static, logit_bias_static)
        return graph, outputs
