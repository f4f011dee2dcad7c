"""ctypes binding of libmoeffn (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch tensors supply device memory, pinned host memory and streams.
The library is loaded on first use and a missing or stale build is an error:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoeffn.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8 = 0, 1, 2, 3, 4
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ECAPACITY, MOE_ENOMEM, MOE_ESTATE = 0, -1, -2, -3, -4, -5, -6
STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EHIP", -4: "MOE_ECAPACITY",
          -5: "MOE_ENOMEM", -6: "MOE_ESTATE"}

DTYPE_CODE = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_FP8_E4M3,
              torch.float8_e4m3fn: MOE_FP8_E4M3}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class RouteCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("score_fn", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("group_topn", ctypes.c_int32), ("act_dtype", ctypes.c_int32)]


class ExpertTable(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("slot_stride", ctypes.c_int64), ("slot_of_expert", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32)]


class FfnProblem(ctypes.Structure):
    _fields_ = [("table", ctypes.POINTER(ExpertTable)), ("rows", ctypes.c_int32), ("offsets", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("a_scale", ctypes.c_void_p), ("act_dtype", ctypes.c_int32),
                ("a_row_src", ctypes.c_void_p), ("a_row_div", ctypes.c_int32), ("y", ctypes.c_void_p),
                ("y_dtype", ctypes.c_int32)]


class CombineArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("k", ctypes.c_int32), ("perm_dst", ctypes.c_void_p),
                ("topk_gate", ctypes.c_void_p), ("shared_gate", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32)]


class DecodeOut(ctypes.Structure):
    _fields_ = [("shared_gate", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk_gate", ctypes.c_void_p), ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm_src", ctypes.c_void_p), ("perm_dst", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32)]


class CacheCfg(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("bundle_bytes", ctypes.c_int64),
                ("slot_stride", ctypes.c_int64), ("bundles_host", ctypes.c_void_p), ("pool", ctypes.c_void_p),
                ("blocking", ctypes.c_int32), ("dry_run", ctypes.c_int32)]


class CacheStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("evictions", ctypes.c_int64), ("waves", ctypes.c_int64), ("h2d_bytes", ctypes.c_int64),
                ("d2h_bytes", ctypes.c_int64), ("copy_ms", ctypes.c_double), ("prefetches", ctypes.c_int64),
                ("prefetch_used", ctypes.c_int64), ("wait_ms", ctypes.c_double)]


class Profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 8), ("launches", ctypes.c_int64 * 8)]


class CacheEntry(ctypes.Structure):
    _fields_ = [("expert", ctypes.c_int32), ("slot", ctypes.c_int32), ("hit", ctypes.c_int32),
                ("evicted", ctypes.c_int32)]


EXPORTS = {
    # name: (restype, argtypes)
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_route": (ctypes.c_int32, [ctypes.POINTER(RouteCfg)] + [ctypes.c_void_p] * 11),
    "moe_route_permute": (ctypes.c_int32, [ctypes.POINTER(RouteCfg)] + [ctypes.c_void_p] * 14 +
                          [ctypes.c_size_t, ctypes.c_void_p]),
    "moe_route_permute_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 4),
    "moe_permute_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "moe_permute": (ctypes.c_int32, [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p,
                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_bundle_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "moe_pack_expert": (ctypes.c_int32, [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 7),
    "moe_grouped_ffn_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(ExpertTable), ctypes.c_int32, ctypes.c_int32]),
    "moe_grouped_ffn": (ctypes.c_int32, [ctypes.POINTER(ExpertTable), ctypes.c_int32, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_grouped_ffn_batch_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FfnProblem), ctypes.c_int32]),
    "moe_grouped_ffn_batch": (ctypes.c_int32, [ctypes.POINTER(FfnProblem), ctypes.c_int32, ctypes.c_void_p,
                              ctypes.c_size_t, ctypes.c_void_p]),
    "moe_combine": (ctypes.c_int32, [ctypes.c_int32] * 3 + [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                    ctypes.c_void_p]),
    "moe_grouped_ffn_combine_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(FfnProblem),
                                               ctypes.POINTER(FfnProblem)]),
    "moe_grouped_ffn_combine": (ctypes.c_int32, [ctypes.POINTER(FfnProblem), ctypes.POINTER(FfnProblem),
                                ctypes.POINTER(CombineArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_grouped_ffn_combine_noalloc": (ctypes.c_int32, [ctypes.POINTER(FfnProblem), ctypes.POINTER(FfnProblem),
                                        ctypes.POINTER(CombineArgs), ctypes.c_void_p]),
    "moe_decode_step_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(RouteCfg), ctypes.POINTER(ExpertTable),
                                       ctypes.POINTER(ExpertTable)]),
    "moe_decode_step": (ctypes.c_int32, [ctypes.POINTER(RouteCfg)] + [ctypes.c_void_p] * 5 +
                        [ctypes.POINTER(ExpertTable), ctypes.POINTER(ExpertTable), ctypes.POINTER(DecodeOut),
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "expert_slot_cache_create": (ctypes.c_int32, [ctypes.POINTER(CacheCfg), ctypes.POINTER(ctypes.c_void_p)]),
    "expert_slot_cache_destroy": (ctypes.c_int32, [ctypes.c_void_p]),
    "expert_slot_cache_reset": (ctypes.c_int32, [ctypes.c_void_p]),
    "expert_slot_cache_acquire": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_int32)]),
    "expert_slot_cache_plan_host": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    "expert_slot_cache_wave": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
    "expert_slot_cache_release": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "expert_slot_cache_set_layers": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32]),
    "expert_slot_cache_set_frequency": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_double]),
    "expert_slot_cache_prefetch": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32)]),
    "expert_slot_cache_wave_plan": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(CacheEntry),
                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "expert_slot_cache_stats": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(CacheStats)]),
    "expert_slot_cache_dev_create": (ctypes.c_int32, [ctypes.POINTER(CacheCfg), ctypes.POINTER(ctypes.c_void_p)]),
    "expert_slot_cache_dev_destroy": (ctypes.c_int32, [ctypes.c_void_p]),
    "expert_slot_cache_dev_reset": (ctypes.c_int32, [ctypes.c_void_p]),
    "expert_slot_cache_dev_max_waves": (ctypes.c_int32, [ctypes.c_void_p]),
    "expert_slot_cache_dev_set_frequency": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_double]),
    "expert_slot_cache_dev_set_layers": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32]),
    "expert_slot_cache_dev_step": (ctypes.c_int32, [ctypes.c_void_p] * 5),
    "expert_slot_cache_dev_copy": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "expert_slot_cache_dev_join": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "expert_slot_cache_dev_stats": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(CacheStats)]),
    "moe_profile_enable": (ctypes.c_int32, [ctypes.c_int32]),
    "moe_profile_label": (ctypes.c_int32, [ctypes.c_int32]),
    "moe_profile_read": (ctypes.c_int32, [ctypes.POINTER(Profile)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m expert_offloaded_ffn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def stream_ptr(stream=None) -> int | None:
    """The hipStream_t of `stream` (default: torch's current stream); None without a device."""
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# --------------------------------------------------------------- calls ---

def route(x, w_router_t, *, k, score_fn=MOE_SOFTMAX, renormalize=1, route_scale=1.0, n_groups=1, topk_groups=1,
          group_topn=0, logit_bias=None, select_bias=None, w_shared_gate=None, out=None, stream=None):
    """moe_route. x [T, d]; w_router_t [E, d] (row e = expert e). Returns dict of device tensors."""
    T, d = x.shape
    E = w_router_t.shape[0]
    dev = x.device
    o = out or {}
    scores = o.get("scores") if o.get("scores") is not None else torch.empty(T, E, device=dev, dtype=torch.float32)
    idx = o.get("idx") if o.get("idx") is not None else torch.empty(T, k, device=dev, dtype=torch.int32)
    gate = o.get("gate") if o.get("gate") is not None else torch.empty(T, k, device=dev, dtype=torch.float32)
    counts = o.get("counts") if o.get("counts") is not None else torch.empty(E, device=dev, dtype=torch.int32)
    sg = None
    if w_shared_gate is not None:
        sg = o.get("shared_gate") if o.get("shared_gate") is not None else torch.empty(T, device=dev, dtype=torch.float32)
    cfg = RouteCfg(T, d, E, k, score_fn, renormalize, route_scale, n_groups, topk_groups, group_topn,
                   DTYPE_CODE[x.dtype])
    _check(lib().moe_route(ctypes.byref(cfg), ptr(x), ptr(w_router_t), ptr(logit_bias), ptr(select_bias),
                           ptr(w_shared_gate), ptr(sg), ptr(scores), ptr(idx), ptr(gate), ptr(counts),
                           stream_ptr(stream)))
    return {"scores": scores, "idx": idx, "gate": gate, "counts": counts, "shared_gate": sg}


def permute_workspace_size(T, k, E) -> int:
    return int(lib().moe_permute_workspace_size(T, k, E))


def permute(idx, E, *, x=None, out_dtype=None, gather=1, ws=None, out=None, stream=None):
    """moe_permute. Returns dict(offsets, perm_src, perm_dst, x_out, x_out_scale)."""
    T, k = idx.shape
    dev = idx.device
    o = out or {}
    offsets = o.get("offsets") if o.get("offsets") is not None else torch.empty(E + 1, device=dev, dtype=torch.int32)
    src = o.get("perm_src") if o.get("perm_src") is not None else torch.empty(T * k, device=dev, dtype=torch.int32)
    dst = o.get("perm_dst") if o.get("perm_dst") is not None else torch.empty(T * k, device=dev, dtype=torch.int32)
    if ws is None:
        ws = torch.empty(max(permute_workspace_size(T, k, E), 256), device=dev, dtype=torch.uint8)
    x_out = xs = None
    d = 0
    xdt = odt = 0
    if x is not None:
        d = x.shape[1]
        xdt = DTYPE_CODE[x.dtype]
        odt = xdt if out_dtype is None else out_dtype
        rows = T * k if gather else T
        x_out = o.get("x_out")
        if x_out is None:
            x_out = torch.empty(rows, d, device=dev,
                                dtype=torch.uint8 if odt in (MOE_FP8_E4M3, MOE_MXFP8) else x.dtype)
        if odt == MOE_FP8_E4M3:
            xs = o.get("x_out_scale")
            if xs is None:
                xs = torch.empty(rows, d // 128, device=dev, dtype=torch.float32)
        elif odt == MOE_MXFP8:   # the E8M0 bytes, one per 32 values
            xs = o.get("x_out_scale")
            if xs is None:
                xs = torch.empty(rows, d // 32, device=dev, dtype=torch.uint8)
    _check(lib().moe_permute(T, k, E, ptr(idx), ptr(offsets), ptr(src), ptr(dst), d, ptr(x), xdt, ptr(x_out), odt,
                             ptr(xs), int(gather), ptr(ws), ws.numel(), stream_ptr(stream)))
    return {"offsets": offsets, "perm_src": src, "perm_dst": dst, "x_out": x_out, "x_out_scale": xs}


def route_permute_workspace_size(T, k, E, d) -> int:
    return int(lib().moe_route_permute_workspace_size(T, k, E, d))


def route_permute(x, w_router_t, *, k, score_fn=MOE_SOFTMAX, renormalize=1, route_scale=1.0, n_groups=1,
                  topk_groups=1, group_topn=0, logit_bias=None, select_bias=None, w_shared_gate=None, ws=None,
                  out=None, stream=None):
    """moe_route_permute. Returns the dicts of route() and permute() (without x_out) merged."""
    T, d = x.shape
    E = w_router_t.shape[0]
    dev = x.device
    o = out or {}

    def get(name, shape, dtype):
        t = o.get(name)
        return t if t is not None else torch.empty(*shape, device=dev, dtype=dtype)

    scores = get("scores", (T, E), torch.float32)
    idx = get("idx", (T, k), torch.int32)
    gate = get("gate", (T, k), torch.float32)
    counts = get("counts", (E,), torch.int32)
    sg = get("shared_gate", (T,), torch.float32) if w_shared_gate is not None else None
    offsets = get("offsets", (E + 1,), torch.int32)
    src = get("perm_src", (T * k,), torch.int32)
    dst = get("perm_dst", (T * k,), torch.int32)
    if ws is None:
        ws = torch.empty(max(route_permute_workspace_size(T, k, E, d), 256), device=dev, dtype=torch.uint8)
    cfg = RouteCfg(T, d, E, k, score_fn, renormalize, route_scale, n_groups, topk_groups, group_topn,
                   DTYPE_CODE[x.dtype])
    _check(lib().moe_route_permute(ctypes.byref(cfg), ptr(x), ptr(w_router_t), ptr(logit_bias), ptr(select_bias),
                                   ptr(w_shared_gate), ptr(sg), ptr(scores), ptr(idx), ptr(gate), ptr(counts),
                                   ptr(offsets), ptr(src), ptr(dst), ptr(ws), ws.numel(), stream_ptr(stream)))
    return {"scores": scores, "idx": idx, "gate": gate, "counts": counts, "shared_gate": sg,
            "offsets": offsets, "perm_src": src, "perm_dst": dst, "x_out": None, "x_out_scale": None}


def bundle_bytes(d, F, w_dtype) -> int:
    return int(lib().moe_bundle_bytes(d, F, w_dtype))


def pack_expert(d, F, w_dtype, wg, wu, wd, sg=None, su=None, sd=None, out=None):
    """Packs one expert (numpy arrays in storage format: f32, bf16 bits as uint16, e4m3 codes as uint8,
    FP4 codes as one uint8 each; fp8 block scales or MXFP4 power-of-two scales as fp32 grids) into a
    host bundle (a uint8 tensor, pinned if `out` is pinned)."""
    import numpy as np

    nb = bundle_bytes(d, F, w_dtype)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8)
    arrs = [np.ascontiguousarray(a) for a in (wg, wu, wd)]
    sc = [None if s is None else np.ascontiguousarray(s, dtype=np.float32) for s in (sg, su, sd)]
    p = lambda a: None if a is None else a.ctypes.data
    _check(lib().moe_pack_expert(d, F, w_dtype, p(arrs[0]), p(arrs[1]), p(arrs[2]), p(sc[0]), p(sc[1]), p(sc[2]),
                                 out.data_ptr()))
    return out


def expert_table(pool, slot_stride, slot_of_expert, n_experts, d, F, w_dtype) -> ExpertTable:
    return ExpertTable(ptr(pool), int(slot_stride), ptr(slot_of_expert), n_experts, d, F, w_dtype)


def grouped_ffn_workspace_size(table: ExpertTable, rows, act_dtype) -> int:
    return int(lib().moe_grouped_ffn_workspace_size(ctypes.byref(table), rows, act_dtype))


def grouped_ffn(table: ExpertTable, rows, offsets, a, *, a_scale=None, act_dtype=None, a_row_src=None, a_row_div=1,
                y=None, y_dtype=MOE_BF16, ws=None, stream=None):
    act = DTYPE_CODE[a.dtype] if act_dtype is None else act_dtype
    if y is None:
        y = torch.empty(rows, table.d_model, device=a.device,
                        dtype=torch.bfloat16 if y_dtype == MOE_BF16 else torch.float32)
    if ws is None:
        ws = torch.empty(max(grouped_ffn_workspace_size(table, rows, act), 256), device=a.device, dtype=torch.uint8)
    _check(lib().moe_grouped_ffn(ctypes.byref(table), rows, ptr(offsets), ptr(a), ptr(a_scale), act, ptr(a_row_src),
                                 int(a_row_div), ptr(y), y_dtype, ptr(ws), ws.numel(), stream_ptr(stream)))
    return y


def ffn_problem(table: ExpertTable, rows, offsets, a, *, a_scale=None, act_dtype=None, a_row_src=None, a_row_div=1,
                y=None, y_dtype=MOE_BF16) -> FfnProblem:
    """The fields of one moe_grouped_ffn call; `y` is allocated when not given (read it back as .y_tensor)."""
    act = DTYPE_CODE[a.dtype] if act_dtype is None else act_dtype
    if y is None:
        y = torch.empty(rows, table.d_model, device=a.device,
                        dtype=torch.bfloat16 if y_dtype == MOE_BF16 else torch.float32)
    pr = FfnProblem(ctypes.pointer(table), rows, ptr(offsets), ptr(a), ptr(a_scale), act, ptr(a_row_src),
                    int(a_row_div), ptr(y), y_dtype)
    pr.y_tensor = y
    pr.keep = (table, offsets, a, a_scale, a_row_src)   # the tensors stay alive with the struct
    return pr


def grouped_ffn_batch_workspace_size(problems) -> int:
    arr = (FfnProblem * len(problems))(*problems)
    return int(lib().moe_grouped_ffn_batch_workspace_size(arr, len(problems)))


def grouped_ffn_batch(problems, *, ws=None, stream=None):
    """moe_grouped_ffn_batch over 1 or 2 FfnProblem structs (see ffn_problem). Returns their y tensors."""
    arr = (FfnProblem * len(problems))(*problems)
    dev = problems[0].y_tensor.device
    if ws is None:
        ws = torch.empty(max(grouped_ffn_batch_workspace_size(problems), 256), device=dev, dtype=torch.uint8)
    _check(lib().moe_grouped_ffn_batch(arr, len(problems), ptr(ws), ws.numel(), stream_ptr(stream)))
    return [pr.y_tensor for pr in problems]


def combine(y, perm_dst, gate, *, shared_y=None, shared_gate=None, out=None, out_dtype=None, stream=None):
    T, k = gate.shape
    d = y.shape[1]
    ydt = DTYPE_CODE[y.dtype]
    odt = ydt if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(T, d, device=y.device, dtype=torch.bfloat16 if odt == MOE_BF16 else torch.float32)
    _check(lib().moe_combine(T, k, d, ptr(y), ydt, ptr(perm_dst), ptr(gate), ptr(shared_y), ptr(shared_gate),
                             ptr(out), odt, stream_ptr(stream)))
    return out


def grouped_ffn_combine_workspace_size(routed: FfnProblem, shared: FfnProblem | None = None) -> int:
    return int(lib().moe_grouped_ffn_combine_workspace_size(ctypes.byref(routed),
                                                             ctypes.byref(shared) if shared is not None else None))


def grouped_ffn_combine(routed: FfnProblem, shared, perm_dst, gate, *, shared_gate=None, out=None, out_dtype=MOE_BF16,
                        ws=None, stream=None):
    """moe_grouped_ffn_combine: the decode FFN of the routed (and shared) problem with the combine
    folded into its down launch. Returns out [T, d]."""
    T, k = gate.shape
    d = routed.table.contents.d_model
    dev = gate.device
    if out is None:
        out = torch.empty(T, d, device=dev, dtype=torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32)
    if ws is None:
        ws = torch.empty(max(grouped_ffn_combine_workspace_size(routed, shared), 256), device=dev, dtype=torch.uint8)
    cb = CombineArgs(T, k, ptr(perm_dst), ptr(gate), ptr(shared_gate), ptr(out), out_dtype)
    _check(lib().moe_grouped_ffn_combine(ctypes.byref(routed), ctypes.byref(shared) if shared is not None else None,
                                         ctypes.byref(cb), ptr(ws), ws.numel(), stream_ptr(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def grouped_ffn_combine_noalloc(routed: FfnProblem, shared, perm_dst, gate, out, *, shared_gate=None,
                                out_dtype=MOE_BF16, stream=None):
    """moe_grouped_ffn_combine_noalloc: as grouped_ffn_combine, with the workspace in the library's
    per-device static scratch array; `out` [T, d] is the caller's. Returns out."""
    T, k = gate.shape
    cb = CombineArgs(T, k, ptr(perm_dst), ptr(gate), ptr(shared_gate), ptr(out), out_dtype)
    _check(lib().moe_grouped_ffn_combine_noalloc(ctypes.byref(routed),
                                                 ctypes.byref(shared) if shared is not None else None,
                                                 ctypes.byref(cb), stream_ptr(stream)))
    return out


def decode_step_workspace_size(T, d, E, k, routed: ExpertTable, shared=None) -> int:
    cfg = RouteCfg(T, d, E, k, MOE_SOFTMAX, 1, 1.0, 1, 1, 0, MOE_BF16)
    return int(lib().moe_decode_step_workspace_size(ctypes.byref(cfg), ctypes.byref(routed),
                                                    ctypes.byref(shared) if shared is not None else None))


def decode_step(x, w_router_t, routed: ExpertTable, shared=None, *, k, score_fn=MOE_SOFTMAX, renormalize=1,
                route_scale=1.0, n_groups=1, topk_groups=1, group_topn=0, logit_bias=None, select_bias=None,
                w_shared_gate=None, out_dtype=MOE_BF16, ws=None, out=None, stream=None):
    """moe_decode_step: routing, the routed and shared experts' FFN and the combine of one decode
    step. `ws` must have been zero-filled before its first use (the call leaves its counters at
    zero); a new one is allocated zero-filled when None. Returns route_permute()'s dict plus "out"."""
    T, d = x.shape
    E = w_router_t.shape[0]
    dev = x.device
    o = out or {}

    def get(name, shape, dtype):
        t = o.get(name)
        return t if t is not None else torch.empty(*shape, device=dev, dtype=dtype)

    res = {"scores": get("scores", (T, E), torch.float32), "idx": get("idx", (T, k), torch.int32),
           "gate": get("gate", (T, k), torch.float32), "counts": get("counts", (E,), torch.int32),
           "shared_gate": get("shared_gate", (T,), torch.float32) if w_shared_gate is not None else None,
           "offsets": get("offsets", (E + 1,), torch.int32), "perm_src": get("perm_src", (T * k,), torch.int32),
           "perm_dst": get("perm_dst", (T * k,), torch.int32),
           "out": get("out", (T, d), torch.bfloat16 if out_dtype == MOE_BF16 else torch.float32)}
    cfg = RouteCfg(T, d, E, k, score_fn, renormalize, route_scale, n_groups, topk_groups, group_topn,
                   DTYPE_CODE[x.dtype])
    if ws is None:
        need = lib().moe_decode_step_workspace_size(ctypes.byref(cfg), ctypes.byref(routed),
                                                    ctypes.byref(shared) if shared is not None else None)
        ws = torch.zeros(max(int(need), 256), device=dev, dtype=torch.uint8)
    do = DecodeOut(ptr(res["shared_gate"]), ptr(res["scores"]), ptr(res["idx"]), ptr(res["gate"]), ptr(res["counts"]),
                   ptr(res["offsets"]), ptr(res["perm_src"]), ptr(res["perm_dst"]), ptr(res["out"]), out_dtype)
    _check(lib().moe_decode_step(ctypes.byref(cfg), ptr(x), ptr(w_router_t), ptr(logit_bias), ptr(select_bias),
                                 ptr(w_shared_gate), ctypes.byref(routed),
                                 ctypes.byref(shared) if shared is not None else None, ctypes.byref(do), ptr(ws),
                                 ws.numel(), stream_ptr(stream)))
    res.update(x_out=None, x_out_scale=None)
    return res


# ---------------------------------------------------------- slot cache ---

class SlotCache:
    """expert_slot_cache over a caller pool tensor and pinned host bundles."""

    def __init__(self, n_experts, n_slots, bundle_bytes_, slot_stride, bundles_host=None, pool=None, blocking=False,
                 dry_run=False):
        self._keep = bundles_host
        arr = None
        if bundles_host is not None:
            arr = (ctypes.c_void_p * n_experts)(*[b.data_ptr() for b in bundles_host])
        self._arr = arr
        cfg = CacheCfg(n_experts, n_slots, int(bundle_bytes_), int(slot_stride),
                       ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, ptr(pool), int(blocking),
                       int(dry_run))
        h = ctypes.c_void_p()
        _check(lib().expert_slot_cache_create(ctypes.byref(cfg), ctypes.byref(h)))
        self.h = h
        self.E = n_experts

    def close(self):
        if self.h:
            lib().expert_slot_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _check(lib().expert_slot_cache_reset(self.h))

    def acquire(self, counts, stream=None) -> int:
        n = ctypes.c_int32()
        _check(lib().expert_slot_cache_acquire(self.h, ptr(counts), stream_ptr(stream), ctypes.byref(n)))
        return n.value

    def plan_host(self, counts_host) -> int:
        import numpy as np

        c = np.ascontiguousarray(counts_host, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().expert_slot_cache_plan_host(self.h, c.ctypes.data, ctypes.byref(n)))
        return n.value

    def wave(self, w, part, slot_table, stream=None) -> int:
        n = ctypes.c_int32()
        _check(lib().expert_slot_cache_wave(self.h, w, part, stream_ptr(stream), ptr(slot_table), ctypes.byref(n)))
        return n.value

    def release(self, w, stream=None):
        _check(lib().expert_slot_cache_release(self.h, w, stream_ptr(stream)))

    def set_layers(self, n_layers: int):
        """Entries are n_layers layer-major groups run in cyclic order: evict from the layer that
        runs furthest ahead, then LRU (1 = plain LRU)."""
        _check(lib().expert_slot_cache_set_layers(self.h, int(n_layers)))

    def set_frequency(self, decay: float):
        """Victims by decayed routing frequency (freq = decay*freq + counts per step), then recency;
        0 = plain recency."""
        _check(lib().expert_slot_cache_set_frequency(self.h, float(decay)))

    def prefetch(self, experts) -> int:
        """Copies the listed (predicted) experts ahead of their step; returns the copies issued."""
        import numpy as np

        e = np.ascontiguousarray(experts, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().expert_slot_cache_prefetch(self.h, e.ctypes.data if e.size else None, int(e.size),
                                                ctypes.byref(n)))
        return n.value

    def wave_plan(self, w):
        n = ctypes.c_int32()
        _check(lib().expert_slot_cache_wave_plan(self.h, w, None, 0, ctypes.byref(n)))
        buf = (CacheEntry * max(n.value, 1))()
        _check(lib().expert_slot_cache_wave_plan(self.h, w, buf, n.value, ctypes.byref(n)))
        return [(buf[i].expert, buf[i].slot, buf[i].hit, buf[i].evicted) for i in range(n.value)]

    def stats(self) -> dict:
        s = CacheStats()
        _check(lib().expert_slot_cache_stats(self.h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in CacheStats._fields_}


class DeviceSlotCache:
    """expert_slot_cache_dev: the slot pool planned on the device (no host synchronisation)."""

    def __init__(self, n_experts, n_slots, bundle_bytes_, slot_stride, bundles_host, pool):
        self._keep = bundles_host
        self._arr = (ctypes.c_void_p * n_experts)(*[b.data_ptr() for b in bundles_host])
        cfg = CacheCfg(n_experts, n_slots, int(bundle_bytes_), int(slot_stride),
                       ctypes.cast(self._arr, ctypes.c_void_p), ptr(pool), 0, 0)
        h = ctypes.c_void_p()
        _check(lib().expert_slot_cache_dev_create(ctypes.byref(cfg), ctypes.byref(h)))
        self.h = h
        self.E = n_experts

    def close(self):
        if self.h:
            lib().expert_slot_cache_dev_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _check(lib().expert_slot_cache_dev_reset(self.h))

    def set_frequency(self, decay: float):
        _check(lib().expert_slot_cache_dev_set_frequency(self.h, float(decay)))

    def set_layers(self, n_layers: int):
        _check(lib().expert_slot_cache_dev_set_layers(self.h, int(n_layers)))

    @property
    def max_waves(self) -> int:
        return int(lib().expert_slot_cache_dev_max_waves(self.h))

    def step(self, counts, hit_table, miss_tables, stream=None):
        _check(lib().expert_slot_cache_dev_step(self.h, ptr(counts), stream_ptr(stream), ptr(hit_table),
                                                ptr(miss_tables)))

    def copy(self, wave, stream=None):
        _check(lib().expert_slot_cache_dev_copy(self.h, int(wave), stream_ptr(stream)))

    def join(self, wave, stream=None):
        _check(lib().expert_slot_cache_dev_join(self.h, int(wave), stream_ptr(stream)))

    def stats(self) -> dict:
        s = CacheStats()
        _check(lib().expert_slot_cache_dev_stats(self.h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in CacheStats._fields_}


# ------------------------------------------------------------- profile ---

PROF_GATEUP, PROF_DOWN, PROF_DEC_GATEUP, PROF_DEC_DOWN = 0, 1, 2, 3
PROF_LABELED = 4   # kind offset of launches made under label 1 (e.g. a shared expert)


def profile_enable(on: bool = True):
    _check(lib().moe_profile_enable(int(on)))


def profile_label(label: int):
    """Launches from this thread are recorded under kind + 4 while label is 1."""
    _check(lib().moe_profile_label(int(label)))


def profile_read() -> dict:
    """{kind: (total_ms, launches)} since the last profile_enable (kinds 0..7)."""
    p = Profile()
    _check(lib().moe_profile_read(ctypes.byref(p)))
    return {k: (p.ms[k], p.launches[k]) for k in range(8)}
