"""Host-side checks of the C ABI (no device work): every symbol the header declares
is exported, argument validation fails with the documented codes before touching a
device, the bundle packer writes the documented layout, and the slot-pool planner
(dry run) matches the oracle's LRU simulation exactly."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from expert_offloaded_ffn_amd import binding as B
from oracle.slot_cache import LRUSlotCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:moe_status|size_t|int32_t|char\s*\*|const\s+char\s*\*)\s*\**\s*(\w+)\s*\(",
                       src, flags=re.M)
    names += re.findall(r"^\s*const char\*\s+(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared_functions()
    assert names == sorted(B.EXPORTS), names   # the binding covers exactly the header
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe.h but not exported"
    assert b"gfx950" in L.moe_version()


def test_route_validation_codes():
    L = B.lib()
    cfg = B.RouteCfg(16, 128, 8, 2, 0, 1, 1.0, 1, 1, 0, B.MOE_BF16)
    null = None
    assert L.moe_route(None, *([null] * 10), null) == -1
    bad = B.RouteCfg(16, 128, 8, 9, 0, 1, 1.0, 1, 1, 0, B.MOE_BF16)        # k > E
    assert L.moe_route(ctypes.byref(bad), *([null] * 10), null) == -1
    assert b"top_k" in L.moe_last_error()
    bad = B.RouteCfg(16, 128, 256, 8, 1, 1, 2.5, 7, 4, 2, B.MOE_BF16)      # groups do not divide E
    assert L.moe_route(ctypes.byref(bad), *([null] * 10), null) == -1
    bad = B.RouteCfg(16, 128, 256, 8, 1, 1, 2.5, 8, 4, 2, B.MOE_FP8_E4M3)  # fp8 router input
    assert L.moe_route(ctypes.byref(bad), *([null] * 10), null) == -2
    ok_empty = B.RouteCfg(0, 128, 8, 2, 0, 1, 1.0, 1, 1, 0, B.MOE_BF16)    # T = 0 is a no-op
    assert L.moe_route(ctypes.byref(ok_empty), *([null] * 10), null) == 0
    sb = (ctypes.c_float * 8)()
    args = [null, null, null, ctypes.cast(sb, ctypes.c_void_p)] + [null] * 6
    assert L.moe_route(ctypes.byref(cfg), *args, null) == -1               # select_bias with softmax


def test_permute_and_combine_validation_codes():
    L = B.lib()
    assert L.moe_permute(16, 0, 8, *([None] * 4), 0, None, 0, None, 0, None, 1, None, 0, None) == -1
    need = L.moe_permute_workspace_size(16, 2, 8)
    assert need > 0
    fake = ctypes.c_void_p(0x1000)
    assert L.moe_permute(16, 2, 8, fake, fake, fake, fake, 0, None, 0, None, 0, None, 1, fake, need - 1, None) == -4
    assert L.moe_combine(4, 40, 128, None, 1, None, None, None, None, None, 1, None) == -1
    assert L.moe_combine(0, 2, 128, None, 1, None, None, None, None, None, 1, None) == 0


def test_grouped_ffn_validation_codes():
    L = B.lib()
    t = B.ExpertTable(None, 0, None, 8, 4096, 14336, B.MOE_BF16)
    assert L.moe_grouped_ffn(ctypes.byref(t), 16, *([None] * 3), 1, None, 1, None, 1, None, 0, None) == -1
    nb = B.bundle_bytes(4096, 14336, B.MOE_BF16)
    assert nb == 3 * 4096 * 14336 * 2
    assert B.bundle_bytes(7168, 2048, B.MOE_FP8_E4M3) == 3 * 7168 * 2048 + 3 * 16 * 56 * 4
    assert B.bundle_bytes(4096, 1536, B.MOE_BF16) == 37748736
    assert B.bundle_bytes(100, 256, B.MOE_BF16) == 0          # d % 32 != 0
    t = B.ExpertTable(ctypes.c_void_p(256), nb - 256, ctypes.c_void_p(256), 8, 4096, 14336, B.MOE_BF16)
    assert L.moe_grouped_ffn(ctypes.byref(t), 16, *([None] * 3), 1, None, 1, None, 1, None, 0, None) == -1
    assert b"slot_stride" in L.moe_last_error()


_STRUCTS = [("moe_route_cfg", B.RouteCfg), ("moe_expert_table", B.ExpertTable), ("moe_ffn_problem", B.FfnProblem),
            ("moe_cache_cfg", B.CacheCfg), ("moe_cache_stats", B.CacheStats), ("moe_cache_entry", B.CacheEntry),
            ("moe_profile", B.Profile), ("moe_combine_args", B.CombineArgs), ("moe_decode_out", B.DecodeOut)]


def test_struct_layouts_match_header(tmp_path):
    """Every ctypes mirror has the size and field offsets the C compiler gives the header's struct."""
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe.h"', "int main(void) {"]
    for cname, py in _STRUCTS:
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                           text=True).stdout.splitlines())
    for cname, py in _STRUCTS:
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, f"{cname}.{f}"


def test_batch_and_route_permute_validation_codes():
    L = B.lib()
    assert L.moe_grouped_ffn_batch(None, 1, None, 0, None) == -1
    t = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(256, 512, B.MOE_BF16), ctypes.c_void_p(256), 8, 256, 512,
                      B.MOE_BF16)
    fake = ctypes.c_void_p(0x1000)
    pr = B.FfnProblem(ctypes.pointer(t), 16, fake, fake, None, B.MOE_BF16, None, 1, fake, B.MOE_BF16)
    arr = (B.FfnProblem * 3)(pr, pr, pr)
    assert L.moe_grouped_ffn_batch(arr, 3, fake, 1 << 20, None) == -1               # n outside [1, 2]
    one = L.moe_grouped_ffn_workspace_size(ctypes.byref(t), 16, B.MOE_BF16)
    need = L.moe_grouped_ffn_batch_workspace_size(arr, 2)
    assert need == 2 * ((one + 255) // 256 * 256)
    assert L.moe_grouped_ffn_batch(arr, 2, None, need, None) == -1                 # no workspace
    assert L.moe_grouped_ffn_batch(arr, 2, fake, need - 1, None) == -4             # short workspace
    empty = B.FfnProblem(ctypes.pointer(t), 0, None, None, None, B.MOE_BF16, None, 1, None, B.MOE_BF16)
    assert L.moe_grouped_ffn_batch((B.FfnProblem * 2)(empty, empty), 2, None, 0, None) == 0
    nul = B.FfnProblem(None, 4, None, None, None, B.MOE_BF16, None, 1, None, B.MOE_BF16)
    assert L.moe_grouped_ffn_batch((B.FfnProblem * 1)(nul), 1, fake, need, None) == -1
    assert b"no table" in L.moe_last_error()
    null = None
    assert L.moe_route_permute(None, *([null] * 14), 0, null) == -1
    bad = B.RouteCfg(4, 128, 8, 9, 0, 1, 1.0, 1, 1, 0, B.MOE_BF16)                # k > E
    assert L.moe_route_permute(ctypes.byref(bad), *([null] * 14), 0, null) == -1
    assert b"moe_route_permute" in L.moe_last_error()
    cfg = B.RouteCfg(4, 128, 8, 2, 0, 1, 1.0, 1, 1, 0, B.MOE_BF16)
    args = [fake] * 14                                                              # 13 tensors and ws
    args[3] = None                                                                  # select_bias: softmax has none
    assert L.moe_route_permute(ctypes.byref(cfg), *args, 0, null) == -4             # short workspace
    args[1] = ctypes.c_void_p(0x1001)                                               # misaligned router weights
    assert L.moe_route_permute(ctypes.byref(cfg), *args, 1 << 16, null) == -1


def test_grouped_ffn_combine_validation_codes():
    """The fused decode FFN + combine rejects, before any launch, what the two-call sequence would
    reject, rows that do not match T and k, non-decode problems and short workspaces."""
    L = B.lib()
    t = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(256, 512, B.MOE_BF16), ctypes.c_void_p(256), 8, 256, 512,
                      B.MOE_BF16)
    fake = ctypes.c_void_p(0x1000)
    T, k = 4, 2
    routed = B.FfnProblem(ctypes.pointer(t), T * k, fake, fake, None, B.MOE_BF16, fake, k, None, B.MOE_BF16)
    shared = B.FfnProblem(ctypes.pointer(t), T, fake, fake, None, B.MOE_BF16, None, 1, None, B.MOE_BF16)
    cb = B.CombineArgs(T, k, fake, fake, fake, fake, B.MOE_BF16)
    need = L.moe_grouped_ffn_combine_workspace_size(ctypes.byref(routed), ctypes.byref(shared))
    batch = L.moe_grouped_ffn_batch_workspace_size((B.FfnProblem * 2)(shared, routed), 2)
    # the batch workspace, fp32 expert outputs of both problems, then the group counts
    assert need == batch + T * k * 256 * 4 + T * 256 * 4 + 256
    assert L.moe_grouped_ffn_combine(None, None, ctypes.byref(cb), fake, need, None) == -1
    assert L.moe_grouped_ffn_combine(ctypes.byref(routed), None, None, fake, need, None) == -1
    assert L.moe_grouped_ffn_combine(ctypes.byref(routed), ctypes.byref(shared), ctypes.byref(cb), fake, need - 1,
                                     None) == -4
    bad_rows = B.CombineArgs(T + 1, k, fake, fake, fake, fake, B.MOE_BF16)
    assert L.moe_grouped_ffn_combine(ctypes.byref(routed), None, ctypes.byref(bad_rows), fake, need, None) == -1
    assert b"routed rows" in L.moe_last_error()
    big = B.CombineArgs(65, 1, fake, fake, fake, fake, B.MOE_BF16)
    assert L.moe_grouped_ffn_combine(ctypes.byref(routed), None, ctypes.byref(big), fake, need, None) == -2
    t32 = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(256, 512, B.MOE_F32), ctypes.c_void_p(256), 8, 256, 512,
                        B.MOE_F32)
    r32 = B.FfnProblem(ctypes.pointer(t32), T * k, fake, fake, None, B.MOE_F32, fake, k, None, B.MOE_F32)
    need32 = L.moe_grouped_ffn_combine_workspace_size(ctypes.byref(r32), None)
    assert L.moe_grouped_ffn_combine(ctypes.byref(r32), None, ctypes.byref(cb), ctypes.c_void_p(0x10000), need32,
                                     None) == -2
    assert b"not a decode problem" in L.moe_last_error()
    empty = B.CombineArgs(0, k, None, None, None, None, B.MOE_BF16)
    r0 = B.FfnProblem(ctypes.pointer(t), 0, None, None, None, B.MOE_BF16, None, k, None, B.MOE_BF16)
    assert L.moe_grouped_ffn_combine(ctypes.byref(r0), None, ctypes.byref(empty), None, 0, None) == 0


def test_decode_step_validation_codes():
    """The fused decode step rejects, before any launch, what the separate calls would reject and
    the sizes it does not cover (more than 64 tokens, more than 256 experts, fp8 weights), and
    sizes its workspace as documented."""
    L = B.lib()
    fake = ctypes.c_void_p(0x1000)
    T, d, E, k, F = 4, 256, 8, 2, 512
    t = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(d, F, B.MOE_BF16), ctypes.c_void_p(256), E, d, F,
                      B.MOE_BF16)
    ts = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(d, 1024, B.MOE_BF16), ctypes.c_void_p(256), 1, d, 1024,
                       B.MOE_BF16)
    cfg = B.RouteCfg(T, d, E, k, B.MOE_SOFTMAX, 1, 1.0, 1, 1, 0, B.MOE_BF16)
    out = B.DecodeOut(None, fake, fake, fake, None, fake, fake, fake, fake, B.MOE_BF16)
    need = L.moe_decode_step_workspace_size(ctypes.byref(cfg), ctypes.byref(t), ctypes.byref(ts))
    need0 = L.moe_decode_step_workspace_size(ctypes.byref(cfg), ctypes.byref(t), None)
    one = lambda n: (n + 255) // 256 * 256
    # counters, logit slices (d/128 slices x T x (E + 1)), the selection, the two FFN workspaces,
    # fp32 expert outputs, the combine's group counts
    ffn_s = L.moe_grouped_ffn_workspace_size(ctypes.byref(ts), T, B.MOE_BF16)
    ffn_r = L.moe_grouped_ffn_workspace_size(ctypes.byref(t), T * k, B.MOE_BF16)
    assert need == (256 + one(d // 128 * T * (E + 1) * 4) + one(T * k * 4) + one(ffn_s) + one(ffn_r) +
                    one(T * k * d * 4) + one(T * d * 4) + one(d // 32 * 4))
    assert need0 == need - one(ffn_s) - one(T * d * 4)
    go = lambda c, o, ws, n, shared=ctypes.byref(ts): L.moe_decode_step(
        ctypes.byref(c), fake, fake, None, None, None, ctypes.byref(t), shared, o, ws, n, None)
    assert L.moe_decode_step(None, fake, fake, None, None, None, ctypes.byref(t), None, ctypes.byref(out), fake, need,
                             None) == -1
    assert go(cfg, ctypes.byref(out), fake, need - 1) == -4                          # short workspace
    assert go(cfg, ctypes.byref(out), ctypes.c_void_p(0x1010), need) == -1           # misaligned workspace
    big = B.RouteCfg(65, d, E, k, B.MOE_SOFTMAX, 1, 1.0, 1, 1, 0, B.MOE_BF16)
    assert go(big, ctypes.byref(out), fake, 1 << 30) == -2                           # not a decode step
    assert b"decode steps only" in L.moe_last_error()
    f32 = B.RouteCfg(T, d, E, k, B.MOE_SOFTMAX, 1, 1.0, 1, 1, 0, B.MOE_F32)
    assert go(f32, ctypes.byref(out), fake, need) == -2
    with_gate = B.DecodeOut(fake, fake, fake, fake, None, fake, fake, fake, fake, B.MOE_BF16)
    assert go(cfg, ctypes.byref(with_gate), fake, need) == -1                         # gate output, no weights
    assert b"go together" in L.moe_last_error()
    t8 = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(d, F, B.MOE_FP8_E4M3), ctypes.c_void_p(256), E, d, F,
                       B.MOE_FP8_E4M3)
    assert L.moe_decode_step(ctypes.byref(cfg), fake, fake, None, None, None, ctypes.byref(t8), None,
                             ctypes.byref(out), fake, 1 << 30, None) == -2
    wrong_e = B.ExpertTable(ctypes.c_void_p(256), B.bundle_bytes(d, F, B.MOE_BF16), ctypes.c_void_p(256), E + 1, d,
                            F, B.MOE_BF16)
    assert L.moe_decode_step(ctypes.byref(cfg), fake, fake, None, None, None, ctypes.byref(wrong_e), None,
                             ctypes.byref(out), fake, 1 << 30, None) == -1
    assert L.moe_decode_step_workspace_size(ctypes.byref(big), ctypes.byref(t), None) == 0


def test_route_permute_workspace_only_holds_slices_when_used():
    """The logit slices (K slices x T x (E + 1) fp32) are part of the workspace only for the
    batches that take the sliced path (1..64 tokens, E <= 256, d % 32 == 0)."""
    assert B.route_permute_workspace_size(8192, 8, 256, 7168) == B.permute_workspace_size(8192, 8, 256)
    assert B.route_permute_workspace_size(65, 4, 60, 2048) == B.permute_workspace_size(65, 4, 60)
    assert B.route_permute_workspace_size(64, 4, 300, 2048) == B.permute_workspace_size(64, 4, 300)
    slices = (2048 // 32 + 3) // 4           # 4 k-steps of 32 per slice
    assert B.route_permute_workspace_size(64, 4, 60, 2048) >= slices * 64 * 61 * 4
    assert B.route_permute_workspace_size(1, 4, 60, 2048) >= slices * 1 * 61 * 4


def test_pack_bf16_layout():
    d, F = 64, 32
    rng = np.random.default_rng(0)
    wg = rng.integers(0, 2 ** 16, (d, F), dtype=np.uint16)
    wu = rng.integers(0, 2 ** 16, (d, F), dtype=np.uint16)
    wd = rng.integers(0, 2 ** 16, (F, d), dtype=np.uint16)
    b = B.pack_expert(d, F, B.MOE_BF16, wg, wu, wd).numpy().view(np.uint16)
    gu = b[:2 * F * d]

    def tiled(buf, n, k, K):   # header: tile (n//16, k//32) at (nb*K/32 + kb)*512 elems; lane = n%16 + 16*((k%32)//8)
        tile = (n // 16) * (K // 32) + k // 32
        lane = n % 16 + 16 * ((k % 32) // 8)
        return buf[tile * 512 + lane * 8 + k % 8]

    for _ in range(200):
        R, kk = rng.integers(0, 2 * F), rng.integers(0, d)
        j, rr = R // 32, R % 32
        want = (wu if rr >= 16 else wg)[kk, 16 * j + rr % 16]
        assert tiled(gu, R, kk, d) == want
    dn = b[2 * F * d:]
    for _ in range(200):
        n, f = rng.integers(0, d), rng.integers(0, F)
        assert tiled(dn, n, f, F) == wd[f, n]


def test_pack_mxfp4_layout_and_scales():
    """MXFP4 bundle: two codes per byte in 16 x 128 chunks and E8M0 exponents per 32-input
    block, as the header lays them out; bad codes and non-power-of-two scales are refused."""
    d, F = 256, 128
    rng = np.random.default_rng(2)
    wg, wu = rng.integers(0, 16, (d, F), dtype=np.uint8), rng.integers(0, 16, (d, F), dtype=np.uint8)
    wd = rng.integers(0, 16, (F, d), dtype=np.uint8)
    eg, eu = rng.integers(100, 150, (d // 32, F)), rng.integers(100, 150, (d // 32, F))
    ed = rng.integers(100, 150, (F // 32, d))
    p2 = lambda e: np.ldexp(np.float32(1.0), e - 127).astype(np.float32)
    b = B.pack_expert(d, F, B.MOE_MXFP4, wg, wu, wd, p2(eg), p2(eu), p2(ed)).numpy()
    al = lambda v: (v + 255) // 256 * 256
    gu_s = al(2 * F * d // 2)
    dn_c = gu_s + al(2 * F * d // 32)
    dn_s = dn_c + al(d * F // 2)
    assert b.size == dn_s + al(d * F // 32) == B.bundle_bytes(d, F, B.MOE_MXFP4)

    def code_at(base, n, k, K):
        kc, c, q, j = k // 128, (k % 128) // 32, (k % 32) // 8, (k % 8) // 2
        lane = n % 16 + 16 * q
        byte = b[base + ((n // 16) * (K // 128) + kc) * 1024 + 16 * lane + 4 * c + j]
        return (byte >> 4) if k % 2 else (byte & 15)

    def exp_at(base, n, k, K):
        kc, c = k // 128, (k % 128) // 32
        return b[base + ((n // 16) * (K // 128) + kc) * 64 + 4 * (n % 16) + c]

    for _ in range(300):
        R, kk = rng.integers(0, 2 * F), rng.integers(0, d)
        j, rr = R // 32, R % 32
        up, col = rr >= 16, 16 * j + rr % 16
        assert code_at(0, R, kk, d) == (wu if up else wg)[kk, col]
        assert exp_at(gu_s, R, kk, d) == (eu if up else eg)[kk // 32, col]
        n, f = rng.integers(0, d), rng.integers(0, F)
        assert code_at(dn_c, n, f, F) == wd[f, n]
        assert exp_at(dn_s, n, f, F) == ed[f // 32, n]
    bad = wg.copy()
    bad[3, 4] = 16
    with pytest.raises(B.MoeError):
        B.pack_expert(d, F, B.MOE_MXFP4, bad, wu, wd, p2(eg), p2(eu), p2(ed))
    s_bad = p2(eg)
    s_bad[0, 0] = 0.75
    with pytest.raises(B.MoeError):
        B.pack_expert(d, F, B.MOE_MXFP4, wg, wu, wd, s_bad, p2(eu), p2(ed))


def test_pack_fp8_layout_and_scales():
    d, F = 256, 128
    rng = np.random.default_rng(1)
    wg, wu = rng.integers(0, 255, (d, F), dtype=np.uint8), rng.integers(0, 255, (d, F), dtype=np.uint8)
    wd = rng.integers(0, 255, (F, d), dtype=np.uint8)
    sg, su = rng.random((2, 1), dtype=np.float32), rng.random((2, 1), dtype=np.float32)
    sd = rng.random((1, 2), dtype=np.float32)
    b = B.pack_expert(d, F, B.MOE_FP8_E4M3, wg, wu, wd, sg, su, sd).numpy()
    for _ in range(200):
        R, kk = rng.integers(0, 2 * F), rng.integers(0, d)
        tile = (R // 16) * (d // 128) + kk // 128
        lane = R % 16 + 16 * ((kk % 128) // 32)
        half, byte = (kk % 32) // 16, kk % 16
        j, rr = R // 32, R % 32
        assert b[tile * 2048 + half * 1024 + lane * 16 + byte] == (wu if rr >= 16 else wg)[kk, 16 * j + rr % 16]
    off = 2 * F * d + d * F
    s = b[off:].view(np.float32)
    assert s[0] == sg[0, 0] and s[1] == sg[1, 0]                # gate stored [F/128][d/128]
    assert s[64] == su[0, 0] and s[65] == su[1, 0]              # next grid at +256 B
    assert s[128] == sd[0, 0] and s[129] == sd[0, 1]            # down stored [d/128][F/128]


@pytest.mark.parametrize("E,S,k,T", [(8, 3, 2, 4), (60, 16, 4, 8), (128, 32, 8, 32)])
def test_planner_matches_oracle_simulation(E, S, k, T):
    rng = np.random.default_rng(E + S)
    c = B.SlotCache(E, S, 1 << 20, 1 << 20, dry_run=True)
    sim = LRUSlotCache(E, S)
    for step in range(60):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        n = c.plan_host(counts)
        plan = sim.step(idx.ravel())
        assert n == len(plan.waves)
        for w, wave in enumerate(plan.waves):
            assert c.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
    st = c.stats()
    assert (st["hits"], st["misses"], st["evictions"], st["waves"], st["steps"]) == \
        (sim.stats.hits, sim.stats.misses, sim.stats.evictions, sim.stats.waves, sim.stats.steps)
    c.reset()
    assert c.stats()["misses"] == 0
    c.close()


@pytest.mark.parametrize("E,S,k,T", [(8, 5, 2, 2), (60, 24, 4, 4), (128, 48, 8, 4), (128, 32, 8, 32)])
def test_planner_prefetch_matches_oracle_simulation(E, S, k, T):
    """Steps interleaved with predictions (the previous step's set, random lists, resident
    experts): the library's plans, copy counts and counters equal the oracle's."""
    rng = np.random.default_rng(7 * E + S)
    c = B.SlotCache(E, S, 1 << 20, 1 << 20, dry_run=True)
    sim = LRUSlotCache(E, S)
    prev = None
    for step in range(60):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        n = c.plan_host(counts)
        plan = sim.step(idx.ravel())
        assert n == len(plan.waves)
        for w, wave in enumerate(plan.waves):
            assert c.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
        pred = rng.choice(E, size=rng.integers(0, S + 4)).tolist()
        if prev is not None and step % 2:
            pred = np.flatnonzero(prev).tolist() + pred
        assert c.prefetch(pred) == len(sim.prefetch(pred))
        prev = counts
    st = c.stats()
    s = sim.stats
    assert (st["hits"], st["misses"], st["evictions"], st["prefetches"], st["prefetch_used"]) == \
        (s.hits, s.misses, s.evictions, s.prefetches, s.prefetch_used)
    if S > T * k:   # else every slot holds an expert of the last step and nothing is copied
        assert s.prefetches > 0 and s.prefetch_used > 0
    with pytest.raises(B.MoeError) as ei:
        c.prefetch([E])
    assert ei.value.status == -1
    c.close()
    blocking = B.SlotCache(E, S, 1 << 20, 1 << 20, blocking=True, dry_run=True)
    with pytest.raises(B.MoeError) as ei:
        blocking.prefetch([0])
    assert ei.value.status == -6
    blocking.close()


@pytest.mark.parametrize("L,per,S,k,T", [(2, 8, 5, 2, 2), (4, 32, 40, 4, 4), (4, 128, 128, 8, 32)])
def test_planner_layer_order_matches_oracle_simulation(L, per, S, k, T):
    """A stack's cyclic layer steps, with and without predictions, under the layer order."""
    rng = np.random.default_rng(L * per + S)
    E = L * per
    c = B.SlotCache(E, S, 1 << 20, 1 << 20, dry_run=True)
    c.set_layers(L)
    sim = LRUSlotCache(E, S, n_layers=L)
    for step in range(30 * L):
        l = step % L
        idx = l * per + np.stack([rng.choice(per, size=k, replace=False) for _ in range(T)])
        counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        n = c.plan_host(counts)
        plan = sim.step(idx.ravel())
        assert n == len(plan.waves)
        for w, wave in enumerate(plan.waves):
            assert c.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
        if step % 3 == 1:
            nxt = (l + 1) % L
            pred = (nxt * per + rng.choice(per, size=rng.integers(0, per // 2 + 1), replace=False)).tolist()
            assert c.prefetch(pred) == len(sim.prefetch(pred))
    st, s = c.stats(), sim.stats
    assert (st["hits"], st["misses"], st["evictions"], st["prefetches"]) == (s.hits, s.misses, s.evictions, s.prefetches)
    bad = np.zeros(E, np.int32)
    bad[0] = bad[per] = 1   # entries of layers 0 and 1 in one step
    with pytest.raises(B.MoeError) as ei:
        c.plan_host(bad)
    assert ei.value.status == -1
    with pytest.raises(B.MoeError):
        c.set_layers(E + 1)
    c.close()


@pytest.mark.parametrize("L,decay", [(1, 0.8), (1, 1.0), (4, 0.8)])
def test_planner_frequency_matches_oracle_simulation(L, decay):
    """Frequency-aware victims (alone and after the layer order), with predictions."""
    rng = np.random.default_rng(int(decay * 10) + L)
    per, S, k, T = 32, 24, 4, 6
    E = L * per
    c = B.SlotCache(E, S, 1 << 20, 1 << 20, dry_run=True)
    if L > 1:
        c.set_layers(L)
    c.set_frequency(decay)
    sim = LRUSlotCache(E, S, n_layers=L, freq_decay=decay)
    p = rng.dirichlet(np.full(per, 0.5))
    for step in range(40 * L):
        l = step % L
        idx = l * per + np.stack([rng.choice(per, size=k, replace=False, p=p) for _ in range(T)])
        counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        n = c.plan_host(counts)
        plan = sim.step(idx.ravel())
        assert n == len(plan.waves)
        for w, wave in enumerate(plan.waves):
            assert c.wave_plan(w) == [(en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
        if step % 4 == 3:
            pred = (((l + 1) % L) * per + rng.choice(per, size=5, replace=False)).tolist()
            assert c.prefetch(pred) == len(sim.prefetch(pred))
    st, s = c.stats(), sim.stats
    assert (st["hits"], st["misses"], st["evictions"]) == (s.hits, s.misses, s.evictions)
    with pytest.raises(B.MoeError):
        c.set_frequency(1.5)
    c.close()


def test_cache_create_validation():
    with pytest.raises(B.MoeError) as ei:
        B.SlotCache(8, 0, 1024, 1024, dry_run=True)
    assert ei.value.status == -4
    with pytest.raises(B.MoeError) as ei:
        B.SlotCache(8, 2, 1024, 512, dry_run=True)
    assert ei.value.status == -4
    c = B.SlotCache(8, 2, 1024, 1024, dry_run=True)
    with pytest.raises(B.MoeError) as ei:
        c.acquire(None)
    assert ei.value.status in (-1, -6)


def test_profile_label_validation():
    L = B.lib()
    assert L.moe_profile_label(2) == -1
    assert b"label" in L.moe_last_error()
    assert L.moe_profile_label(1) == 0
    assert L.moe_profile_label(0) == 0
    assert ctypes.sizeof(B.Profile) == 8 * 8 + 8 * 8   # ms[8] doubles, launches[8] int64


def test_device_cache_validation_without_a_device():
    """Argument checks of the device-planned cache fail before any HIP call."""
    L = B.lib()
    h = ctypes.c_void_p()
    for blocking, dry_run, E, S, nb in [(1, 0, 8, 2, 1024), (0, 1, 8, 2, 1024), (0, 0, 0, 2, 1024),
                                        (0, 0, 2048, 2, 1024), (0, 0, 8, 0, 1024), (0, 0, 8, 2, 1000)]:
        cfg = B.CacheCfg(E, S, nb, 1024, None, None, blocking, dry_run)
        st = L.expert_slot_cache_dev_create(ctypes.byref(cfg), ctypes.byref(h))
        assert st in (-1, -4), (blocking, dry_run, E, S, nb, st)
        assert not h.value
    assert L.expert_slot_cache_dev_set_frequency(None, 0.5) == -1
    assert L.expert_slot_cache_dev_set_layers(None, 2) == -1
    assert L.expert_slot_cache_dev_step(None, None, None, None, None) == -1
    assert L.expert_slot_cache_dev_copy(None, 0, None) == -1
    assert L.expert_slot_cache_dev_join(None, 0, None) == -1
    assert L.expert_slot_cache_dev_max_waves(None) == 0
    assert L.expert_slot_cache_dev_destroy(None) == 0
