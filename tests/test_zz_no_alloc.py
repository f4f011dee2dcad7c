"""moe_grouped_ffn_combine_noalloc (the decode FFN + combine with its workspace in the library's
per-device static scratch array) against moe_grouped_ffn_combine with a caller workspace: bit
for bit on two calls in a row (the second with fewer tokens, so it runs on what the first left
in the array), and a step larger than the array is rejected before any launch."""
import numpy as np
import pytest
import torch

from expert_offloaded_ffn_amd import binding as B
from expert_offloaded_ffn_amd import synth
from expert_offloaded_ffn_amd.layer import MoELayer
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(layer, x, noalloc):
    """Routing, then the routed and shared experts with the combine in one call."""
    T = x.shape[0]
    r = B.route_permute(x, layer.w_router_t, w_shared_gate=layer.w_sg, **layer.route_args())
    probs = [B.ffn_problem(layer.shared.table, T, layer._shared_offsets(T), x, act_dtype=B.MOE_BF16),
             B.ffn_problem(layer.table, T * layer.k, r["offsets"], x, act_dtype=B.MOE_BF16, a_row_src=r["perm_src"],
                           a_row_div=layer.k)]
    if noalloc:
        out = torch.empty(T, layer.d, device=DEV, dtype=torch.bfloat16)
        return B.grouped_ffn_combine_noalloc(probs[1], probs[0], r["perm_dst"], r["gate"], out,
                                             shared_gate=r["shared_gate"])
    return B.grouped_ffn_combine(probs[1], probs[0], r["perm_dst"], r["gate"], shared_gate=r["shared_gate"])


def test_noalloc_matches_workspace_call_two_calls():
    cfg = synth.get_config("qwen_decode_bf16")
    layer = MoELayer(cfg, router=synth.gen_router(cfg), experts=synth.gen_experts(cfg), shared=synth.gen_shared(cfg),
                     w_shared_gate=synth.gen_shared_gate(cfg), device=DEV)
    for call, T in enumerate((8, 3)):     # the second call is smaller and reuses the scratch array
        x = torch.from_numpy(synth.gen_x(cfg, 40 + call, T=T).view(np.int16)).view(torch.bfloat16).to(DEV)
        say(f"  case no-alloc call {call} T={T}: launching")
        want = _step(layer, x, noalloc=False)
        got = _step(layer, x, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {call} (T={T}) differs"
        # and the layer's own (workspace) path agrees
        assert torch.equal(got.view(torch.int16), layer.forward(x)["out"].view(torch.int16))


def test_noalloc_rejects_a_step_larger_than_the_array():
    """1024 experts with Mixtral-sized F at top-32 over 64 tokens need about 70 MB of scratch: the
    call returns MOE_ECAPACITY before touching the device (the tensors are never read)."""
    dummy = torch.zeros(256, dtype=torch.uint8, device=DEV)
    slots = torch.zeros(1024, dtype=torch.int32, device=DEV)
    table = B.expert_table(dummy, B.bundle_bytes(4096, 14336, B.MOE_BF16), slots, 1024, 4096, 14336, B.MOE_BF16)
    x = torch.zeros(64, 4096, dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros(64 * 32, dtype=torch.int32, device=DEV)
    routed = B.ffn_problem(table, 64 * 32, idx, x, a_row_src=idx, a_row_div=32)
    assert B.grouped_ffn_combine_workspace_size(routed, None) > B.NOALLOC_SCRATCH_BYTES
    gate = torch.zeros(64, 32, dtype=torch.float32, device=DEV)
    out = torch.zeros(64, 4096, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.MoeError) as ei:
        B.grouped_ffn_combine_noalloc(routed, None, idx, gate, out)
    assert ei.value.status == B.MOE_ECAPACITY
