"""CPU oracle for one Mixture-of-Experts FFN layer (test infrastructure only).

This package is the slow, plain, float64 reference that the HIP library is
checked against. It is test infrastructure: only the test suite, the smoke
check of the package entry point and the CPU-baseline leg of the benchmark may
import it. The product path never imports, links or calls anything here, and
nothing here imports the product package.

Modules
-------
``formats``     bf16 decoding and the OCP 8-bit E4M3 codec (from the OCP
                8-bit floating point specification), plus the per-token
                per-128 activation quantisation and per-block weight scales.
``moe``         router scores, group-limited top-k with ties to the lower
                expert index, renormalised gates, expert histogram, the stable
                expert-major permutation, the SwiGLU expert FFN, the shared
                expert and the gate-weighted combine.
``slot_cache``  an exact simulation of the expert slot pool under LRU with
                deterministic transfer waves.

Sources. The pages define the setting, not the arithmetic: experts are
feed-forward networks chosen per token by a router ("The Billion-Token
Bottleneck", section "The Geometry of the Problem: Why MoE is Different");
only the chosen experts' weights are touched ("NovaLLM: Running Massive MoE
Models Fully In-Memory", sections 2-3); the expert cache intercepts the
router's expert list, keeps whole expert bundles (weights and quantisation
scales) resident in VRAM under LRU eviction, and a step that needs more
experts than there are slots waits for each wave's copies before that wave's
experts compute ("Running 35B MoE Models on
8GB GPUs: How vvllm-ms Caches Experts in System RAM", section "Technical
Insight"). The router math (softmax or sigmoid, renormalisation, group limit,
tie-break), the SwiGLU form and the fp8 formats are not on the pages; each
function states the reading it takes.

Every function here is pinned by tests in ``tests/test_oracle_*.py`` against
brute force, closed forms, invariants or an independent library routine.
"""
