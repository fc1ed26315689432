"""The verify-step workloads, named by what they are.

Sizes follow the operating points the pages discuss: group size G in {8, 32},
draft length chosen so that G*(1+D) = 128 (the attention tile the translated
co-design page's "Draft length and attention performance" section singles out),
KV lengths of 32K and 128K (its Figure 4), the D sweep across G*(1+D) = 128 and
256 (Figure 5), and a fixed acceptance rate alpha in {0.4, 0.6, 0.8} (the LLM
inference handbook's section on how the acceptance rate affects performance).
Value distributions not stated for a workload borrow those of the G=8 one.
"""

from __future__ import annotations

from .generate import WorkloadSpec

PRESETS = {
    # tiny, checkable on the CPU in well under a second
    "tiny": WorkloadSpec(
        name="tiny_b2_hkv2_g4_d64_kv256_D3_v1000", batch=2, kv_heads=2, group=4, head_dim=64,
        kv_len=256, draft_len=3, vocab=1000, mode="stochastic", target_std=2.0, draft_noise_std=0.5),
    # attention-dominated decode, G*(1+D) = 128
    "g8_kv32k_D15": WorkloadSpec(
        name="b16_hkv8_g8_d128_kv32768_D15_v131072", batch=16, kv_heads=8, group=8, head_dim=128,
        kv_len=32768, draft_len=15, vocab=131072, mode="stochastic", target_std=3.0, draft_noise_std=1.0),
    # long context, large group, greedy acceptance
    "g32_kv128k_D3_greedy": WorkloadSpec(
        name="b4_hkv2_g32_d128_kv131072_D3_v131072_greedy", batch=4, kv_heads=2, group=32, head_dim=128,
        kv_len=131072, draft_len=3, vocab=131072, mode="greedy", target_std=3.0, draft_noise_std=1.0,
        draft_pick="argmax"),
    # tile-boundary sweep point (D and alpha are overridden per point)
    "g8_kv32k_sweep": WorkloadSpec(
        name="b32_hkv8_g8_d128_kv32768_v32000_sweep", batch=32, kv_heads=8, group=8, head_dim=128,
        kv_len=32768, draft_len=15, vocab=32000, mode="stochastic", target_std=3.0, alpha=0.6),
    # ragged mixed batch from one shared page pool
    "ragged_b64": WorkloadSpec(
        name="b64_hkv8_g8_d128_kvlognormal1k-128k_D3-7-15_v151936", batch=64, kv_heads=8, group=8,
        head_dim=128, kv_len=("lognormal", 8192, 1.0, 1024, 131072), draft_len=(3, 7, 15), vocab=151936,
        mode="stochastic", target_std=3.0, draft_noise_std=1.0),
}


def preset(name: str, **overrides) -> WorkloadSpec:
    spec = PRESETS[name]
    if overrides:
        spec = spec.with_(**overrides)
        if "draft_len" in overrides and "name" not in overrides and spec.name.endswith("_sweep"):
            spec = spec.with_(name=spec.name.replace("_sweep", f"_D{overrides['draft_len']}"))
    return spec
