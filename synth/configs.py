"""The five workload configurations and their cases, by shape and seed.

Every case is synthetic: bf16 N(0,1) values from the seeded generator, the
shapes of the draft-block attention layers the pages measure (Kimi-style TP8
rank 8q/2kv, wide 64q/16kv drafter, 16q/1kv and 64q/4kv windowed DSpark
layers), paged "HND" pools with disjoint shuffled page ranges.

Seeds are 1000 * config + case index. Context "32K" is 32768 tokens, "128K"
is 131072; the K block keys are appended after the context, so a request
holds context + K keys.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Case:
    name: str
    cfg: int
    index: int
    batch: int
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    context: int = 0                        # tokens before the block (fixed contexts)
    context_range: tuple | None = None      # (lo, hi) inclusive, drawn per request
    window_left: int = -1                   # -1: unwindowed non-causal
    window_right: int = -1
    outlier_rate: float = 0.0
    outlier_scale: float = 8.0
    sm_scale: float = field(default=0.0)
    kv_dtype: str = "bf16"                  # "bf16" or "fp8_e4m3": element type of the K and V pools
    k_scale: float = 1.0                    # a stored key element stands for k_scale times its value
    v_scale: float = 1.0

    @property
    def seed(self) -> int:
        return 1000 * self.cfg + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        return self.block_size * self.group

    @property
    def windowed(self) -> bool:
        return self.window_left != -1

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale else 1.0 / math.sqrt(self.head_dim)


def _cfg1():
    return [Case("cfg1", 1, 0, batch=1, block_size=3, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=32,
                 context=256, sm_scale=1.0 / 8.0)]


def _cfg2():
    out, idx = [], 0
    for ctx in (32768, 131072):
        for b in (1, 2, 4, 8, 16, 32):
            out.append(Case(f"cfg2_b{b}_{ctx // 1024}k", 2, idx, batch=b, block_size=7, num_q_heads=8,
                            num_kv_heads=2, head_dim=64, page_size=32, context=ctx))
            idx += 1
    return out


def _cfg3():
    out, idx = [], 0
    for ctx in (32768, 131072):
        for b in (1, 4, 16, 32):
            out.append(Case(f"cfg3_b{b}_{ctx // 1024}k", 3, idx, batch=b, block_size=7, num_q_heads=64,
                            num_kv_heads=16, head_dim=64, page_size=32, context=ctx))
            idx += 1
    return out


def _cfg4():
    out, idx = [], 0
    for ctx in (2048, 8192, 16384):
        for k in (1, 3, 7):
            for b in (1, 8, 64):
                out.append(Case(f"cfg4_b{b}_k{k}_{ctx // 1024}k", 4, idx, batch=b, block_size=k, num_q_heads=16,
                                num_kv_heads=1, head_dim=128, page_size=64, context=ctx, window_left=4096,
                                window_right=-1))
                idx += 1
    return out


def _cfg5():
    return [Case(f"cfg5_k{k}", 5, i, batch=64, block_size=k, num_q_heads=64, num_kv_heads=4, head_dim=128,
                 page_size=64, context_range=(2048, 16384), window_left=4096, window_right=-1, outlier_rate=0.01)
            for i, k in enumerate((3, 7))]


def cases_for_config(cfg: int) -> list:
    return {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}[cfg]()


def all_cases() -> list:
    return [c for cfg in range(1, 6) for c in cases_for_config(cfg)]


def find_case(name: str) -> Case:
    """A configuration case by name; a "_fp8" suffix selects its fp8 E4M3 variant."""
    if name.endswith("_fp8"):
        return fp8_variant(find_case(name[: -len("_fp8")]))
    for c in all_cases():
        if c.name == name:
            return c
    raise KeyError(name)


# fp8 context storage: the same case with both pools held as OCP fp8 E4M3 bytes.
# The N(0,1) draws are divided by the pool scale before encoding; 1/16 maps them
# (|x| < 6) below 96, inside the format's range (448), and off its subnormals for
# |x| > 2^-10. Outlier keys scaled x8 may saturate at 448.
FP8_SCALE = 0.0625


def fp8_variant(case: Case, k_scale: float = FP8_SCALE, v_scale: float = FP8_SCALE) -> Case:
    """A copy of `case` whose K and V pools are fp8 E4M3 with the given per-pool scales."""
    return replace(case, name=case.name + "_fp8", kv_dtype="fp8_e4m3", k_scale=k_scale, v_scale=v_scale)
