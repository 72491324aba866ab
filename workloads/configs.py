"""The five synthetic ISD workloads.

Shapes follow the 8B serving setup the I-DLM pages describe: a Qwen3-8B-shaped
model (32 query heads, 8 KV heads, head dim 128, vocabulary 151936, hidden size
4096) served in bfloat16 at up to 32 concurrent requests on one GPU
("Introspective Diffusion Language Models" blog, section on reusing the AR
inference stack: the SGLang launch command with --max-running-requests 32 and
--dtype bfloat16).  The stride size N=4 is the configuration the hotdry.top
article tabulates (section on core parameters: N=4, p=0.90, about 7 queries).

Every workload uses 16-token KV pages handed out in a seeded shuffled order,
so every run exercises the page-table gather.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    batch: int                 # B, concurrent requests
    n_q_heads: int             # Hq
    n_kv_heads: int            # Hkv
    head_dim: int              # D
    stride_n: int              # N: proposals per stride; Q = 2N-1 query rows
    vocab: int                 # V
    dtype: str                 # "f32" or "bf16" (q, k/v, pages, logits)
    ctx: Optional[int] = None  # fixed context length, or None with ctx_range
    ctx_range: Optional[Tuple[int, int]] = None  # inclusive uniform range
    accept_targets: Tuple[float, ...] = (0.9,)   # one value, or a set drawn per request
    page_size: int = 16
    lora: bool = False
    lora_dim: int = 4096       # d_in = d_out of the adapted projection
    lora_rank: int = 128
    lora_std: float = 0.02
    logit_std: float = 3.0
    seed_base: int = 0
    description: str = ""

    @property
    def q_rows(self) -> int:
        return 2 * self.stride_n - 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "tiny_fp32": WorkloadConfig(
        name="tiny_fp32", batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, stride_n=2,
        vocab=1024, dtype="f32", ctx=256, seed_base=0,
        description="tiny fp32 step: B=1, 2/1 heads, D=64, ctx 256, N=2 (Q=3), V=1024"),
    "b8_ctx2k": WorkloadConfig(
        name="b8_ctx2k", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, stride_n=4,
        vocab=151936, dtype="bf16", ctx=2048, seed_base=1000,
        description="B=8, 32/8 heads, D=128, ctx 2048, N=4 (Q=7), V=151936, bf16"),
    "c32_ctx4k": WorkloadConfig(
        name="c32_ctx4k", batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128, stride_n=4,
        vocab=151936, dtype="bf16", ctx=4096, seed_base=2000,
        description="concurrency 32, ctx 4096, N=4 (Q=7), V=151936, bf16, shuffled pages"),
    "c64_ragged": WorkloadConfig(
        name="c64_ragged", batch=64, n_q_heads=32, n_kv_heads=8, head_dim=128, stride_n=8,
        vocab=151936, dtype="bf16", ctx_range=(512, 8192), accept_targets=(0.7, 0.8, 0.9, 0.95),
        seed_base=3000,
        description="concurrency 64, ctx ~ U[512, 8192], N=8 (Q=15), per-request acceptance "
                    "target in {0.7, 0.8, 0.9, 0.95}, bf16"),
    "c128_lora": WorkloadConfig(
        name="c128_lora", batch=128, n_q_heads=32, n_kv_heads=8, head_dim=128, stride_n=4,
        vocab=151936, dtype="bf16", ctx=2048, lora=True, seed_base=4000,
        description="concurrency 128, ctx 2048, N=4, plus a rank-128 gated LoRA delta on a "
                    "4096->4096 projection at the N MASK rows"),
}

# The configuration the throughput figure is quoted on.
HEADLINE = "c32_ctx4k"


def get_config(name: str, **overrides) -> WorkloadConfig:
    """Return a named config, optionally with fields replaced (for scaled-down tests)."""
    cfg = CONFIGS[name]
    if overrides:
        from dataclasses import replace
        cfg = replace(cfg, **overrides)
    return cfg
