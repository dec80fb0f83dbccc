"""Workload presets: model shapes, seeds and run parameters.

Each preset describes one synthetic workload (shapes, dtype, seeds, context,
draft length, batch).  Shapes follow the Gemma-4-family descriptions on the
pages (drafter four layers wide 256 reading the backbone hidden state, page 5
"What is different about Gemma 4's drafter"; 2048 centroids, same section)
and the five workload lines the build is measured on.  Nothing here computes
any part of the decoding method.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

__all__ = ["ModelConfig", "PRESETS", "preset", "truncated"]


@dataclass(frozen=True)
class ModelConfig:
    name: str
    # target decoder
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    # mixture of experts (n_experts == 0 means a dense gated FFN)
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    shared_ffn: int = 0
    # drafter
    d_layers: int = 4
    d_dim: int = 256
    d_ffn: int = 1024
    n_centroids: int = 2048
    kv_src_layer: int = -1  # -1 means the target's last layer
    # numerics
    dtype: str = "bf16"  # storage dtype of weights / KV / GEMM inputs: "bf16" or "f32"
    # "dense" (weights in dtype) or "q4" (every weight matrix in 32-element blocks of 4-bit codes
    # and an fp16 step; bf16 activations)
    weight_format: str = "dense"
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    # weight generator: "normal" (numpy default_rng per tensor) or "hash" (counter hash, bf16)
    init: str = "hash"
    seed: int = 0
    weight_std: float = 0.02
    norm_jitter: float = 0.0  # 0 => all norm weights are exactly 1
    # run parameters
    ctx: int = 0  # committed context at the start of the timed window (synthetic KV)
    prompt_len: int = 0  # real prompt (tiny config) instead of synthetic KV
    gen_tokens: int = 64
    draft_k: int = 3
    batch: int = 1
    p_inject: float = 0.7
    kv_seed: int = 100
    state_seed: int = 300
    perm_seed: int = 500
    inject_seed: int = 700

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def cluster_size(self) -> int:
        return self.vocab // self.n_centroids

    @property
    def src_layer(self) -> int:
        return self.n_layers - 1 if self.kv_src_layer < 0 else self.kv_src_layer

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)

    def target_params(self) -> int:
        d, L = self.d_model, self.n_layers
        attn = d * (self.q_dim + 2 * self.kv_dim) + self.q_dim * d
        if self.is_moe:
            ffn = self.n_experts * 3 * d * self.expert_ffn + 3 * d * self.shared_ffn + self.n_experts * d
        else:
            ffn = 3 * d * self.ffn_dim
        return self.vocab * d + L * (attn + ffn + 2 * d) + d

    def drafter_params(self) -> int:
        D, d = self.d_dim, self.d_model
        per = D * self.q_dim * 2 + 3 * D * self.d_ffn + 2 * D
        return (self.vocab * D + self.n_centroids * D + D * (d + D) + self.d_layers * per
                + d * D + d + 2 * D)


PRESETS = {
    # Tiny CPU-seconds configuration: 2 layers, d=256, 4/2 heads of 64, FFN 1024,
    # vocab 4096, fp32 N(0, 0.02); drafter 1 layer d=128, 64 centroids x 64 tokens;
    # prompt of 64 uniform ids, 64 generated tokens, K=3, batch 1.
    "tiny": ModelConfig(
        name="tiny", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        ffn_dim=1024, vocab=4096, d_layers=1, d_dim=128, d_ffn=512, n_centroids=64,
        dtype="f32", init="normal", seed=0, prompt_len=64, gen_tokens=64, draft_k=3,
        p_inject=0.6),
    # The tiny configuration's mixture-of-experts twin: each layer's FFN is the softmax-weighted
    # sum of its top-4 of 16 gated experts of width 128 plus a shared gated FFN of 256.
    "tiny-moe": ModelConfig(
        name="tiny-moe", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        ffn_dim=0, vocab=4096, n_experts=16, top_k=4, expert_ffn=128, shared_ffn=256,
        d_layers=1, d_dim=128, d_ffn=512, n_centroids=64, dtype="f32", init="normal", seed=8,
        prompt_len=64, gen_tokens=64, draft_k=3, p_inject=0.6),
    # E2B-shaped
    "e2b": ModelConfig(
        name="e2b", n_layers=24, d_model=1536, n_q_heads=8, n_kv_heads=1, head_dim=256,
        ffn_dim=6144, vocab=262144, seed=1, ctx=2048, draft_k=3, kv_seed=101),
    # E4B-shaped
    "e4b": ModelConfig(
        name="e4b", n_layers=34, d_model=2560, n_q_heads=8, n_kv_heads=2, head_dim=256,
        ffn_dim=10240, vocab=262144, seed=2, ctx=4096, draft_k=4, kv_seed=102),
    # 31B-class dense
    "31b": ModelConfig(
        name="31b", n_layers=64, d_model=5120, n_q_heads=40, n_kv_heads=8, head_dim=128,
        ffn_dim=25600, vocab=262144, seed=3, ctx=8192, draft_k=3, kv_seed=103),
    # One GPU's share of the 31B-class model under 8-way tensor parallelism: q/k/v and gate/up
    # split by output columns (5 of 40 query heads, 1 of 8 KV heads, 3200 of 25600 FFN columns),
    # o and down by input rows (the residual stream keeps its full width), the tied LM head by
    # vocabulary (32768 of 262144 rows).  The drafter covers the same vocabulary slice with 512
    # centroids of 64 tokens (the sharded design replicates the full drafter instead).
    "31b-tp8": ModelConfig(
        name="31b-tp8", n_layers=64, d_model=5120, n_q_heads=5, n_kv_heads=1, head_dim=128,
        ffn_dim=3200, vocab=32768, n_centroids=512, seed=5, ctx=8192, draft_k=3, kv_seed=105),
    # 26B-class MoE
    "moe": ModelConfig(
        name="moe", n_layers=30, d_model=2816, n_q_heads=16, n_kv_heads=4, head_dim=176,
        ffn_dim=0, vocab=262144, n_experts=128, top_k=8, expert_ffn=1408, shared_ffn=5632,
        seed=4, ctx=4096, draft_k=3, kv_seed=104),
}


def preset(name: str, **overrides) -> ModelConfig:
    return PRESETS[name].replace(**overrides)


def truncated(name: str, n_layers: int, **overrides) -> ModelConfig:
    """Depth-truncated variant of a preset: full width and vocab, fewer layers."""
    return PRESETS[name].replace(n_layers=n_layers, name=f"{name}-L{n_layers}", **overrides)
