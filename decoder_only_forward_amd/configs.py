"""Model shapes of the decoder-block forward, as plain numbers.

Each shape follows the model table of the Pantheon page "Llama Forward Pass"
(sections "Grouped Query Attention", "Architecture Differences") and the
rml page "The decoder" (section "The model config"): one recipe with switches
(q/k/v bias, sliding window, experts).  Nothing here computes anything; the
same objects describe a model to the HIP library and to the CPU oracle.

Readings where the pages leave a value open:
  * eps defaults to 1e-5 (Pantheon, "RMSNorm") where a shape names none;
  * the Qwen2.5-0.5B shape ties its LM head to the embedding, as that model does;
  * Mixtral uses rope theta 10000 (Pantheon, "Architecture Differences").
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

WEIGHT_BF16 = 0
WEIGHT_F32 = 1


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    n_experts: int = 0          # 0 = dense SwiGLU FFN
    top_k: int = 0
    qkv_bias: bool = False
    tied_embedding: bool = False
    sliding_window: int = 0     # 0 = full causal range
    max_seq: int = 0            # KV positions per sequence (ring size when windowed)
    weight_dtype: int = WEIGHT_BF16
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    # RoPE variants (rml "The decoder", "Rotary embeddings"): pairing 0 rotates
    # adjacent elements (2i, 2i+1), 1 rotates halves (i, i + hd/2); scaling 1 is
    # llama3 frequency scaling with these parameters.
    rope_pairing: int = 0
    rope_scaling: int = 0
    rope_factor: float = 8.0
    rope_low_freq_factor: float = 1.0
    rope_high_freq_factor: float = 4.0
    rope_orig_ctx: int = 8192
    # K/V cache element type: fp32 by default; kv_bf16: bf16 (rounded to
    # nearest even); kv_f24: a 24-bit float (fp32 rounded to nearest even at
    # 15 stored mantissa bits, 16 significant bits).  At most one is set.
    kv_bf16: bool = False
    kv_f24: bool = False
    # Prefill projections (more than 64 rows) on fp16 + fp8 split operands
    # instead of the bf16 (hi, lo) pair: an arithmetic choice of the GPU path
    # (DEC_PREFILL_F16_F8), not part of the model; the oracle ignores it.
    prefill_fp8: bool = False

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_heads // self.n_kv_heads

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)

    def matrix_params(self) -> int:
        """Matrix parameters (the counting rule of rml's ParameterCount,
        "The decoder", section "From GGUF metadata"), without fp32 norms and biases."""
        d, q, kv, f = self.hidden, self.q_dim, self.kv_dim, self.ffn_dim
        attn = d * q + 2 * d * kv + q * d
        if self.n_experts:
            ffn = self.n_experts * 3 * d * f + self.n_experts * d
        else:
            ffn = 3 * d * f
        emb = self.vocab * d
        head = 0 if self.tied_embedding else self.vocab * d
        return self.n_layers * (attn + ffn) + emb + head


# The five shapes of the build, with their workloads in the docstrings of tests/bench.
TINY = ModelConfig("tiny", n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16,
                   ffn_dim=172, vocab=256, max_seq=16, weight_dtype=WEIGHT_F32,
                   rms_eps=1e-5, rope_theta=1e4)
SMOLLM2 = ModelConfig("smollm2-135m", n_layers=30, hidden=576, n_heads=9, n_kv_heads=3,
                      head_dim=64, ffn_dim=1536, vocab=49152, tied_embedding=True,
                      max_seq=256, rms_eps=1e-5, rope_theta=1e4)
QWEN25 = ModelConfig("qwen2.5-0.5b", n_layers=24, hidden=896, n_heads=14, n_kv_heads=2,
                     head_dim=64, ffn_dim=4864, vocab=151936, qkv_bias=True,
                     tied_embedding=True, max_seq=2304, rms_eps=1e-6, rope_theta=1e6)
MISTRAL = ModelConfig("mistral-7b", n_layers=32, hidden=4096, n_heads=32, n_kv_heads=8,
                      head_dim=128, ffn_dim=14336, vocab=32000, sliding_window=4096,
                      max_seq=4096, rms_eps=1e-5, rope_theta=1e4)
MIXTRAL = ModelConfig("mixtral-8x7b", n_layers=32, hidden=4096, n_heads=32, n_kv_heads=8,
                      head_dim=128, ffn_dim=14336, vocab=32000, n_experts=8, top_k=2,
                      max_seq=768, rms_eps=1e-5, rope_theta=1e4)

CONFIGS = {c.name: c for c in (TINY, SMOLLM2, QWEN25, MISTRAL, MIXTRAL)}

# Small variants that exercise the switches the tiny shape leaves off.
TINY_WINDOW = TINY.replace(name="tiny-window", sliding_window=5, max_seq=5)
TINY_MOE = TINY.replace(name="tiny-moe", n_experts=8, top_k=2)
TINY_BIAS = TINY.replace(name="tiny-bias", qkv_bias=True, tied_embedding=True)
TINY_BF16 = TINY.replace(name="tiny-bf16", weight_dtype=WEIGHT_BF16, ffn_dim=192)
# llama3 scaling with a context short enough that all three frequency bands occur
TINY_LLAMA3 = TINY.replace(name="tiny-llama3", rope_scaling=1, rope_factor=8.0, rope_low_freq_factor=1.0,
                           rope_high_freq_factor=4.0, rope_orig_ctx=64)
TINY_HALF = TINY.replace(name="tiny-half", rope_pairing=1)
TINY_KVBF16 = TINY_BF16.replace(name="tiny-kvbf16", kv_bf16=True)
TINY_KVF24 = TINY_BF16.replace(name="tiny-kvf24", kv_f24=True)


def one_layer(cfg: ModelConfig) -> ModelConfig:
    """Full-width shape with a single block: every kernel runs at its real size
    while a CPU oracle can still recompute sampled rows."""
    return cfg.replace(name=cfg.name + "-1l", n_layers=1)
