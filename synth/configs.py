"""Model geometry and workload presets for the DSpark draft pass.

This module holds sizes and storage choices only: no arithmetic of the method.
It is shared by the oracle tests and by the GPU tests / bench, which is why it
lives outside both `oracle/` and `mla_block_drafter_amd/`.

Geometry sources (pages on "mla_block_drafter"):
  * alphaneural.io "kimi-k3-dspark-gguf", section "How it works" and the GGUF
    metadata table: 5 MLA layers, q_lora_rank 1536, kv_lora_rank 512, block 7,
    hidden 7168, vocab 163,840.
  * graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", section "Architecture
    metadata": Markov rank 256, YaRN-16 from a 65,536 window, five captured
    target states feeding fc.
  * huggingface.co "Kimi-K3-DSpark-NVFP4", section "Model Overview" of the
    original card: 576-element latent per token (512 + 64 rope), non-causal
    block attention; section "What is quantized to what": which tensors are
    quantised.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional

# Storage formats (mirrors DSPARK_DT_* in include/dspark.h).
F32 = "f32"
BF16 = "bf16"
Q8_0 = "q8_0"
FP8 = "fp8_e4m3"
MXFP4 = "mxfp4"


@dataclass(frozen=True)
class ModelConfig:
    hidden: int = 7168
    n_layers: int = 5
    n_heads: int = 64
    q_lora: int = 1536
    kv_lora: int = 512
    qk_nope: int = 128
    qk_rope: int = 64
    v_head: int = 128
    inter: int = 14336
    vocab: int = 163840
    markov_rank: int = 256
    block: int = 7
    n_captured: int = 5
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    yarn_factor: float = 16.0       # 1.0 = plain RoPE
    yarn_orig_ctx: int = 65536
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0

    @property
    def latent(self) -> int:
        return self.kv_lora + self.qk_rope

    @property
    def qk_head(self) -> int:
        return self.qk_nope + self.qk_rope


@dataclass(frozen=True)
class Formats:
    """Storage format per tensor group."""
    fc: str = Q8_0
    q_a: str = BF16          # q_a and kv_a (fused on the device)
    q_b: str = Q8_0
    kv_b: str = BF16
    o: str = Q8_0
    mlp: str = Q8_0          # gate, up, down
    lm_head: str = BF16
    markov: str = BF16       # W1, W2
    kv_cache: str = BF16
    captured: str = BF16
    # norms and confidence head are always f32


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    formats: Formats
    seed: int
    kv_lens: tuple          # cache length per sequence
    attn_only: bool = False  # one decoder layer, attention half only (a2-a8)
    fixture_gains: bool = False  # norm gains ~U(0.5,1.5), conf bias != 0
    sharp_attention: bool = False  # kv_b rows for W_UK scaled x10
    markov_dominant: bool = False  # W1, W2 ~ N(0, R^-1/2); lm_head = 0
    weight_std: float = 0.02
    spike: tuple = ()        # (cache row, factor): that row of every cache scaled (a far-away dominant key)
    captured_dist: str = "gauss"  # captured states: "gauss" N(0,1) or "heavy" (Student-t, 3 dof, unit variance)

    @property
    def n_seq(self) -> int:
        return len(self.kv_lens)

    @property
    def total_ctx(self) -> int:
        return int(sum(self.kv_lens))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = ModelConfig(hidden=512, n_layers=1, n_heads=8, q_lora=128, kv_lora=64,
                   qk_nope=32, qk_rope=16, v_head=32, inter=1024, vocab=4096,
                   markov_rank=16, yarn_factor=1.0)
FULL = ModelConfig()

ALL_F32 = Formats(fc=F32, q_a=F32, q_b=F32, kv_b=F32, o=F32, mlp=F32,
                  lm_head=F32, markov=F32, kv_cache=F32, captured=F32)
ALL_BF16 = Formats(fc=BF16, q_a=BF16, q_b=BF16, kv_b=BF16, o=BF16, mlp=BF16,
                   lm_head=BF16, markov=BF16)
Q8 = Formats()
FP8_PC = Formats(fc=FP8, q_b=FP8, o=FP8, mlp=FP8)
MX4 = Formats(fc=MXFP4, q_b=MXFP4, o=MXFP4, mlp=MXFP4)  # same tensor selection as FP8

SEED_BASE = 20261200


def _cfg5_lens(n: int = 16, lo: int = 1024, hi: int = 16384) -> tuple:
    import numpy as np
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 5, spawn_key=(9999,)))
    return tuple(int(v) for v in rng.integers(lo, hi + 1, size=n))


# The five workloads of the pass. cfg1 is the tiny all-fp32 drafter.
CFG1 = Workload("tiny_f32_ctx256", TINY, ALL_F32, SEED_BASE + 1, (256,))
CFG2 = Workload("mla_layer_bf16_ctx4096", ModelConfig(n_layers=1), ALL_BF16,
                SEED_BASE + 2, (4096,), attn_only=True)
CFG3 = Workload("full_q8_0_bs1_ctx8192", FULL, Q8, SEED_BASE + 3, (8192,))
CFG4 = Workload("full_bf16_bs1_ctx98304", FULL, ALL_BF16, SEED_BASE + 4, (98304,))
CFG5 = Workload("full_fp8_bs16_ragged", FULL, FP8_PC, SEED_BASE + 5, _cfg5_lens())

CFG6 = Workload("full_mxfp4_bs1_ctx8192", FULL, MX4, SEED_BASE + 6, (8192,))
CFG7 = Workload("full_fp8_bs1_ctx8192", FULL, FP8_PC, SEED_BASE + 7, (8192,))
PRESETS = {1: CFG1, 2: CFG2, 3: CFG3, 4: CFG4, 5: CFG5, 6: CFG6, 7: CFG7}


def small_model(**kw) -> ModelConfig:
    """A mid-size geometry with ragged (non tile-multiple) sizes for parity tests.

    hidden 352 (= 11 x 32, not a multiple of 64), 2 layers, 4 heads, vocab 1000
    (not a multiple of 16), inter 480, markov rank 24.
    """
    base = dict(hidden=352, n_layers=2, n_heads=4, q_lora=96, kv_lora=64,
                qk_nope=32, qk_rope=16, v_head=24, inter=480, vocab=1000,
                markov_rank=24, yarn_factor=4.0, yarn_orig_ctx=128)
    base.update(kw)
    return ModelConfig(**base)


def tensor_names(m: ModelConfig, attn_only: bool = False) -> List[str]:
    """Fixed, ordered tensor list; the index of a name seeds its random stream."""
    names = [] if attn_only else ["fc", "fc_norm"]
    for l in range(m.n_layers):
        p = f"L{l}."
        names += [p + "in_norm", p + "q_a", p + "q_a_norm", p + "kv_a", p + "kv_a_norm",
                  p + "q_b", p + "kv_b", p + "o"]
        if not attn_only:
            names += [p + "post_norm", p + "gate", p + "up", p + "down"]
    if not attn_only:
        names += ["final_norm", "lm_head", "markov_w1", "markov_w2", "conf_w", "conf_b"]
    return names


def tensor_shape(m: ModelConfig, name: str) -> tuple:
    base = name.split(".")[-1]
    H, nh = m.hidden, m.n_heads
    shapes = {
        "fc": (H, m.n_captured * H), "fc_norm": (H,), "in_norm": (H,),
        "q_a": (m.q_lora, H), "q_a_norm": (m.q_lora,),
        "kv_a": (m.latent, H), "kv_a_norm": (m.kv_lora,),
        "q_b": (nh * m.qk_head, m.q_lora),
        "kv_b": (nh * (m.qk_nope + m.v_head), m.kv_lora),
        "o": (H, nh * m.v_head), "post_norm": (H,),
        "gate": (m.inter, H), "up": (m.inter, H), "down": (H, m.inter),
        "final_norm": (H,), "lm_head": (m.vocab, H),
        "markov_w1": (m.vocab, m.markov_rank), "markov_w2": (m.vocab, m.markov_rank),
        "conf_w": (H + m.markov_rank,), "conf_b": (1,),
    }
    return shapes[base]


def tensor_format(f: Formats, name: str) -> str:
    base = name.split(".")[-1]
    if base in ("fc_norm", "in_norm", "q_a_norm", "kv_a_norm", "post_norm",
                "final_norm", "conf_w", "conf_b"):
        return F32
    return {"fc": f.fc, "q_a": f.q_a, "kv_a": f.q_a, "q_b": f.q_b, "kv_b": f.kv_b,
            "o": f.o, "gate": f.mlp, "up": f.mlp, "down": f.mlp,
            "lm_head": f.lm_head, "markov_w1": f.markov, "markov_w2": f.markov}[base]
