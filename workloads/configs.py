"""Model shapes and workloads.

Shapes follow the draft models the pages describe: a Qwen3-8B-shaped draft
with block size 16 (SGLang PR "Spec V2 DFlash Support", Benchmarks) and the
Kimi-K2.6-DFlash draft (CSDN DFlash article, the config.json sample: 6 layers,
5 sliding-window layers of 2048 and one full layer, 64 q / 8 kv heads,
head_dim 128, block size 8, mask token id 163838).

Values the pages leave open are fixed here and applied identically by the HIP
path and the oracle: RMSNorm epsilon 1e-6, RoPE theta 1e6, a page size of 16
tokens, the mask token id V-2 for the Qwen3-shaped drafts and an intermediate
size of 3*hidden for the Kimi-shaped draft.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class DFlashConfig:
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    n_target_layers: int
    target_hidden: int
    block_size: int
    mask_token_id: int
    page_size: int = 16
    sliding_window: Tuple[int, ...] = ()   # per layer; 0 = full attention
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    act_dtype: str = "bf16"                # "f32" | "bf16": weights, features, logits
    kv_dtype: str = "bf16"                 # "f32" | "bf16" | "fp8_e4m3"
    context_window: int = 0                # draft window: last N context rows (0 = all)

    @property
    def feat_dim(self) -> int:
        return self.n_target_layers * self.target_hidden

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def window(self, layer: int) -> int:
        if not self.sliding_window:
            return 0
        return int(self.sliding_window[layer])

    @property
    def kv_bytes_per_token(self) -> int:
        nb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[self.kv_dtype]
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim * nb


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: DFlashConfig
    batch: int
    ctx: Tuple[int, int]            # prefix length range, inclusive (lo == hi: fixed)
    commit: Tuple[int, int] = (1, 0)  # planted commit lengths range; hi 0 = block size
    inject_rows: int = 0            # prefill rows per request injected before drafting
    seed: int = 0
    desc: str = ""
    extra: dict = field(default_factory=dict)


TINY = DFlashConfig(hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    inter=512, vocab=1024, n_target_layers=2, target_hidden=256,
                    block_size=4, mask_token_id=1022, act_dtype="f32", kv_dtype="f32")

QWEN3_8B_DRAFT = DFlashConfig(hidden=4096, n_layers=5, n_q_heads=32, n_kv_heads=8,
                              head_dim=128, inter=12288, vocab=151936, n_target_layers=5,
                              target_hidden=4096, block_size=16, mask_token_id=151934)

KIMI_DRAFT = DFlashConfig(hidden=7168, n_layers=6, n_q_heads=64, n_kv_heads=8, head_dim=128,
                          inter=21504, vocab=163840, n_target_layers=6, target_hidden=7168,
                          block_size=8, mask_token_id=163838,
                          sliding_window=(2048, 2048, 2048, 2048, 2048, 0),
                          kv_dtype="fp8_e4m3")

# Small shapes for parity at sizes the oracle finishes in seconds: several
# tiles in every dimension plus ragged tails (vocab and feature widths that are
# not multiples of the kernel tiles, ragged prefixes, partial pages).
SMALL_BF16 = DFlashConfig(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                          inter=1536, vocab=5003, n_target_layers=3, target_hidden=352,
                          block_size=16, mask_token_id=5001)
SMALL_SWA_FP8 = DFlashConfig(hidden=512, n_layers=3, n_q_heads=8, n_kv_heads=1, head_dim=128,
                             inter=1024, vocab=3001, n_target_layers=2, target_hidden=384,
                             block_size=8, mask_token_id=2999, sliding_window=(40, 0, 24),
                             kv_dtype="fp8_e4m3")
SMALL_F32_D64 = DFlashConfig(hidden=192, n_layers=2, n_q_heads=6, n_kv_heads=3, head_dim=64,
                             inter=320, vocab=777, n_target_layers=3, target_hidden=96,
                             block_size=5, mask_token_id=775, sliding_window=(0, 33),
                             act_dtype="f32", kv_dtype="f32")
# Wide enough (hidden 2048) and batched enough (24 x 16 rows) that every GEMM
# of the draft pass and of a >128-row injection takes the LDS-tiled path with
# a split K and a ragged last row tile.
SMALL_BF16_WIDE = DFlashConfig(hidden=2048, n_layers=1, n_q_heads=16, n_kv_heads=4,
                               head_dim=128, inter=2560, vocab=4099, n_target_layers=2,
                               target_hidden=1088, block_size=16, mask_token_id=4097,
                               sliding_window=(96,))
# A vocabulary of 70001 (547 128-column tiles, the last one ragged): at 65..128
# rows the lm_head takes the tall-tile path.
SMALL_BF16_VOCAB_WIDE = DFlashConfig(hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=1,
                                     head_dim=64, inter=512, vocab=70001, n_target_layers=2,
                                     target_hidden=256, block_size=16, mask_token_id=69990)
# A vocabulary wide enough (32777, an odd number of 128-column tiles) that the
# lm_head of 24 x 15 rows takes the 256 x 256-tile path with a ragged last
# row tile and a half-empty last column tile.
SMALL_BF16_VOCAB = DFlashConfig(hidden=512, n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                inter=1024, vocab=32777, n_target_layers=2, target_hidden=256,
                                block_size=16, mask_token_id=32770)

WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", TINY, batch=1, ctx=(64, 64), inject_rows=64,
                         desc="tiny DFlash draft, fp32, 1 layer, block 4, 64 context tokens"),
    "qwen3_8b_b16": Workload("qwen3_8b_b16", QWEN3_8B_DRAFT, batch=1, ctx=(4096, 4096),
                             inject_rows=4096,
                             desc="Qwen3-8B-shaped draft, bf16, block 16, batch 1, 4096 context"),
    "qwen3_8b_b16_bs32": Workload("qwen3_8b_b16_bs32", QWEN3_8B_DRAFT, batch=32,
                                  ctx=(512, 8192), commit=(1, 16),
                                  desc="Qwen3-8B-shaped draft, batch 32, ragged context 512..8192"),
    "qwen3_8b_prefill": Workload("qwen3_8b_prefill", QWEN3_8B_DRAFT, batch=8,
                                 ctx=(16384, 16384), inject_rows=16384,
                                 desc="prefill injection of 8 x 16384 rows, then one draft pass"),
    "kimi_k26_b8": Workload("kimi_k26_b8", KIMI_DRAFT, batch=16, ctx=(32768, 32768),
                            commit=(1, 8),
                            desc="Kimi-K2.6-DFlash-shaped draft, fp8 KV, batch 16, 32768 context"),
    "kimi_k26_b8_w4096": Workload("kimi_k26_b8_w4096",
                                  replace(KIMI_DRAFT, context_window=4096),
                                  batch=16, ctx=(32768, 32768), commit=(1, 8),
                                  desc="the Kimi-shaped workload with a 4096-row draft window"),
    # small parity workloads
    "small_bf16": Workload("small_bf16", SMALL_BF16, batch=3, ctx=(37, 301), commit=(1, 16),
                           inject_rows=0, seed=1),
    "small_swa_fp8": Workload("small_swa_fp8", SMALL_SWA_FP8, batch=4, ctx=(5, 150),
                              commit=(1, 8), seed=2),
    "small_f32_d64": Workload("small_f32_d64", SMALL_F32_D64, batch=2, ctx=(1, 70),
                              commit=(1, 5), seed=3),
    "small_bf16_wide": Workload("small_bf16_wide", SMALL_BF16_WIDE, batch=24, ctx=(20, 200),
                                commit=(1, 16), seed=4),
    "small_bf16_vocab": Workload("small_bf16_vocab", SMALL_BF16_VOCAB, batch=24, ctx=(3, 90),
                                 commit=(1, 16), seed=5),
    # 65..128 rows: 7 x 16 = 112 rows (128-row tiles, every GEMM with a split
    # K); 8 x 16 = 128 rows over a 70001-token vocabulary (the lm_head's 120
    # rows on the tall-tile path)
    "small_bf16_tall": Workload("small_bf16_tall", SMALL_BF16_WIDE, batch=7, ctx=(20, 200),
                                commit=(1, 16), seed=6),
    "small_bf16_vocab_tall": Workload("small_bf16_vocab_tall", SMALL_BF16_VOCAB_WIDE, batch=8,
                                      ctx=(3, 90), commit=(1, 16), seed=7),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
