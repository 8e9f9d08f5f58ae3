"""Model shapes and workload descriptions.

The five workloads are the tiny OPT-style case, OPT-1.3B, OPT-13B (batch 64,
the headline), the OPT-6.7B high-rank factorized case and the Qwen3-8B mixed
co-serving batch.  The pages name the OPT family 1.3B-13B ("Zeroth-Order
Fine-Tuning Was an Inference Workload All Along", section "The System
Reorganization") and Qwen3-8B co-serving (arXiv abstract page of
"Inference-Native Zeroth-Order Optimization"); the layer shapes are the public
architecture shapes of those families, with random weights.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple

KIND_NAMES_OPT = ("q", "k", "v", "o", "fc1", "fc2")
KIND_NAMES_QWEN3 = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass(frozen=True)
class ModelCfg:
    arch: str            # "opt" or "qwen3"
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    max_pos: int
    dtype: str           # "f32", "bf16" or "fp8" (OPT: e4m3 layer linears and linear inputs)
    norm_eps: float
    rope_theta: float = 0.0

    @property
    def kind_names(self):
        return KIND_NAMES_OPT if self.arch == "opt" else KIND_NAMES_QWEN3

    def linear_shape(self, kind: str) -> Tuple[int, int]:
        """(n_out, n_in) of the linear named `kind`."""
        d, hq, hkv, hd, f = self.d_model, self.n_heads, self.n_kv_heads, self.head_dim, self.d_ffn
        table = {
            "q": (hq * hd, d), "k": (hkv * hd, d), "v": (hkv * hd, d), "o": (d, hq * hd),
            "fc1": (f, d), "fc2": (d, f), "gate": (f, d), "up": (f, d), "down": (d, f),
        }
        return table[kind]


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelCfg
    n_prompts: int                 # probe prompts (each scored under every candidate)
    len_lo: int
    len_hi: int
    token_dist: str                # "uniform" or "zipf"
    score_mode: str                # score mode of the probe sequences: "last_label" or "all_next"
    rank: int
    eps: float
    dir_seeds: Tuple[int, ...]     # one seed per direction
    targets: Tuple[str, ...]       # linear kinds that carry the side path
    nu: int = 1024                 # lazy-sampling window (V fixed for nu steps)
    n_fg: int = 0                  # foreground sequences (no adapter)
    fg_score_mode: str = "all_next"
    verbalizers: Tuple[int, int] = (11, 13)
    model_seed: int = 0
    data_seed: int = 0
    scale_inv_sqrt_r: bool = False
    # score with two-term bf16 activations (hi + lo), fp32 attention and three-term side
    # products: a precision choice of the GPU path for summed long-sequence losses and deep
    # stacks; the oracle is exact either way
    act_split: bool = False
    # the same at single rounding sites only (a mask of the library's two-term site flags)
    split_sites: int = 0

    @property
    def n_dirs(self):
        return len(self.dir_seeds)

    @property
    def candidates(self):
        """(direction, sign) pairs: direction-major, + before -."""
        return tuple((d, s) for d in range(self.n_dirs) for s in (+1, -1))

    def with_(self, **kw):
        return replace(self, **kw)


TINY = ModelCfg("opt", 2, 128, 4, 4, 32, 512, 512, 2048, "f32", 1e-5)
OPT_1_3B = ModelCfg("opt", 24, 2048, 32, 32, 64, 8192, 50272, 2048, "bf16", 1e-5)
OPT_13B = ModelCfg("opt", 40, 5120, 40, 40, 128, 20480, 50272, 2048, "bf16", 1e-5)
OPT_6_7B = ModelCfg("opt", 32, 4096, 32, 32, 128, 16384, 50272, 2048, "bf16", 1e-5)
# the fp8-quantized OPT-13B (e4m3 layer linears and linear inputs, bf16 embeddings)
OPT_13B_FP8 = ModelCfg("opt", 40, 5120, 40, 40, 128, 20480, 50272, 2048, "fp8", 1e-5)
QWEN3_8B = ModelCfg("qwen3", 36, 4096, 32, 8, 128, 12288, 151936, 40960, "bf16", 1e-6, 1e6)
QWEN3_8B_FP8 = ModelCfg("qwen3", 36, 4096, 32, 8, 128, 12288, 151936, 40960, "fp8", 1e-6, 1e6)

_ALL_OPT = ("q", "k", "v", "o", "fc1", "fc2")
_ALL_QWEN = ("q", "k", "v", "o", "gate", "up", "down")

CONFIGS = {
    "tiny": Workload("tiny", TINY, 4, 32, 32, "uniform", "last_label", 2, 1e-3, (0,), ("q", "v")),
    "opt1.3b": Workload("opt1.3b", OPT_1_3B, 16, 16, 64, "zipf", "last_label", 2, 1e-3, (0,), _ALL_OPT),
    "opt13b": Workload("opt13b", OPT_13B, 64, 16, 128, "zipf", "last_label", 2, 1e-3, (0,), _ALL_OPT),
    # one GPU's share of the batch-64 step split data-parallel over 8 GPUs (8 prompts)
    "opt13b-share8": Workload("opt13b-share8", OPT_13B, 8, 16, 128, "zipf", "last_label", 2, 1e-3, (0,), _ALL_OPT),
    "opt13b-fp8": Workload("opt13b-fp8", OPT_13B_FP8, 64, 16, 128, "zipf", "last_label", 2, 1e-3, (0,), _ALL_OPT),
    "opt6.7b-mezo": Workload("opt6.7b-mezo", OPT_6_7B, 32, 128, 128, "zipf", "all_next", 64, 1e-3,
                             (0, 1, 2, 3), _ALL_OPT, scale_inv_sqrt_r=True, act_split=True),
    "qwen3-8b-mixed": Workload("qwen3-8b-mixed", QWEN3_8B, 16, 32, 512, "zipf", "last_label", 4, 1e-3,
                               (0,), _ALL_QWEN, n_fg=32, fg_score_mode="all_next", act_split=True),
    # the same mixed batch on the fp8-quantized model (e4m3 layer linears and linear inputs)
    "qwen3-8b-fp8": Workload("qwen3-8b-fp8", QWEN3_8B_FP8, 16, 32, 512, "zipf", "last_label", 4, 1e-3,
                             (0,), _ALL_QWEN, n_fg=32, fg_score_mode="all_next"),
}


def get(name: str) -> Workload:
    return CONFIGS[name]
