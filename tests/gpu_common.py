"""Shared helpers of the GPU tests: run the HIP path and the oracle on the same
seeded inputs."""
import numpy as np
import pytest

from oracle import zo as ozo
from synth import configs, inputs
from synth.configs import ModelCfg


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def flush(msg):
    print(msg, flush=True)


SMALL_OPT_BF16 = ModelCfg("opt", 2, 256, 4, 4, 64, 512, 1000, 512, "bf16", 1e-5)
# kind boundaries of the packed QKV (q | k | v) fall on 256-column tiles, as in the real shapes
SMALL_QWEN_BF16 = ModelCfg("qwen3", 2, 512, 4, 2, 128, 768, 1200, 1024, "bf16", 1e-6, 1e6)
# projection widths that are not multiples of the 256-wide tile (o-proj N = 320, fc1 N = 1280)
SMALL_OPT_ODD = ModelCfg("opt", 2, 320, 5, 5, 64, 1280, 1000, 512, "bf16", 1e-5)
# the fp8-quantized OPT (e4m3 layer linears and linear inputs; d and FFN multiples of 128)
SMALL_OPT_FP8 = ModelCfg("opt", 2, 256, 4, 4, 64, 512, 1000, 512, "fp8", 1e-5)
SMALL_QWEN_FP8 = ModelCfg("qwen3", 2, 512, 4, 2, 128, 768, 1200, 1024, "fp8", 1e-6, 1e6)
SMALL_QWEN_F32 = ModelCfg("qwen3", 2, 128, 4, 2, 32, 256, 300, 1024, "f32", 1e-6, 1e6)


def workload(cfg, **kw):
    base = dict(name="t", model=cfg, n_prompts=3, len_lo=5, len_hi=150, token_dist="zipf", score_mode="last_label",
                rank=2, eps=1e-3, dir_seeds=(0,), targets=cfg.kind_names, nu=4)
    base.update(kw)
    return configs.Workload(**base)


class GpuRun:
    """Model + plan + bank on the GPU for a workload, one call per step."""

    def __init__(self, wl, n_slots=4):
        import zeroth_order_fine_amd as zo
        self.zo = zo
        self.wl = wl
        self.model = zo.Model(wl.model)
        self.model.init_weights(wl.model_seed)
        self.bank = zo.Bank(self.model, n_slots, wl.rank, wl.targets)

    def plan(self, t, **kw):
        return self.zo.Plan.from_workload(self.model, self.wl, t=t, **kw)

    def score(self, t, batch, want_tokens=True, bank=True, **kw):
        return self.zo.score(self.model, self.plan(t, **kw), self.bank if bank else None,
                             self.zo.DeviceBatch(batch), want_tokens=want_tokens)

    def update(self, t, c, lr):
        self.zo.update(self.model, self.plan(t), self.bank, c, lr)


class OracleRun:
    def __init__(self, wl, n_slots=4):
        self.wl = wl
        self.W = ozo.Weights(wl.model, wl.model_seed, cache_layers=True)
        self.bank = ozo.Bank(n_slots, wl.rank, wl.targets)

    def score(self, t, batch, bank=True, **kw):
        plan = ozo.plan_from_workload(self.wl, t)
        for k, v in kw.items():
            setattr(plan, k, v)
        return ozo.score(self.wl.model, self.W, plan, self.bank if bank else None, batch)

    def update(self, t, c, lr):
        ozo.update(self.wl.model, ozo.plan_from_workload(self.wl, t), self.bank, c, lr)
