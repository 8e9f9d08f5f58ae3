"""Pins of the oracle's fp8 (OCP e4m3) model (oracle/params.py e4m3_round,
oracle/model.py quantization points).

* e4m3_round against PyTorch's float8_e4m3fn conversion (an independent
  implementation of the same format, round to nearest even) on random values,
  on every representable value and on every midpoint between neighbours;
* saturation at +-448 (the format's largest finite value) beyond the range;
* the fp8 weights are e4m3 values times 2^-11 and stay inside the range;
* the factorized side state equals dense mutation of the (quantized) weights.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import params, zo
from oracle.zo import Weights
from synth import configs, inputs

from .test_oracle_model import OPT_SMALL, QWEN_SMALL
from .test_oracle_zo import _bank_after_updates, _small_wl

OPT_FP8 = dataclasses.replace(OPT_SMALL, dtype="fp8")
QWEN_FP8 = dataclasses.replace(QWEN_SMALL, dtype="fp8")


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).double().numpy()


def _all_finite_values():
    v = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    return np.unique(v[np.isfinite(v)])


def test_e4m3_matches_library_on_random_values():
    rs = np.random.default_rng(3)
    x = np.concatenate([rs.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x[np.abs(x) < 448]
    assert np.array_equal(params.e4m3_round(x), _torch_e4m3(x))


def test_e4m3_fixed_points_and_ties_to_even():
    v = _all_finite_values()                      # 253 values (+0 and -0 merge)
    assert len(v) == 253 and v.max() == 448.0 and v[v > 0].min() == 2.0 ** -9
    assert np.array_equal(params.e4m3_round(v), v)
    mids = (v[:-1] + v[1:]) / 2                   # exactly representable in binary64
    got, ref = params.e4m3_round(mids), _torch_e4m3(mids)
    assert np.array_equal(got, ref)
    # each midpoint goes to the neighbour with an even mantissa (code bit 0 clear)
    codes = torch.from_numpy(got).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.all((codes & 1) == 0)


def test_e4m3_saturates():
    assert np.array_equal(params.e4m3_round(np.array([1e4, -1e4, 464.0, -500.0])), [448.0, -448.0, 448.0, -448.0])
    assert params.e4m3_round(np.array([2.0 ** -11]))[0] == 0.0      # below half the smallest subnormal


def test_fp8_weights_are_scaled_e4m3_values():
    W = Weights(OPT_FP8, 2, cache_layers=False)
    Wl = W.get_layer(0)
    for name in ("wq", "wk", "wv", "wo", "w_fc1", "w_fc2"):
        s = Wl[name] * 2.0 ** params.FP8_WEIGHT_EXP
        assert np.array_equal(params.e4m3_round(s), s) and np.abs(s).max() < 448
        assert len(np.unique(s)) > 100
    G = W.get_global()                             # embeddings stay bf16
    t = G["tok_embed"].astype(np.float32)
    assert np.array_equal(params.bf16_round(t), t)


@pytest.mark.parametrize("cfg", [OPT_FP8, QWEN_FP8], ids=["opt", "qwen3"])
def test_fp8_factorized_equals_dense_mutation(cfg):
    kinds = configs.KIND_NAMES_OPT if cfg.arch == "opt" else configs.KIND_NAMES_QWEN3
    wl = _small_wl(cfg, kinds, dirs=(0, 5), n_fg=1)
    bank = _bank_after_updates(cfg, wl)
    batch = inputs.make_batch(wl)
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 2)
    a = zo.score(cfg, W, plan, bank, batch)
    b = zo.score(cfg, W, plan, bank, batch, dense=True)
    assert np.allclose(a["seq_logp"], b["seq_logp"], rtol=1e-12, atol=0)
    assert np.ptp(a["S"]) > 0


@pytest.mark.parametrize("which", ["opt", "qwen3"])
def test_activation_rounding_is_visible_at_the_gpu_bound(which):
    """Rounding the four linear inputs to e4m3 moves the per-sequence sums of the GPU
    tests' models (same workload shape) by far more than the fp8 parity bound derived for
    them (tests/golden/fp8floor_*.json): a kernel that skipped it would fail those tests."""
    import dataclasses as dc
    from tests.gpu_common import SMALL_OPT_FP8, SMALL_QWEN_FP8, workload
    cfg_fp8 = SMALL_OPT_FP8 if which == "opt" else SMALL_QWEN_FP8
    cfg_noq = dc.replace(cfg_fp8, dtype="bf16")          # same weights, unrounded inputs
    wl = workload(cfg_fp8, dir_seeds=(3, 8), n_fg=2, n_prompts=3)
    batch = inputs.make_batch(wl)
    W = Weights(cfg_fp8, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 0)
    a = zo.score(cfg_fp8, W, plan, None, batch)
    b = zo.score(cfg_noq, W, plan, None, batch)
    gap = np.abs(np.asarray(a["seq_logp"]) - np.asarray(b["seq_logp"]))
    import json, os
    case = "opt-small-fp8" if which == "opt" else "qwen3-small-fp8"
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8floor_%s.json" % case)) as f:
        bound = json.load(f)["bound_seq"]
    # twice the derived bound (0.059 OPT, 0.119 Qwen3); measured max 0.20 / 0.66
    assert gap.max() > 2 * bound, (gap.max(), bound)


def test_error_model_is_off_by_default_and_exact_at_zero():
    """The tolerance error model (oracle.model jitter) changes nothing at delta = 0 and
    moves the sums once deltas reach e4m3-boundary distances (pinned: it is the knob the
    fp8 bounds are measured with)."""
    from tests.gpu_common import SMALL_OPT_FP8, workload
    wl = workload(SMALL_OPT_FP8, dir_seeds=(3,), n_prompts=2)
    batch = inputs.make_batch(wl)
    W = Weights(SMALL_OPT_FP8, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 0)
    a = zo.score(SMALL_OPT_FP8, W, plan, None, batch)
    z = zo.score(SMALL_OPT_FP8, W, plan, None, batch, e4m3_jitter=({"attn": 0.0, "norm": 0.0, "ffn": 0.0}, 1))
    assert np.array_equal(a["seq_logp"], z["seq_logp"])
    j = zo.score(SMALL_OPT_FP8, W, plan, None, batch, e4m3_jitter=({"attn": 2.0 ** -8, "norm": 0.0, "ffn": 0.0}, 1))
    assert not np.array_equal(a["seq_logp"], j["seq_logp"])
