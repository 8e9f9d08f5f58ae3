"""GPU parity of zo_generate (greedy generation with the K/V cache) against the oracle's
full-recompute greedy generation.

fp8 models follow the same checks with the fp8 scoring bounds (6e-2 OPT, 1.2e-1 Qwen3).

Several continuations can be correct where two logits are closer than the arithmetic's
error, so the comparison follows the GPU's own choices: the oracle re-runs every step
along the GPU's tokens (teacher forcing) and checks that
  * each GPU token is a valid greedy choice: its oracle log-prob is within CHOICE_TOL of
    the oracle's maximum at that step (exactly the argmax unless two logits nearly tie);
  * each GPU log-prob equals the oracle's for that token (fp32 models 1e-4 absolute,
    bf16 models 2e-2, the per-token bound of scoring);
  * the per-candidate sums S agree to the per-token bound times the tokens summed.
"""
import numpy as np
import pytest

from oracle import zo as ozo
from synth import configs, inputs

from .gpu_common import (SMALL_OPT_BF16, SMALL_OPT_FP8, SMALL_QWEN_BF16, SMALL_QWEN_FP8, GpuRun, OracleRun, flush,
                         need_gpu, workload)

pytestmark = pytest.mark.gpu

TINY_F32 = configs.CONFIGS["tiny"].model


@pytest.mark.parametrize("cfg,n_prompts,len_lo,len_hi,n_new",
                         [(TINY_F32, 2, 5, 70, 12), (SMALL_OPT_BF16, 2, 5, 70, 12), (SMALL_QWEN_BF16, 2, 5, 70, 12),
                          (SMALL_QWEN_BF16, 1, 600, 700, 3), (SMALL_OPT_FP8, 2, 5, 70, 12),
                          (SMALL_QWEN_FP8, 2, 5, 70, 12)],
                         ids=["tiny-f32", "opt-bf16", "qwen3-bf16", "qwen3-bf16-long", "opt-fp8", "qwen3-fp8"])
def test_generation_matches_oracle(cfg, n_prompts, len_lo, len_hi, n_new):
    """Two directions, a bank entry, a foreground prompt; prompts of 5..70 tokens and 12
    new tokens, so the cached keys of the longer ones span two 64-key chunks; "long":
    prompts of 600..700 tokens, where decode attention splits the keys over four waves."""
    need_gpu()
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=1, n_prompts=n_prompts, len_lo=len_lo, len_hi=len_hi)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c0 = np.array([0.9, -1.7])
    g.update(0, c0, 5e-3)
    o.update(0, c0, 5e-3)
    flush("generate %s, prompts %d..%d" % (cfg.arch, len_lo, len_hi))
    out = g.zo.generate(g.model, g.plan(1), g.bank, g.zo.DeviceBatch(batch), n_new)
    tok = out["tokens"].cpu().numpy()
    lp = out["logp"].cpu().numpy()
    ref = ozo.generate(cfg, o.W, ozo.plan_from_workload(wl, 1), o.bank, batch, n_new, forced=tok)
    # fp8 models: the per-token bound that tests/golden/make_fp8_floor.py derives from the
    # oracle for the same small model (tests/test_gpu_parity.py fp8_bounds)
    if cfg.dtype == "fp8":
        from .test_gpu_parity import fp8_bounds
        b = fp8_bounds("opt-small-fp8" if cfg.arch == "opt" else "qwen3-small-fp8")[1]
        lp_tol, choice_tol = b, b
    else:
        lp_tol, choice_tol = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}[cfg.dtype]
    gap = ref["best_logp"] - ref["logp"]
    flush("max choice gap %.3g, max |dlogp| %.3g, exact argmax %d of %d" % (
        gap.max(), np.abs(lp - ref["logp"]).max(), int((tok == ref["best_tok"]).sum()), tok.size))
    assert np.all(gap <= choice_tol)
    assert np.max(np.abs(lp - ref["logp"])) <= lp_tol
    per_cand = sum(1 for li, c in ref["phys"] if c == 0) * n_new
    assert np.all(np.abs(out["S"] - ref["S"]) <= lp_tol * per_cand)
    assert np.mean(tok == ref["best_tok"]) >= 0.8


def test_generation_rejections():
    """Two-term plans are refused (ZO_E_INVAL), and so is a continuation past max_pos
    (ZO_E_SHAPE)."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl2 = workload(SMALL_OPT_BF16, n_prompts=2, len_lo=500, len_hi=510)
    g2 = GpuRun(wl2)
    db2 = zo.DeviceBatch(inputs.make_batch(wl2))
    with pytest.raises(zo.ZoError) as ei:
        zo.generate(g2.model, g2.plan(0, flags=zo.api.PLAN_ACT_SPLIT), None, db2, 4)
    assert ei.value.code == -1
    with pytest.raises(zo.ZoError) as ei:
        zo.generate(g2.model, g2.plan(0), None, db2, 16)     # 510 + 15 > max_pos 512
    assert ei.value.code == -2


def test_generative_zo_step_matches_oracle():
    """A whole ZO step on a generative objective (fp32 tiny model): S from zo_generate, c
    from zo_estimate, the factor update; the oracle follows the GPU's continuations, its
    c agrees within 1e-2 relative and, given the same c, the updated factors are equal."""
    need_gpu()
    wl = workload(TINY_F32, dir_seeds=(3, 8), n_fg=1, n_prompts=2, len_lo=5, len_hi=40)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    n_new = 8
    for t in range(2):
        out = g.zo.generate(g.model, g.plan(t), g.bank, g.zo.DeviceBatch(batch), n_new)
        plan_o = ozo.plan_from_workload(wl, t)
        ref = ozo.generate(TINY_F32, o.W, plan_o, o.bank, batch, n_new, forced=out["tokens"].cpu().numpy())
        assert np.array_equal(out["tokens"].cpu().numpy(), ref["best_tok"])
        cg = g.zo.estimate(g.plan(t), out["S"])
        co = ozo.estimate(plan_o, ref["S"])
        flush("step %d: c gpu %s oracle %s" % (t, cg, co))
        assert np.all(np.abs(cg - co) <= 1e-2 * np.abs(co))
        g.update(t, cg, 1e-2)
        o.update(t, cg, 1e-2)
        for slot, e in enumerate(o.bank.entries):
            if e is None:
                continue
            for (layer, kind), U in e.U.items():
                assert np.array_equal(g.bank.entry(slot, layer, kind).cpu().numpy(), U.astype(np.float32))


def test_generation_edge_cases():
    """Foreground-only batch (no candidate: S is zero, tokens as the oracle's under W), one
    new token (prefill only), and an empty batch."""
    need_gpu()
    wl = workload(SMALL_OPT_BF16, n_fg=2, n_prompts=0, len_lo=5, len_hi=40)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    for n_new in (1, 5):
        out = g.zo.generate(g.model, g.plan(0), None, g.zo.DeviceBatch(batch), n_new)
        tok = out["tokens"].cpu().numpy()
        ref = ozo.generate(SMALL_OPT_BF16, o.W, ozo.plan_from_workload(wl, 0), None, batch, n_new, forced=tok)
        assert np.all(out["S"] == 0.0) and tok.shape == (2, n_new)
        assert np.all(ref["best_logp"] - ref["logp"] <= 2e-2)
        assert np.max(np.abs(out["logp"].cpu().numpy() - ref["logp"])) <= 2e-2
    empty = g.zo.generate(g.model, g.plan(0), None, g.zo.DeviceBatch(batch.subset([])), 3)
    assert empty["n_phys"] == 0 and np.all(empty["S"] == 0.0)
