"""Full-size parity: every workload at its real shape, in the launch
configuration bench.py times (whole batch, one zo_score call), against expected
values written by tests/golden/make_golden.py from the oracle alone.

State: one zo_update at step 0 with fixed coefficients, then zo_score at step 1.

Bound (bf16): the contract is on the per-candidate L+/- (S_c, a sum over the
candidate's sequences): |S_c - S_c(oracle)| <= 2e-2 per summed sequence.  Where
a workload scores with two-term activations (ZO_PLAN_ACT_SPLIT) every single
sequence is also held to 2e-2; with plain bf16 activations the per-sequence
error is reported (at the OPT-13B shape a few of 128 sequences reach 0.026 by
bf16 rounding alone) and held to a 5e-2 sanity bound, and the same batch is
also scored with two-term activations and held to 1e-3 per sequence, so the
arithmetic itself is checked tightly at full size.  Foreground rows are checked
per scored token (2e-2) and must be bitwise identical to a run of the same
batch without probes.
"""
import gc
import json
import os

import numpy as np
import pytest

from synth import configs, inputs

from .gpu_common import flush, need_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(name, split=None):
    import torch
    import zeroth_order_fine_amd as zo
    with open(os.path.join(GOLDEN, "%s_step1.json" % name)) as f:
        gold = json.load(f)
    wl = configs.CONFIGS[name]
    if split is not None:
        wl = wl.with_(act_split=split)
    batch = inputs.make_batch(wl)
    flush("full-size %s (split %s): init" % (name, wl.act_split))
    model = zo.Model(wl.model)
    model.init_weights(wl.model_seed)
    bank = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
    db = zo.DeviceBatch(batch)
    zo.update(model, zo.Plan.from_workload(model, wl, t=0), bank, gold["state"]["c"], gold["state"]["lr"])
    flush("full-size %s: score" % name)
    out = zo.score(model, zo.Plan.from_workload(model, wl, t=1), bank, db, want_tokens=True)
    phys_seq, phys_cand, first = zo.pack(model, zo.Plan.from_workload(model, wl, t=1), db)
    return gold, wl, batch, model, bank, db, out, list(zip(phys_seq, phys_cand)), first


def _check(name, gold, wl, out, phys, first, seq_bound, c_gpu=None, fg_tok_bound=2e-2, fg_median_bound=None):
    seq = out["seq_logp"].cpu().numpy()
    tok = out["tok_logp"].cpu().numpy()
    errs, fg_errs = [], []
    for p, (ls, c), g, gt in zip(gold["phys_index"], gold["phys"], gold["seq_logp"], gold["tok_logp"]):
        assert tuple(phys[p]) == (ls, c)                        # packing agrees with the oracle's
        t = tok[first[p]:first[p + 1]]
        assert len(t) == len(gt)
        if c >= 0:
            errs.append(abs(seq[p] - g))
        else:
            d = np.abs(t - np.array(gt))
            fg_errs.append((p, len(d), float(d.max()), float(np.median(d))))
    if fg_errs:
        flush("%s: foreground sequences (index, tokens, max, median |err|): %s" % (name, fg_errs))
        assert max(e[2] for e in fg_errs) <= fg_tok_bound, (name, fg_errs)
        if fg_median_bound is not None:
            assert max(e[3] for e in fg_errs) <= fg_median_bound, (name, fg_errs)
    errs = np.array(errs)
    flush("%s (split %s): %d probe sequences, max per-sequence |err| %.4f, %d above 2e-2" % (
        name, wl.act_split, len(errs), errs.max(), int((errs > 2e-2).sum())))
    assert np.all(errs <= seq_bound), (name, errs.max())
    if "S" in gold:
        S = out["S"]
        n_seq = np.array([sum(1 for _, c in phys if c == k) for k in range(len(S))])
        dS = np.abs(S - np.array(gold["S"]))
        flush("%s: per-candidate |dS| %s (budget %s)" % (name, np.round(dS, 4), 2e-2 * n_seq))
        assert np.all(dS <= 2e-2 * n_seq), (S, gold["S"])
        if "c" in gold and c_gpu is not None:
            c = np.asarray(c_gpu)
            rel = np.abs(c - np.array(gold["c"])) / np.abs(np.array(gold["c"]))
            flush("%s (split %s): c %s oracle %s, relative error %s" % (name, wl.act_split, c, gold["c"], rel))
            if wl.act_split:
                # the estimate divides the score difference by 2 eps: only two-term
                # activations keep it within the fp32 contract's 1e-2 relative
                assert np.all(rel <= 1e-2), (c, gold["c"])
    return seq, tok


@pytest.mark.parametrize("name", ["opt1.3b", "opt13b", "opt6.7b-mezo", "qwen3-8b-mixed"])
def test_full_size_against_oracle(name):
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    gold, wl, batch, model, bank, db, out, phys, first = _run(name)
    c_gpu = zo.estimate(zo.Plan.from_workload(model, wl, t=1), out["S"])
    seq, tok = _check(name, gold, wl, out, phys, first, 2e-2 if wl.act_split else 5e-2, c_gpu)
    if name == "qwen3-8b-mixed":
        # co-serving: the foreground rows are bitwise identical without the probes
        import zeroth_order_fine_amd as zo
        fg = batch.subset([i for i in range(batch.n_seq) if batch.role[i] == inputs.ROLE_FOREGROUND])
        alone = zo.score(model, zo.Plan.from_workload(model, wl, t=1), bank, zo.DeviceBatch(fg), want_tokens=True)
        nf = fg.n_seq
        assert np.array_equal(alone["seq_logp"].cpu().numpy().view(np.uint64), seq[:nf].view(np.uint64))
        nt = alone["n_scored"]
        assert np.array_equal(alone["tok_logp"].cpu().numpy().view(np.uint32), tok[:nt].view(np.uint32))
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["opt1.3b", "opt13b"])
def test_full_size_two_term_activations(name):
    """The plain-bf16 workloads scored with two-term activations: every sequence within
    1e-3 of the oracle (measured about 3e-5), and c = (L+ - L-)/2eps within 1e-2
    relative (with plain bf16 activations c at eps = 1e-3 is off by about 20 % at the
    OPT-13B shape: the score difference is divided by 2 eps)."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    gold, wl, batch, model, bank, db, out, phys, first = _run(name, split=True)
    c_gpu = zo.estimate(zo.Plan.from_workload(model, wl, t=1), out["S"])
    _check(name, gold, wl, out, phys, first, 1e-3, c_gpu)
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()


# fp8 OPT-13B: see the fp8 bound of tests/test_gpu_parity.py.  Over 40 layers the kernels'
# residual stream drifts from the oracle's (fp32 and bf16 against fp64), so more and more
# linear inputs land on the other side of an e4m3 rounding boundary (one e4m3 step, 1/16
# to 1/8 relative, each).  Bound: the small fp8 model's measured 0.023 grown by the factor
# the bf16 difference grows from the small model to OPT-13B (about 0.002 to 0.026, 13x):
# 0.3.  Measured 0.033 / 0.050 / 0.036 / 0.159.  An indexing or tiling fault at these
# shapes moves a log-prob by units, not tenths.
FP8_FULL_SEQ_BOUND = 3e-1


# Qwen3-8B fp8: at the Qwen3-8B width the fp8 model's GPU-oracle difference is about 10x
# the bf16 model's at the same depth (measured on 2- and 8-layer cuts: foreground tokens
# max 0.20 / 0.42, median 0.076 / 0.12 against bf16 0.025 / 0.041 and 0.0075 / 0.015:
# 4096-wide rows hold more elements near an e4m3 boundary), and both grow with depth.
# Full depth measured: foreground tokens max 1.08 / 1.29, median 0.26 / 0.27.  Bounds: 2.0
# per probe sequence and foreground token, 0.5 on a foreground sequence's median token; an
# indexing fault at these shapes moves log-probs by many nats.
FP8_FULL_SEQ_BOUND_QWEN3 = 2.0
FP8_FULL_MEDIAN_BOUND_QWEN3 = 0.5


@pytest.mark.parametrize("name", ["opt13b-fp8", "qwen3-8b-fp8"])
def test_full_size_fp8_against_oracle(name):
    """The fp8 workloads in the launch configuration bench.py times (e4m3 projections on
    128x128 tiles): the shortest and the longest probe prompt under every candidate (and,
    for the Qwen3 mixed batch, the two shortest foreground sequences, every token) against
    the oracle's e4m3 model."""
    need_gpu()
    import torch
    gold, wl, batch, model, bank, db, out, phys, first = _run(name)
    if name == "opt13b-fp8":
        _check(name, gold, wl, out, phys, first, FP8_FULL_SEQ_BOUND)
    else:
        _check(name, gold, wl, out, phys, first, FP8_FULL_SEQ_BOUND_QWEN3, fg_tok_bound=FP8_FULL_SEQ_BOUND_QWEN3,
               fg_median_bound=FP8_FULL_MEDIAN_BOUND_QWEN3)
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()
