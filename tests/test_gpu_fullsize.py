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


def _run(name, split=None, sites=0):
    import torch
    import zeroth_order_fine_amd as zo
    with open(os.path.join(GOLDEN, "%s_step1.json" % name)) as f:
        gold = json.load(f)
    wl = configs.CONFIGS[name]
    if split is not None:
        wl = wl.with_(act_split=split)
    if sites:
        wl = wl.with_(split_sites=sites)
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
    if name in ("opt13b", "qwen3-8b-mixed"):
        # the o and fc2 / down projections run as split-tail launches at this batch (the last
        # rounds of 256x256 tiles in K-slices dealt over every CU); the slices continue the
        # same MFMA sequence, so the data-parallel launch gives the same bits
        os.environ["ZO_GEMM_SPLIT_TAIL"] = "0"
        try:
            dp = zo.score(model, zo.Plan.from_workload(model, wl, t=1), bank, db, want_tokens=True)
        finally:
            del os.environ["ZO_GEMM_SPLIT_TAIL"]
        assert np.array_equal(dp["seq_logp"].cpu().numpy().view(np.uint64), seq.view(np.uint64))
        assert np.array_equal(dp["tok_logp"].cpu().numpy().view(np.uint32), tok.view(np.uint32))
        flush("%s: split-tail and data-parallel projections bitwise equal" % name)
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


def test_full_size_opt13b_three_split_sites():
    """OPT-13B batch 64 with two-term activations at three rounding sites only (attention,
    the q|k|v input and the fc1 input: ZO_PLAN_SPLIT_ATTN | _QKV_IN | _FC1_IN), about 1.6x
    the plain-bf16 step instead of 2x: every probe sequence within the contract's 2e-2 (the
    site set is the one whose single-site runs cut the mean per-sequence error most per unit
    of cost at this shape; the fc2 input, the costliest site, moved it least)."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    A = zo.api
    gold, wl, batch, model, bank, db, out, phys, first = _run(
        "opt13b", sites=A.PLAN_SPLIT_ATTN | A.PLAN_SPLIT_QKV_IN | A.PLAN_SPLIT_FC1_IN)
    _check("opt13b", gold, wl, out, phys, first, 2e-2)
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


# fp8 workloads: the bounds are written by tests/golden/make_fp8_floor.py from the oracle
# alone (fp8floor_<workload>.json: the oracle's own log-probs perturbed by a relative 2^-9
# before every e4m3 rounding, three seeds, times two, never below 2e-2) - see
# tests/test_gpu_parity.py fp8_bounds.
def _floor(case):
    with open(os.path.join(GOLDEN, "fp8floor_%s.json" % case)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["opt13b-fp8", "qwen3-8b-fp8"])
def test_full_size_fp8_against_oracle(name):
    """The fp8 workloads in the launch configuration bench.py times (e4m3 projections on
    128x128 tiles): the shortest and the longest probe prompt under every candidate (and,
    for the Qwen3 mixed batch, the two shortest foreground sequences, every token) against
    the oracle's e4m3 model."""
    need_gpu()
    import torch
    rec = _floor(name)
    gold, wl, batch, model, bank, db, out, phys, first = _run(name)
    assert rec["phys_index"] == gold["phys_index"] and np.allclose(rec["seq_logp"], gold["seq_logp"])
    flush("%s: bounds per sequence %.3g, per foreground token %.3g (oracle floors %.3g / %.3g)" % (
        name, rec["bound_seq"], rec["bound_tok"], rec["floor_seq_max"], rec["floor_tok_max"]))
    _check(name, gold, wl, out, phys, first, rec["bound_seq"], fg_tok_bound=rec["bound_tok"])
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()


CUT_BASE = {"opt13b-fp8": "opt13b-fp8", "qwen3-8b-fp8": "qwen3-8b-fp8", "opt13b": "opt13b",
            "qwen3-8b": "qwen3-8b-mixed"}


@pytest.mark.parametrize("case,split", [("opt13b-fp8-L1", False), ("opt13b-fp8-L2", False),
                                        ("qwen3-8b-fp8-L1", False), ("qwen3-8b-fp8-L2", False),
                                        ("opt13b-L2", True), ("qwen3-8b-L2", True)])
def test_full_width_layer_cuts(case, split):
    """The first one or two layers of the OPT-13B and Qwen3-8B shapes at full width (same
    embeddings, head and batch as the full workloads, whole batch in one zo_score call)
    against tests/golden/fp8floor_<case>.json (oracle only): the first eight probe prompts
    under both candidates and the two shortest foreground sequences.  fp8: the bounds
    derived from the oracle's floor for the same cut.  bf16 with two-term activations: every
    probe sequence and every foreground token within 2e-2.  (Plain bf16 activations already
    miss 2e-2 here on a few sequences: 0.024 on the OPT-13B cut, 0.021 on the Qwen3-8B cut,
    by the rounding of the activations alone; bench.py reports that mode's error at full
    size.)"""
    need_gpu()
    import dataclasses
    import torch
    import zeroth_order_fine_amd as zo
    rec = _floor(case)
    base, layers = case.rsplit("-L", 1)
    wl0 = configs.CONFIGS[CUT_BASE[base]]
    wl = wl0.with_(model=dataclasses.replace(wl0.model, n_layers=int(layers)), act_split=split)
    batch = inputs.make_batch(wl)
    flush("cut %s (split %s): init" % (case, split))
    model = zo.Model(wl.model)
    model.init_weights(wl.model_seed)
    bank = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
    db = zo.DeviceBatch(batch)
    zo.update(model, zo.Plan.from_workload(model, wl, t=0), bank, [2.5, -1.75, 0.5, -3.0][:wl.n_dirs], 1e-3)
    out = zo.score(model, zo.Plan.from_workload(model, wl, t=1), bank, db, want_tokens=True)
    phys_seq, phys_cand, first = zo.pack(model, zo.Plan.from_workload(model, wl, t=1), db)
    phys = list(zip(phys_seq, phys_cand))
    fp8 = wl.model.dtype == "fp8"
    bseq = rec["bound_seq"] if fp8 else 2e-2
    btok = rec["bound_tok"] if fp8 else (2e-2 if split else None)
    seq = out["seq_logp"].cpu().numpy()
    tok = out["tok_logp"].cpu().numpy()
    perr, ferr = [], []
    for p, (ls, c), g, gt in zip(rec["phys_index"], rec["phys"], rec["seq_logp"], rec["tok_logp"]):
        assert tuple(phys[p]) == (ls, c)
        if c >= 0:
            perr.append(abs(seq[p] - g))
        else:
            ferr.append(float(np.max(np.abs(tok[first[p]:first[p + 1]] - np.array(gt)))))
    flush("cut %s (split %s): probe sequences max |err| %.4f (bound %.3g), foreground tokens max %s (bound %s)%s" % (
        case, split, max(perr), bseq, ["%.4f" % e for e in ferr], btok,
        " oracle floors %.3g / %.3g" % (rec["floor_seq_max"], rec["floor_tok_max"]) if fp8 else ""))
    assert max(perr) <= bseq
    if btok is not None and ferr:
        assert max(ferr) <= btok
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()


def test_full_size_opt13b_graph_replays():
    """OPT-13B batch 64 scored from a captured HIP graph: the split-tail fc2 launches (their
    flags cleared before every call, outside the graph) and every other launch replayed give
    bitwise the eager results, across replays and a step change of the plan."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    gold, wl, batch, model, bank, db, out, phys, first = _run("opt13b")
    bits = lambda o: (o["seq_logp"].cpu().numpy().view(np.uint64).copy(), o["tok_logp"].cpu().numpy().view(np.uint32).copy())
    ref1 = bits(out)
    ref2 = bits(zo.score(model, zo.Plan.from_workload(model, wl, t=2), bank, db, want_tokens=True))
    model.set_graphs(True)
    stream = torch.cuda.Stream()             # graphs are captured on the call's (non-default) stream
    try:
        with torch.cuda.stream(stream):
            for k, t in enumerate((1, 1, 1, 2, 1)):
                flush("opt13b graph call %d (t=%d)" % (k, t))
                got = bits(zo.score(model, zo.Plan.from_workload(model, wl, t=t), bank, db, want_tokens=True))
                ref = ref1 if t == 1 else ref2
                assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (k, t)
                torch.cuda.synchronize()
    finally:
        model.set_graphs(False)
    del model, bank, db, out
    gc.collect()
    torch.cuda.empty_cache()
