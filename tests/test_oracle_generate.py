"""Pins of the oracle's greedy generation (oracle/zo.py generate).

* under W (a foreground prompt) the continuation equals greedy decoding by the
  transformers library's OPT and Qwen3 models in fp64 on the same weights: an
  independent implementation of the architecture and of the token-by-token loop
  (its own positions, its own attention over the grown sequence);
* under a candidate state the generated tokens' log-probs equal teacher-forced
  scoring of prompt + continuation by the scoring path (another code path through the
  forward: all positions of one pass instead of one pass per token);
* forcing the generated continuation reproduces it; the per-candidate sums are the
  sums of the generated tokens' log-probs.
"""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import zo
from oracle.zo import Weights
from synth import configs, inputs

from .test_oracle_model import OPT_SMALL, QWEN_SMALL, _opt_hf, _qwen_hf
from .test_oracle_zo import _bank_after_updates, _small_wl


def _workload(cfg):
    kinds = configs.KIND_NAMES_OPT if cfg.arch == "opt" else configs.KIND_NAMES_QWEN3
    return _small_wl(cfg, kinds, dirs=(0, 5), n_fg=1)


@pytest.mark.parametrize("cfg,build", [(OPT_SMALL, _opt_hf), (QWEN_SMALL, _qwen_hf)], ids=["opt", "qwen3"])
def test_greedy_generation_under_W_matches_library(cfg, build):
    wl = _workload(cfg)
    batch = inputs.make_batch(wl).subset([0])            # the foreground prompt
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 0)
    n_new = 7
    g = zo.generate(cfg, W, plan, None, batch, n_new)
    fg = [p for p, (li, c) in enumerate(g["phys"]) if c < 0]
    assert len(fg) == 1
    m = build(cfg, W)
    ids = torch.tensor(np.asarray(batch.tokens[0], np.int64))[None]
    ref_tok, ref_lp = [], []
    with torch.no_grad():
        for _ in range(n_new):
            lsm = torch.log_softmax(m(input_ids=ids).logits[0, -1], -1)
            t = int(torch.argmax(lsm))
            ref_tok.append(t)
            ref_lp.append(float(lsm[t]))
            ids = torch.cat([ids, torch.tensor([[t]])], 1)
    assert list(g["tokens"][fg[0]]) == ref_tok
    assert np.max(np.abs(g["logp"][fg[0]] - np.array(ref_lp))) < 1e-6


@pytest.mark.parametrize("cfg", [OPT_SMALL, QWEN_SMALL], ids=["opt", "qwen3"])
def test_generated_logprobs_equal_teacher_forced_scores(cfg):
    wl = _workload(cfg)
    bank = _bank_after_updates(cfg, wl)
    batch = inputs.make_batch(wl)
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 2)
    n_new = 5
    g = zo.generate(cfg, W, plan, bank, batch, n_new)
    assert np.array_equal(g["tokens"], g["best_tok"]) and np.array_equal(g["logp"], g["best_logp"])
    seqs = []
    for p, (li, c) in enumerate(g["phys"]):
        prompt = np.asarray(batch.tokens[li], np.int64)
        full = np.concatenate([prompt, g["tokens"][p]])
        seqs.append(dict(tokens=full, side=zo.side_terms(cfg, plan, bank, c),
                         positions=np.arange(len(prompt) - 1, len(full) - 1), labels=g["tokens"][p]))
    ref = om.forward_logprobs(cfg, W.get_global, W.get_layer, seqs)
    for p in range(len(seqs)):
        assert np.max(np.abs(g["logp"][p] - ref[p])) < 1e-10, p
    # candidates differ (the side path is on), and S sums the generated log-probs
    S = np.zeros(len(plan.candidates))
    for p, (li, c) in enumerate(g["phys"]):
        if c >= 0:
            S[c] += g["logp"][p].sum()
    assert np.allclose(S, g["S"], rtol=1e-13, atol=0) and np.ptp(g["S"]) > 0
    f = zo.generate(cfg, W, plan, bank, batch, n_new, forced=g["tokens"])
    assert np.array_equal(f["tokens"], g["tokens"]) and np.array_equal(f["logp"], g["logp"])
