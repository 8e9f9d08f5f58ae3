"""Tolerances of the fp8 parity tests, derived from the oracle alone, and the expected
values of the full-width layer cuts.

fp8 models round every linear input to e4m3, a step function.  Wherever the kernels'
value before a rounding and the fp64 definition's straddle an e4m3 rounding boundary,
the rounded values are one e4m3 step (1/16 to 1/8 relative) apart, and every later layer
sees the difference.  How far that moves a log-prob depends on the model and the
sequence, not on the kernels, so it is measured on the oracle: the same forward with every
pre-rounding value multiplied by (1 + delta u), u uniform on [-1, 1] (oracle.model's error
model), with delta the precision the kernels form that value in:
  attention output   2^-8   (bf16 q, k, v and probabilities: a few bf16 roundings, 2^-9 each)
  norm outputs, GELU / SwiGLU outputs   2^-20   (fp32 arithmetic on an fp32 residual or on
                     fp32 sums of exact e4m3 products)
for SEEDS seeds.  The floor of a case is the largest change of a probe sequence's sum (and
of a foreground token's log-prob) over the seeds; the bound a test applies is FACTOR times
the floor, and never below the bf16 bound 2e-2 (the head and the side path run in bf16 as
in bf16 models).

Cases (each written to fp8floor_<case>.json):
  opt-small-fp8, qwen3-small-fp8  the small fp8 models of tests/test_gpu_parity.py
  opt13b-fp8, qwen3-8b-fp8        the full-size goldens' samples (tests/golden/*_step1.json)
  opt13b-fp8-L1/L2, qwen3-8b-fp8-L1/L2
                                  full-width cuts (the first 1 or 2 layers of those models,
                                  same embeddings and head): plain values + floors
  opt13b-L2, qwen3-8b-L2          the bf16 models cut the same way (plain values only)

    python tests/golden/make_fp8_floor.py [case ...]
"""
import dataclasses
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import zo as ozo          # noqa: E402
from synth import configs, inputs     # noqa: E402

DELTAS = {"attn": 2.0 ** -8, "norm": 2.0 ** -20, "ffn": 2.0 ** -20}
SEEDS = (1, 2, 3)
SEEDS_FULL = (1, 2)         # the full-depth workloads (each seed is a whole oracle run)
FACTOR = 2.0
BF16_BOUND = 2e-2
LR = 1e-3
C_FIXED = [2.5, -1.75, 0.5, -3.0]


def _small(arch):
    from tests.gpu_common import SMALL_OPT_FP8, SMALL_QWEN_FP8, workload
    cfg = SMALL_OPT_FP8 if arch == "opt" else SMALL_QWEN_FP8
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=2, n_prompts=3)
    bank = ozo.Bank(4, wl.rank, wl.targets)
    c_fixed = [np.array([0.9, -1.7]), np.array([-2.5, 0.4]), np.array([1.1, 0.8])]
    for k, t in enumerate((0, 3, 5)):
        ozo.update(cfg, ozo.plan_from_workload(wl, t), bank, c_fixed[k], 5e-3)
    return wl, bank, 6, None


def _cut(name, layers):
    wl0 = configs.CONFIGS[name]
    return wl0.with_(model=dataclasses.replace(wl0.model, n_layers=layers), act_split=False)


def _golden_state(wl):
    bank = ozo.Bank(2 * wl.n_dirs, wl.rank, wl.targets)
    ozo.update(wl.model, ozo.plan_from_workload(wl, 0), bank, np.array(C_FIXED[:wl.n_dirs]), LR)
    return bank


def cut_sample(wl, batch, phys):
    """Physical sequences of a layer cut: the first eight probe prompts under every
    candidate, and the two shortest foreground sequences."""
    probes = [i for i in range(batch.n_seq) if batch.role[i] == 0][:8]
    fg = sorted([i for i in range(batch.n_seq) if batch.role[i] == 1], key=lambda i: len(batch.tokens[i]))[:2]
    keep = set(probes) | set(fg)
    return [p for p, (li, c) in enumerate(phys) if li in keep]


CASES = {
    "opt-small-fp8": lambda: _small("opt"),
    "qwen3-small-fp8": lambda: _small("qwen3"),
    "opt13b-fp8": lambda: (configs.CONFIGS["opt13b-fp8"], None, 1, "golden"),
    "qwen3-8b-fp8": lambda: (configs.CONFIGS["qwen3-8b-fp8"], None, 1, "golden"),
    "opt13b-fp8-L1": lambda: (_cut("opt13b-fp8", 1), None, 1, "cut"),
    "opt13b-fp8-L2": lambda: (_cut("opt13b-fp8", 2), None, 1, "cut"),
    "qwen3-8b-fp8-L1": lambda: (_cut("qwen3-8b-fp8", 1), None, 1, "cut"),
    "qwen3-8b-fp8-L2": lambda: (_cut("qwen3-8b-fp8", 2), None, 1, "cut"),
    "opt13b-L2": lambda: (_cut("opt13b", 2), None, 1, "cut"),
    "qwen3-8b-L2": lambda: (_cut("qwen3-8b-mixed", 2), None, 1, "cut"),
}


def make(case):
    wl, bank, t, sample = CASES[case]()
    cfg = wl.model
    if bank is None:
        bank = _golden_state(wl)
    batch = inputs.make_batch(wl)
    plan = ozo.plan_from_workload(wl, t)
    phys = ozo.pack(batch, plan)
    t0 = time.time()
    W = ozo.Weights(cfg, wl.model_seed, cache_layers=cfg.n_layers <= 2)
    if sample == "golden":
        with open(os.path.join(HERE, "%s_step1.json" % case)) as f:
            gold = json.load(f)
        idx = gold["phys_index"]
        plain_seq = np.full(len(phys), np.nan)
        plain_tok = {}
        for p, s, tl in zip(idx, gold["seq_logp"], gold["tok_logp"]):
            plain_seq[p] = s
            plain_tok[p] = np.array(tl)
    else:
        idx = cut_sample(wl, batch, phys) if sample == "cut" else list(range(len(phys)))
        out = ozo.score(cfg, W, plan, bank, batch, phys_subset=idx)
        plain_seq, plain_tok = out["seq_logp"], out["tok_logp"]
    rec = {"case": case, "written_by": "tests/golden/make_fp8_floor.py (oracle/ only)",
           "layers": cfg.n_layers, "dtype": cfg.dtype, "score_step": t,
           "phys_index": [int(p) for p in idx], "phys": [list(map(int, phys[p])) for p in idx],
           "seq_logp": [float(plain_seq[p]) for p in idx],
           "tok_logp": [[float(v) for v in plain_tok[p]] for p in idx]}
    if cfg.dtype == "fp8":
        floor_seq = np.zeros(len(idx))
        floor_tok = np.zeros(len(idx))
        seeds = SEEDS_FULL if sample == "golden" else SEEDS
        for seed in seeds:
            j = ozo.score(cfg, W, plan, bank, batch, phys_subset=idx, e4m3_jitter=(DELTAS, seed))
            for i, p in enumerate(idx):
                floor_seq[i] = max(floor_seq[i], abs(j["seq_logp"][p] - plain_seq[p]))
                floor_tok[i] = max(floor_tok[i], float(np.max(np.abs(j["tok_logp"][p] - plain_tok[p]))))
            print(case, "seed", seed, "done %.0f s" % (time.time() - t0), flush=True)
        probe = np.array([phys[p][1] >= 0 for p in idx])
        fs = float(floor_seq[probe].max())
        ft = float(floor_tok[~probe].max()) if (~probe).any() else 0.0
        rec.update({"deltas": DELTAS, "seeds": list(seeds), "factor": FACTOR,
                    "floor_seq": floor_seq.tolist(), "floor_tok": floor_tok.tolist(),
                    "floor_seq_max": fs, "floor_tok_max": ft,
                    "bound_seq": max(BF16_BOUND, FACTOR * fs), "bound_tok": max(BF16_BOUND, FACTOR * ft)})
    rec["oracle_seconds"] = round(time.time() - t0, 1)
    with open(os.path.join(HERE, "fp8floor_%s.json" % case), "w") as f:
        json.dump(rec, f)
    print(case, "floor seq %s tok %s bound seq %s tok %s (%.0f s)" % (
        rec.get("floor_seq_max"), rec.get("floor_tok_max"), rec.get("bound_seq"), rec.get("bound_tok"),
        rec["oracle_seconds"]), flush=True)


if __name__ == "__main__":
    for c in (sys.argv[1:] or list(CASES)):
        make(c)
