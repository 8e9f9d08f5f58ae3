"""Write the expected values of the full-size parity tests.

Calls only oracle/ (and the seeded input generators in synth/).  For each
workload, the state is: one lazy update at step 0 with the fixed coefficients
C_FIXED and learning rate LR, then scoring at step 1 (so the bank holds a
non-zero entry, as in a running fine-tuning job).  The oracle scores a sample
of the physical sequences of the full batch (all of them for opt1.3b and
opt13b, which also gives S and c per candidate) in fp64 on the bf16-rounded
weights (the e4m3 weights and e4m3-rounded linear inputs for the fp8 workloads).

    python tests/golden/make_golden.py [workload ...]
"""
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

LR = 1e-3
C_FIXED = [2.5, -1.75, 0.5, -3.0]


def sample(wl, batch, phys):
    """Physical sequences checked at full size."""
    if wl.name in ("opt1.3b", "opt13b"):          # every sequence: S and c per candidate
        return list(range(len(phys)))
    lens = batch.lengths
    probes = [i for i in range(batch.n_seq) if batch.role[i] == 0]
    by_len = sorted(probes, key=lambda i: lens[i])
    if wl.name == "opt6.7b-mezo":
        pick = [probes[0]]
    else:                                          # qwen3 mixed (bf16, fp8), opt13b fp8: shortest and longest probe
        pick = [by_len[0], by_len[-1]]
    out = [p for p, (li, c) in enumerate(phys) if li in pick]
    if wl.name in ("qwen3-8b-mixed", "qwen3-8b-fp8"):
        fg = [i for i in range(batch.n_seq) if batch.role[i] == 1]
        fg_short = sorted(fg, key=lambda i: lens[i])[:2]
        out += [p for p, (li, c) in enumerate(phys) if li in fg_short]
    return sorted(out)


def make(name):
    wl = configs.CONFIGS[name]
    cfg = wl.model
    batch = inputs.make_batch(wl)
    t0 = time.time()
    W = ozo.Weights(cfg, wl.model_seed, cache_layers=False)
    bank = ozo.Bank(2 * wl.n_dirs, wl.rank, wl.targets)
    c0 = np.array(C_FIXED[:wl.n_dirs])
    ozo.update(cfg, ozo.plan_from_workload(wl, 0), bank, c0, LR)
    plan = ozo.plan_from_workload(wl, 1)
    phys = ozo.pack(batch, plan)
    idx = sample(wl, batch, phys)
    out = ozo.score(cfg, W, plan, bank, batch, phys_subset=idx if len(idx) < len(phys) else None)
    rec = {"workload": name, "written_by": "tests/golden/make_golden.py (oracle/ only)",
           "state": {"update_step": 0, "c": c0.tolist(), "lr": LR, "score_step": 1},
           "phys": [list(map(int, phys[p])) for p in idx], "phys_index": idx,
           "seq_logp": [float(out["seq_logp"][p]) for p in idx],
           "tok_logp": [[float(v) for v in out["tok_logp"][p]] for p in idx],
           "oracle_seconds": round(time.time() - t0, 1)}
    if "S" in out:
        rec["S"] = out["S"].tolist()
        rec["c"] = ozo.estimate(plan, out["S"]).tolist()
    path = os.path.join(HERE, "%s_step1.json" % name)
    with open(path, "w") as f:
        json.dump(rec, f)
    print(name, "done in %.0f s" % rec["oracle_seconds"], flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["opt1.3b", "opt13b", "opt6.7b-mezo", "qwen3-8b-mixed"]):
        make(n)
