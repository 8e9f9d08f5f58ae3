"""Full-size parity: every workload at its real shape, in the launch
configuration bench.py times (whole batch, one zo_score call), against expected
values written by tests/golden/make_golden.py from the oracle alone.

State: one zo_update at step 0 with fixed coefficients, then zo_score at step 1.
Bound (bf16): 2e-2 absolute per candidate (probe) sequence; foreground rows are
checked per scored token (2e-2) and must be bitwise identical to a run of the
same batch without probes.
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


def _run(name):
    import torch
    import zeroth_order_fine_amd as zo
    with open(os.path.join(GOLDEN, "%s_step1.json" % name)) as f:
        gold = json.load(f)
    wl = configs.CONFIGS[name]
    batch = inputs.make_batch(wl)
    flush("full-size %s: init" % name)
    model = zo.Model(wl.model)
    model.init_weights(wl.model_seed)
    bank = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
    db = zo.DeviceBatch(batch)
    zo.update(model, zo.Plan.from_workload(model, wl, t=0), bank, gold["state"]["c"], gold["state"]["lr"])
    flush("full-size %s: score" % name)
    out = zo.score(model, zo.Plan.from_workload(model, wl, t=1), bank, db, want_tokens=True)
    phys_seq, phys_cand, first = zo.pack(model, zo.Plan.from_workload(model, wl, t=1), db)
    return gold, wl, batch, model, bank, db, out, list(zip(phys_seq, phys_cand)), first


@pytest.mark.parametrize("name", ["opt1.3b", "opt13b", "opt6.7b-mezo", "qwen3-8b-mixed"])
def test_full_size_against_oracle(name):
    need_gpu()
    import torch
    gold, wl, batch, model, bank, db, out, phys, first = _run(name)
    seq = out["seq_logp"].cpu().numpy()
    tok = out["tok_logp"].cpu().numpy()
    worst = 0.0
    for p, (ls, c), g, gt in zip(gold["phys_index"], gold["phys"], gold["seq_logp"], gold["tok_logp"]):
        assert tuple(phys[p]) == (ls, c)                        # packing agrees with the oracle's
        t = tok[first[p]:first[p + 1]]
        assert len(t) == len(gt)
        if c >= 0:
            err = abs(seq[p] - g)
            worst = max(worst, err)
            assert err <= 2e-2, (name, p, seq[p], g)
        else:
            assert np.max(np.abs(t - np.array(gt))) <= 2e-2, (name, p)
    flush("%s: %d sequences, max per-sequence |err| %.4f" % (name, len(gold["phys_index"]), worst))
    if "S" in gold:
        S = out["S"]
        n_probe = sum(1 for _, c in phys if c == 0)
        assert np.all(np.abs(S - np.array(gold["S"])) <= 2e-2 * n_probe), (S, gold["S"])
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
