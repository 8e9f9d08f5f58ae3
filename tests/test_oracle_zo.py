"""Pins of the oracle's ProbePlan / score / estimate / update (oracle/zo.py).

What the pages fix and the tests check:
* the factorized side state equals explicit dense mutation of the weights
  (arXiv abstract of "Inference-Native Zeroth-Order Optimization"), both in
  the oracle (fp64, 1e-12) and against the transformers library run on the
  mutated weights;
* eps = 0 makes S+ and S- bitwise equal; swapping the signs negates c
  exactly ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along",
  equations for L+, L- and c);
* c converges to the analytic directional derivative at rate O(eps^2) on a
  single linear + log-softmax layer with a closed-form gradient;
* the 1/r flag divides c by r (section "The System Reorganization");
* the lazy update U_{t+1} = U_t - eta c_t G_t and the m-step identity
  Delta W = (U_t - eta sum c_s G_s) V^T (same section);
* packing: a batch scores the same as its sequences scored one by one.
"""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import params, zo
from oracle.zo import Bank, Plan, Weights
from synth import configs, inputs
from synth.configs import ModelCfg

from .test_oracle_model import OPT_SMALL, QWEN_SMALL, _opt_hf, _qwen_hf, T


def _small_wl(cfg, targets, n_prompts=3, rank=2, dirs=(0,), n_fg=0, mode="last_label"):
    return configs.Workload("t", cfg, n_prompts, 6, 11, "uniform", mode, rank, 1e-2, dirs, targets,
                            nu=4, n_fg=n_fg, model_seed=2, data_seed=5)


def _bank_after_updates(cfg, wl, steps=2, c=(0.7, -1.3)):
    bank = Bank(4, wl.rank, wl.targets)
    for t in range(steps):
        plan = zo.plan_from_workload(wl, t)
        zo.update(cfg, plan, bank, np.array([c[t % 2]] * wl.n_dirs), 0.5)
    return bank


@pytest.mark.parametrize("cfg,targets", [(OPT_SMALL, configs.KIND_NAMES_OPT),
                                         (QWEN_SMALL, configs.KIND_NAMES_QWEN3),
                                         (OPT_SMALL, ("q", "v"))])
def test_factorized_equals_dense_mutation(cfg, targets):
    wl = _small_wl(cfg, targets, dirs=(0, 5), n_fg=1)
    bank = _bank_after_updates(cfg, wl)
    batch = inputs.make_batch(wl)
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    plan = zo.plan_from_workload(wl, 2)
    a = zo.score(cfg, W, plan, bank, batch)
    b = zo.score(cfg, W, plan, bank, batch, dense=True)
    assert np.allclose(a["seq_logp"], b["seq_logp"], rtol=1e-12, atol=0)
    assert np.allclose(a["S"], b["S"], rtol=1e-12, atol=0)
    # the perturbation is actually visible
    assert np.ptp(a["S"]) > 0


@pytest.mark.parametrize("cfg,build", [(OPT_SMALL, _opt_hf), (QWEN_SMALL, _qwen_hf)])
def test_candidate_state_matches_library_on_mutated_weights(cfg, build):
    targets = cfg.kind_names
    wl = _small_wl(cfg, targets, n_prompts=1)
    bank = _bank_after_updates(cfg, wl, steps=1)
    batch = inputs.make_batch(wl)
    plan = zo.plan_from_workload(wl, 1)
    Wbase = Weights(cfg, wl.model_seed, cache_layers=True)
    got = zo.score(cfg, Wbase, plan, bank, batch)
    for cand in range(2):
        side = zo.side_terms(cfg, plan, bank, cand)
        Wm = Weights(cfg, wl.model_seed, cache_layers=True)
        names = {"q": "wq", "k": "wk", "v": "wv", "o": "wo", "fc1": "w_fc1", "fc2": "w_fc2",
                 "gate": "w_gate", "up": "w_up", "down": "w_down"}
        for l in range(cfg.n_layers):
            Wl = Wm.get_layer(l)
            for kind in targets:
                for V, B in side(l, kind):
                    Wl[names[kind]] = Wl[names[kind]] + B @ V.T
        m = build(cfg, Wm)
        toks = batch.tokens[0]
        with torch.no_grad():
            logits = m(input_ids=torch.tensor(toks, dtype=torch.long)[None]).logits[0]
        ref = torch.log_softmax(logits, -1)[len(toks) - 2, int(toks[-1])].item()
        p = [i for i, (li, c) in enumerate(got["phys"]) if c == cand][0]
        assert abs(got["seq_logp"][p] - ref) < 1e-6


def test_eps_zero_gives_equal_scores():
    cfg = OPT_SMALL
    wl = _small_wl(cfg, ("q", "v", "fc1"))
    bank = _bank_after_updates(cfg, wl)
    plan = zo.plan_from_workload(wl, 2)
    plan.eps, plan.allow_zero_eps = 0.0, True
    out = zo.score(cfg, Weights(cfg, 2, True), plan, bank, inputs.make_batch(wl))
    assert out["S"][0] == out["S"][1]
    with pytest.raises(ValueError):
        Plan(0, 1, 2, 0.0, (0,), ((0, 1), (0, -1)), ("q",)).validate()


def test_swapping_signs_negates_c_exactly():
    S = np.array([-12.25, -12.875, -3.1, -2.9])
    p1 = Plan(0, 1, 2, 1e-3, (0, 1), ((0, 1), (0, -1), (1, 1), (1, -1)), ("q",))
    p2 = Plan(0, 1, 2, 1e-3, (0, 1), ((0, -1), (0, 1), (1, -1), (1, 1)), ("q",))
    c1, c2 = zo.estimate(p1, S), zo.estimate(p2, S)
    assert np.array_equal(c1, -c2)
    # closed form: L = -S
    assert c1[0] == ((-S[0]) - (-S[1])) / (2 * 1e-3)


def test_inv_rank_and_mean_flags():
    S = np.array([-10.0, -10.5])
    p = Plan(0, 1, 4, 1e-2, (0,), ((0, 1), (0, -1)), ("q",))
    c = zo.estimate(p, S)
    cr = zo.estimate(p, S, zo.EST_INV_RANK)
    assert abs(cr[0] * 4 - c[0]) <= np.spacing(abs(c[0]))
    cm = zo.estimate(p, S, zo.EST_MEAN, n_scored=np.array([5, 5]))
    # (L+/5 - L-/5) rounds the two quotients before the difference: bound relative to |L|
    assert abs(cm[0] * 5 - c[0]) <= 1e-12 * abs(S).max() / 1e-2
    with pytest.raises(FloatingPointError):
        zo.estimate(p, np.array([np.nan, 1.0]))


def test_c_converges_to_directional_derivative():
    """L(W) = -sum log softmax(x W^T)_y; grad = (P - Y)^T X; D = <grad, G V^T>."""
    r = np.random.default_rng(9)
    n, din, V, rank = 6, 24, 40, 2
    X, W = r.normal(size=(n, din)), r.normal(size=(V, din)) * 0.3
    y = r.integers(0, V, size=n)
    G, Vf = params.factor(3, 0, 0, 0, 0, V, rank), params.factor(3, 0, 0, 1, 0, din, rank)
    logits = X @ W.T
    P = np.exp(logits - logits.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Y = np.zeros_like(P)
    Y[np.arange(n), y] = 1
    D = np.sum(((P - Y).T @ X) * (G @ Vf.T))
    errs = []
    for eps in (4e-3, 2e-3, 1e-3):
        plan = Plan(0, 1, rank, eps, (3,), ((0, 1), (0, -1)), ("q",))
        S = np.array([om.log_softmax_gather(om.linear(X, W, None, [(Vf, s * eps * G)], False), y).sum()
                      for s in (1, -1)])
        errs.append(abs(zo.estimate(plan, S)[0] - D))
    assert errs[-1] / abs(D) < 5e-5
    assert 3.0 < errs[0] / errs[1] < 5.0 and 3.0 < errs[1] / errs[2] < 5.0


def test_update_closed_form_and_m_step_identity():
    cfg = OPT_SMALL
    wl = _small_wl(cfg, ("q", "fc2"), dirs=(4, 9))
    bank = Bank(2, wl.rank, wl.targets)
    cs = [np.array([0.8, -0.3]), np.array([-1.1, 0.6]), np.array([0.25, 0.4])]
    lr = 0.05
    for t, c in enumerate(cs):
        zo.update(cfg, zo.plan_from_workload(wl, t), bank, c, lr)
        if t == 0:
            for d, e in enumerate(bank.active()):
                G = params.factor(wl.dir_seeds[d], 1, 0, 0, 0, cfg.d_model, wl.rank)
                exact = (0.0 - ((lr / 2) * c[d]) * G).astype(np.float32)
                assert np.array_equal(e.U[(1, "q")], exact.astype(np.float64))
    assert len(bank.active()) == 2          # nu = 4: all three steps in window 0
    for d, e in enumerate(bank.active()):
        n_out, n_in = cfg.linear_shape("fc2")
        kid = cfg.kind_names.index("fc2")
        dense = np.zeros((n_out, n_in))
        V = params.factor(wl.dir_seeds[d], 0, kid, 1, 0, n_in, wl.rank)
        for t, c in enumerate(cs):
            G = params.factor(wl.dir_seeds[d], 0, kid, 0, t, n_out, wl.rank)
            dense = dense - (lr / 2) * c[d] * (G @ V.T)       # three explicit dense updates
        lazy = e.U[(0, "fc2")] @ V.T
        assert np.allclose(lazy, dense, rtol=0, atol=1e-6 * np.abs(dense).max())


def test_window_rollover_makes_new_entry():
    cfg = OPT_SMALL
    wl = _small_wl(cfg, ("v",))
    bank = Bank(2, wl.rank, wl.targets)
    for t in range(6):                                       # nu = 4: windows 0 and 1
        zo.update(cfg, zo.plan_from_workload(wl, t), bank, np.array([1.0]), 0.1)
    keys = sorted((e.seed, e.window) for e in bank.active())
    assert keys == [(0, 0), (0, 1)]
    with pytest.raises(RuntimeError):
        for t in range(8, 9):
            zo.update(cfg, zo.plan_from_workload(wl, t), bank, np.array([1.0]), 0.1)


def test_packing_order_and_batch_equals_single():
    cfg = OPT_SMALL
    wl = _small_wl(cfg, ("q", "v"), n_fg=2, n_prompts=2)
    batch = inputs.make_batch(wl)
    plan = zo.plan_from_workload(wl, 0)
    phys = zo.pack(batch, plan)
    assert phys == [(0, -1), (1, -1), (2, 0), (3, 0), (2, 1), (3, 1)]
    W = Weights(cfg, 2, True)
    full = zo.score(cfg, W, plan, None, batch)
    for li in range(batch.n_seq):
        one = zo.score(cfg, W, plan, None, batch.subset([li]))
        for p1, (l1, c1) in enumerate(one["phys"]):
            p = phys.index((li, c1))
            assert full["seq_logp"][p] == one["seq_logp"][p1]


def test_all_next_scores_every_position():
    toks = np.array([4, 8, 15, 16, 23])
    pos, lab = zo.scored_positions(toks, zo.MODE_ALL_NEXT)
    assert list(pos) == [0, 1, 2, 3] and list(lab) == [8, 15, 16, 23]
    pos, lab = zo.scored_positions(toks, zo.MODE_LAST_LABEL)
    assert list(pos) == [3] and list(lab) == [23]
    with pytest.raises(ValueError):
        zo.scored_positions(np.array([3]), zo.MODE_LAST_LABEL)


@pytest.mark.parametrize("cfg", [OPT_SMALL, QWEN_SMALL], ids=["opt", "qwen3"])
def test_fold_commits_entry_into_weights(cfg):
    """Folding a finished window's entry into W (Delta W = U V^T of the lazy update) leaves
    every score unchanged up to the fp32 rounding of W, and the folded values are the
    rounded W + U V^T."""
    wl = _small_wl(cfg, cfg.kind_names, dirs=(0, 5))
    bank = _bank_after_updates(cfg, wl, steps=2)            # window 0 entries for both seeds
    batch = inputs.make_batch(wl)
    plan = zo.plan_from_workload(wl, 4)                     # window 1: directions do not alias
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    before = zo.score(cfg, W, plan, bank, batch)
    plain = zo.score(cfg, W, plan, Bank(4, wl.rank, wl.targets), batch)
    assert np.max(np.abs(before["seq_logp"] - plain["seq_logp"])) > 1e-2   # the entry matters
    slot = [i for i, e in enumerate(bank.entries) if e is not None and e.seed == 0][0]
    e = bank.entries[slot]
    old = {(l, k): W.get_layer(l)[zo.WEIGHT_NAME[k]].copy() for l in range(cfg.n_layers) for k in wl.targets}
    zo.fold(cfg, W, bank, slot)
    assert bank.entries[slot] is None
    for (l, k), w0 in old.items():
        n_out, n_in = cfg.linear_shape(k)
        V = params.factor(0, l, cfg.kind_names.index(k), params.rng.FACTOR_V, 0, n_in, wl.rank)
        ref = (w0 + e.U[(l, k)] @ V.T).astype(np.float32)        # another summation order
        got = W.get_layer(l)[zo.WEIGHT_NAME[k]].astype(np.float32)
        ulp = np.spacing(np.abs(ref))
        assert np.all(np.abs(got - ref) <= ulp), (l, k)
        assert np.mean(got == ref) > 0.99
    after = zo.score(cfg, W, plan, bank, batch)
    assert np.allclose(after["seq_logp"], before["seq_logp"], rtol=1e-6, atol=0)
    assert np.allclose(after["S"], before["S"], rtol=1e-6, atol=0)


def test_fold_rounds_bf16_weights():
    """bf16 weights: the fold rounds fp64 -> fp32 -> bf16 (each to nearest even)."""
    cfg = configs.ModelCfg("opt", 1, 64, 4, 4, 16, 128, 97, 64, "bf16", 1e-5)
    wl = _small_wl(cfg, ("q", "fc2"), dirs=(3,))
    bank = _bank_after_updates(cfg, wl, steps=1)
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    w0 = W.get_layer(0)["wq"].copy()
    e = bank.entries[0]
    zo.fold(cfg, W, bank, 0)
    V = params.factor(3, 0, 0, params.rng.FACTOR_V, 0, cfg.d_model, wl.rank)
    exact = w0 + e.U[(0, "q")] @ V.T
    got = W.get_layer(0)["wq"]
    assert np.all(params.bf16_round(got.astype(np.float32)) == got.astype(np.float32))   # bf16 values
    # within half a bf16 step of the exact sum (plus the fp32 step of the first rounding)
    step = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64) * 2.0 ** 16
    assert np.all(np.abs(got - exact) <= 0.5 * step + np.spacing(np.abs(exact).astype(np.float32)))
    assert not np.array_equal(got, w0)


@pytest.mark.parametrize("scaled", [False, True])
def test_update_follows_the_probed_direction(scaled):
    """theta <- theta - (eta/q) sum_d c_d z_d with z_d the direction the candidates probed:
    the + candidate's dense weight is W + eps z_d, so after one update from an empty bank
    the applied Delta W = U V^T must equal -(eta/q) c_d (W_plus - W) / eps, with or without
    the 1/sqrt(r) scaling of the MeZO-style factorized probes."""
    cfg = OPT_SMALL
    wl = _small_wl(cfg, ("q", "fc1"), rank=4, dirs=(2, 7))
    plan = zo.plan_from_workload(wl, 0)
    plan.scale_inv_sqrt_r = scaled
    c, lr, q = np.array([0.9, -0.4]), 0.3, 2
    bank = Bank(2, wl.rank, wl.targets)
    zo.update(cfg, plan, bank, c, lr)
    for d in range(q):
        e = [x for x in bank.active() if x.seed == wl.dir_seeds[d]][0]
        for l in range(cfg.n_layers):
            for kind in wl.targets:
                n_out, n_in = cfg.linear_shape(kind)
                kid = cfg.kind_names.index(kind)
                V = params.factor(wl.dir_seeds[d], l, kid, 1, 0, n_in, wl.rank)
                # the probed direction, read off the + candidate's side term (V, s eps~ G)
                probe = Plan(plan.t, plan.nu, plan.rank, plan.eps, plan.dir_seeds, ((d, 1), (d, -1)),
                             plan.targets, scaled)
                (Vp, B), = zo.side_terms(cfg, probe, None, 0)(l, kind)
                z = (B @ Vp.T) / plan.eps
                applied = e.U[(l, kind)] @ V.T
                ref = -(lr / q) * c[d] * z
                assert np.allclose(applied, ref, rtol=0, atol=1e-6 * np.abs(ref).max())
                # and z has unit-variance entries exactly when scaled (within sampling error)
                var = float(np.mean(z * z))
                assert (abs(var - 1.0) < 0.35) if scaled else (abs(var - wl.rank) < 0.35 * wl.rank)


def test_fold_requantizes_fp8_weights():
    """fp8 models: the fold adds U V^T to the dequantized weights and requantizes, i.e. each
    folded weight is the e4m3 value nearest to (w + sum_k U V^T) * 2^11, times 2^-11; checked
    against PyTorch's float8_e4m3fn conversion of the fp32 sum."""
    import dataclasses
    cfg = dataclasses.replace(OPT_SMALL, dtype="fp8", d_model=128, d_ffn=256, n_heads=4, head_dim=32)
    wl = _small_wl(cfg, ("q", "fc2"), dirs=(3,))
    bank = Bank(4, wl.rank, wl.targets)
    for t in range(2):
        zo.update(cfg, zo.plan_from_workload(wl, t), bank, np.array([0.02 * (t + 1)]), 0.5)
    W = Weights(cfg, wl.model_seed, cache_layers=True)
    w0 = {k: W.get_layer(0)[k].copy() for k in ("wq", "w_fc2")}
    e = bank.entries[0]
    zo.fold(cfg, W, bank, 0)
    for kind, name in (("q", "wq"), ("fc2", "w_fc2")):
        n_out, n_in = cfg.linear_shape(kind)
        V = params.factor(3, 0, cfg.kind_names.index(kind), params.rng.FACTOR_V, 0, n_in, wl.rank)
        exact32 = (w0[name] + e.U[(0, kind)] @ V.T).astype(np.float32)      # another summation order
        scaled = exact32.astype(np.float64) * 2048.0
        inside = np.abs(scaled) < 448.0                   # PyTorch's conversion gives NaN beyond the range
        ref = torch.from_numpy(np.where(inside, scaled, 0.0)).to(torch.float8_e4m3fn).double().numpy() / 2048.0
        got = W.get_layer(0)[name]
        # identical except where the two fp32 sums round differently next to an e4m3 midpoint
        assert np.mean(got[inside] == ref[inside]) > 0.999
        assert np.all(np.abs(got - ref)[inside] <= np.abs(ref[inside]) / 8 + 2.0 ** -20)
        assert np.all(got[~inside] == np.sign(scaled[~inside]) * 448.0 / 2048.0)   # saturated
        assert np.mean(got != w0[name]) > 0.01                                # the update is visible


def test_cap_trajectory_crosses_the_cap():
    """Eight steps with nu = 2 (four windows) and at most one frozen entry: after each update
    the oldest frozen entries are folded into W.  The frozen count never exceeds the cap, the
    active window's entry is never folded, and the capped state scores like the uncapped one
    (every window's entry kept as a side term) up to the fp32 rounding of the folds."""
    cfg = configs.CONFIGS["tiny"].model
    wl = configs.CONFIGS["tiny"].with_(nu=2)
    batch = inputs.make_batch(wl)
    Wc = Weights(cfg, wl.model_seed, cache_layers=True)
    Wf = Weights(cfg, wl.model_seed, cache_layers=True)
    capped, full = Bank(3, wl.rank, wl.targets), Bank(5, wl.rank, wl.targets)
    folds = []
    for t in range(8):
        plan = zo.plan_from_workload(wl, t)
        c = np.array([1.5 * (-1) ** t + 0.25 * t])
        zo.update(cfg, plan, capped, c, 1e-2)
        zo.update(cfg, plan, full, c, 1e-2)
        folds.append(zo.cap(cfg, Wc, capped, plan, 1))
        frozen = [e for e in capped.active() if e.window != plan.window]
        assert len(frozen) <= 1 and any(e.window == plan.window for e in capped.active())
    assert folds == [0, 0, 0, 0, 1, 0, 1, 0]               # windows 0 and 1 folded at t = 4 and 6
    plan = zo.plan_from_workload(wl, 7)
    a = zo.score(cfg, Wc, plan, capped, batch)
    b = zo.score(cfg, Wf, plan, full, batch)
    assert np.allclose(a["seq_logp"], b["seq_logp"], rtol=1e-6, atol=0)
    assert not np.array_equal(Wc.get_layer(0)["wq"], Wf.get_layer(0)["wq"])
