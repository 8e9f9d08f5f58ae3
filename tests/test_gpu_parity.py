"""GPU parity of zo_score / zo_estimate / zo_update against the oracle.

Tolerances (stated by the method's parity contract):
  fp32 models: per-candidate S within 1e-4 relative; c within 1e-2 relative at eps = 1e-3;
  bf16 models: per-sequence summed log-prob within 2e-2 absolute, against the oracle run on
               the same bf16-rounded weights with fp64 activations;
  fp8 models: per-sequence summed log-prob (and foreground token) within the bound that
               tests/golden/make_fp8_floor.py derives from the oracle alone (fp8_bounds),
               against the oracle run on the same e4m3 weights with its e4m3-rounded inputs;
  updated factors: equal to the oracle's (the same fp64 formula rounded once to fp32),
               given the same c;
  packing offsets: bit-exact; foreground rows: bitwise identical with and without probes.
"""
import numpy as np
import pytest

from oracle import zo as ozo
from synth import configs, inputs

from .gpu_common import (SMALL_OPT_BF16, SMALL_OPT_FP8, SMALL_OPT_ODD, SMALL_QWEN_BF16, SMALL_QWEN_F32, SMALL_QWEN_FP8,
                         GpuRun, OracleRun, flush, need_gpu, workload)

pytestmark = pytest.mark.gpu


def _seq_close(gpu, ref, atol, probes_only=True):
    """Per physical sequence.  The bound applies to candidate (probe) sequences, whose
    sums make up L+/-; foreground sequences are checked per token by the callers."""
    g = gpu["seq_logp"].cpu().numpy()
    r = ref["seq_logp"]
    err = np.abs(g - r)
    if probes_only:
        err = np.where(np.array([c >= 0 for _, c in ref["phys"]]), err, 0.0)
    assert np.all(err <= atol), "max |err| %.3g at %d (gpu %.6f oracle %.6f)" % (
        err.max(), err.argmax(), g[err.argmax()], r[err.argmax()])
    return err.max()


def test_tiny_fp32_two_point_step():
    """The tiny OPT-style workload: L+, L-, c and the updated factors; then a second
    step that scores with the accumulated bank state."""
    need_gpu()
    wl = configs.CONFIGS["tiny"]
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    for t in range(3):
        flush("tiny step %d" % t)
        gs = g.score(t, batch)
        os_ = o.score(t, batch)
        assert np.all(np.abs(gs["S"] - os_["S"]) <= 1e-4 * np.abs(os_["S"])), (gs["S"], os_["S"])
        plan_o = ozo.plan_from_workload(wl, t)
        cg = g.zo.estimate(g.plan(t), gs["S"])
        co = ozo.estimate(plan_o, os_["S"])
        assert np.all(np.abs(cg - co) <= 1e-2 * np.abs(co)), (cg, co)
        g.update(t, cg, 1e-3)
        o.update(t, cg, 1e-3)          # same c on both sides: the factors must agree exactly
        for slot, e in enumerate(o.bank.entries):
            if e is None:
                continue
            for (layer, kind), U in e.U.items():
                got = g.bank.entry(slot, layer, kind).cpu().numpy()
                assert np.array_equal(got, U.astype(np.float32)), (t, slot, layer, kind)


@pytest.mark.parametrize("cfg,split", [(SMALL_OPT_BF16, False), (SMALL_QWEN_BF16, False), (SMALL_QWEN_F32, False),
                                       (SMALL_OPT_BF16, True), (SMALL_QWEN_BF16, True)],
                         ids=["opt-bf16", "qwen3-bf16", "qwen3-f32", "opt-bf16-split", "qwen3-bf16-split"])
def test_small_models_with_bank_and_ragged_rows(cfg, split):
    """Lengths 5..150 (1-3 query blocks, ragged row count), foreground + probes, two
    directions, a bank with entries from two windows (nu = 4: a frozen entry and an
    active one).  `split`: two-term bf16 activations (ZO_PLAN_ACT_SPLIT)."""
    need_gpu()
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=2, n_prompts=3, act_split=split)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c_fixed = [np.array([0.9, -1.7]), np.array([-2.5, 0.4]), np.array([1.1, 0.8])]
    for t in (0, 3, 5):                      # windows 0, 0, 1
        g.update(t, c_fixed[0 if t == 0 else (1 if t == 3 else 2)], 5e-3)
        o.update(t, c_fixed[0 if t == 0 else (1 if t == 3 else 2)], 5e-3)
    flush("score %s" % cfg.arch)
    gs, os_ = g.score(6, batch), o.score(6, batch)
    if cfg.dtype == "f32":      # relative bound, every sequence
        g_ = gs["seq_logp"].cpu().numpy()
        err = np.max(np.abs(g_ - os_["seq_logp"]) / np.abs(os_["seq_logp"]))
        assert err <= 1e-4, err
    else:
        # two-term activations carry ~16 significant bits: the bf16 bound shrinks by far more
        # than 10x, so a dropped lo term (bf16-level error) fails here
        err = _seq_close(gs, os_, 5e-4 if split else 2e-2)
    flush("max per-sequence err %.3g" % err)
    if cfg.dtype == "f32":
        assert np.all(np.abs(gs["S"] - os_["S"]) <= 1e-4 * np.abs(os_["S"]))
    # per-token agreement on every scored row (foreground rows score ALL_NEXT)
    tok = gs["tok_logp"].cpu().numpy()
    first = 0
    for p, (li, c) in enumerate(os_["phys"]):
        ref = os_["tok_logp"][p]
        assert np.all(np.abs(tok[first:first + len(ref)] - ref) <= (1e-4 if cfg.dtype == "f32" else 2e-2))
        first += len(ref)


@pytest.mark.parametrize("cfg", [SMALL_OPT_BF16, SMALL_QWEN_BF16], ids=["opt-bf16", "qwen3-bf16"])
def test_single_split_sites(cfg):
    """Two-term activations at one rounding site at a time (ZO_PLAN_SPLIT_*): every site alone
    and two combinations score within the bf16 bound of the oracle, and the five site flags
    together give bitwise the results of ZO_PLAN_ACT_SPLIT (so each site's buffers, pitches
    and wraps are the ones the all-sites mode uses)."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    A = zo.api
    sites = {"qkv": A.PLAN_SPLIT_QKV_IN, "attn": A.PLAN_SPLIT_ATTN, "fc1": A.PLAN_SPLIT_FC1_IN,
             "fc2": A.PLAN_SPLIT_FC2_IN, "head": A.PLAN_SPLIT_HEAD,
             "attn+fc2": A.PLAN_SPLIT_ATTN | A.PLAN_SPLIT_FC2_IN, "qkv+head": A.PLAN_SPLIT_QKV_IN | A.PLAN_SPLIT_HEAD}
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=2, n_prompts=3)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    for t in (0, 3, 5):                      # windows 0, 0, 1: a frozen entry and an active one
        c = np.array([0.9, -1.7]) if t == 0 else np.array([-2.5, 0.4])
        g.update(t, c, 5e-3)
        o.update(t, c, 5e-3)
    ref = o.score(6, batch)
    for name, bits in sites.items():
        out = g.score(6, batch, flags=bits)
        err = _seq_close(out, ref, 2e-2)
        flush("site %s: max per-sequence err %.3g" % (name, err))
    all5 = g.score(6, batch, flags=sum(v for k, v in sites.items() if "+" not in k))
    act = g.score(6, batch, flags=A.PLAN_ACT_SPLIT)
    for key in ("seq_logp", "tok_logp"):
        a, b = all5[key].cpu().numpy(), act[key].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key


@pytest.mark.parametrize("n_prompts,len_lo", [(4, 5), (72, 100)], ids=["small-batch", "tile-switch"])
def test_foreground_bitwise_invariance(n_prompts, len_lo):
    """Foreground rows are bitwise identical whether batched alone or alongside probes.
    "tile-switch": the mixed batch (about 18k rows) runs every projection in 256x256
    tiles of 128x64 wave tiles, the foreground batch alone (about 400 rows) in 128x128
    tiles of 64x64 wave tiles."""
    need_gpu()
    wl = workload(SMALL_QWEN_BF16, n_fg=3, n_prompts=n_prompts, len_lo=len_lo, dir_seeds=(1,))
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    g.update(0, np.array([1.3]), 1e-2)
    mixed = g.score(1, batch)
    fg = batch.subset([i for i in range(batch.n_seq) if batch.role[i] == inputs.ROLE_FOREGROUND])
    alone = g.score(1, fg)
    n_fg = fg.n_seq
    flush("rows: mixed %d, foreground alone %d" % (int(mixed["n_rows"]), int(alone["n_rows"])))
    a = mixed["seq_logp"].cpu().numpy()[:n_fg]
    b = alone["seq_logp"].cpu().numpy()[:n_fg]
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    nt = alone["n_scored"]
    ta = mixed["tok_logp"].cpu().numpy()[:nt]
    tb = alone["tok_logp"].cpu().numpy()[:nt]
    assert np.array_equal(ta.view(np.uint32), tb.view(np.uint32))


def test_probe_rows_bitwise_across_tile_shapes():
    """A probe sequence's log-prob, side path included, is bitwise the same whether its
    batch is large (more than 16k rows: every projection in 256x256 tiles of 128x64 wave
    tiles) or small (two prompts: 128x128 tiles of 64x64 wave tiles)."""
    need_gpu()
    wl = workload(SMALL_QWEN_BF16, n_prompts=72, len_lo=100, dir_seeds=(1,))
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    g.update(0, np.array([0.9]), 1e-2)
    big = g.score(1, batch)
    small = g.score(1, batch.subset([0, 1]))
    flush("rows: large batch %d, small batch %d" % (int(big["n_rows"]), int(small["n_rows"])))
    # o-proj output (N = d = 512) in 256x256 tiles needs more than 63 row tiles
    assert int(big["n_rows"]) > 63 * 256 and int(small["n_rows"]) < 4 * 256
    n = batch.n_seq
    a = big["seq_logp"].cpu().numpy()
    b = small["seq_logp"].cpu().numpy()
    # packing: candidate-major, prompts in input order
    for ia, ib in ((0, 0), (1, 1), (n, 2), (n + 1, 3)):
        assert a[ia:ia + 1].view(np.uint64)[0] == b[ib:ib + 1].view(np.uint64)[0], (ia, ib)


def test_eps_zero_and_sign_swap_and_repeatability():
    need_gpu()
    wl = workload(SMALL_OPT_BF16, n_prompts=4)
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    g.update(0, np.array([0.7]), 1e-2)
    z = g.score(1, batch, eps=0.0, flags=2)
    assert z["S"][0] == z["S"][1]
    a = g.score(1, batch)
    b = g.score(1, batch)
    assert np.array_equal(a["S"], b["S"])
    assert np.array_equal(a["seq_logp"].cpu().numpy(), b["seq_logp"].cpu().numpy())
    # the same candidates listed in the other order: every sequence lands elsewhere in the
    # packed batch, yet each candidate's score is bitwise the same (row results do not
    # depend on their position); exchanging the two scores negates c exactly
    import zeroth_order_fine_amd as zo
    p1 = g.plan(1)
    p2 = zo.Plan(g.model, 1, wl.nu, wl.rank, wl.eps, wl.dir_seeds, ((0, -1), (0, 1)), wl.targets)
    s1 = zo.score(g.model, p1, g.bank, zo.DeviceBatch(batch))["S"]
    s2 = zo.score(g.model, p2, g.bank, zo.DeviceBatch(batch))["S"]
    assert np.array_equal(s1, s2[::-1])
    assert np.array_equal(zo.estimate(p1, s1), zo.estimate(p2, s2))
    assert np.array_equal(zo.estimate(p1, s1[::-1]), -zo.estimate(p1, s1))


def test_empty_and_foreground_only_batches():
    need_gpu()
    wl = workload(SMALL_OPT_BF16, n_fg=2, n_prompts=0)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    gs, os_ = g.score(0, batch), o.score(0, batch)
    assert np.all(gs["S"] == 0.0)
    tok = gs["tok_logp"].cpu().numpy()
    ref = np.concatenate([os_["tok_logp"][p] for p in range(len(os_["phys"]))])
    assert np.max(np.abs(tok - ref)) <= 2e-2
    empty = batch.subset([])
    ge = g.score(0, empty)
    assert ge["n_phys"] == 0 and np.all(ge["S"] == 0.0)


def test_token_ids_outside_vocab_rejected():
    """Token ids are device data, checked by the kernels that read them: a label (the
    last token of a probe prompt) or a prompt token outside [0, vocab) makes zo_score
    return ZO_E_INVAL instead of a wrong S; the next call with valid ids is unaffected."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl = workload(SMALL_OPT_BF16, n_prompts=3, n_fg=1, fg_score_mode="all_next")
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    good = g.score(0, batch)
    vocab = wl.model.vocab
    for where, value in (("label", vocab), ("label", -3), ("prompt", vocab + 7), ("foreground", -1)):
        bad = inputs.Batch([t.copy() for t in batch.tokens], batch.role.copy(), batch.score_mode.copy())
        if where == "label":
            bad.tokens[2][-1] = value
        elif where == "prompt":
            bad.tokens[3][1] = value
        else:
            bad.tokens[0][4] = value
        flush("bad id %d at %s" % (value, where))
        with pytest.raises(zo.ZoError) as ei:
            g.score(0, bad)
        assert ei.value.code == -1 and "vocab" in str(ei.value)
    again = g.score(0, batch)
    assert np.array_equal(again["S"], good["S"])


def test_length_one_all_next_foreground_sequence():
    """A foreground sequence of one token scores no position (ALL_NEXT scores tokens
    1..n-1): its sum is 0 and it changes no other sequence's result (bitwise)."""
    need_gpu()
    wl = workload(SMALL_OPT_BF16, n_prompts=3, n_fg=2, fg_score_mode="all_next", dir_seeds=(4,))
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    g.update(0, np.array([0.6]), 1e-2)
    base = g.score(1, batch)
    one = inputs.Batch([np.array([17], np.int32)] + list(batch.tokens),
                       np.concatenate([[inputs.ROLE_FOREGROUND], batch.role]).astype(np.int32),
                       np.concatenate([[inputs.MODE_ALL_NEXT], batch.score_mode]).astype(np.int32))
    got = g.score(1, one)
    assert got["n_phys"] == base["n_phys"] + 1 and got["n_scored"] == base["n_scored"]
    a = got["seq_logp"].cpu().numpy()
    b = base["seq_logp"].cpu().numpy()
    assert a[0] == 0.0
    assert np.array_equal(a[1:].view(np.uint64), b.view(np.uint64))
    assert np.array_equal(got["S"], base["S"])


def test_high_rank_multi_direction():
    """r = 64, four directions, eight candidates sharing one base pass, loss summed over
    every next-token position, eps / sqrt(r) scaling; bank holding all four entries."""
    need_gpu()
    wl = workload(SMALL_OPT_BF16, rank=64, dir_seeds=(0, 1, 2, 3), n_prompts=2, len_lo=40, len_hi=70,
                  score_mode="all_next", scale_inv_sqrt_r=True, nu=1024, act_split=True)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c = np.array([0.5, -0.25, 1.5, -2.0])
    g.update(0, c, 2e-3)
    o.update(0, c, 2e-3)
    gs, os_ = g.score(1, batch), o.score(1, batch)
    err = _seq_close(gs, os_, 5e-4)          # two-term activations (see the small-model test)
    flush("r=64 max per-sequence |err| %.3g over %d tokens" % (err, len(os_["tok_logp"][0])))
    tok = gs["tok_logp"].cpu().numpy()
    allref = np.concatenate([os_["tok_logp"][p] for p in range(len(os_["phys"]))])
    assert np.max(np.abs(tok - allref)) <= 2e-2


@pytest.mark.parametrize("split", [False, True], ids=["bf16", "split"])
def test_projection_widths_not_multiple_of_tile(split):
    """d = 320, FFN 1280: the o-proj and fc2 outputs (N = 320) end inside a 256-wide
    column tile, and so does the QKV output (N = 960); side path on o, fc1, fc2 (the
    q/k/v boundaries are not tile multiples, which the library rejects for targets)."""
    need_gpu()
    wl = workload(SMALL_OPT_ODD, targets=("o", "fc1", "fc2"), dir_seeds=(2, 5), n_fg=2, n_prompts=3,
                  act_split=split)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c = np.array([1.3, -0.6])
    g.update(0, c, 5e-3)
    o.update(0, c, 5e-3)
    gs, os_ = g.score(1, batch), o.score(1, batch)
    err = _seq_close(gs, os_, 5e-4 if split else 2e-2)
    flush("odd widths (split %s): max per-sequence err %.3g" % (split, err))
    tok = gs["tok_logp"].cpu().numpy()
    allref = np.concatenate([os_["tok_logp"][p] for p in range(len(os_["phys"]))])
    assert np.max(np.abs(tok - allref)) <= (5e-4 if split else 2e-2)


@pytest.mark.parametrize("split", [False, True], ids=["bf16", "split"])
def test_wide_side_projection_in_k_slices(split):
    """r = 64 with four directions on o, fc1, fc2 of the d = 320, FFN 1280 model: every
    side-input projection has 256 factor columns per kind and runs on the pipelined kernel;
    the fc2 input (K = 1280, or 3840 as two-term products) is split into two K-slices with
    the ordered reduction, the others run whole."""
    need_gpu()
    wl = workload(SMALL_OPT_ODD, targets=("o", "fc1", "fc2"), rank=64, dir_seeds=(0, 1, 2, 3), n_prompts=2,
                  len_lo=20, len_hi=60, score_mode="all_next" if split else "last_label", scale_inv_sqrt_r=True,
                  nu=1024, act_split=split)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c = np.array([0.5, -0.25, 1.5, -2.0])
    g.update(0, c, 2e-3)
    o.update(0, c, 2e-3)
    gs, os_ = g.score(1, batch), o.score(1, batch)
    err = _seq_close(gs, os_, 5e-4 if split else 2e-2)
    flush("wide side projection (split %s): max per-sequence err %.3g" % (split, err))


def test_qkv_side_targets_off_tile_boundary_rejected():
    """q/k/v targets on a model whose q|k|v boundaries are not column-tile multiples:
    zo_score refuses with ZO_E_SHAPE instead of mixing kinds inside a tile."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl = workload(SMALL_OPT_ODD, targets=("q", "v"), n_prompts=2)
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    with pytest.raises(zo.ZoError) as ei:
        g.score(0, batch)
    assert ei.value.code == -2


@pytest.mark.parametrize("cfg", [SMALL_OPT_BF16, SMALL_QWEN_BF16], ids=["opt", "qwen3"])
def test_fold_matches_oracle_bitwise_then_scores(cfg):
    """zo_bank_fold commits a window-0 entry into the bf16 weights: every target weight
    (packed q|k|v rows, the interleaved gate/up pack) equals the oracle's fold bit for
    bit; the slot is freed; scoring at window 1 with the folded weights and the remaining
    entry matches the oracle (two-term activations, 5e-4)."""
    need_gpu()
    from oracle import params
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=1, n_prompts=2, act_split=True)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    for t, c in enumerate([np.array([0.9, -1.7]), np.array([-2.5, 0.4])]):
        g.update(t, c, 5e-3)
        o.update(t, c, 5e-3)
    seeds, wins = g.bank.keys()
    gslot = [i for i in range(len(seeds)) if seeds[i] == 3 and wins[i] == 0][0]
    oslot = [i for i, e in enumerate(o.bank.entries) if e is not None and e.seed == 3 and e.window == 0][0]
    flush("fold %s slot %d" % (cfg.arch, gslot))
    g.zo.fold(g.model, g.bank, gslot)
    ozo.fold(cfg, o.W, o.bank, oslot)
    assert g.bank.keys()[1][gslot] == -1
    pid = {"q": params.WQ, "k": params.WK, "v": params.WV, "o": params.WO, "fc1": params.W_FC1,
           "fc2": params.W_FC2, "gate": params.W_GATE, "up": params.W_UP, "down": params.W_DOWN}
    for layer in range(cfg.n_layers):
        for kind in wl.targets:
            got = g.model.tensor(layer + 1, pid[kind]).float().cpu().numpy()
            ref = o.W.get_layer(layer)[ozo.WEIGHT_NAME[kind]].astype(np.float32)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (layer, kind)
    gs, os_ = g.score(4, batch), o.score(4, batch)
    err = _seq_close(gs, os_, 5e-4)
    flush("after fold: max per-sequence err %.3g" % err)


def test_multi_step_trajectory_with_window_rollover():
    """Eight steps of score -> estimate -> update with nu = 4 (two windows: the
    bank gains a second entry at t = 4 and the first stays as a frozen term).  The
    oracle applies the GPU's c, so both states stay identical; S and c are checked at
    every step and the bank keys and factors at the end."""
    need_gpu()
    wl = configs.CONFIGS["tiny"].with_(nu=4)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl, n_slots=3), OracleRun(wl, n_slots=3)
    for t in range(8):
        gs, os_ = g.score(t, batch), o.score(t, batch)
        assert np.all(np.abs(gs["S"] - os_["S"]) <= 1e-4 * np.abs(os_["S"])), (t, gs["S"], os_["S"])
        cg = g.zo.estimate(g.plan(t), gs["S"])
        co = ozo.estimate(ozo.plan_from_workload(wl, t), os_["S"])
        assert np.all(np.abs(cg - co) <= 1e-2 * np.abs(co)), (t, cg, co)
        g.update(t, cg, 1e-2)
        o.update(t, cg, 1e-2)
    seeds, windows = g.bank.keys()
    assert sorted(w for w in windows if w >= 0) == [0, 1]
    for slot, e in enumerate(o.bank.entries):
        if e is None:
            continue
        gslot = [i for i in range(3) if windows[i] == e.window][0]
        for (layer, kind), U in e.U.items():
            assert np.array_equal(g.bank.entry(gslot, layer, kind).cpu().numpy(), U.astype(np.float32))


def test_trajectory_with_fold_at_rollover():
    """Twelve steps, nu = 4, a one-slot bank: at every window start the finished window's
    entry is folded into W (zo_bank_fold) before the new window's first update, on the
    GPU and in the oracle alike (the oracle applies the GPU's c).  S and c at every step,
    the folded weights and the final entry are checked."""
    need_gpu()
    wl = configs.CONFIGS["tiny"].with_(nu=4)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl, n_slots=1), OracleRun(wl, n_slots=1)
    for t in range(12):
        if t > 0 and t % wl.nu == 0:
            g.zo.fold(g.model, g.bank, 0)
            ozo.fold(wl.model, o.W, o.bank, 0)
        gs, os_ = g.score(t, batch), o.score(t, batch)
        assert np.all(np.abs(gs["S"] - os_["S"]) <= 1e-4 * np.abs(os_["S"])), (t, gs["S"], os_["S"])
        cg = g.zo.estimate(g.plan(t), gs["S"])
        co = ozo.estimate(ozo.plan_from_workload(wl, t), os_["S"])
        assert np.all(np.abs(cg - co) <= 1e-2 * np.abs(co)), (t, cg, co)
        g.update(t, cg, 1e-2)
        o.update(t, cg, 1e-2)
    assert g.bank.keys()[1] == [2]
    from oracle import params
    for layer in range(wl.model.n_layers):
        for kind, pid in (("q", params.WQ), ("v", params.WV)):
            got = g.model.tensor(layer + 1, pid).cpu().numpy()
            assert np.array_equal(got, o.W.get_layer(layer)[ozo.WEIGHT_NAME[kind]].astype(np.float32))
            assert np.array_equal(g.bank.entry(0, layer, kind).cpu().numpy(),
                                  o.bank.entries[0].U[(layer, kind)].astype(np.float32))


def test_bank_checkpoint_restore_is_bitwise():
    """The state is the bank memory plus its keys: restoring both into a fresh bank
    gives bitwise the same scores."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl = workload(SMALL_OPT_BF16, dir_seeds=(2, 9), nu=2)
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    for t in range(3):
        g.update(t, np.array([0.4 * (t + 1), -0.3]), 1e-2)
    a = g.score(3, batch)
    saved_mem = g.bank.mem.clone()
    saved_keys = g.bank.keys()
    fresh = zo.Bank(g.model, 4, wl.rank, wl.targets)
    fresh.mem.copy_(saved_mem)
    fresh.set_keys(*saved_keys)
    b = zo.score(g.model, g.plan(3), fresh, zo.DeviceBatch(batch))
    assert np.array_equal(a["S"], b["S"])
    assert np.array_equal(a["seq_logp"].cpu().numpy(), b["seq_logp"].cpu().numpy())


# fp8 models: every linear input is rounded to e4m3, a step function.  The kernels compute
# the values being rounded in fp32 from bf16 q, k, v and bf16 attention probabilities (up to
# a relative 2^-9 from the fp64 definition), so wherever the two straddle an e4m3 rounding
# boundary they land one e4m3 step apart.  The bounds are written by
# tests/golden/make_fp8_floor.py from the oracle alone: the oracle's own log-probs moved by
# perturbing every pre-rounding value by a relative 2^-9 (three seeds), times two, and never
# below the bf16 bound.
def fp8_bounds(case):
    import json, os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8floor_%s.json" % case)) as f:
        rec = json.load(f)
    return rec["bound_seq"], rec["bound_tok"], rec


@pytest.mark.parametrize("cfg", [SMALL_OPT_FP8, SMALL_QWEN_FP8], ids=["opt", "qwen3"])
def test_fp8_model_with_bank_matches_oracle(cfg):
    """fp8 models: e4m3 x e4m3 projections with the bf16 side path (two directions, a bank
    with entries of two windows), ragged rows; Qwen3: GQA, QK-norm + RoPE on bf16 q|k|v,
    SwiGLU written as e4m3 from the interleaved gate/up tile."""
    need_gpu()
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=2, n_prompts=3)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    c_fixed = [np.array([0.9, -1.7]), np.array([-2.5, 0.4]), np.array([1.1, 0.8])]
    for k, t in enumerate((0, 3, 5)):
        g.update(t, c_fixed[k], 5e-3)
        o.update(t, c_fixed[k], 5e-3)
    flush("fp8 score")
    gs, os_ = g.score(6, batch), o.score(6, batch)
    flush("rows %d" % int(gs["n_rows"]))
    bound_seq, bound_tok, rec = fp8_bounds("opt-small-fp8" if cfg.arch == "opt" else "qwen3-small-fp8")
    # the stored expected values are the oracle's own (the same state): a stale file fails here
    assert np.allclose(rec["seq_logp"], os_["seq_logp"], rtol=0, atol=1e-9)
    err = _seq_close(gs, os_, bound_seq)
    flush("fp8: max per-sequence err %.3g (bound %.3g from the oracle's floor %.3g)" % (
        err, bound_seq, rec["floor_seq_max"]))
    tok = gs["tok_logp"].cpu().numpy()
    first = 0
    tok_err = []
    for p, (li, c) in enumerate(os_["phys"]):
        ref = os_["tok_logp"][p]
        tok_err.append(np.max(np.abs(tok[first:first + len(ref)] - ref)))
        first += len(ref)
    flush("fp8 %s: max per-token err %.3g (per sequence %s)" % (cfg.arch, max(tok_err), np.round(tok_err, 3)))
    fg = [i for i, (li, c) in enumerate(os_["phys"]) if c < 0]
    assert max(tok_err[i] for i in fg) <= bound_tok
    # the probes' differences, what c is made of: each candidate sums its probe sequences, so
    # |dS_c| is at most the sequence bound times their number
    S_g, S_o = np.asarray(gs["S"]), np.asarray(os_["S"])
    n_seq = np.array([sum(1 for _, c in os_["phys"] if c == k) for k in range(len(S_o))])
    flush("S gpu %s oracle %s" % (S_g, S_o))
    assert np.all(np.abs(S_g - S_o) <= bound_seq * n_seq)


def test_fp8_probe_rows_bitwise_across_batch_sizes():
    """As for bf16 models: a probe sequence's log-prob is bitwise the same in a large batch
    (about 45k rows) and in a two-prompt batch."""
    need_gpu()
    wl = workload(SMALL_OPT_FP8, n_prompts=72, len_lo=100, dir_seeds=(1,))
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    g.update(0, np.array([0.9]), 1e-2)
    big = g.score(1, batch)
    small = g.score(1, batch.subset([0, 1]))
    assert int(big["n_rows"]) > 43 * 256 and int(small["n_rows"]) < 4 * 256
    n = batch.n_seq
    a = big["seq_logp"].cpu().numpy()
    b = small["seq_logp"].cpu().numpy()
    for ia, ib in ((0, 0), (1, 1), (n, 2), (n + 1, 3)):
        assert a[ia:ia + 1].view(np.uint64)[0] == b[ib:ib + 1].view(np.uint64)[0], (ia, ib)


def test_fp8_model_rejections():
    """fp8 models refuse two-term activations (ZO_E_INVAL) and side-input projections wider
    than 128 columns (ZO_E_SHAPE)."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl = workload(SMALL_OPT_FP8, n_prompts=2)
    batch = inputs.make_batch(wl)
    g = GpuRun(wl)
    with pytest.raises(zo.ZoError) as ei:
        g.score(0, batch, flags=zo.api.PLAN_ACT_SPLIT)
    assert ei.value.code == -1
    wide = workload(SMALL_OPT_FP8, targets=("o",), rank=64, dir_seeds=(0, 1, 2, 3), n_prompts=2, nu=1024)
    gw = GpuRun(wide)
    with pytest.raises(zo.ZoError) as ei:
        gw.score(0, inputs.make_batch(wide))
    assert ei.value.code == -2


@pytest.mark.parametrize("cfg", [SMALL_OPT_FP8, SMALL_QWEN_FP8], ids=["opt", "qwen3"])
def test_fp8_fold_requantizes_like_the_oracle(cfg):
    """zo_bank_fold on an fp8 model: W <- e4m3(W + U V^T) (the fp64 sum rounded to fp32, then
    to the e4m3 code of w * 2^11): every folded weight code equals the oracle's, and scoring
    after the fold matches the oracle under the small fp8 model's bound."""
    need_gpu()
    import json, os, torch
    from oracle import params
    wl = workload(cfg, dir_seeds=(3, 8), n_fg=1, n_prompts=2)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl), OracleRun(wl)
    for t, c in enumerate([np.array([0.9, -1.7]), np.array([-2.5, 0.4])]):
        g.update(t, c, 5e-3)
        o.update(t, c, 5e-3)
    seeds, wins = g.bank.keys()
    gslot = [i for i in range(len(seeds)) if seeds[i] == 3 and wins[i] == 0][0]
    oslot = [i for i, e in enumerate(o.bank.entries) if e is not None and e.seed == 3 and e.window == 0][0]
    g.zo.fold(g.model, g.bank, gslot)
    ozo.fold(cfg, o.W, o.bank, oslot)
    pid = {"q": params.WQ, "k": params.WK, "v": params.WV, "o": params.WO, "fc1": params.W_FC1,
           "fc2": params.W_FC2, "gate": params.W_GATE, "up": params.W_UP, "down": params.W_DOWN}
    changed = 0
    for layer in range(cfg.n_layers):
        for kind in wl.targets:
            got = g.model.tensor(layer + 1, pid[kind]).double().cpu().numpy() / 2048.0
            ref = o.W.get_layer(layer)[ozo.WEIGHT_NAME[kind]]
            assert np.array_equal(got, ref), (layer, kind, np.mean(got != ref))
            changed += int(np.sum(got != params.make_tensor(cfg, wl.model_seed, layer + 1, pid[kind],
                                                            cfg.linear_shape(kind), "matrix")))
    assert changed > 0
    gs, os_ = g.score(4, batch), o.score(4, batch)
    name = "opt-small-fp8" if cfg.arch == "opt" else "qwen3-small-fp8"
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8floor_%s.json" % name)) as f:
        bound = json.load(f)["bound_seq"]
    err = _seq_close(gs, os_, bound)
    flush("fp8 fold %s: %d weights changed, max per-sequence err after the fold %.3g (bound %.3g)" % (
        cfg.arch, changed, err, bound))


def test_bank_cap_trajectory():
    """Eight steps of score -> estimate -> update -> zo_bank_cap(max_frozen = 1) with nu = 2
    (four windows): the oldest frozen entry is folded into W at t = 4 and t = 6, on the GPU
    and in the oracle alike (the oracle applies the GPU's c).  S and c at every step, the
    number folded, the bank keys and the folded weights are checked."""
    need_gpu()
    import zeroth_order_fine_amd as zo
    from oracle import params
    wl = configs.CONFIGS["tiny"].with_(nu=2)
    batch = inputs.make_batch(wl)
    g, o = GpuRun(wl, n_slots=3), OracleRun(wl, n_slots=3)
    for t in range(8):
        gs, os_ = g.score(t, batch), o.score(t, batch)
        assert np.all(np.abs(gs["S"] - os_["S"]) <= 1e-4 * np.abs(os_["S"])), (t, gs["S"], os_["S"])
        cg = g.zo.estimate(g.plan(t), gs["S"])
        co = ozo.estimate(ozo.plan_from_workload(wl, t), os_["S"])
        assert np.all(np.abs(cg - co) <= 1e-2 * np.abs(co)), (t, cg, co)
        g.update(t, cg, 1e-2)
        o.update(t, cg, 1e-2)
        nf = zo.bank_cap(g.model, g.bank, g.plan(t), 1)
        assert nf == ozo.cap(wl.model, o.W, o.bank, ozo.plan_from_workload(wl, t), 1), t
        assert nf == (1 if t in (4, 6) else 0), (t, nf)
    seeds, windows = g.bank.keys()
    assert sorted(w for w in windows if w >= 0) == [2, 3]
    for layer in range(wl.model.n_layers):
        for kind, pid in (("q", params.WQ), ("v", params.WV)):
            got = g.model.tensor(layer + 1, pid).cpu().numpy()
            assert np.array_equal(got, o.W.get_layer(layer)[ozo.WEIGHT_NAME[kind]].astype(np.float32))
