#!/usr/bin/env python3
"""Throughput of the inference-native ZO step on one MI355X.

A step is the whole hot path on one batch: zo_plan (ProbePlan for step t),
zo_score (one batched forward over every candidate state with the fused
vocabulary log-softmax + label gather), zo_estimate and zo_update (lazy
low-rank bank update), with t advancing.  Default workload: the OPT-13B-shaped
batch-64 configuration (40 layers, d 5120, FFN 20480, vocab 50272, bf16
random-init weights resident in HBM, 64 ragged prompts of U[16,128] tokens,
LoZO rank 2 on every linear, 2 candidates, persistent bank).

Prints one JSON line.  `value` = probe token rows scored per second over the
whole step (sum of the lengths of every probe physical sequence / step time).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ZO probe scored tokens/sec + ZO steps/sec (OPT-13B shape, batch 64, 1 GPU)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "%s_gemm_base_traffic.md")   # per workload
GEMM_SOURCE = os.path.join(ROOT, "zeroth_order_fine_amd", "csrc", "gemm.hip")


def measured_traffic(workload):
    """HBM bytes per projection launch from the committed rocprofv3 PMC summary, if it
    was taken on the current GEMM source (else None)."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_FILE % workload).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except Exception:
        return None
    if rec.get("gemm_source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration():
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 3}))


def measured_peaks():
    """Ceilings measured on this GPU by the committed microbenchmarks (libzo_peaks.so): a
    dense bf16 MFMA loop on constant and on random operands, and 1 GiB streaming copy / read
    / mixed kernels; reported beside the published peaks."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "zeroth_order_fine_amd", "libzo_peaks.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    for f in (L.zo_peak_mfma_bf16, L.zo_peak_mfma_bf16_random, L.zo_peak_copy, L.zo_peak_read, L.zo_peak_mix):
        f.restype = ctypes.c_double
    L.zo_peak_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    L.zo_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    L.zo_peak_mfma_bf16_random.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    L.zo_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    L.zo_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    blocks = 1024
    out = torch.empty(blocks * 256 * 4, dtype=torch.float32, device="cuda")
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    res = {"mfma_bf16_tflops": round(L.zo_peak_mfma_bf16(ctypes.c_void_p(out.data_ptr()), blocks, 2000), 1),
           # the same loop on random operands: the clock the matrix cores hold on real data
           "mfma_bf16_random_tflops": round(L.zo_peak_mfma_bf16_random(ctypes.c_void_p(out.data_ptr()), blocks,
                                                                       2000), 1),
           "copy_gbs": round(L.zo_peak_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, 4096), 1),
           "read_gbs": round(L.zo_peak_read(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(out.data_ptr()), n, 4096), 1),
           # read:write byte mixes of the norms (2:1) and of attention (3:1)
           "mix2_gbs": round(L.zo_peak_mix(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n // 4, 2,
                                           4096), 1),
           "mix3_gbs": round(L.zo_peak_mix(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n // 4, 3,
                                           4096), 1)}
    del a, b, out
    torch.cuda.empty_cache()
    return res


def base_gemm_flops(cfg, rows):
    """Algorithmic FLOPs of the shared-weight projections for `rows` token rows."""
    total = 0
    for kind in cfg.kind_names:
        n_out, n_in = cfg.linear_shape(kind)
        total += 2 * rows * n_out * n_in
    return total * cfg.n_layers


def group_kinds(cfg):
    """Input groups of the side-input projection: linears that read the same activations."""
    if cfg.arch == "opt":
        return [("q", "k", "v"), ("o",), ("fc1",), ("fc2",)]
    return [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]


def hbm_bytes_per_step(cfg, wl, rows, scored, n_entries, n_shared=0):
    """Algorithmic HBM bytes per step of the bandwidth-bound kernel classes: every tensor
    read or written once, no padding, no re-reads (the unit the HBM fractions use).
    n_shared of the n_entries bank entries are the directions' own entries of the current
    window, whose V is the direction's, so they add no side-input columns."""
    split = wl.act_split
    a = 2 * (2 if split else 1)          # bytes per activation element fed to a bf16 GEMM
    d, f, L = cfg.d_model, cfg.d_ffn, cfg.n_layers
    nq, nkv = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    w = 4 if cfg.dtype == "f32" else 2   # embeddings, head, q|k|v (bf16 in fp8 models too)
    if cfg.dtype == "f32":
        a = 4
    ai = 1 if cfg.dtype == "fp8" else a  # layer-linear inputs (e4m3 in fp8 models)
    r, q = wl.rank, wl.n_dirs
    used = (n_entries - n_shared + q) * r
    out = {}
    # embedding (+ learned positions), two norms per layer, final norm, QK-norm + RoPE
    nb = rows * d * (w * (2 if cfg.arch == "opt" else 1) + 4)
    nb += 2 * L * rows * d * (4 + ai) + scored * d * (4 + a)
    if cfg.arch != "opt":
        nb += L * rows * (nq + nkv) * 2 * (4 if split else w)
    out["norm"] = nb
    qkv_b = 4 if split else w
    out["attention"] = L * rows * ((nq + 2 * nkv) * qkv_b + nq * ai)
    side = 0
    prep = 0
    for g, kinds in enumerate(group_kinds(cfg)):
        tk = [k for k in kinds if k in wl.targets]
        if not tk:
            continue
        n_in = cfg.linear_shape(tk[0])[1]
        # groups 0 and 2 read a norm's output: with one-term activations and at most 16 used
        # factor columns the norm kernel forms t from the row it holds (no re-read)
        if g in (0, 2) and cfg.dtype != "f32" and not split and len(kinds) * used <= 16:
            out["norm"] += len(tk) * used * n_in * 2 + rows * len(tk) * used * a
            continue
        # group 3 (fc2 / down) with at most 4 used columns: the fc1 / gate-up epilogue writes
        # per-64-column partial sums; the side-input class is then their ordered reduction
        # (partials read once, t written once)
        if g == 3 and cfg.dtype != "f32" and not split and used <= 4:
            n1 = cfg.d_ffn * (1 if cfg.arch == "opt" else 2)
            side += rows * ((n1 + 63) // 64) * used * 4 + rows * used * a
            n_out = cfg.linear_shape(tk[0])[0]
            prep += used * (n_in + n_out) * 2 + n_entries * r * n_out * 4
            continue
        side += rows * n_in * ai + len(tk) * used * n_in * 2 * (3 if split else 1) + rows * len(tk) * used * a
        for k in tk:
            n_out = cfg.linear_shape(k)[0]
            prep += used * (n_in + n_out) * 2 * (3 if split else 1) + n_entries * r * n_out * 4
    out["gemm_side"] = L * side
    out["side_prep"] = L * prep
    out["gemm_head"] = cfg.vocab * d * w + scored * d * a + scored * ((cfg.vocab + 127) // 128) * 8
    out["update"] = q * L * sum(cfg.linear_shape(k)[0] * r * 8 for k in wl.targets)
    return out


def accuracy_vs_golden(name, wl, model, db):
    """The timed precision mode against the expected values the oracle wrote for this
    workload (tests/golden/<workload>_step1.json: one update at step 0 with fixed
    coefficients, scoring at step 1): per probe sequence |error|, how many exceed the bf16
    bound 2e-2, and the relative error of c = (L+ - L-)/2eps where the file has S."""
    import numpy as np

    import zeroth_order_fine_amd as zo
    path = os.path.join(ROOT, "tests", "golden", "%s_step1.json" % name)
    if not os.path.exists(path):
        return None
    gold = json.load(open(path))
    bank = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
    zo.update(model, zo.Plan.from_workload(model, wl, t=0), bank, gold["state"]["c"], gold["state"]["lr"])
    plan = zo.Plan.from_workload(model, wl, t=1)
    out = zo.score(model, plan, bank, db)
    seq = out["seq_logp"].cpu().numpy()
    err = np.array([abs(seq[p] - g) for p, (li, c), g in zip(gold["phys_index"], gold["phys"], gold["seq_logp"])
                    if c >= 0])
    res = {"probe_sequences": int(err.size), "max_seq_err": round(float(err.max()), 5),
           "mean_seq_err": round(float(err.mean()), 5), "seq_above_2e-2": int((err > 2e-2).sum())}
    if "c" in gold:
        c = zo.estimate(plan, out["S"])
        res["c"] = [round(float(x), 4) for x in c]
        res["c_oracle"] = [round(float(x), 4) for x in gold["c"]]
        res["c_rel_err"] = round(float(np.max(np.abs(c - np.array(gold["c"])) / np.abs(np.array(gold["c"])))), 4)
    del bank
    return res


def describe(wl):
    m = wl.model
    return ("%s: %s-shaped %d x d%d, heads %d/%d x %d, FFN %d, vocab %d, %s weights; %d prompts U[%d,%d]%s, "
            "%d candidates (%d directions x +-), r=%d on %s, eps=%g" % (
                wl.name, m.arch.upper(), m.n_layers, m.d_model, m.n_heads, m.n_kv_heads, m.head_dim, m.d_ffn,
                m.vocab, m.dtype, wl.n_prompts, wl.len_lo, wl.len_hi,
                (" + %d foreground" % wl.n_fg) if wl.n_fg else "", len(wl.candidates), wl.n_dirs, wl.rank,
                ",".join(wl.targets), wl.eps))


def cpu_baseline(wl, batch, n_prompts=8, n_layers=3):
    """Time the oracle (as it stands) on a bounded sample: the first `n_prompts` probe
    prompts under every candidate, through the first `n_layers` decoder layers plus the
    vocabulary head; the per-token rate for the whole model is extrapolated as
    (n_layers_total / n_layers) x layer time + head time."""
    import numpy as np

    from oracle import model as om
    from oracle import zo as ozo
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    cfg = wl.model
    nl = min(n_layers, cfg.n_layers)
    t0 = time.perf_counter()
    W = ozo.Weights(cfg, wl.model_seed, cache_layers=False)
    G = W.get_global()
    t_gen = time.perf_counter() - t0
    plan = ozo.plan_from_workload(wl, 0)
    phys = ozo.pack(batch, plan)
    probes = [i for i in range(batch.n_seq) if batch.role[i] == 0][:n_prompts]
    sample = [(li, c) for li, c in phys if li in probes]
    toks = [np.asarray(batch.tokens[li], np.int64) for li, c in sample]
    hs = [om.embed(cfg, G, t) for t in toks]
    sides = [ozo.side_terms(cfg, plan, None, c) for li, c in sample]
    t_layer = 0.0
    for l in range(nl):
        a = time.perf_counter()
        Wl = W.get_layer(l)
        t_gen += time.perf_counter() - a
        a = time.perf_counter()
        hs = [om.layer_forward(cfg, Wl, h, lambda kind, s=s, l=l: s(l, kind), False) for h, s in zip(hs, sides)]
        t_layer += time.perf_counter() - a
    a = time.perf_counter()
    for h, t, (li, c) in zip(hs, toks, sample):
        pos, lab = ozo.scored_positions(t, int(batch.score_mode[li]))
        om.final_logprobs(cfg, G, h, pos, lab)
    t_head = time.perf_counter() - a
    rows = sum(len(t) for t in toks)
    est = cfg.n_layers / nl * t_layer + t_head
    return {"value": rows / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": ("probe prompts %s (%d token rows) under all %d candidates through layers 0-%d of %d and "
                       "the head; layers %.2f s, head %.2f s, extrapolated x%.1f; oracle weight generation "
                       "%.1f s not counted" % (probes, rows, len(plan.candidates), nl - 1, cfg.n_layers, t_layer,
                                               t_head, cfg.n_layers / nl, t_gen))}


def generation_bench(args, wl, model, bank, batch, db):
    """Greedy generation of args.generate tokens for every physical sequence of the
    workload (every probe prompt under every candidate state, with a bank entry): one
    zo_generate call = prefill + (N - 1) decode steps.  value = generated tokens/s; the
    roofline is the decode attention's (HBM: every cached K and V row read once per
    decode step and kv head)."""
    import torch

    import zeroth_order_fine_amd as zo
    cfg = wl.model
    n_new = args.generate
    for t in range(2):                       # steady state: the bank holds an entry
        plan = zo.Plan.from_workload(model, wl, t=t)
        zo.update(model, plan, bank, zo.estimate(plan, zo.score(model, plan, bank, db)["S"]), args.lr)
    plan = zo.Plan.from_workload(model, wl, t=2)
    for _ in range(args.warmup):
        zo.generate(model, plan, bank, db, n_new)
    torch.cuda.synchronize()
    a = time.perf_counter()
    for _ in range(args.steps):
        out = zo.generate(model, plan, bank, db, n_new)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - a) / args.steps * 1e3
    zo.api.profile_begin()
    zo.generate(model, plan, bank, db, n_new)
    torch.cuda.synchronize()
    prof = zo.api.profile_end()
    phys = zo.pack(model, plan, db)
    lengths = [len(t) for t in batch.tokens]
    n_phys = out["n_phys"]
    esz = 4 if cfg.dtype == "f32" else 2
    nq, nkv = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    dec_bytes = 0
    for li in phys[0]:
        for j in range(1, n_new):
            keys = lengths[li] + j
            # cached K and V rows, q row in, output row out, appended k and v (read + write)
            dec_bytes += cfg.n_layers * esz * (2 * keys * nkv + 2 * nq + 4 * nkv)
    n_dec, ms_dec = prof["decode_attention"]
    gbs = dec_bytes / (ms_dec / 1e3) / 1e9 if ms_dec > 0 else None
    line = {
        "metric": "ZO generation: generated tokens/s under candidate states (greedy, 1 GPU)",
        "value": round(n_phys * n_new / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_call": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": describe(wl), "sequences": n_phys, "new_tokens": n_new,
                   "prompt_tokens": int(sum(lengths[li] for li in phys[0])), "hip_graph_replay": args.graphs},
        "roofline": {"kernel": "decode attention (single-query attention over the K/V cache)", "bound": "hbm",
                     "achieved": round(gbs, 1) if gbs else None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4) if gbs else None, "traffic": None,
                     "launches_per_call": n_dec, "algorithmic_mb_per_call": round(dec_bytes / 1e6, 2)},
        "breakdown_ms_per_call": {k: round(v[1], 3) for k, v in prof.items()},
    }
    print(json.dumps(line), flush=True)


def sites_bench(args, wl, model, db):
    """The precision / cost trade-off of two-term activations at single rounding sites
    (ZO_PLAN_SPLIT_*): for each site mask, score time and the per-sequence error against the
    oracle's expected values for this workload (tests/golden/<workload>_step1.json)."""
    import torch

    import zeroth_order_fine_amd as zo
    A = zo.api
    sites = {"none": 0, "qkv_in": A.PLAN_SPLIT_QKV_IN, "attn": A.PLAN_SPLIT_ATTN, "fc1_in": A.PLAN_SPLIT_FC1_IN,
             "fc2_in": A.PLAN_SPLIT_FC2_IN, "head": A.PLAN_SPLIT_HEAD,
             "attn+qkv_in": A.PLAN_SPLIT_ATTN | A.PLAN_SPLIT_QKV_IN,
             "attn+qkv_in+fc1_in": A.PLAN_SPLIT_ATTN | A.PLAN_SPLIT_QKV_IN | A.PLAN_SPLIT_FC1_IN,
             "all": A.PLAN_ACT_SPLIT}
    base = wl.with_(act_split=False)
    rows = []
    for name, bits in sites.items():
        w = base.with_(split_sites=bits)
        acc = accuracy_vs_golden(args.workload, w, model, db)
        bank = zo.Bank(model, 2 * w.n_dirs, w.rank, w.targets)
        plan = zo.Plan.from_workload(model, w, t=1)
        zo.score(model, plan, bank, db)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(max(1, args.steps)):
            zo.score(model, plan, bank, db)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / max(1, args.steps) * 1e3
        del bank, plan
        row = {"sites": name, "flags": bits, "score_ms": round(ms, 2)}
        if acc:
            row.update(acc)
        rows.append(row)
        print(json.dumps(row), flush=True)
    print(json.dumps({"workload": args.workload, "split_sites": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt13b")
    ap.add_argument("--lr", type=float, default=1e-4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the MFMA-loop and copy microbenchmarks of the measured ceilings")
    ap.add_argument("--no-side-check", action="store_true",
                    help="skip the extra scoring without side path that measures its cost (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for the traffic figure)")
    ap.add_argument("--graphs", action="store_true",
                    help="replay zo_score's forward pass from a captured HIP graph (launch-bound small "
                         "workloads); the timed steps then carry no per-launch events and the roofline "
                         "comes from the eagerly launched breakdown steps")
    ap.add_argument("--sites", action="store_true",
                    help="score time and accuracy against the oracle's expected values of two-term activations "
                         "at each single rounding site (and a few combinations) instead of the ZO step")
    ap.add_argument("--generate", type=int, default=0, metavar="N",
                    help="time greedy generation of N tokens per sequence (zo_generate) instead of the ZO step")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py: the library scores on one GPU (got --gpus %d); a multi-GPU run is not "
              "provided" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import zeroth_order_fine_amd as zo
    from synth import configs, inputs

    wl = configs.CONFIGS[args.workload]
    cfg = wl.model
    torch.cuda.set_device(0)
    # a stream of its own (default priority): graph capture needs a stream other than the null one
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    model = zo.Model(cfg)
    model.init_weights(wl.model_seed)
    batch = inputs.make_batch(wl)
    db = zo.DeviceBatch(batch)
    bank = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
    torch.cuda.synchronize()
    model.set_graphs(args.graphs)
    if args.generate:
        generation_bench(args, wl, model, bank, batch, db)
        return
    if args.sites:
        sites_bench(args, wl, model, db)
        return

    score_s = [0.0]

    def step(t):
        plan = zo.Plan.from_workload(model, wl, t=t)
        a = time.perf_counter()
        out = zo.score(model, plan, bank, db)
        score_s[0] += time.perf_counter() - a
        c = zo.estimate(plan, out["S"])
        zo.update(model, plan, bank, c, args.lr)
        return out

    out = None
    for t in range(args.warmup):
        out = step(t)
    torch.cuda.synchronize()
    score_s[0] = 0.0
    # timed region: events only around the projections (the roofline kernel)
    if not args.graphs:
        zo.api.profile_begin(["gemm_base"])
    t0 = time.perf_counter()
    marks = [t0]
    for k in range(args.steps):
        out = step(args.warmup + k)
        marks.append(time.perf_counter())   # zo_score ends in a stream synchronisation
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted((b - a) * 1e3 for a, b in zip(marks, marks[1:]))
    score_timed = score_s[0]
    prof_timed = zo.api.profile_end() if not args.graphs else None
    # per-class breakdown: a few more steps with every class timed
    n_bd = max(1, min(args.steps, 5))
    zo.api.profile_begin()
    for k in range(n_bd):
        out = step(args.warmup + args.steps + k)
    torch.cuda.synchronize()
    prof = zo.api.profile_end()
    t_next = args.warmup + args.steps + n_bd

    phys = zo.pack(model, zo.Plan.from_workload(model, wl, t=0), db)
    lengths = batch.lengths
    probe_tokens = int(sum(lengths[li] for li, c in zip(phys[0], phys[1]) if c >= 0))
    fg_tokens = int(sum(lengths[li] for li, c in zip(phys[0], phys[1]) if c < 0))
    rows = probe_tokens + fg_tokens
    ms_step = elapsed / args.steps * 1e3
    value = probe_tokens / (ms_step / 1e3)

    # projection launch times: the timed steps' events, or with graph replay the breakdown steps'
    n_base, ms_base = (prof_timed or prof)["gemm_base"]
    flops_step = base_gemm_flops(cfg, rows)
    launches_per_step = n_base / (args.steps if prof_timed else n_bd)
    avg_launch_ms = ms_base / max(n_base, 1)
    achieved = (flops_step / launches_per_step) / (avg_launch_ms / 1e3) / 1e12 if n_base else None
    peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(cfg.dtype, PEAK_F32_TFLOPS)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "median_step_ms": round(step_ms[len(step_ms) // 2], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": describe(wl), "prompts": wl.n_prompts, "candidates": len(wl.candidates),
                   "rank": wl.rank, "probe_tokens_per_step": probe_tokens, "foreground_tokens_per_step": fg_tokens,
                   "scored_positions_per_step": int(out["n_scored"]), "hip_graph_replay": args.graphs},
        "steps_per_s": round(args.steps / elapsed, 4),
        "score_only_tokens_per_s": round(probe_tokens * args.steps / score_timed, 1),
        "score_share_of_step": round(score_timed / elapsed, 4),
        "roofline": {"kernel": {"bf16": "gemm_base (shared-weight projections, bf16 MFMA)",
                                "fp8": "gemm_base (shared-weight projections, e4m3 x e4m3 MFMA)"}.get(
                                    cfg.dtype, "gemm_base (fp32 VALU)"),
                     "bound": "mfma", "achieved": round(achieved, 1) if achieved else None, "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4) if achieved else None,
                     "traffic": measured_traffic(args.workload),
                     "launches_per_step": launches_per_step, "avg_launch_ms": round(avg_launch_ms, 4),
                     "algorithmic_gflop_per_step": round(flops_step / 1e9, 1)},
        "breakdown_ms_per_step": {k: round(v[1] / n_bd, 3) for k, v in prof.items()},
        "launches_per_step": {k: v[0] / n_bd for k, v in prof.items()},
    }
    # bandwidth-bound classes: algorithmic bytes per step / class time per step
    seeds, wins = bank.keys()
    n_entries = sum(1 for w in wins if w >= 0)
    window = (args.warmup + args.steps - 1) // wl.nu
    n_shared = sum(1 for s_, w in zip(seeds, wins) if w == window and s_ in wl.dir_seeds)
    hb = hbm_bytes_per_step(cfg, wl, rows, int(out["n_scored"]), n_entries, n_shared)
    hbm = {}
    for k, b in hb.items():
        ms = prof[k][1] / n_bd
        if ms > 0:
            gbs = b / (ms / 1e3) / 1e9
            hbm[k] = {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_mb_per_step": round(b / 1e6, 2)}
    line["hbm_kernels"] = hbm
    if not args.no_peaks:
        pk = measured_peaks()
        if pk:
            line["measured_peaks"] = pk
            if achieved and cfg.dtype == "bf16":
                line["roofline"]["frac_of_measured_mfma"] = round(achieved / pk["mfma_bf16_tflops"], 4)
                line["roofline"]["frac_of_random_operand_mfma"] = round(achieved / pk["mfma_bf16_random_tflops"], 4)
            # each class against the streaming microbenchmark with its own read:write mix
            matched = {"norm": "mix2_gbs", "attention": "mix3_gbs", "gemm_side": "read_gbs", "gemm_head": "read_gbs",
                       "side_prep": "copy_gbs", "update": "copy_gbs"}
            for k, v in hbm.items():
                ref = matched.get(k, "copy_gbs")
                v["matched_ceiling"] = ref
                v["frac_of_matched_ceiling"] = round(v["achieved"] / pk[ref], 4)
    # side-path cost: the projections' time with the side columns vs a plan with no targets
    if wl.targets and not args.no_side_check:
        # scores with and without the side path, alternated so that clock drift between
        # the two phases does not masquerade as side-path cost
        n_off = 4
        wl0 = wl.with_(targets=())
        on, off = {}, {}
        for k in range(n_off):
            for tgt, plan_ in ((on, zo.Plan.from_workload(model, wl, t=t_next)),
                               (off, zo.Plan.from_workload(model, wl0, t=0))):
                zo.api.profile_begin()
                zo.score(model, plan_, bank if tgt is on else None, db)
                torch.cuda.synchronize()
                for cls, (n_, ms_) in zo.api.profile_end().items():
                    tgt[cls] = tgt.get(cls, 0.0) + ms_ / n_off
        base_on, base_off = on["gemm_base"], off["gemm_base"]
        norm_on, norm_off = on["norm"], off["norm"]
        total = base_on - base_off + norm_on - norm_off + on["gemm_side"] + on["side_prep"]
        line["side_path"] = {
            "gemm_base_ms_with_side": round(base_on, 3), "gemm_base_ms_without": round(base_off, 3),
            "extended_k_overhead": round(base_on / base_off - 1.0, 4),
            "norm_ms_with_side": round(norm_on, 3), "norm_ms_without": round(norm_off, 3),
            "total_ms_per_step": round(total, 3), "share_of_step": round(total / ms_step, 4)}
    # other states of the same workload, scored after the timed region (score only)
    extra = {}

    def score_ms(bank_, db_, n=3):
        torch.cuda.synchronize()
        a = time.perf_counter()
        for k in range(n):
            zo.score(model, zo.Plan.from_workload(model, wl, t=t_next), bank_, db_)
        torch.cuda.synchronize()
        return (time.perf_counter() - a) / n * 1e3

    if not args.no_side_check:
        # bank growth: score time with E frozen entries (windows 0 .. E-1, each a rank-r side
        # term of every probe row) besides the plan's direction
        # (single-direction plans: each window leaves one entry; the MeZO-style workload's
        # four rank-64 directions a window would make 16 windows a rank-4096 side path)
        growth = {}
        for E in ((0, 1, 4, 16) if wl.n_dirs == 1 else ()):
            bE = zo.Bank(model, E + 2 * wl.n_dirs, wl.rank, wl.targets)
            for win in range(E):
                zo.update(model, zo.Plan.from_workload(model, wl, t=win * wl.nu), bE, [0.5] * wl.n_dirs, args.lr)
            pE = zo.Plan.from_workload(model, wl, t=E * wl.nu)
            try:
                zo.score(model, pE, bE, db)
            except zo.ZoError as e:      # e.g. fp8 models: side-input projections of at most 128 columns
                growth[str(E)] = "refused: %s" % e
                del bE
                continue
            torch.cuda.synchronize()
            a = time.perf_counter()
            for k in range(3):
                zo.score(model, pE, bE, db)
            torch.cuda.synchronize()
            growth[str(E)] = round((time.perf_counter() - a) / 3 * 1e3, 3)
            del bE
        if growth:
            extra["score_ms_by_frozen_entries"] = growth
        extra["score_ms_steady_bank"] = round(score_ms(bank, db), 3)
        extra["score_ms_empty_bank"] = round(score_ms(None, db), 3)
        if wl.n_fg:
            fg = batch.subset([i for i in range(batch.n_seq) if batch.role[i] == inputs.ROLE_FOREGROUND])
            extra["score_ms_foreground_only"] = round(score_ms(bank, zo.DeviceBatch(fg)), 3)
            extra["foreground_only_tokens_per_s"] = round(fg_tokens / (extra["score_ms_foreground_only"] / 1e3), 1)
        if not wl.act_split and cfg.dtype == "bf16":
            def step_ms(wl2):
                bank2 = zo.Bank(model, 2 * wl.n_dirs, wl.rank, wl.targets)
                for t in range(2):
                    p2 = zo.Plan.from_workload(model, wl2, t=t)
                    zo.update(model, p2, bank2, zo.estimate(p2, zo.score(model, p2, bank2, db)["S"]), args.lr)
                torch.cuda.synchronize()
                a = time.perf_counter()
                n2 = 3
                for t in range(2, 2 + n2):
                    p2 = zo.Plan.from_workload(model, wl2, t=t)
                    zo.update(model, p2, bank2, zo.estimate(p2, zo.score(model, p2, bank2, db)["S"]), args.lr)
                torch.cuda.synchronize()
                del bank2
                return (time.perf_counter() - a) / n2 * 1e3
            # the same step with two-term activations everywhere (what keeps c within 1e-2 at
            # eps = 1e-3), and at the three rounding sites that carry most of the error here
            # (attention, and the inputs of the q|k|v and fc1 projections; not the fc2 input)
            ms2 = step_ms(wl.with_(act_split=True))
            extra["two_term_ms_per_step"] = round(ms2, 3)
            extra["two_term_tokens_per_s"] = round(probe_tokens / (ms2 / 1e3), 1)
            A = zo.api
            wl3 = wl.with_(split_sites=A.PLAN_SPLIT_ATTN | A.PLAN_SPLIT_QKV_IN | A.PLAN_SPLIT_FC1_IN)
            ms3 = step_ms(wl3)
            three = {"flags": wl3.split_sites, "ms_per_step": round(ms3, 3),
                     "tokens_per_s": round(probe_tokens / (ms3 / 1e3), 1)}
            if not args.no_side_check:
                acc3 = accuracy_vs_golden(args.workload, wl3, model, db)
                if acc3:
                    three["accuracy_vs_oracle"] = acc3
            extra["split_attn_qkv_fc1"] = three
        line["other_states"] = extra
    if not args.no_side_check:
        acc = accuracy_vs_golden(args.workload, wl, model, db)
        if acc:
            line["accuracy_vs_oracle"] = acc
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, batch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
