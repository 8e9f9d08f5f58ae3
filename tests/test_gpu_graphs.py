"""zo_model_set_graphs: zo_score's forward pass captured as a HIP graph and replayed.

Every replay must give bitwise the eager result of the same call.  The replays run with
the program's own eager work between them (scoring without graphs on another model,
updates of the bank, host synchronisations), the plan's step (so the regenerated side
factors) and the bank contents change between replays under one graph, and a batch of
another shape falls back to eager launches and gets its own graph."""
import numpy as np
import pytest

from synth import configs, inputs

from .gpu_common import SMALL_OPT_BF16, SMALL_QWEN_BF16, GpuRun, flush, need_gpu, workload

pytestmark = pytest.mark.gpu


def _bits(out):
    return (out["S"].copy(), out["seq_logp"].cpu().numpy().view(np.uint64).copy(),
            out["tok_logp"].cpu().numpy().view(np.uint32).copy())


def _same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


@pytest.mark.parametrize("name", ["tiny", "opt-bf16", "qwen3-bf16"])
def test_graph_replays_match_eager(name):
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    if name == "tiny":
        wl = configs.CONFIGS["tiny"].with_(n_fg=1)
    else:
        wl = workload(SMALL_OPT_BF16 if name == "opt-bf16" else SMALL_QWEN_BF16, dir_seeds=(3, 8), n_fg=2,
                      n_prompts=3)
    batch = inputs.make_batch(wl)
    g, ref = GpuRun(wl), GpuRun(wl)          # same weights; ref always launches eagerly
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        db = zo.DeviceBatch(batch)
        g.model.set_graphs(True)
        c = np.array([0.7, -1.1][:wl.n_dirs])
        for t in range(7):
            flush("%s graph step %d" % (name, t))
            # the program's own eager work between replays
            eager = zo.score(ref.model, ref.plan(t), ref.bank, zo.DeviceBatch(batch), want_tokens=True)
            torch.cuda.synchronize()
            got = zo.score(g.model, g.plan(t), g.bank, db, want_tokens=True)
            assert _same(_bits(got), _bits(eager)), (name, t)
            # the bank changes under the graph (its factors are rewritten before each replay)
            if t % 2 == 1:
                g.update(t, c, 1e-2)
                ref.update(t, c, 1e-2)
            x = torch.randn(1 << 16, device="cuda").sum()   # unrelated eager work on the same stream
            torch.cuda.synchronize()
        # another batch shape: eager once, then captured; the first graph is replaced
        sub = batch.subset([0, batch.n_seq - 1])
        dbs = zo.DeviceBatch(sub)
        for t in range(7, 10):
            got = zo.score(g.model, g.plan(t), g.bank, dbs, want_tokens=True)
            eager = zo.score(ref.model, ref.plan(t), ref.bank, zo.DeviceBatch(sub), want_tokens=True)
            assert _same(_bits(got), _bits(eager)), (name, "subset", t)
        g.model.set_graphs(False)
        got = zo.score(g.model, g.plan(10), g.bank, db, want_tokens=True)
        eager = zo.score(ref.model, ref.plan(10), ref.bank, zo.DeviceBatch(batch), want_tokens=True)
        assert _same(_bits(got), _bits(eager))
    torch.cuda.synchronize()
    del x


@pytest.mark.parametrize("cfg", [SMALL_OPT_BF16, SMALL_QWEN_BF16], ids=["opt", "qwen3"])
def test_generation_decode_steps_replayed_from_graph(cfg):
    """zo_generate with graph replay: the decode steps after the first two run from one
    captured graph; tokens and log-probs are bitwise those of eager launches, on two calls
    in a row (the second replays from the start) with eager work between them."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    wl = workload(cfg, dir_seeds=(3,), n_fg=1, n_prompts=2, len_lo=5, len_hi=70)
    batch = inputs.make_batch(wl)
    g, ref = GpuRun(wl), GpuRun(wl)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for r in (g, ref):
            r.update(0, np.array([0.8]), 1e-2)
        db = zo.DeviceBatch(batch)
        g.model.set_graphs(True)
        for call in range(2):
            flush("generation with graphs, call %d" % call)
            got = zo.generate(g.model, g.plan(1), g.bank, db, 9)
            eager = zo.generate(ref.model, ref.plan(1), ref.bank, zo.DeviceBatch(batch), 9)
            assert np.array_equal(got["tokens"].cpu().numpy(), eager["tokens"].cpu().numpy())
            assert np.array_equal(got["logp"].cpu().numpy().view(np.uint32), eager["logp"].cpu().numpy().view(np.uint32))
            assert np.array_equal(got["S"], eager["S"])
            x = torch.randn(1 << 12, device="cuda").sum()
            torch.cuda.synchronize()
    torch.cuda.synchronize()
