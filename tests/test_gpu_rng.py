"""GPU parity of the random streams: raw Philox words, Gaussian stream, the
plan's direction factors and the weight initialisation, bit-exact against the
oracle's independent CPU implementation."""
import numpy as np
import pytest

from oracle import params, rng
from synth import configs

from .gpu_common import SMALL_OPT_FP8, SMALL_QWEN_BF16, SMALL_QWEN_FP8, flush, need_gpu

pytestmark = pytest.mark.gpu


def test_philox_words_bit_exact():
    need_gpu()
    import zeroth_order_fine_amd as zo
    for seed, tag, tau, first, n in [(0, 0, 0, 0, 1000), (0x123456789ABCDEF, 77, (5 << 32) | 9, 10, 4096),
                                     (2**64 - 1, 2**32 - 1, 2**64 - 1, 2**32 - 5000, 5000)]:
        flush("philox %x %d" % (seed, first))
        got = zo.philox_words(seed, tag, tau, first, n).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, rng.words(seed, tag, tau, first, n))


def test_normal_stream_bit_exact():
    need_gpu()
    import zeroth_order_fine_amd as zo
    for seed, tag, tau, first, n in [(0, 5, 0, 0, 1 << 20), (9, rng.weight_tag(3, 12), 0, 123457, 300001),
                                     (3, rng.direction_tag(39, 5, 1), 7, 2**33, 40000)]:
        flush("normal seed %d tag %x first %d" % (seed, tag, first))
        got = zo.normal_fill(seed, tag, tau, n, first).cpu().numpy()
        ref = rng.normal(seed, tag, tau, n, first)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_direction_factors_bit_exact():
    need_gpu()
    import zeroth_order_fine_amd as zo
    wl = configs.CONFIGS["opt13b"]
    # only the plan is needed; the model's weights are never touched
    import torch
    cfg = wl.model
    w = torch.empty(1, dtype=torch.uint8, device="cuda")
    from zeroth_order_fine_amd import api
    model = object.__new__(api.Model)
    model.L = api._lib.load()
    model.cfg = cfg
    model.desc = api.model_desc(cfg)
    import ctypes
    h = ctypes.c_void_p()
    n = ctypes.c_size_t()
    model.L.zo_weights_size(ctypes.byref(model.desc), ctypes.byref(n))
    fake = torch.empty(1, dtype=torch.uint8, device="cuda")
    assert model.L.zo_model_create(ctypes.byref(model.desc), ctypes.c_void_p(fake.data_ptr()), n.value,
                                   ctypes.byref(h)) == 0
    model.h = h
    model.weights = fake
    for t in (0, 5, 1030):
        plan = zo.Plan(model, t, 1024, 2, 1e-3, (11, 22), ((0, 1), (0, -1), (1, 1), (1, -1)), wl.targets)
        for d, layer, kind in [(0, 0, "q"), (1, 39, "fc2"), (0, 17, "fc1")]:
            kid = cfg.kind_names.index(kind)
            n_out, n_in = cfg.linear_shape(kind)
            for which, rows, tau in ((0, n_out, t), (1, n_in, t // 1024)):
                got = zo.direction(model, plan, d, layer, kind, which).cpu().numpy()
                ref = params.factor((11, 22)[d], layer, kid, which, tau, rows, 2).astype(np.float32)
                assert np.array_equal(got, ref), (t, d, layer, kind, which)
    model.close()


@pytest.mark.parametrize("name", ["tiny", "qwen_small", "opt_fp8", "qwen_fp8"])
def test_weight_init_bit_exact(name):
    """fp8: every layer linear's e4m3 code equals the oracle's e4m3(w * 2^11) (decoded by
    PyTorch's float8_e4m3fn), the embeddings are bf16 as in bf16 models."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    cfg = {"tiny": configs.CONFIGS["tiny"].model, "qwen_small": SMALL_QWEN_BF16, "opt_fp8": SMALL_OPT_FP8,
           "qwen_fp8": SMALL_QWEN_FP8}[name]
    model = zo.Model(cfg)
    model.init_weights(7)
    torch.cuda.synchronize()
    n_fp8 = 0
    for slot, plist in [(0, params.global_params(cfg))] + [(l + 1, params.layer_params(cfg))
                                                           for l in range(cfg.n_layers)]:
        for pid, pname, shape, init in plist:
            got = model.tensor(slot, pid).float().cpu().numpy().reshape(shape)
            if model.locate(slot, pid)[3] == 2:
                got = got * np.float32(2.0 ** -params.FP8_WEIGHT_EXP)
                n_fp8 += 1
            ref = params.make_tensor(cfg, 7, slot, pid, shape, init).astype(np.float32)
            assert np.array_equal(got, ref), (slot, pname)
    # q, k, v, o, fc1, fc2 (OPT) or q, k, v, o, gate, up, down (Qwen3)
    assert n_fp8 == ((6 if cfg.arch == "opt" else 7) * cfg.n_layers if cfg.dtype == "fp8" else 0)
    model.close()


def test_weight_init_bit_exact_full_size_sampled():
    """OPT-13B-shaped blob (25.7 GB): sampled rows of every kind of tensor."""
    need_gpu()
    import torch
    import zeroth_order_fine_amd as zo
    cfg = configs.CONFIGS["opt13b"].model
    flush("init OPT-13B weights")
    model = zo.Model(cfg)
    model.init_weights(0)
    torch.cuda.synchronize()
    rs = np.random.default_rng(0)
    for slot, pid, shape, init in [(0, params.TOK_EMBED, (cfg.vocab, cfg.d_model), "matrix"),
                                   (0, params.POS_EMBED, (cfg.max_pos, cfg.d_model), "matrix"),
                                   (1, params.WQ, (5120, 5120), "matrix"), (40, params.W_FC2, (5120, 20480), "matrix"),
                                   (23, params.W_FC1, (20480, 5120), "matrix"), (40, params.LN2_W, (5120,), "gain"),
                                   (17, params.B_FC1, (20480,), "bias")]:
        t = model.tensor(slot, pid)
        if len(shape) == 1:
            assert np.array_equal(t.float().cpu().numpy().reshape(-1),
                                  params.make_tensor(cfg, 0, slot, pid, shape, init).astype(np.float32))
            continue
        for r0 in list(rs.integers(0, shape[0] - 2, size=3)) + [shape[0] - 2]:
            got = t[r0:r0 + 2].float().cpu().numpy()
            ref = params.make_tensor(cfg, 0, slot, pid, shape, init, rows=(int(r0), int(r0) + 2)).astype(np.float32)
            assert np.array_equal(got, ref), (slot, pid, r0)
    del model
    torch.cuda.empty_cache()
