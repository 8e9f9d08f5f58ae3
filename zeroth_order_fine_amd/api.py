"""Thin Python front of libzo: argument marshalling only.

PyTorch supplies device memory (weights blob, workspace, bank, outputs) and the
HIP stream; every step of the path runs inside libzo's kernels.
"""
import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import BatchDesc, ModelDesc, PlanDesc

ARCH = {"opt": 0, "qwen3": 1}
DTYPE = {"f32": 0, "bf16": 1, "fp8": 2}
KINDS = {"opt": ("q", "k", "v", "o", "fc1", "fc2"), "qwen3": ("q", "k", "v", "o", "gate", "up", "down")}
PLAN_SCALE_INV_SQRT_R, PLAN_ALLOW_ZERO_EPS, PLAN_ACT_SPLIT = 1, 2, 4
# two-term activations at single rounding sites (PLAN_ACT_SPLIT = all five)
PLAN_SPLIT_QKV_IN, PLAN_SPLIT_ATTN, PLAN_SPLIT_FC1_IN, PLAN_SPLIT_FC2_IN, PLAN_SPLIT_HEAD = 8, 16, 32, 64, 128
EST_INV_RANK, EST_MEAN = 1, 2
NOALLOC_SCRATCH_BYTES = 256 << 20    # ZO_NOALLOC_SCRATCH_BYTES
ROLE_PROBE, ROLE_FOREGROUND = 0, 1
SCORE_LAST_LABEL, SCORE_ALL_NEXT = 0, 1


class ZoError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libzo error %d: %s" % (code, msg))
        self.code = code


def _check(rc):
    if rc != 0:
        raise ZoError(rc, _lib.load().zo_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _arr(ctype, values):
    values = list(values)
    return (ctype * max(len(values), 1))(*values)


def model_desc(cfg):
    return ModelDesc(1, ARCH[cfg.arch], DTYPE[cfg.dtype], cfg.n_layers, cfg.d_model, cfg.n_heads,
                     cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn, cfg.vocab, cfg.max_pos, cfg.norm_eps,
                     cfg.rope_theta)


def kind_mask(cfg, kinds):
    names = KINDS[cfg.arch]
    m = 0
    for k in kinds:
        m |= 1 << names.index(k)
    return m


class Model:
    """A model over a caller-side (torch) weights blob."""

    def __init__(self, cfg, weights=None, device="cuda"):
        self.L = _lib.load()
        self.cfg = cfg
        self.desc = model_desc(cfg)
        n = ctypes.c_size_t()
        _check(self.L.zo_weights_size(ctypes.byref(self.desc), ctypes.byref(n)))
        self.weight_bytes = n.value
        if weights is None:
            weights = torch.empty(self.weight_bytes, dtype=torch.uint8, device=device)
        self.weights = weights
        h = ctypes.c_void_p()
        _check(self.L.zo_model_create(ctypes.byref(self.desc), _ptr(weights), weights.numel(), ctypes.byref(h)))
        self.h = h
        self._ws = None

    def close(self):
        if self.h:
            self.L.zo_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_graphs(self, enable=True):
        """Replay zo_score's forward pass from a captured HIP graph while shapes and buffers
        repeat (zo_model_set_graphs)."""
        _check(self.L.zo_model_set_graphs(self.h, 1 if enable else 0))

    def init_weights(self, seed):
        _check(self.L.zo_init_weights(self.h, seed, _stream()))

    def locate(self, slot, param):
        off, rows, cols = ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64()
        dt, lay = ctypes.c_int32(), ctypes.c_int32()
        _check(self.L.zo_weight_locate(ctypes.byref(self.desc), slot, param, ctypes.byref(off), ctypes.byref(rows),
                                       ctypes.byref(cols), ctypes.byref(dt), ctypes.byref(lay)))
        return off.value, rows.value, cols.value, dt.value, lay.value

    def tensor(self, slot, param):
        """Logical tensor as a torch tensor (a view for plain layouts, a gathered copy for
        the interleaved gate/up pack).  fp8 layer linears come back as stored: e4m3 codes
        (torch.float8_e4m3fn) of w * 2^11."""
        off, rows, cols, dt, lay = self.locate(slot, param)
        tdt, es = {0: (torch.float32, 4), 1: (torch.bfloat16, 2), 2: (torch.float8_e4m3fn, 1)}[dt]
        if lay == 0:
            return self.weights[off:off + rows * cols * es].view(tdt).view(rows, cols)
        packed = self.weights[off:off + 2 * rows * cols * es].view(tdt).view(2 * rows, cols)
        idx = torch.arange(rows, device=packed.device)
        prow = (idx // 16) * 32 + (16 if lay == 2 else 0) + idx % 16
        return packed[prow]

    def workspace(self, nbytes):
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.weights.device)
        return self._ws


class Plan:
    def __init__(self, model, t, nu, rank, eps, dir_seeds, candidates, targets, flags=0):
        self.L = model.L
        self.model = model
        self.t, self.nu, self.rank, self.eps = t, nu, rank, eps
        self.dir_seeds = tuple(dir_seeds)
        self.candidates = tuple(candidates)
        self.targets = tuple(targets)
        self.mask = kind_mask(model.cfg, targets)
        seeds = _arr(ctypes.c_uint64, self.dir_seeds)
        cd = _arr(ctypes.c_int32, [c[0] for c in candidates])
        cs = _arr(ctypes.c_int32, [c[1] for c in candidates])
        self.desc = PlanDesc(t, nu, rank, eps, len(self.dir_seeds), seeds, len(candidates), cd, cs, self.mask, flags)
        self._keep = (seeds, cd, cs)
        h = ctypes.c_void_p()
        _check(self.L.zo_plan(model.h, ctypes.byref(self.desc), ctypes.byref(h)))
        self.h = h

    @classmethod
    def from_workload(cls, model, wl, t=0, eps=None, flags=None, candidates=None):
        if flags is None:
            flags = ((PLAN_SCALE_INV_SQRT_R if wl.scale_inv_sqrt_r else 0) | (PLAN_ACT_SPLIT if wl.act_split else 0)
                     | wl.split_sites)
        return cls(model, t, wl.nu, wl.rank, wl.eps if eps is None else eps, wl.dir_seeds,
                   wl.candidates if candidates is None else candidates, wl.targets, flags)

    def close(self):
        if self.h:
            self.L.zo_plan_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Bank:
    def __init__(self, model, n_slots, rank, targets):
        self.L = model.L
        self.model = model
        self.n_slots, self.rank = n_slots, rank
        self.mask = kind_mask(model.cfg, targets)
        n = ctypes.c_size_t()
        _check(self.L.zo_bank_size(model.h, n_slots, rank, self.mask, ctypes.byref(n)))
        self.mem = torch.zeros(max(n.value // 4, 1), dtype=torch.float32, device=model.weights.device)
        h = ctypes.c_void_p()
        _check(self.L.zo_bank_create(model.h, n_slots, rank, self.mask, _ptr(self.mem), n.value, ctypes.byref(h)))
        self.h = h

    def keys(self):
        s = (ctypes.c_uint64 * self.n_slots)()
        w = (ctypes.c_int64 * self.n_slots)()
        _check(self.L.zo_bank_keys(self.h, s, w))
        return list(s), list(w)

    def set_keys(self, seeds, windows):
        _check(self.L.zo_bank_set_keys(self.h, _arr(ctypes.c_uint64, seeds), _arr(ctypes.c_int64, windows)))

    def entry(self, slot, layer, kind_name):
        kind = KINDS[self.model.cfg.arch].index(kind_name)
        off = ctypes.c_size_t()
        _check(self.L.zo_bank_entry_offset(self.h, slot, layer, kind, ctypes.byref(off)))
        n_out = self.model.cfg.linear_shape(kind_name)[0]
        i0 = off.value // 4
        return self.mem[i0:i0 + n_out * self.rank].view(n_out, self.rank)

    def close(self):
        if self.h:
            self.L.zo_bank_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceBatch:
    """A synth.Batch with its tokens on the device."""

    def __init__(self, batch, device="cuda"):
        self.batch = batch
        self.cu = np.ascontiguousarray(batch.cu_seqlens, np.int32)
        self.role = np.ascontiguousarray(batch.role, np.int32)
        self.mode = np.ascontiguousarray(batch.score_mode, np.int32)
        flat = batch.flat_tokens
        self.tokens = torch.from_numpy(flat if flat.size else np.zeros(1, np.int32)).to(device)
        i32p = ctypes.POINTER(ctypes.c_int32)
        self.desc = BatchDesc(batch.n_seq, self.cu.ctypes.data_as(i32p), ctypes.c_void_p(self.tokens.data_ptr()),
                              self.role.ctypes.data_as(i32p), self.mode.ctypes.data_as(i32p))


def batch_layout(model, plan, bank, db):
    n_phys, n_rows, n_sc, ws = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check(model.L.zo_batch_layout(model.h, plan.h, bank.h if bank else None, ctypes.byref(db.desc),
                                   ctypes.byref(n_phys), ctypes.byref(n_rows), ctypes.byref(n_sc), ctypes.byref(ws)))
    return n_phys.value, n_rows.value, n_sc.value, ws.value


def pack(model, plan, db):
    n_phys = batch_layout(model, plan, None, db)[0]
    ps = (ctypes.c_int32 * max(n_phys, 1))()
    pc = (ctypes.c_int32 * max(n_phys, 1))()
    pf = (ctypes.c_int32 * (n_phys + 1))()
    _check(model.L.zo_pack(plan.h, ctypes.byref(db.desc), ps, pc, pf))
    return list(ps)[:n_phys], list(pc)[:n_phys], list(pf)


def score(model, plan, bank, db, want_tokens=False):
    """Returns dict(S [n_cand] numpy fp64, seq_logp torch fp64 [n_phys], tok_logp torch fp32 or None)."""
    n_phys, n_rows, n_sc, ws_bytes = batch_layout(model, plan, bank, db)
    ws = model.workspace(ws_bytes)
    dev = model.weights.device
    seq = torch.empty(max(n_phys, 1), dtype=torch.float64, device=dev)
    tok = torch.empty(max(n_sc, 1), dtype=torch.float32, device=dev) if want_tokens else None
    S = (ctypes.c_double * len(plan.candidates))()
    _check(model.L.zo_score(model.h, plan.h, bank.h if bank else None, ctypes.byref(db.desc), _ptr(ws), ws.numel(),
                            _ptr(seq), _ptr(tok), S, _stream()))
    return dict(S=np.array(list(S)), seq_logp=seq[:n_phys], tok_logp=tok[:n_sc] if tok is not None else None,
                n_phys=n_phys, n_rows=n_rows, n_scored=n_sc)


def score_noalloc(model, plan, bank, db, seq_out, tok_out=None):
    """zo_score_noalloc: the workspace is the library's own device scratch; the outputs
    (seq_out fp64 [n_phys], tok_out fp32 [n_scored] or None) are the caller's tensors.
    Returns the per-candidate sums S (numpy fp64)."""
    S = (ctypes.c_double * len(plan.candidates))()
    _check(model.L.zo_score_noalloc(model.h, plan.h, bank.h if bank else None, ctypes.byref(db.desc),
                                    _ptr(seq_out), _ptr(tok_out), S, _stream()))
    return np.array(list(S))


def generate(model, plan, bank, db, n_new):
    """Greedy generation of n_new tokens for every physical sequence (zo_pack order).
    Returns dict(tokens torch int32 [n_phys, n_new], logp torch fp32 [n_phys, n_new],
    S numpy fp64 [n_cand] = per-candidate sums of the generated tokens' log-probs)."""
    n_phys, ws_bytes = ctypes.c_int32(), ctypes.c_size_t()
    _check(model.L.zo_generate_layout(model.h, plan.h, bank.h if bank else None, ctypes.byref(db.desc), n_new,
                                      ctypes.byref(n_phys), ctypes.byref(ws_bytes)))
    ws = model.workspace(ws_bytes.value)
    dev = model.weights.device
    n = n_phys.value
    tok = torch.empty((max(n, 1), n_new), dtype=torch.int32, device=dev)
    lp = torch.empty((max(n, 1), n_new), dtype=torch.float32, device=dev)
    S = (ctypes.c_double * len(plan.candidates))()
    _check(model.L.zo_generate(model.h, plan.h, bank.h if bank else None, ctypes.byref(db.desc), n_new, _ptr(ws),
                               ws.numel(), _ptr(tok), _ptr(lp), S, _stream()))
    return dict(tokens=tok[:n], logp=lp[:n], S=np.array(list(S)), n_phys=n)


def estimate(plan, S, flags=0, n_scored=None):
    L = plan.L
    q = len(plan.dir_seeds)
    out = (ctypes.c_double * q)()
    ns = _arr(ctypes.c_int64, n_scored) if n_scored is not None else None
    _check(L.zo_estimate(plan.h, _arr(ctypes.c_double, S), ns, flags, out))
    return np.array(list(out))


def update(model, plan, bank, c, lr):
    _check(model.L.zo_update(model.h, plan.h, bank.h, _arr(ctypes.c_double, c), lr, _stream()))


def fold(model, bank, slot):
    """Fold bank entry `slot` into the model's weights (W <- round(W + U V^T) for every
    target linear) and free the slot."""
    n = ctypes.c_size_t()
    _check(model.L.zo_bank_fold_size(model.h, bank.h, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    _check(model.L.zo_bank_fold(model.h, bank.h, slot, _ptr(ws), n.value, _stream()))


def bank_cap(model, bank, plan, max_frozen):
    """Fold the oldest frozen entries (windows other than the plan's) into the weights until
    at most max_frozen remain; returns the number folded."""
    n = ctypes.c_size_t()
    _check(model.L.zo_bank_fold_size(model.h, bank.h, ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    k = ctypes.c_int32()
    _check(model.L.zo_bank_cap(model.h, bank.h, plan.h, max_frozen, _ptr(ws), n.value, _stream(), ctypes.byref(k)))
    return k.value


def philox_words(seed, tag, tau, first_block, n_blocks):
    L = _lib.load()
    out = torch.empty(max(4 * n_blocks, 1), dtype=torch.int32, device="cuda")
    _check(L.zo_philox_words(seed, tag, tau, first_block, n_blocks, _ptr(out), _stream()))
    return out[:4 * n_blocks].view(n_blocks, 4)


def normal_fill(seed, tag, tau, n, first=0):
    L = _lib.load()
    out = torch.empty(max(n, 1), dtype=torch.float64, device="cuda")
    _check(L.zo_normal_fill(seed, tag, tau, first, n, _ptr(out), _stream()))
    return out[:n]


def direction(model, plan, dir_index, layer, kind_name, which):
    kind = KINDS[model.cfg.arch].index(kind_name)
    n_out, n_in = model.cfg.linear_shape(kind_name)
    n = n_out if which == 0 else n_in
    out = torch.empty(n * plan.rank, dtype=torch.float32, device=model.weights.device)
    _check(model.L.zo_direction(model.h, plan.h, dir_index, layer, kind, which, _ptr(out), _stream()))
    return out.view(n, plan.rank)


PROFILE_CLASSES = ("gemm_base", "gemm_side", "gemm_head", "attention", "norm", "side_prep", "reduce", "update",
                   "decode_attention")


def profile_begin(classes=None):
    """Start timing every launch of the named classes (default: all)."""
    L = _lib.load()
    mask = 0xFFFFFFFF if classes is None else sum(1 << PROFILE_CLASSES.index(c) for c in classes)
    _check(L.zo_profile_select(mask))
    _check(L.zo_profile_begin())


def profile_end():
    """{class: (launches, total ms)} for the launches since profile_begin."""
    n = len(PROFILE_CLASSES)
    counts = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    _check(_lib.load().zo_profile_end(n, counts, ms))
    return {k: (counts[i], ms[i]) for i, k in enumerate(PROFILE_CLASSES)}
