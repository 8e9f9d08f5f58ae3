"""ProbePlan, packing, score, estimate, update and bank (test infrastructure only).

Pages: "Zeroth-Order Fine-Tuning Was an Inference Workload All Along",
section "Why ZO Fine-Tuning Is Really Scoring" (two-point estimator L+, L-,
c = (L+ - L-)/2eps, update theta <- theta - eta c z; LoZO's low-rank z),
section "The System Reorganization" (the 1/r note; lazy sampling: V held
for a nu-step window; U_{t+1} = U_t - eta c_t G_t, Delta W = U_{t+1} V^T),
and the arXiv abstract of "Inference-Native Zeroth-Order Optimization"
(query process, ProbePlan, candidate evaluation, factorized side states,
persistent banked state).

Readings where the pages are silent:
  * z = G V^T per target linear; G [n_out, r], V [n_in, r], entries N(0,1),
    and eps_tilde = eps (or eps/sqrt(r) with scale_inv_sqrt_r, the
    MeZO-factorized variant whose entries have unit variance).
  * score returns S = summed label log-probs; the loss is L = -S.
  * candidate (d, s) sees W + sum_j U_j V_j^T + s*eps_tilde*G_d V_d^T, where j
    runs over the bank's entries; a foreground sequence sees W only.
  * the update accumulates into the bank entry keyed (seed_d, floor(t/nu)),
    U <- U - (eta/q) c_d sigma G_d, with q the number of directions and sigma =
    eps_tilde/eps, so that the step follows the probed direction z_d = sigma G_d V_d^T.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import params
from .model import forward_logprobs

ROLE_PROBE, ROLE_FOREGROUND = 0, 1
MODE_LAST_LABEL, MODE_ALL_NEXT = 0, 1
EST_INV_RANK = 1
EST_MEAN = 2


@dataclass
class Plan:
    t: int
    nu: int
    rank: int
    eps: float
    dir_seeds: Tuple[int, ...]
    candidates: Tuple[Tuple[int, int], ...]     # (direction, sign)
    targets: Tuple[str, ...]
    scale_inv_sqrt_r: bool = False
    allow_zero_eps: bool = False

    @property
    def window(self):
        return self.t // self.nu

    @property
    def eps_tilde(self):
        if self.scale_inv_sqrt_r:
            return self.eps / np.sqrt(float(self.rank))
        return self.eps

    def validate(self):
        if self.rank < 1 or self.nu < 1 or self.t < 0:
            raise ValueError("rank, nu must be >= 1 and t >= 0")
        if not (np.isfinite(self.eps) and (self.eps > 0 or (self.allow_zero_eps and self.eps == 0))):
            raise ValueError("eps must be finite and > 0")
        for d, s in self.candidates:
            if not (0 <= d < len(self.dir_seeds)) or s not in (1, -1):
                raise ValueError("bad candidate")


def plan_from_workload(wl, t=0):
    return Plan(t, wl.nu, wl.rank, wl.eps, tuple(wl.dir_seeds), wl.candidates, tuple(wl.targets),
                wl.scale_inv_sqrt_r)


@dataclass
class BankEntry:
    seed: int
    window: int
    U: Dict[Tuple[int, str], np.ndarray]      # (layer, kind) -> fp32-valued [n_out, r]


@dataclass
class Bank:
    n_slots: int
    rank: int
    targets: Tuple[str, ...]
    entries: List[Optional[BankEntry]] = field(default_factory=list)

    def __post_init__(self):
        if not self.entries:
            self.entries = [None] * self.n_slots

    def active(self):
        return [e for e in self.entries if e is not None]

    def find_or_alloc(self, cfg, seed, window):
        for e in self.entries:
            if e is not None and e.seed == seed and e.window == window:
                return e
        for i, e in enumerate(self.entries):
            if e is None:
                U = {(l, k): np.zeros((cfg.linear_shape(k)[0], self.rank))
                     for l in range(cfg.n_layers) for k in self.targets}
                self.entries[i] = BankEntry(seed, window, U)
                return self.entries[i]
        raise RuntimeError("bank full")


def pack(batch, plan):
    """Canonical physical order: foreground sequences in input order, then for
    each candidate in plan order the probe sequences in input order.
    Returns [(logical index, candidate index or -1)]."""
    phys = [(i, -1) for i in range(batch.n_seq) if batch.role[i] == ROLE_FOREGROUND]
    probes = [i for i in range(batch.n_seq) if batch.role[i] == ROLE_PROBE]
    for c in range(len(plan.candidates)):
        phys += [(i, c) for i in probes]
    return phys


def scored_positions(tokens, mode):
    """LAST_LABEL: the row before the last predicts the last token.
    ALL_NEXT: rows 0..n-2 predict tokens 1..n-1."""
    n = len(tokens)
    if mode == MODE_LAST_LABEL:
        if n < 2:
            raise ValueError("a LAST_LABEL sequence needs at least 2 tokens")
        return np.array([n - 2]), np.array([tokens[n - 1]])
    return np.arange(n - 1), np.asarray(tokens[1:])


def _kind_id(cfg, kind):
    return cfg.kind_names.index(kind)


def side_terms(cfg, plan, bank, cand):
    """side(layer, kind) -> [(V, B)] for a physical sequence with candidate `cand`."""
    r, w = plan.rank, plan.window
    cache = {}          # factors of the layer being processed only (layers run in order)

    def side(layer, kind):
        if cand < 0 or kind not in plan.targets:
            return []
        key = (layer, kind)
        if key not in cache:
            for k in [k for k in cache if k[0] != layer]:
                del cache[k]
            kid = _kind_id(cfg, kind)
            n_out, n_in = cfg.linear_shape(kind)
            terms = []
            if bank is not None:
                for e in bank.active():
                    V = params.factor(e.seed, layer, kid, params.rng.FACTOR_V, e.window, n_in, r)
                    terms.append((V, e.U[(layer, kind)]))
            d, s = plan.candidates[cand]
            seed = plan.dir_seeds[d]
            Vd = params.factor(seed, layer, kid, params.rng.FACTOR_V, w, n_in, r)
            Gd = params.factor(seed, layer, kid, params.rng.FACTOR_G, plan.t, n_out, r)
            terms.append((Vd, (s * plan.eps_tilde) * Gd))
            cache[key] = terms
        return cache[key]
    return side


class Weights:
    """Lazily generated fp64 weights (one layer at a time for large models)."""

    def __init__(self, cfg, seed, cache_layers=False):
        self.cfg, self.seed, self.cache_layers = cfg, seed, cache_layers
        self._g = None
        self._layers = {}

    def get_global(self):
        if self._g is None:
            self._g = params.global_weights(self.cfg, self.seed)
        return self._g

    def get_layer(self, l):
        if l in self._layers:
            return self._layers[l]
        W = params.layer_weights(self.cfg, self.seed, l)
        if self.cache_layers:
            self._layers[l] = W
        return W


def score(cfg, weights, plan, bank, batch, dense=False, phys_subset=None, e4m3_jitter=None):
    """Score every physical sequence (or the given subset of physical indices).
    e4m3_jitter = ({site: delta}, seed): fp8 models only, the error model of oracle.model
    (values perturbed by a relative delta before their e4m3 rounding), for sizing tolerances.
    Returns dict(phys, seq_logp [n_phys] (nan where not computed),
                 tok_logp {phys index: fp64 array}, S [n_cand] (only when all computed))."""
    plan.validate()
    phys = pack(batch, plan)
    idx = list(range(len(phys))) if phys_subset is None else list(phys_subset)
    seqs = []
    for p in idx:
        li, c = phys[p]
        toks = batch.tokens[li]
        pos, lab = scored_positions(toks, int(batch.score_mode[li]))
        seqs.append(dict(tokens=np.asarray(toks, np.int64), side=side_terms(cfg, plan, bank, c),
                         positions=pos, labels=lab))
    jitter = None
    if e4m3_jitter is not None:
        jitter = ({k: float(v) for k, v in e4m3_jitter[0].items()}, np.random.default_rng(int(e4m3_jitter[1])))
    lps = forward_logprobs(cfg, weights.get_global, weights.get_layer, seqs, dense=dense,
                           jitter=jitter) if seqs else []
    seq_logp = np.full(len(phys), np.nan)
    tok = {}
    for p, lp in zip(idx, lps):
        s = 0.0
        for v in lp:
            s += v
        seq_logp[p] = s
        tok[p] = lp
    out = dict(phys=phys, seq_logp=seq_logp, tok_logp=tok)
    if phys_subset is None:
        S = np.zeros(len(plan.candidates))
        for p, (li, c) in enumerate(phys):
            if c >= 0:
                S[c] += seq_logp[p]
        out["S"] = S
        out["n_scored"] = np.array([sum(len(tok[p]) for p, (li, cc) in enumerate(phys) if cc == c)
                                    for c in range(len(plan.candidates))])
    return out


def generate(cfg, weights, plan, bank, batch, n_new, forced=None):
    """Greedy generation of n_new tokens for every physical sequence (the packing of
    score): at each step the whole sequence so far (prompt + tokens chosen so far) is run
    through the model at its candidate state again - no cache, the plain definition - and
    the next token is the first vocabulary id holding the largest log-probability at the
    last position ("Inference-Native Zeroth-Order Optimization", arXiv abstract:
    candidate-state queries cover autoregressive generation).  forced (optional,
    [n_phys x n_new] ids): continue with these tokens instead of the argmax, so that the
    log-probabilities can be compared along another implementation's choices.
    Returns dict(phys, tokens (the continuation used), logp (its tokens' log-probs),
    best_tok and best_logp (the argmax and its log-prob at every step), S [n_cand])."""
    from .model import forward_last_logsoftmax
    plan.validate()
    phys = pack(batch, plan)
    n = len(phys)
    toks = [list(np.asarray(batch.tokens[li], np.int64)) for li, c in phys]
    out_tok = np.zeros((n, n_new), np.int64)
    logp = np.zeros((n, n_new))
    best_tok = np.zeros((n, n_new), np.int64)
    best_lp = np.zeros((n, n_new))
    sides = [side_terms(cfg, plan, bank, c) for li, c in phys]
    for j in range(n_new):
        seqs = [dict(tokens=np.asarray(toks[p], np.int64), side=sides[p]) for p in range(n)]
        lsm = forward_last_logsoftmax(cfg, weights.get_global, weights.get_layer, seqs)
        for p in range(n):
            b = int(np.argmax(lsm[p]))                 # first index of the maximum
            t = b if forced is None else int(forced[p][j])
            best_tok[p, j], best_lp[p, j] = b, lsm[p][b]
            out_tok[p, j], logp[p, j] = t, lsm[p][t]
            toks[p].append(t)
    S = np.zeros(len(plan.candidates))
    for p, (li, c) in enumerate(phys):
        if c >= 0:
            for v in logp[p]:
                S[c] += v
    return dict(phys=phys, tokens=out_tok, logp=logp, best_tok=best_tok, best_logp=best_lp, S=S)


def estimate(plan, S, flags=0, n_scored=None):
    """c_d = (L_{d,+} - L_{d,-}) / (2 eps) with L = -S (optionally / n_scored);
    divided by r when EST_INV_RANK is set (the estimator's explicit 1/r, which
    the released LoZO code omits)."""
    S = np.asarray(S, np.float64)
    if not np.all(np.isfinite(S)):
        raise FloatingPointError("non-finite score")
    q = len(plan.dir_seeds)
    c = np.zeros(q)
    two_eps = 2.0 * plan.eps
    for d in range(q):
        ip = [i for i, (dd, s) in enumerate(plan.candidates) if dd == d and s == 1]
        im = [i for i, (dd, s) in enumerate(plan.candidates) if dd == d and s == -1]
        if len(ip) != 1 or len(im) != 1:
            raise ValueError("direction %d needs exactly one + and one - candidate" % d)
        Lp, Lm = -S[ip[0]], -S[im[0]]
        if flags & EST_MEAN:
            Lp, Lm = Lp / float(n_scored[ip[0]]), Lm / float(n_scored[im[0]])
        cd = (Lp - Lm) / two_eps
        if flags & EST_INV_RANK:
            cd = cd / float(plan.rank)
        c[d] = cd
    return c


WEIGHT_NAME = {"q": "wq", "k": "wk", "v": "wv", "o": "wo", "fc1": "w_fc1", "fc2": "w_fc2",
               "gate": "w_gate", "up": "w_up", "down": "w_down"}


def fold(cfg, weights, bank, slot):
    """Commit bank entry `slot` into the weights (the low-rank state of a finished window,
    Delta W = U V^T of the lazy update) and free the slot:
        W <- round(W + sum_k U[:, k] V[:, k]^T),
    the sum in fp64 in k order (each product rounded, then added), rounded fp64 -> fp32,
    then fp32 -> bf16 for bf16 models, or for fp8 models fp32 -> the e4m3 value of w * 2^11
    (nearest even, saturating) times 2^-11, the quantized base requantized.  `weights` must
    cache its layers (the folded values replace the generated ones)."""
    if not weights.cache_layers:
        raise ValueError("fold needs Weights(cache_layers=True)")
    e = bank.entries[slot]
    if e is None:
        raise ValueError("slot %d is empty" % slot)
    r = bank.rank
    for l in range(cfg.n_layers):
        W = weights.get_layer(l)
        for kind in bank.targets:
            n_out, n_in = cfg.linear_shape(kind)
            V = params.factor(e.seed, l, _kind_id(cfg, kind), params.rng.FACTOR_V, e.window, n_in, r)
            U = e.U[(l, kind)]
            w = W[WEIGHT_NAME[kind]].copy()
            for k in range(r):
                w = w + np.outer(U[:, k], V[:, k])
            w32 = w.astype(np.float32)
            if cfg.dtype == "bf16":
                w32 = params.bf16_round(w32)
            if cfg.dtype == "fp8":       # requantized: the e4m3 value of w * 2^11, times 2^-11
                scale = 2.0 ** params.FP8_WEIGHT_EXP
                W[WEIGHT_NAME[kind]] = params.e4m3_round(w32.astype(np.float64) * scale) / scale
            else:
                W[WEIGHT_NAME[kind]] = w32.astype(np.float64)
    bank.entries[slot] = None
    return bank


def cap(cfg, weights, bank, plan, max_frozen):
    """Keep at most max_frozen frozen entries (entries of windows other than the plan's):
    fold the oldest ones into the weights, lowest window first, then lowest slot.  The pages
    commit a finished window's low-rank state as Delta W = U V^T ("Zeroth-Order Fine-Tuning
    Was an Inference Workload All Along", section "The System Reorganization"); they do not
    say when, so this bounds how many finished windows stay as side terms.  Returns the
    number folded."""
    frozen = sorted((e.window, i) for i, e in enumerate(bank.entries)
                    if e is not None and e.window != plan.window)
    n = max(0, len(frozen) - max_frozen)
    for _, slot in frozen[:n]:
        fold(cfg, weights, bank, slot)
    return n


def update(cfg, plan, bank, c, lr):
    """U_{seed_d, window} <- fp32(U - (((lr / q) * c_d) * sigma) * G_d), one entry per direction.

    The step is theta <- theta - (eta / q) sum_d c_d z_d along the directions the probes
    used ("Zeroth-Order Fine-Tuning Was an Inference Workload All Along", section "Why ZO
    Fine-Tuning Is Really Scoring": theta <- theta - eta c z, with c measured along z).  A
    candidate sits at theta + s eps z_d with z_d = sigma G_d V_d^T (sigma = eps_tilde / eps:
    1, or 1/sqrt(r) with scale_inv_sqrt_r), so the accumulated factor takes sigma too."""
    q = len(plan.dir_seeds)
    r = plan.rank
    sigma = 1.0 / np.sqrt(float(r)) if plan.scale_inv_sqrt_r else 1.0
    for d in range(q):
        seed = plan.dir_seeds[d]
        e = bank.find_or_alloc(cfg, seed, plan.window)
        coef = ((lr / float(q)) * float(c[d])) * sigma
        for l in range(cfg.n_layers):
            for kind in plan.targets:
                n_out, _ = cfg.linear_shape(kind)
                G = params.factor(seed, l, _kind_id(cfg, kind), params.rng.FACTOR_G, plan.t, n_out, r)
                e.U[(l, kind)] = (e.U[(l, kind)] - coef * G).astype(np.float32).astype(np.float64)
    return bank
