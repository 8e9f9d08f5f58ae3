"""Seeded token batches.

Probe prompts stand in for the pages' SST-2 workload (binary sentiment with
short option-token completions; "Zeroth-Order Fine-Tuning Was an Inference
Workload All Along", section "Limitations and Open Questions"): the last token
of every probe prompt is a label drawn from two fixed verbalizer ids.  No
dataset item is reproduced; ids are uniform or Zipf(s=1) over the vocabulary.
"""
from dataclasses import dataclass
from typing import List

import numpy as np

ROLE_PROBE = 0
ROLE_FOREGROUND = 1
MODE_LAST_LABEL = 0
MODE_ALL_NEXT = 1


@dataclass
class Batch:
    tokens: List[np.ndarray]   # one int32 array per logical sequence
    role: np.ndarray           # int32 [n_seq]
    score_mode: np.ndarray     # int32 [n_seq]

    @property
    def n_seq(self):
        return len(self.tokens)

    @property
    def lengths(self):
        return np.array([len(t) for t in self.tokens], dtype=np.int32)

    @property
    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)

    @property
    def flat_tokens(self):
        if not self.tokens:
            return np.zeros(0, np.int32)
        return np.concatenate(self.tokens).astype(np.int32)

    def subset(self, idx):
        idx = list(idx)
        return Batch([self.tokens[i] for i in idx], self.role[idx].copy(), self.score_mode[idx].copy())


def _zipf_ids(rng, vocab, n):
    ranks = np.arange(vocab, dtype=np.float64)
    w = 1.0 / (ranks + 1.0)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1).astype(np.int32)


def _ids(rng, dist, vocab, n):
    if dist == "uniform":
        return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
    if dist == "zipf":
        return _zipf_ids(rng, vocab, n)
    raise ValueError(dist)


def make_batch(wl, seed=None) -> Batch:
    """Foreground sequences first (if any), then the probe prompts."""
    rng = np.random.default_rng(wl.data_seed if seed is None else seed)
    vocab = wl.model.vocab
    toks, role, mode = [], [], []
    for _ in range(wl.n_fg):
        n = int(rng.integers(wl.len_lo, wl.len_hi + 1))
        toks.append(_ids(rng, wl.token_dist, vocab, n))
        role.append(ROLE_FOREGROUND)
        mode.append(MODE_ALL_NEXT if wl.fg_score_mode == "all_next" else MODE_LAST_LABEL)
    for _ in range(wl.n_prompts):
        n = int(rng.integers(wl.len_lo, wl.len_hi + 1))
        t = _ids(rng, wl.token_dist, vocab, n)
        if wl.score_mode == "last_label":
            t[-1] = wl.verbalizers[int(rng.integers(0, 2))]
        toks.append(t)
        role.append(ROLE_PROBE)
        mode.append(MODE_LAST_LABEL if wl.score_mode == "last_label" else MODE_ALL_NEXT)
    return Batch(toks, np.array(role, np.int32), np.array(mode, np.int32))
