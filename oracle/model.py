"""Decoder forward in fp64 numpy (test infrastructure only).

Plain definitions, one sequence at a time, no fusion:
  OPT-style (pre-LN): h = E[tok] + P[pos];  per layer
      h += Wo Attn(LN1 h) + bo;  h += W2 GELU(W1 LN2 h + b1) + b2
  Qwen3-style: h = E[tok];  per layer
      a = RMS(h);  q,k = RMS_head(Wq a), RMS_head(Wk a), RoPE;  h += Wo Attn(q,k,Wv a)
      h += Wdown (silu(Wgate RMS h) * Wup RMS h)
  final norm, logits over the whole vocabulary, log-softmax, label gather.

Every target linear also carries the factorized side term of its candidate
state (see oracle.zo): y += sum_j (x V_j) B_j^T.  With dense=True the same
candidate state is realised by mutating the weight, W + sum_j B_j V_j^T,
which is what conventional implementations do (arXiv abstract of
"Inference-Native Zeroth-Order Optimization": candidate states created by
mutating model weights vs. factorized side states).

fp8 models are the quantized model: the layer linears hold e4m3 weights (see
oracle.params) and every activation a layer linear reads - the two norm outputs,
the attention output and the GELU (OPT) or SwiGLU (Qwen3) output - is rounded to
e4m3 (oracle.params.e4m3_round, no scale) before the product; q, k, v (with
Qwen3's QK-norm and RoPE), the residual stream, the final norm and the head stay
as in bf16 models.

Error model for fp8 tolerances (not part of the definition): with
jitter = ({site: delta}, numpy Generator), every value about to be rounded to e4m3 at a
site ("norm": the two norm outputs, "attn": the attention output, "ffn": the GELU or
SwiGLU output) is first multiplied by (1 + delta u), u uniform on [-1, 1] per element.
e4m3 rounding is a step function, so an implementation whose values before a rounding
differ from the definition's by a relative delta lands one e4m3 step away wherever the
two straddle a rounding boundary, and every later layer sees the difference; running the
definition with and without the jitter measures how far the log-probs move when that
happens (the floor that an implementation of that precision meets).

The architecture facts (pre-LN, learned positions, tied head for OPT;
RMSNorm, QK-norm, rotate-half RoPE, GQA, SwiGLU, untied head for Qwen3) are
the public definitions of those families; the pages only name the families.
"""
import math

import numpy as np
from scipy.special import erf

from .params import e4m3_round


def layer_norm(x, w, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * w + b


def rms_norm(x, w, eps):
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def gelu(x):
    """Exact (erf) GELU."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, pos, theta):
    """Rotate-half rotary embedding: pairs (i, i + hd/2), inv_freq_i = theta^(-2i/hd).
    x [n, H, hd], pos [n] (position within the sequence, from 0)."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def causal_attention(q, k, v):
    """softmax(q k^T / sqrt(hd) + causal mask) v per head; GQA maps query head h
    to key/value head h // (Hq/Hkv).  q [n,Hq,hd], k,v [n,Hkv,hd]."""
    n, hq, hd = q.shape
    group = hq // k.shape[1]
    out = np.empty_like(q)
    mask = np.triu(np.ones((n, n), dtype=bool), k=1)
    for h in range(hq):
        kh, vh = k[:, h // group], v[:, h // group]
        s = q[:, h] @ kh.T / math.sqrt(hd)
        s[mask] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vh
    return out


def linear(x, W, b, side, dense):
    """y = x W^T (+ b) plus the side terms [(V, B)], each adding (x V) B^T."""
    if dense and side:
        Weff = W.copy()
        for V, B in side:
            Weff = Weff + B @ V.T
        y = x @ Weff.T
    else:
        y = x @ W.T
        for V, B in side:
            y = y + (x @ V) @ B.T
    if b is not None:
        y = y + b
    return y


def log_softmax_gather(logits, labels):
    """log p(label) = z_label - logsumexp(z), per row, over the whole row."""
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    return logits[np.arange(len(labels)), labels] - lse


def embed(cfg, G, tokens):
    h = G["tok_embed"][tokens]
    if cfg.arch == "opt":
        h = h + G["pos_embed"][np.arange(len(tokens))]
    return h.astype(np.float64)


def _e4m3_input(jitter):
    """The rounding of an fp8 model's linear inputs (qa(x, site)), optionally under the
    error model."""
    if jitter is None:
        return lambda x, site: e4m3_round(x)
    deltas, rs = jitter

    def qa(x, site):
        x = np.asarray(x, np.float64)
        return e4m3_round(x * (1.0 + deltas[site] * rs.uniform(-1.0, 1.0, size=x.shape)))
    return qa


def layer_forward(cfg, Wl, h, side, dense, jitter=None):
    """One decoder layer on one sequence.  side(kind) -> [(V, B)]."""
    n = h.shape[0]
    hq, hkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    qa = _e4m3_input(jitter) if cfg.dtype == "fp8" else (lambda x, site: x)   # linear inputs of fp8 models
    if cfg.arch == "opt":
        a = qa(layer_norm(h, Wl["ln1_w"], Wl["ln1_b"], cfg.norm_eps), "norm")
        q = linear(a, Wl["wq"], Wl["bq"], side("q"), dense).reshape(n, hq, hd)
        k = linear(a, Wl["wk"], Wl["bk"], side("k"), dense).reshape(n, hkv, hd)
        v = linear(a, Wl["wv"], Wl["bv"], side("v"), dense).reshape(n, hkv, hd)
        o = qa(causal_attention(q, k, v).reshape(n, hq * hd), "attn")
        h = h + linear(o, Wl["wo"], Wl["bo"], side("o"), dense)
        a = qa(layer_norm(h, Wl["ln2_w"], Wl["ln2_b"], cfg.norm_eps), "norm")
        f = qa(gelu(linear(a, Wl["w_fc1"], Wl["b_fc1"], side("fc1"), dense)), "ffn")
        h = h + linear(f, Wl["w_fc2"], Wl["b_fc2"], side("fc2"), dense)
        return h
    a = qa(rms_norm(h, Wl["ln1_w"], cfg.norm_eps), "norm")
    q = linear(a, Wl["wq"], None, side("q"), dense).reshape(n, hq, hd)
    k = linear(a, Wl["wk"], None, side("k"), dense).reshape(n, hkv, hd)
    v = linear(a, Wl["wv"], None, side("v"), dense).reshape(n, hkv, hd)
    q = rms_norm(q, Wl["q_norm_w"], cfg.norm_eps)
    k = rms_norm(k, Wl["k_norm_w"], cfg.norm_eps)
    pos = np.arange(n)
    q, k = rope(q, pos, cfg.rope_theta), rope(k, pos, cfg.rope_theta)
    o = qa(causal_attention(q, k, v).reshape(n, hq * hd), "attn")
    h = h + linear(o, Wl["wo"], None, side("o"), dense)
    a = qa(rms_norm(h, Wl["ln2_w"], cfg.norm_eps), "norm")
    g = linear(a, Wl["w_gate"], None, side("gate"), dense)
    u = linear(a, Wl["w_up"], None, side("up"), dense)
    h = h + linear(qa(silu(g) * u, "ffn"), Wl["w_down"], None, side("down"), dense)
    return h


def final_logprobs(cfg, G, h, positions, labels, row_chunk=64):
    """Log-probs of labels at the given row positions of one sequence."""
    if len(positions) == 0:
        return np.zeros(0)
    x = h[positions]
    if cfg.arch == "opt":
        x = layer_norm(x, G["final_norm_w"], G["final_norm_b"], cfg.norm_eps)
        head = G["tok_embed"]
    else:
        x = rms_norm(x, G["final_norm_w"], cfg.norm_eps)
        head = G["lm_head"]
    out = np.empty(len(positions))
    for i in range(0, len(positions), row_chunk):
        logits = x[i:i + row_chunk] @ head.T
        out[i:i + row_chunk] = log_softmax_gather(logits, labels[i:i + row_chunk])
    return out


def final_logsoftmax(cfg, G, h, position):
    """Log-softmax over the whole vocabulary at one row of one sequence (final norm, head)."""
    x = h[position:position + 1]
    if cfg.arch == "opt":
        x = layer_norm(x, G["final_norm_w"], G["final_norm_b"], cfg.norm_eps)
        head = G["tok_embed"]
    else:
        x = rms_norm(x, G["final_norm_w"], cfg.norm_eps)
        head = G["lm_head"]
    z = (x @ head.T)[0]
    m = z.max()
    return z - (m + np.log(np.sum(np.exp(z - m))))


def forward_last_logsoftmax(cfg, get_global, get_layer, seqs):
    """Full-vocabulary log-softmax at the last position of each sequence (dicts with
    tokens and side, as for forward_logprobs)."""
    G = get_global()
    hs = [embed(cfg, G, s["tokens"]) for s in seqs]
    for l in range(cfg.n_layers):
        Wl = get_layer(l)
        for i, s in enumerate(seqs):
            hs[i] = layer_forward(cfg, Wl, hs[i], lambda kind, s=s, l=l: s["side"](l, kind), False)
        del Wl
    return [final_logsoftmax(cfg, G, hs[i], len(s["tokens"]) - 1) for i, s in enumerate(seqs)]


def forward_logprobs(cfg, get_global, get_layer, seqs, dense=False, jitter=None):
    """Run a list of sequences through the model, layer by layer (so that only
    one layer's weights are resident).  Each seq is a dict with
      tokens    int array
      side      callable(layer, kind) -> [(V, B)]
      positions rows whose next token is scored
      labels    the scored token ids
    Returns one fp64 array of log-probs per sequence."""
    G = get_global()
    hs = [embed(cfg, G, s["tokens"]) for s in seqs]
    for l in range(cfg.n_layers):
        Wl = get_layer(l)
        for i, s in enumerate(seqs):
            hs[i] = layer_forward(cfg, Wl, hs[i], lambda kind, s=s, l=l: s["side"](l, kind), dense, jitter)
        del Wl
    return [final_logprobs(cfg, G, hs[i], np.asarray(s["positions"], np.int64),
                           np.asarray(s["labels"], np.int64)) for i, s in enumerate(seqs)]
