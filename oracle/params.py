"""Weight-initialisation spec and direction factors (test infrastructure only).

Weights are synthetic (the pages use pretrained OPT and Qwen3 checkpoints,
which are not available; the workloads ask for random-init N(0, 0.02)).
Every logical tensor is a Gaussian stream (see oracle.rng) keyed by the model
seed and the tensor's tag, element index = row-major index:
  matrices and biases : 0.02 * z
  norm gains          : 1 + 0.02 * z
computed in fp64, rounded to fp32 (round to nearest even), and for bf16
models the matrices are then rounded fp32 -> bf16 (round to nearest even).
Vectors (biases, norm gains) stay fp32.  fp8 models keep the
embedding matrices in bf16 and store every layer linear as OCP e4m3 codes of
w * 2^11 (round to nearest even, saturating at 448): |0.02 z| < 0.14 for every
stream value (u >= 2^-33 bounds |z| below 6.8), so the fixed power-of-two
scale keeps the whole range below 448 and the stored value is exactly
e4m3(w * 2^11) * 2^-11.

Direction factors (pages: "Zeroth-Order Fine-Tuning Was an Inference Workload
All Along", section "Why ZO Fine-Tuning Is Really Scoring" - LoZO samples
low-rank factors; section "The System Reorganization" - V is held for a
nu-step window, the other factor is resampled every step):
  G[l, kind] : n_out x r, stream (dir_seed, direction_tag(l, kind, 0), t)
  V[l, kind] : n_in  x r, stream (dir_seed, direction_tag(l, kind, 1), floor(t/nu))
each entry a standard normal rounded to fp32.
"""
import numpy as np

from . import rng

# global parameter ids (slot 0)
TOK_EMBED, POS_EMBED, FINAL_NORM_W, FINAL_NORM_B, LM_HEAD = 0, 1, 2, 3, 4
# per-layer parameter ids (slot layer+1)
LN1_W, LN1_B, WQ, BQ, WK, BK, WV, BV, WO, BO = range(10)
LN2_W, LN2_B, W_FC1, B_FC1, W_FC2, B_FC2, W_DOWN, QNORM_W, KNORM_W = range(10, 19)
W_GATE, W_UP = W_FC1, W_FC2

SCALE = 0.02
FP8_WEIGHT_EXP = 11          # fp8 models: layer linears stored as e4m3(w * 2^11)
E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest OCP e4m3 value (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals down to 2^-9, largest finite 448), ties to even, saturating at +-448.
    The quantum of |x| in binade [2^E, 2^(E+1)) is 2^(max(E, -6) - 3); dividing by a
    power of two and rounding to an integer is exact in binary64."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = m 2^e, m in [0.5, 1)
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    y = np.minimum(np.round(a / q) * q, E4M3_MAX)   # np.round: half to even
    return np.where(x < 0, -y, y)


def bf16_round(x32):
    """fp32 -> bf16 by round to nearest even, returned as fp32 values."""
    b = np.ascontiguousarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def global_params(cfg):
    d, V = cfg.d_model, cfg.vocab
    out = [(TOK_EMBED, "tok_embed", (V, d), "matrix")]
    if cfg.arch == "opt":
        out += [(POS_EMBED, "pos_embed", (cfg.max_pos, d), "matrix"),
                (FINAL_NORM_W, "final_norm_w", (d,), "gain"),
                (FINAL_NORM_B, "final_norm_b", (d,), "bias")]
    else:
        out += [(FINAL_NORM_W, "final_norm_w", (d,), "gain"),
                (LM_HEAD, "lm_head", (V, d), "matrix")]
    return out


def layer_params(cfg):
    d, f = cfg.d_model, cfg.d_ffn
    nq, nkv = cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    if cfg.arch == "opt":
        return [(LN1_W, "ln1_w", (d,), "gain"), (LN1_B, "ln1_b", (d,), "bias"),
                (WQ, "wq", (nq, d), "matrix"), (BQ, "bq", (nq,), "bias"),
                (WK, "wk", (nkv, d), "matrix"), (BK, "bk", (nkv,), "bias"),
                (WV, "wv", (nkv, d), "matrix"), (BV, "bv", (nkv,), "bias"),
                (WO, "wo", (d, nq), "matrix"), (BO, "bo", (d,), "bias"),
                (LN2_W, "ln2_w", (d,), "gain"), (LN2_B, "ln2_b", (d,), "bias"),
                (W_FC1, "w_fc1", (f, d), "matrix"), (B_FC1, "b_fc1", (f,), "bias"),
                (W_FC2, "w_fc2", (d, f), "matrix"), (B_FC2, "b_fc2", (d,), "bias")]
    return [(LN1_W, "ln1_w", (d,), "gain"),
            (WQ, "wq", (nq, d), "matrix"), (WK, "wk", (nkv, d), "matrix"),
            (WV, "wv", (nkv, d), "matrix"),
            (QNORM_W, "q_norm_w", (cfg.head_dim,), "gain"),
            (KNORM_W, "k_norm_w", (cfg.head_dim,), "gain"),
            (WO, "wo", (d, nq), "matrix"),
            (LN2_W, "ln2_w", (d,), "gain"),
            (W_GATE, "w_gate", (f, d), "matrix"), (W_UP, "w_up", (f, d), "matrix"),
            (W_DOWN, "w_down", (d, f), "matrix")]


def make_tensor(cfg, seed, slot, pid, shape, init, rows=None):
    """One logical tensor (or a row range of it) as fp64 holding the stored values."""
    n_cols = shape[-1] if len(shape) == 2 else 1
    if rows is None:
        first, n = 0, int(np.prod(shape))
        out_shape = shape
    else:
        r0, r1 = rows
        first, n = r0 * n_cols, (r1 - r0) * n_cols
        out_shape = (r1 - r0, n_cols)
    z = rng.normal(seed, rng.weight_tag(slot, pid), 0, n, first)
    if init == "gain":
        v = 1.0 + SCALE * z
    else:
        v = SCALE * z
    v32 = v.astype(np.float32)
    if init == "matrix" and cfg.dtype == "fp8" and slot >= 1:
        return (e4m3_round(v32.astype(np.float64) * 2.0 ** FP8_WEIGHT_EXP) * 2.0 ** -FP8_WEIGHT_EXP).reshape(out_shape)
    if init == "matrix" and cfg.dtype in ("bf16", "fp8"):
        v32 = bf16_round(v32)
    return v32.astype(np.float64).reshape(out_shape)


def global_weights(cfg, seed):
    return {name: make_tensor(cfg, seed, 0, pid, shape, init)
            for pid, name, shape, init in global_params(cfg)}


def layer_weights(cfg, seed, layer):
    return {name: make_tensor(cfg, seed, layer + 1, pid, shape, init)
            for pid, name, shape, init in layer_params(cfg)}


def factor(seed, layer, kind, which, tau, n_rows, r):
    """fp32-valued direction factor [n_rows, r] as fp64."""
    z = rng.normal(seed, rng.direction_tag(layer, kind, which), tau, n_rows * r)
    return z.astype(np.float32).astype(np.float64).reshape(n_rows, r)
