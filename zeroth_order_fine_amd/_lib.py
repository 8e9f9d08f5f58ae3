"""ctypes declarations of libzo (include/zo.h).  Argument marshalling only."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzo.so")

c_i32, c_u32, c_i64, c_u64, c_dbl, c_sz, c_vp = (ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint64,
                                                 ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p)
P = ctypes.POINTER


class ModelDesc(ctypes.Structure):
    _fields_ = [("abi_version", c_i32), ("arch", c_i32), ("dtype", c_i32), ("n_layers", c_i32),
                ("d_model", c_i32), ("n_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
                ("d_ffn", c_i32), ("vocab", c_i32), ("max_pos", c_i32), ("norm_eps", c_dbl),
                ("rope_theta", c_dbl)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("step", c_u64), ("nu", c_u32), ("rank", c_i32), ("eps", c_dbl), ("n_dirs", c_i32),
                ("dir_seeds", P(c_u64)), ("n_cand", c_i32), ("cand_dir", P(c_i32)), ("cand_sign", P(c_i32)),
                ("target_mask", c_u32), ("flags", c_u32)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("n_seq", c_i32), ("cu_seqlens", P(c_i32)), ("tokens_dev", c_vp), ("role", P(c_i32)),
                ("score_mode", P(c_i32))]


_SIGS = {
    "zo_abi_version": (c_i32, []),
    "zo_last_error": (ctypes.c_char_p, []),
    "zo_weights_size": (c_i32, [P(ModelDesc), P(c_sz)]),
    "zo_weight_locate": (c_i32, [P(ModelDesc), c_i32, c_i32, P(c_sz), P(c_i64), P(c_i64), P(c_i32), P(c_i32)]),
    "zo_model_create": (c_i32, [P(ModelDesc), c_vp, c_sz, P(c_vp)]),
    "zo_model_destroy": (c_i32, [c_vp]),
    "zo_model_set_graphs": (c_i32, [c_vp, c_i32]),
    "zo_init_weights": (c_i32, [c_vp, c_u64, c_vp]),
    "zo_plan": (c_i32, [c_vp, P(PlanDesc), P(c_vp)]),
    "zo_plan_destroy": (c_i32, [c_vp]),
    "zo_bank_size": (c_i32, [c_vp, c_i32, c_i32, c_u32, P(c_sz)]),
    "zo_bank_create": (c_i32, [c_vp, c_i32, c_i32, c_u32, c_vp, c_sz, P(c_vp)]),
    "zo_bank_destroy": (c_i32, [c_vp]),
    "zo_bank_keys": (c_i32, [c_vp, P(c_u64), P(c_i64)]),
    "zo_bank_set_keys": (c_i32, [c_vp, P(c_u64), P(c_i64)]),
    "zo_bank_entry_offset": (c_i32, [c_vp, c_i32, c_i32, c_i32, P(c_sz)]),
    "zo_bank_fold_size": (c_i32, [c_vp, c_vp, P(c_sz)]),
    "zo_bank_fold": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_sz, c_vp]),
    "zo_bank_cap": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_sz, c_vp, P(c_i32)]),
    "zo_batch_layout": (c_i32, [c_vp, c_vp, c_vp, P(BatchDesc), P(c_i32), P(c_i64), P(c_i64), P(c_sz)]),
    "zo_pack": (c_i32, [c_vp, P(BatchDesc), P(c_i32), P(c_i32), P(c_i32)]),
    "zo_score": (c_i32, [c_vp, c_vp, c_vp, P(BatchDesc), c_vp, c_sz, c_vp, c_vp, P(c_dbl), c_vp]),
    "zo_score_noalloc": (c_i32, [c_vp, c_vp, c_vp, P(BatchDesc), c_vp, c_vp, P(c_dbl), c_vp]),
    "zo_generate_layout": (c_i32, [c_vp, c_vp, c_vp, P(BatchDesc), c_i32, P(c_i32), P(c_sz)]),
    "zo_generate": (c_i32, [c_vp, c_vp, c_vp, P(BatchDesc), c_i32, c_vp, c_sz, c_vp, c_vp, P(c_dbl), c_vp]),
    "zo_estimate": (c_i32, [c_vp, P(c_dbl), P(c_i64), c_u32, P(c_dbl)]),
    "zo_update": (c_i32, [c_vp, c_vp, c_vp, P(c_dbl), c_dbl, c_vp]),
    "zo_philox_words": (c_i32, [c_u64, c_u32, c_u64, c_i64, c_i64, c_vp, c_vp]),
    "zo_normal_fill": (c_i32, [c_u64, c_u32, c_u64, c_i64, c_i64, c_vp, c_vp]),
    "zo_direction": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "zo_profile_begin": (c_i32, []),
    "zo_profile_end": (c_i32, [c_i32, P(c_i64), P(c_dbl)]),
    "zo_profile_select": (c_i32, [c_u32]),
}

EXPORTED = tuple(_SIGS)
_lib = None


def load():
    """Load libzo.so from the package directory.  There is no fallback: without
    the built HIP library the package cannot run."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libzo.so is not built (run __graft_entry__.build() or "
                              "python zeroth_order_fine_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
