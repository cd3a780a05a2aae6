"""ctypes view of include/ec.h (libec.so). Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libec.so")

EC_OK, EC_ERR_ARG, EC_ERR_DTYPE, EC_ERR_WORKSPACE, EC_ERR_HIP, EC_ERR_NAN, EC_ERR_UNSUPPORTED = range(7)
EC_F32, EC_BF16 = 0, 1
EC_LAYOUT_PLAIN, EC_LAYOUT_PACKED = 0, 1
EC_CAND_BLOCKS, EC_CAND_WINDOW = 0, 1
EC_MAX_TOKENS_PER_STEP = 64
EC_MAX_SEQ = 16
EC_ENTROPY_NOALLOC_SCRATCH_BYTES = 1 << 20

STATUS_NAMES = {
    0: "EC_OK", 1: "EC_ERR_ARG", 2: "EC_ERR_DTYPE", 3: "EC_ERR_WORKSPACE", 4: "EC_ERR_HIP",
    5: "EC_ERR_NAN", 6: "EC_ERR_UNSUPPORTED",
}

EXPORTS = (
    "ec_entropy_max_workspace_size", "ec_entropy_max", "ec_entropy_max_noalloc", "ec_cache_scatter",
    "ec_partial_attn_workspace_size", "ec_partial_attn_plan", "ec_partial_attn", "ec_rope_table",
    "ec_forward_workspace_size", "ec_forward", "ec_state_plan_words", "ec_state_reset",
    "ec_step_workspace_size", "ec_step", "ec_timing_enable", "ec_timing_select", "ec_timing_read",
    "ec_last_error",
    "ec_version", "ec_pack_weights", "ec_step_batch_workspace_size", "ec_step_batch", "ec_step_probe",
)

EC_T_KINDS = 11
TIMING_KINDS = ("embed", "norm", "qkv", "attn", "oproj", "gateup", "down", "lmhead", "entropy",
                "select", "last")


class ec_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class ec_model_desc(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32), ("dtype", C.c_int),
        ("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
        ("head_dim", C.c_int32), ("ffn_dim", C.c_int32), ("vocab", C.c_int32),
        ("rms_eps", C.c_float),
        ("embed", C.c_void_p), ("layers", C.POINTER(ec_layer_weights)),
        ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
        ("rope_cos", C.c_void_p), ("rope_sin", C.c_void_p), ("rope_max_pos", C.c_int32),
        ("weight_layout", C.c_int32),
    ]


class ec_cache_desc(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("seq_len", C.c_int32),
                ("k", C.POINTER(C.c_void_p)), ("v", C.POINTER(C.c_void_p))]


class ec_params(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("tau", C.c_float), ("k_recent", C.c_int32),
                ("tokens_per_step", C.c_int32), ("block_len", C.c_int32),
                ("prompt_len", C.c_int32), ("seq_len", C.c_int32), ("mask_id", C.c_int32),
                ("candidates", C.c_int32)]


class ec_state(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("tokens", C.c_void_p), ("masked", C.c_void_p),
                ("plan", C.c_void_p), ("t", C.c_int32), ("refresh_next", C.c_int32),
                ("n_masked", C.c_int32), ("n_decoded", C.c_int32), ("next_rows", C.c_int32),
                ("next_cand", C.c_int32)]


class ec_step_out(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("status", C.c_int32), ("refreshed", C.c_int32),
                ("rows", C.c_int32), ("n_cand", C.c_int32), ("n_decoded", C.c_int32),
                ("refresh_next", C.c_int32), ("emax", C.c_float),
                ("positions", C.c_int32 * EC_MAX_TOKENS_PER_STEP),
                ("ids", C.c_int32 * EC_MAX_TOKENS_PER_STEP),
                ("entropy", C.c_float * EC_MAX_TOKENS_PER_STEP),
                ("maxprob", C.c_float * EC_MAX_TOKENS_PER_STEP)]


class ec_timing(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("n_kinds", C.c_int32),
                ("ms", C.c_double * EC_T_KINDS), ("launches", C.c_int64 * EC_T_KINDS),
                ("flops", C.c_double * EC_T_KINDS), ("bytes", C.c_double * EC_T_KINDS)]


_lib = None


class ECError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libec.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libec.so not found at {path}; build it with "
                           "`python -m entropy_guided_kv_amd.build`")
    lib = C.CDLL(path)
    vp, i32, i64, sz, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
    sig = {
        "ec_entropy_max_workspace_size": (sz, [i32, i32]),
        "ec_entropy_max": (C.c_int, [vp, C.c_int, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, sz, vp]),
        "ec_entropy_max_noalloc": (C.c_int, [vp, C.c_int, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp]),
        "ec_cache_scatter": (C.c_int, [vp, vp, i64, i32, C.c_int, vp, vp, vp, i32, vp]),
        "ec_partial_attn_workspace_size": (sz, [i32, i32, i32, i32]),
        "ec_partial_attn_plan": (C.c_int, [i32, i32, i32, i32, C.POINTER(i32), C.POINTER(i32)]),
        "ec_partial_attn": (C.c_int, [vp, vp, vp, i32, i32, i32, i32, f32, C.c_int, vp, vp, sz, vp]),
        "ec_rope_table": (C.c_int, [vp, vp, i32, i32, C.c_double, vp]),
        "ec_forward_workspace_size": (sz, [C.POINTER(ec_model_desc), i32, i32, i32]),
        "ec_forward": (C.c_int, [C.POINTER(ec_model_desc), C.POINTER(ec_cache_desc), vp, vp, i32,
                                 vp, i32, vp, vp, vp, sz, vp]),
        "ec_state_plan_words": (sz, [i32, i32]),
        "ec_state_reset": (C.c_int, [C.POINTER(ec_state), C.POINTER(ec_params), vp]),
        "ec_step_workspace_size": (sz, [C.POINTER(ec_model_desc), C.POINTER(ec_params)]),
        "ec_step": (C.c_int, [C.POINTER(ec_model_desc), C.POINTER(ec_cache_desc), C.POINTER(ec_state),
                              C.POINTER(ec_params), vp, sz, vp, C.POINTER(ec_step_out)]),
        "ec_timing_enable": (C.c_int, [C.c_int]),
        "ec_timing_select": (C.c_int, [C.c_uint32]),
        "ec_timing_read": (C.c_int, [C.POINTER(ec_timing), C.c_int]),
        "ec_last_error": (C.c_char_p, []),
        "ec_version": (C.c_int, []),
        "ec_pack_weights": (C.c_int, [C.c_int, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "ec_step_probe": (C.c_int, [C.POINTER(ec_model_desc), C.POINTER(ec_cache_desc), C.POINTER(ec_state),
                                    C.POINTER(ec_params), vp, sz, vp, C.POINTER(ec_step_out), vp]),
        "ec_step_batch_workspace_size": (sz, [C.POINTER(ec_model_desc), i32, C.POINTER(ec_params)]),
        "ec_step_batch": (C.c_int, [C.POINTER(ec_model_desc), i32, C.POINTER(ec_cache_desc),
                                    C.POINTER(ec_state), C.POINTER(ec_params), vp, sz, vp,
                                    C.POINTER(ec_step_out)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def check(status: int, what: str = "") -> int:
    if status != EC_OK:
        msg = _lib.ec_last_error().decode() if _lib is not None else ""
        raise ECError(status, f"{what}: {msg}" if what else msg)
    return status
