"""ctypes declarations of libspecdec's C ABI (include/specdec.h).  Marshalling only."""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecdec.so")

OK, E_INVAL, E_CAPACITY, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4
STATIC_WORKSPACE_BYTES = 64 << 20  # SPECDEC_STATIC_WORKSPACE_BYTES
TREE_MAX_DEPTH = TREE_MAX_WIDTH = 16
F32, BF16 = 0, 1
HEAD_CLUSTERED, HEAD_FULL = 0, 1
WF_DENSE, WF_Q4 = 0, 1
ACCEPT_COMMIT = 1
DEVERR_CAPACITY, DEVERR_NAN, DEVERR_TOKEN = 1, 2, 4
PACK_PLAIN, PACK_ROPE, PACK_GATE_UP = 0, 1, 2
(LW_ATTN_NORM, LW_QKV, LW_O, LW_FFN_NORM, LW_GATE_UP, LW_DOWN, LW_ROUTER, LW_EXP_GATE_UP, LW_EXP_DOWN,
 N_LAYER_TENSORS) = range(10)
DW_N1, DW_Q, DW_O, DW_N2, DW_GATE_UP, DW_DOWN, N_DRAFT_TENSORS = range(7)
(PROF_GATE_UP, PROF_DOWN, PROF_QKV, PROF_O, PROF_ATTN, PROF_HEAD, PROF_DRAFT_HEAD, PROF_EXP_GATE_UP,
 PROF_EXP_DOWN) = range(9)

EXPORTS = [
    "specdec_workspace_bytes", "specdec_kv_elems", "specdec_create", "specdec_create_static",
    "specdec_destroy",
    "specdec_draft", "specdec_draft_traced", "specdec_draft_tree", "specdec_verify", "specdec_prefill",
    "specdec_verify_tree", "specdec_accept_tree", "specdec_accept", "specdec_kv_commit",
    "specdec_pack_matrix", "specdec_q4_bytes", "specdec_pack_q4", "specdec_set_len_bound", "specdec_read_device_error",
    "specdec_profile_start", "specdec_profile_read", "specdec_query_split", "specdec_query_launch", "specdec_error_string",
    "specdec_moe_usage_start", "specdec_moe_usage_read", "specdec_k_policy_init",
    "specdec_k_policy_observe", "specdec_k_policy_acceptance", "specdec_k_policy_choose",
]


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab",
        "n_experts", "top_k", "expert_ffn", "shared_ffn",
        "d_layers", "d_dim", "d_ffn", "n_centroids", "kv_src_layer", "dtype")] + [
        ("rms_eps", C.c_float), ("rope_theta", C.c_float)] + [
        (n, C.c_int32) for n in ("max_batch", "max_draft", "max_rows", "max_ctx",
                                 "weight_format", "max_prefill")]


class Weights(C.Structure):
    _fields_ = [
        ("embed", C.c_void_p), ("final_norm", C.c_void_p), ("layers", C.POINTER(C.c_void_p)),
        ("table", C.c_void_p), ("centroids", C.c_void_p), ("row_vocab", C.c_void_p),
        ("vocab_row", C.c_void_p), ("norm_h", C.c_void_p), ("norm_e", C.c_void_p),
        ("w_in", C.c_void_p), ("d_layers", C.POINTER(C.c_void_p)), ("norm_f", C.c_void_p),
        ("w_back", C.c_void_p),
    ]


class KPolicy(C.Structure):
    _fields_ = [("k_min", C.c_int32), ("k_max", C.c_int32), ("decay", C.c_float),
                ("prior_accepted", C.c_float), ("prior_rejected", C.c_float),
                ("t_draft_ms", C.c_float), ("t_verify_ms", C.c_float), ("t_row_ms", C.c_float),
                ("accepted", C.c_double), ("rejected", C.c_double)]


class DraftTrace(C.Structure):
    _fields_ = [("state", C.c_void_p), ("hidden", C.c_void_p), ("centroid_scores", C.c_void_p),
                ("table_scores", C.c_void_p), ("raw_drafts", C.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Loads libspecdec.so.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m speculative_decoding_03_amd.build`")
    lib = C.CDLL(path)
    vp, i32, i64, u32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_size_t
    P = C.POINTER
    sig = {
        "specdec_workspace_bytes": (sz, [P(Config)]),
        "specdec_kv_elems": (sz, [P(Config)]),
        "specdec_create": (C.c_int, [P(Config), P(Weights), vp, vp, vp, vp, vp, sz, vp, P(vp)]),
        "specdec_create_static": (C.c_int, [P(Config), P(Weights), vp, vp, vp, vp, vp, P(vp)]),
        "specdec_destroy": (C.c_int, [vp]),
        "specdec_draft": (C.c_int, [vp, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp]),
        "specdec_draft_traced": (C.c_int, [vp, i32, i32, i32, i32, vp, vp, vp, i64, vp,
                                           P(DraftTrace), vp]),
        "specdec_moe_usage_start": (C.c_int, [vp, vp]),
        "specdec_moe_usage_read": (C.c_int, [vp, P(i32), vp]),
        "specdec_verify": (C.c_int, [vp, i32, i32, vp, vp, vp, vp]),
        "specdec_prefill": (C.c_int, [vp, i32, i32, vp, vp, vp, vp]),
        "specdec_draft_tree": (C.c_int, [vp, i32, i32, i32, i32, i32, vp, vp, vp, i64, vp]),
        "specdec_verify_tree": (C.c_int, [vp, i32, i32, P(i32), vp, vp, vp, vp]),
        "specdec_accept_tree": (C.c_int, [vp, i32, i32, P(i32), vp, vp, i32, vp, vp, u32, vp]),
        "specdec_accept": (C.c_int, [vp, i32, i32, vp, vp, vp, vp, u32, vp]),
        "specdec_kv_commit": (C.c_int, [vp, i32, vp, vp]),
        "specdec_pack_matrix": (C.c_int, [vp, vp, i32, i32, i32, i32, i32, i32, vp]),
        "specdec_q4_bytes": (sz, [i32, i32]),
        "specdec_pack_q4": (C.c_int, [vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "specdec_set_len_bound": (C.c_int, [vp, P(i32), i32]),
        "specdec_read_device_error": (C.c_int, [vp, P(i32), i32, vp]),
        "specdec_profile_start": (C.c_int, [vp, i32, i32]),
        "specdec_profile_read": (C.c_int, [vp, P(C.c_float), i32, P(i32)]),
        "specdec_query_split": (C.c_int, [vp, i32, P(i32), P(i32), P(i32), P(i32)]),
        "specdec_query_launch": (C.c_int, [vp, i32, i32, P(i32), P(i32), P(i32), P(i32), P(i32)]),
        "specdec_error_string": (C.c_char_p, [C.c_int]),
        "specdec_k_policy_init": (C.c_int, [P(KPolicy), i32, i32, C.c_float, C.c_float, C.c_float,
                                            C.c_float, C.c_float, C.c_float]),
        "specdec_k_policy_observe": (C.c_int, [P(KPolicy), i32, P(i32), i32]),
        "specdec_k_policy_acceptance": (C.c_double, [P(KPolicy)]),
        "specdec_k_policy_choose": (C.c_int32, [P(KPolicy)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class SpecdecError(RuntimeError):
    def __init__(self, code: int, what: str):
        msg = load().specdec_error_string(code).decode() if _lib else str(code)
        super().__init__(f"{what}: {msg} ({code})")
        self.code = code


def check(code: int, what: str) -> None:
    if code != OK:
        raise SpecdecError(code, what)
