"""ctypes loader of libsparselora.so (the C ABI declared in include/sparselora.h).

Argument marshalling only.  The library must have been built in-tree
(``python -m contextual_sparsity_lora_amd.build`` or ``__graft_entry__.build()``);
there is no fallback: a missing library raises.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparselora.so")

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_int = ctypes.c_int
_f = ctypes.c_float
_st = ctypes.c_int   # sl_status

# name -> (restype, argtypes); mirrors include/sparselora.h
SIGNATURES = {
    "sl_create": (_st, [ctypes.POINTER(_vp), _int]),
    "sl_destroy": (_st, [_vp]),
    "sl_set_stream": (_st, [_vp, _vp]),
    "sl_reserve_workspace": (_st, [_vp, ctypes.c_size_t]),
    "sl_workspace_bytes": (_st, [_vp, ctypes.POINTER(ctypes.c_size_t)]),
    "sl_set_option": (_st, [_vp, ctypes.c_char_p, _i64]),
    "sl_sync": (_st, [_vp]),
    "sl_last_error": (ctypes.c_char_p, [_vp]),
    "sl_status_str": (ctypes.c_char_p, [_st]),
    "sl_version": (ctypes.c_char_p, []),
    "sl_timing_enable": (_st, [_vp, _int]),
    "sl_timing_reset": (_st, [_vp]),
    "sl_timing_query": (_st, [_vp, ctypes.c_char_p, ctypes.POINTER(_i64),
                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_double)]),
    "sl_timing_only": (_st, [_vp, ctypes.c_char_p]),
    "sl_timing_class_name": (ctypes.c_char_p, [_int]),
    "sl_token_split": (_st, [_vp, _vp, _i64, _vp, _i64, _vp, _i64]),
    "sl_svd_estimate": (_st, [_vp, _vp, _int, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "sl_score_select": (_st, [_vp, _int, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                              _i64, _i64, _i64, _vp, _vp]),
    "sl_score_select_noalloc": (_st, [_vp, _int, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                      _i64, _i64, _i64, _vp, _vp]),
    "sl_select_top": (_st, [_vp, _vp, _i64, _i64, _vp]),
    "sl_random_scores": (_st, [_vp, ctypes.c_uint64, _i64, _vp]),
    "sl_dense_scores": (_st, [_vp, _int, _int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]),
    "sl_select_heads": (_st, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "sl_expand_gqa": (_st, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "sl_stack_index": (_st, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "sl_offset_index": (_st, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "sl_qkv_index": (_st, [_vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp]),
    "sl_sparse_linear_fwd": (_st, [_vp, _int, _int, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                   _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int,
                                   _vp, _i64, _vp, _i64, _i64, _f, _vp, _i64, _vp, _i64, _int]),
    "sl_sparse_linear_bwd": (_st, [_vp, _int, _int, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64,
                                   _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _int,
                                   _vp, _i64, _vp, _i64, _i64, _f, _vp, _i64, _vp, _i64, _int]),
    "sl_weight_slice": (_st, [_vp, _int, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64]),
    "sl_lora_fill_unselected": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64,
                                      _i64, _f, _vp, _i64]),
    "sl_lora_fwd_bwd": (_st, [_vp, _int, _int, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _f,
                              _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64]),
    "sl_swiglu_fwd": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64]),
    "sl_swiglu_bwd": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64,
                            _vp, _i64]),
    "sl_swiglu_fwd_lora": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                 _i64, _vp, _i64]),
    "sl_swiglu_fwd_ctx": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                _i64, _f, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64]),
    "sl_swiglu_bwd_lora": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                 _vp, _i64, _vp, _i64, _vp, _i64, _i64, _f, _vp, _vp, _vp]),
    "sl_svd_factors": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_uint64,
                             _vp, _vp]),
    "sl_token_ce": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _vp, _i64, _f, _vp, _i64, _vp]),
    "sl_adamw_step": (_st, [_vp, _vp, _int, _f, _f, _f, _f, _f, _i64]),
    "sl_dot_stats": (_st, [_vp, _vp, _vp, _i64, _vp]),
    "sl_transpose": (_st, [_vp, _int, _vp, _i64, _i64, _i64, _vp, _i64]),
    "sl_rmsnorm_fwd": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _f, _vp, _i64, _vp, _i64,
                             _vp]),
    "sl_rmsnorm_bwd": (_st, [_vp, _int, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64]),
    "sl_add": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _i64, _i64, _vp, _i64]),
    "sl_attention_fwd": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                               _i64, _vp, _i64, _vp]),
    "sl_attention_bwd": (_st, [_vp, _int, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                               _i64, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]),
}

_lib = None


def load():
    """Load the library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run contextual_sparsity_lora_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
