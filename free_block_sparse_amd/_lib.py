"""ctypes binding of libsparsepr (argument marshalling only).

Every computation runs inside the HIP library; this module only turns torch
tensors into device pointers, strides and a stream handle.  It fails loudly
when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsparsepr.so")

SPARSEPR_BF16 = 0
SPARSEPR_FP32 = 1
PART_RESPONSE_COUPLED = 0
PART_INDEPENDENT = 1
RIDGE_RELATIVE = 0
RIDGE_ABSOLUTE = 1
ROUTER_BUDGET = 0
ROUTER_ALPHA = 1


class SparseprConfig(ctypes.Structure):
    _fields_ = [
        ("density", ctypes.c_float),
        ("probe_rows", ctypes.c_int),
        ("n_kv_groups", ctypes.c_int),
        ("n_q_groups", ctypes.c_int),
        ("residual_rank", ctypes.c_int),
        ("ridge_lambda", ctypes.c_float),
        ("kmeans_iters", ctypes.c_int),
        ("n_sample_q", ctypes.c_int),
        ("key_coord_rank", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("rank_cut", ctypes.c_float),
        ("partition_mode", ctypes.c_int),
        ("ridge_mode", ctypes.c_int),
        ("seed", ctypes.c_ulonglong),
        ("router", ctypes.c_int),
        ("alpha", ctypes.c_float),
        ("rank_cap", ctypes.c_float),
        ("svd_weighted", ctypes.c_int),
        ("centred_query_coords", ctypes.c_int),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class SparseprTensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("q_strides", ctypes.c_longlong * 4),
        ("k_strides", ctypes.c_longlong * 4),
        ("v_strides", ctypes.c_longlong * 4),
        ("o_strides", ctypes.c_longlong * 4),
        ("B", ctypes.c_int),
        ("H", ctypes.c_int),
        ("N", ctypes.c_int),
        ("d", ctypes.c_int),
        ("dtype", ctypes.c_int),
    ]


class SparseprHeadStats(ctypes.Structure):
    _fields_ = [
        ("routed_pairs", ctypes.c_longlong),
        ("budget_pairs", ctypes.c_longlong),
        ("mandatory_pairs", ctypes.c_longlong),
        ("probe_pairs", ctypes.c_longlong),
        ("granted_cells", ctypes.c_int),
        ("nonempty_q_groups", ctypes.c_int),
        ("nonempty_kv_groups", ctypes.c_int),
        ("probe_rows", ctypes.c_int),
        ("residual_rank", ctypes.c_int),
        ("over_budget", ctypes.c_int),
        ("q_tiles", ctypes.c_int),
        ("kmeans_redecided", ctypes.c_int),
        ("fit_fallback", ctypes.c_int),
        ("reserved", ctypes.c_int),
        ("rho_route", ctypes.c_double),
        ("rho_exec", ctypes.c_double),
        ("sigma", ctypes.c_double * 4),
    ]


STAGES = ["sample_metric", "key_eigen", "key_coords", "key_kmeans", "key_centres", "query_kmeans",
          "query_centres", "route", "gather", "probes", "fit", "sparse_attention", "restore"]

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small",
          -4: "HIP error", -5: "internal error"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "sparsepr_config_default": (_I, [_I, _I, ctypes.POINTER(SparseprConfig)]),
    "sparsepr_validate": (_I, [ctypes.POINTER(SparseprConfig), _I, _I, _I, _I, _I]),
    "sparsepr_workspace_size": (_I, [ctypes.POINTER(SparseprConfig), _I, _I, _I, _I, _I,
                                     ctypes.POINTER(ctypes.c_size_t)]),
    "sparsepr_attention": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P,
                                ctypes.c_size_t, _P, _P]),
    "sparsepr_attention_with_partition": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors),
                                               _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "sparsepr_key_metric": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P,
                                 ctypes.c_size_t, _P, _P, _P, _P, _P]),
    "sparsepr_partition": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P,
                                ctypes.c_size_t, _P, _P, _P]),
    "sparsepr_route": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P, _P, _P,
                            ctypes.c_size_t, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sparsepr_sparse_attention": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P, _P,
                                       _P, ctypes.c_size_t, _P]),
    "sparsepr_probe_fit": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P, _P, _P,
                                ctypes.c_size_t, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sparsepr_dense_attention": (_I, [ctypes.POINTER(SparseprTensors), ctypes.c_float, _P]),
    "sparsepr_mfma_rounding_check": (_I, [_P, ctypes.c_int, _P, _P]),
    "sparsepr_attention_noalloc": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P, _P]),
    "sparsepr_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "sparsepr_attention_profile": (_I, [ctypes.POINTER(SparseprConfig), ctypes.POINTER(SparseprTensors), _P,
                                        ctypes.c_size_t, _P, _P, ctypes.POINTER(ctypes.c_float)]),
    "sparsepr_status_string": (ctypes.c_char_p, [_I]),
    "sparsepr_last_hip_error": (_I, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m free_block_sparse_amd._build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class SparsePRError(RuntimeError):
    pass


def check(status: int, what: str) -> None:
    if status != 0:
        extra = ""
        if status == -4:
            extra = f" (hipError {lib().sparsepr_last_hip_error()})"
        raise SparsePRError(f"{what}: {STATUS.get(status, status)}{extra}")
