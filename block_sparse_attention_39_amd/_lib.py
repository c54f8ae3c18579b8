"""ctypes loader for libbsa.so and the mirror of ``bsa_desc`` (include/bsa.h).

The library is built in-tree by ``python block_sparse_attention_39_amd/build.py``;
importing this module without it raises at once: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")

BSA_OK = 0
STATUS_NAMES = {0: "BSA_OK", -1: "BSA_ERR_NULL", -2: "BSA_ERR_SHAPE", -3: "BSA_ERR_UNSUPPORTED",
                -4: "BSA_ERR_ALIGN", -5: "BSA_ERR_WORKSPACE", -6: "BSA_ERR_LAUNCH", -7: "BSA_ERR_ARG"}
TILE_STATIC, TILE_DYNAMIC, TILE_STATIC_PADDED = 0, 1, 2
PERM_BUILD, PERM_GATHER, PERM_SCATTER, PERM_GATHER_KF, PERM_GATHER_VF = 0, 1, 2, 3, 4
PERM_GATHER_POOL, PERM_GATHER_KF_POOL, PERM_TILED_TO_KF, PERM_TILED_TO_VF, PERM_POOL = 5, 6, 7, 8, 9
MAX_VIDEO_TILES = 8192
MAX_TILES = 16384
# the exported entry points, in the order include/bsa.h declares them
EXPORTS = ("bsa_workspace_size", "bsa_permute", "bsa_plan", "bsa_select", "bsa_forward", "bsa_forward_stats_offset",
           "bsa_forward_noalloc", "bsa_forward_raster",
           "bsa_csr_entries", "bsa_plan_csr", "bsa_select_csr",
           "bsa_forward_csr", "bsa_forward_csr_raster", "bsa_structured_entries", "bsa_plan_structured", "bsa_backward_workspace_size",
           "bsa_backward", "bsa_backward_csr_workspace_size", "bsa_backward_csr", "bsa_backward_stats_offset",
           "bsa_status_string", "bsa_version")
MASK_SPATIAL, MASK_TEMPORAL = 0, 1
MAX_CSR_HEADS = 256


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("n_prefix", ctypes.c_int32), ("tile_mode", ctypes.c_int32), ("tile_t", ctypes.c_int32),
                ("tile_h", ctypes.c_int32), ("tile_w", ctypes.c_int32), ("keep_tiles", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dyn_tau", ctypes.c_float)]

    def __repr__(self):
        return "Desc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class BsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().bsa_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python block_sparse_attention_39_amd/build.py` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(Desc)
        L.bsa_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_permute.argtypes = [D, ctypes.c_int, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.bsa_plan.argtypes = [D, P, P, P, P, ctypes.c_size_t, P]
        L.bsa_select.argtypes = [D, P, P, ctypes.c_size_t, P]
        L.bsa_forward.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.bsa_forward_stats_offset.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_forward_noalloc.argtypes = [D, P, P, P, P, P, P, P]
        L.bsa_forward_raster.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        I64 = ctypes.c_int64
        L.bsa_csr_entries.argtypes = [D, P, ctypes.POINTER(I64)]
        L.bsa_plan_csr.argtypes = [D, P, P, P, P, P, P, I64, P, ctypes.c_size_t, P]
        L.bsa_select_csr.argtypes = [D, P, P, P, P, I64, P, ctypes.c_size_t, P]
        L.bsa_forward_csr.argtypes = [D, P, P, P, P, P, I64, P, P, P, ctypes.c_size_t, P]
        L.bsa_forward_csr_raster.argtypes = [D, P, P, P, P, P, P, I64, P, P, P, ctypes.c_size_t, P]
        I32 = ctypes.c_int32
        L.bsa_structured_entries.argtypes = [D, P, I32, I32, ctypes.POINTER(I64)]
        L.bsa_plan_structured.argtypes = [D, P, I32, I32, P, P, I64, P]
        L.bsa_backward_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_backward.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.bsa_backward_csr_workspace_size.argtypes = [D, I64, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_backward_csr.argtypes = [D, P, P, P, P, P, P, P, P, P, I64, P, P, P, P, ctypes.c_size_t, P]
        L.bsa_backward_stats_offset.argtypes = [D, I64, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_status_string.argtypes = [ctypes.c_int]
        L.bsa_status_string.restype = ctypes.c_char_p
        L.bsa_version.argtypes = []
        for f in ("bsa_workspace_size", "bsa_permute", "bsa_plan", "bsa_select", "bsa_forward",
                  "bsa_forward_stats_offset", "bsa_forward_noalloc", "bsa_forward_raster",
                  "bsa_backward_workspace_size",
                  "bsa_backward", "bsa_backward_csr_workspace_size", "bsa_backward_csr", "bsa_backward_stats_offset",
                  "bsa_version"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib
