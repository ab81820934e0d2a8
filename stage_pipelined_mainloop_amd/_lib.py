"""ctypes binding of libstagegemm.so: the C-ABI functions under the same names.

Argument marshalling only.  Every step of the GEMM runs in the HIP kernels of
the shared library; nothing here computes, and there is no fallback: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstagegemm.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "stagegemm.h")

SG_OK = 0
SG_ERR_NULL = 1
SG_ERR_SHAPE = 2
SG_ERR_ALIGN = 3
SG_ERR_UNSUPPORTED = 4
SG_ERR_ALIAS = 5
SG_ERR_HIP = 6


class SgConfig(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("stages", ctypes.c_int), ("waves", ctypes.c_int), ("schedule", ctypes.c_int)]

    def as_tuple(self):
        return (self.tile_m, self.tile_n, self.tile_k, self.stages, self.waves, self.schedule)

    def __repr__(self):
        return "SgConfig(%d, %d, %d, stages=%d, waves=%d, schedule=%d)" % self.as_tuple()


class SgConfigInfo(ctypes.Structure):
    _fields_ = [("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("lds_total_bytes", ctypes.c_int), ("loads_per_stage", ctypes.c_int), ("wg_per_cu_lds", ctypes.c_int),
                ("regs", ctypes.c_int), ("wg_per_cu_regs", ctypes.c_int),
                ("wg_per_cu", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class SgSplitInfo(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_int), ("whole_tiles", ctypes.c_int), ("cut_tiles", ctypes.c_int),
                ("splits", ctypes.c_int), ("workgroups", ctypes.c_longlong),
                ("workspace_bytes", ctypes.c_size_t), ("chosen_splits", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class SgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {sg_status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libstagegemm.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        # PyTorch-ROCm ships its own libamdhip64 (same soname).  Loading torch
        # first makes this library bind to that already-loaded runtime, so
        # torch's device memory and stream handles belong to the runtime our
        # launches go through.  Loading ours first would bring in a second HIP
        # runtime that rejects torch's streams.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.gemm_fp16_tn.argtypes = [i, i, i, vp, vp, vp, vp]
        L.gemm_fp16_tn.restype = i
        L.gemm_fp16_tn_alpha.argtypes = [i, i, i, f, vp, vp, vp, vp]
        L.gemm_fp16_tn_alpha.restype = i
        L.gemm_fp16_tn_alpha_beta.argtypes = [i, i, i, f, f, vp, vp, vp, vp, vp]
        L.gemm_fp16_tn_alpha_beta.restype = i
        L.attention_fp16_fwd.argtypes = [i, i, i, i, f, vp, vp, vp, vp, vp]
        L.attention_fp16_fwd.restype = i
        L.attention_fp16_fwd_split.argtypes = [i, i, i, i, f, vp, vp, vp, vp, i, vp, ctypes.c_size_t, vp]
        L.attention_fp16_fwd_split.restype = i
        L.attention_fp16_workspace_bytes.argtypes = [i, i, i, i, i]
        L.attention_fp16_workspace_bytes.restype = ctypes.c_size_t
        L.attention_fp16_splits.argtypes = [i, i, i, i]
        L.attention_fp16_splits.restype = i
        L.gemm_fp16_tn_splitk.argtypes = [i, i, i, f, vp, vp, vp, i, vp, ctypes.c_size_t, vp]
        L.gemm_fp16_tn_splitk.restype = i
        L.gemm_fp16_tn_splitk_noalloc.argtypes = [i, i, i, f, vp, vp, vp, i, vp]
        L.gemm_fp16_tn_splitk_noalloc.restype = i
        L.gemm_fp16_tn_splitk_workspace_bytes.argtypes = [i, i, i, i]
        L.gemm_fp16_tn_splitk_workspace_bytes.restype = ctypes.c_size_t
        L.sg_split_plan.argtypes = [i, i, i, i, i, ctypes.POINTER(SgSplitInfo)]
        L.sg_split_plan.restype = i
        L.gemm_fp16_tn_splitk_splits.argtypes = [i, i, i]
        L.gemm_fp16_tn_splitk_splits.restype = i
        L.gemm_fp16_tn_remainder_quarters.argtypes = [i, i, i]
        L.gemm_fp16_tn_remainder_quarters.restype = i
        L.gemm_fp16_tn_cfg.argtypes = [i, i, i, f, vp, vp, vp, ctypes.POINTER(SgConfig), vp]
        L.gemm_fp16_tn_cfg.restype = i
        L.sg_select_config.argtypes = [i, i, i, ctypes.POINTER(SgConfig)]
        L.sg_select_config.restype = i
        L.sg_num_configs.argtypes = []
        L.sg_num_configs.restype = i
        L.sg_get_config.argtypes = [i, ctypes.POINTER(SgConfig)]
        L.sg_get_config.restype = i
        L.sg_query_config.argtypes = [ctypes.POINTER(SgConfig), ctypes.POINTER(SgConfigInfo)]
        L.sg_query_config.restype = i
        L.sg_minimum_stages.argtypes = [ctypes.c_longlong, ctypes.c_longlong]
        L.sg_minimum_stages.restype = i
        L.sg_pipeline_wait_count.argtypes = [i, i, i, i]
        L.sg_pipeline_wait_count.restype = i
        L.sg_persistent_wait_count.argtypes = [i, i, i, i, i, i]
        L.sg_persistent_wait_count.restype = i
        L.sg_status_string.argtypes = [i]
        L.sg_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/stagegemm.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)


# --- the C-ABI under the same names ----------------------------------------

def _check(st: int, what: str) -> int:
    if st != SG_OK:
        raise SgError(st, what)
    return st


def gemm_fp16_tn(M: int, N: int, K: int, A: int, B: int, D: int, stream: int = 0) -> int:
    return _check(lib().gemm_fp16_tn(M, N, K, A, B, D, stream), "gemm_fp16_tn")


def gemm_fp16_tn_alpha(M: int, N: int, K: int, alpha: float, A: int, B: int, D: int,
                       stream: int = 0) -> int:
    return _check(lib().gemm_fp16_tn_alpha(M, N, K, alpha, A, B, D, stream),
                  "gemm_fp16_tn_alpha")


def gemm_fp16_tn_alpha_beta(M: int, N: int, K: int, alpha: float, beta: float, A: int, B: int,
                            C: int, D: int, stream: int = 0) -> int:
    return _check(lib().gemm_fp16_tn_alpha_beta(M, N, K, alpha, beta, A, B, C, D, stream),
                  "gemm_fp16_tn_alpha_beta")


def attention_fp16_fwd(H: int, M: int, N: int, d: int, alpha: float, Q: int, K: int, V: int,
                       O: int, stream: int = 0) -> int:
    return _check(lib().attention_fp16_fwd(H, M, N, d, alpha, Q, K, V, O, stream),
                  "attention_fp16_fwd")


def attention_fp16_fwd_split(H: int, M: int, N: int, d: int, alpha: float, Q: int, K: int, V: int,
                             O: int, splits: int, workspace: int, workspace_bytes: int,
                             stream: int = 0) -> int:
    return _check(lib().attention_fp16_fwd_split(H, M, N, d, alpha, Q, K, V, O, splits, workspace,
                                                 workspace_bytes, stream),
                  "attention_fp16_fwd_split")


def attention_fp16_workspace_bytes(H: int, M: int, N: int, d: int, splits: int) -> int:
    return lib().attention_fp16_workspace_bytes(H, M, N, d, splits)


def attention_fp16_splits(H: int, M: int, N: int, d: int) -> int:
    return lib().attention_fp16_splits(H, M, N, d)


def gemm_fp16_tn_cfg(M: int, N: int, K: int, alpha: float, A: int, B: int, D: int,
                     cfg, stream: int = 0) -> int:
    c = cfg if isinstance(cfg, SgConfig) else SgConfig(*cfg)
    return _check(lib().gemm_fp16_tn_cfg(M, N, K, alpha, A, B, D, ctypes.byref(c), stream),
                  "gemm_fp16_tn_cfg")


def gemm_fp16_tn_splitk(M: int, N: int, K: int, alpha: float, A: int, B: int, D: int, splits: int,
                        workspace: int, workspace_bytes: int, stream: int = 0) -> int:
    return _check(lib().gemm_fp16_tn_splitk(M, N, K, alpha, A, B, D, splits, workspace,
                                            workspace_bytes, stream), "gemm_fp16_tn_splitk")


def gemm_fp16_tn_splitk_noalloc(M: int, N: int, K: int, alpha: float, A: int, B: int, D: int,
                                splits: int, stream: int = 0) -> int:
    return _check(lib().gemm_fp16_tn_splitk_noalloc(M, N, K, alpha, A, B, D, splits, stream),
                  "gemm_fp16_tn_splitk_noalloc")


def gemm_fp16_tn_splitk_workspace_bytes(M: int, N: int, K: int, splits: int) -> int:
    return int(lib().gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits))


def gemm_fp16_tn_splitk_splits(M: int, N: int, K: int) -> int:
    return int(lib().gemm_fp16_tn_splitk_splits(M, N, K))


def gemm_fp16_tn_remainder_quarters(M: int, N: int, K: int) -> int:
    return int(lib().gemm_fp16_tn_remainder_quarters(M, N, K))


def sg_split_plan(M: int, N: int, K: int, splits: int, capacity: int) -> SgSplitInfo:
    info = SgSplitInfo()
    _check(lib().sg_split_plan(M, N, K, splits, capacity, ctypes.byref(info)), "sg_split_plan")
    return info


def sg_select_config(M: int, N: int, K: int) -> SgConfig:
    c = SgConfig()
    _check(lib().sg_select_config(M, N, K, ctypes.byref(c)), "sg_select_config")
    return c


def sg_num_configs() -> int:
    return int(lib().sg_num_configs())


def sg_get_config(index: int) -> SgConfig:
    c = SgConfig()
    _check(lib().sg_get_config(index, ctypes.byref(c)), "sg_get_config")
    return c


def sg_query_config(cfg) -> tuple[int, SgConfigInfo]:
    """Returns (status, info); info's LDS fields are filled even when the
    register / occupancy query needs a device that is not there."""
    c = cfg if isinstance(cfg, SgConfig) else SgConfig(*cfg)
    info = SgConfigInfo()
    st = lib().sg_query_config(ctypes.byref(c), ctypes.byref(info))
    return st, info


def sg_minimum_stages(copy_cycles: int, compute_cycles: int) -> int:
    return int(lib().sg_minimum_stages(copy_cycles, compute_cycles))


def sg_pipeline_wait_count(stages: int, loads_per_stage: int, ntile: int, k: int) -> int:
    return int(lib().sg_pipeline_wait_count(stages, loads_per_stage, ntile, k))


def sg_persistent_wait_count(stages: int, loads_per_stage: int, stores_per_tile: int, ntile: int,
                             total: int, q: int) -> int:
    return int(lib().sg_persistent_wait_count(stages, loads_per_stage, stores_per_tile, ntile,
                                              total, q))


def sg_status_string(status: int) -> str:
    return lib().sg_status_string(status).decode()


def configs() -> list[SgConfig]:
    return [sg_get_config(i) for i in range(sg_num_configs())]
