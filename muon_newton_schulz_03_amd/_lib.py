"""ctypes view of the C ABI declared in include/muon.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon_mi355x.so")

MUON_OK = 0
MUON_E_INVAL = -1
MUON_E_UNSUPPORTED = -2
MUON_E_MISMATCH = -3
MUON_E_WORKSPACE = -4
MUON_SCRATCH_BYTES = 64 << 20
MUON_E_HIP = -5

MUON_DTYPE_F32 = 0
MUON_DTYPE_BF16 = 1
MUON_PATH_BF16 = 0
MUON_PATH_F32 = 1

KIND_MOMENTUM, KIND_GRAM, KIND_POLY, KIND_UPDATE, KIND_APPLY, KIND_NORM, KIND_FUSED = range(7)
KIND_COUNT = 7
KIND_NAMES = ("momentum", "gram", "poly", "update", "apply", "norm", "fused")

EXPORTS = ("muon_version", "muon_workspace_size", "muon_init", "muon_step", "muon_step_schedule", "muon_destroy",
           "muon_last_error", "muon_describe", "muon_profile_enable", "muon_profile_select", "muon_profile_read",
           "muon_step_scratch", "muon_check", "muon_fused_limits")


class MatrixDesc(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld_w", ctypes.c_int64),
                ("ld_g", ctypes.c_int64), ("w_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("reserved", ctypes.c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("x_master_iters", ctypes.c_int32),
                ("zero_momentum", ctypes.c_int32), ("max_T", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("fused", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_int64), ("n_matrices", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("blocks", ctypes.c_int32 * KIND_COUNT), ("x_master_iters", ctypes.c_int32),
                ("path", ctypes.c_int32), ("n_f32_matrices", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("bf16_tile_rows", ctypes.c_int32), ("bf16_tile_cols", ctypes.c_int32), ("fused", ctypes.c_int32)]


class MuonError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"muon error {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree build of the library (fails loudly if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with `python -m muon_newton_schulz_03_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.muon_version.restype = ctypes.c_char_p
    lib.muon_version.argtypes = []
    lib.muon_last_error.restype = ctypes.c_char_p
    lib.muon_last_error.argtypes = []
    lib.muon_workspace_size.restype = ctypes.c_size_t
    lib.muon_workspace_size.argtypes = [P(MatrixDesc), ctypes.c_int, P(Options)]
    lib.muon_init.restype = ctypes.c_int
    lib.muon_init.argtypes = [P(MatrixDesc), ctypes.c_int, P(Options), ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_void_p, P(ctypes.c_void_p)]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step.argtypes = [ctypes.c_void_p, P(MatrixDesc), ctypes.c_int, ctypes.c_float, ctypes.c_float,
                              ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                              ctypes.c_void_p]
    lib.muon_step_schedule.restype = ctypes.c_int
    lib.muon_step_schedule.argtypes = [ctypes.c_void_p, P(MatrixDesc), ctypes.c_int, P(ctypes.c_float), ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
    lib.muon_step_scratch.restype = ctypes.c_int
    lib.muon_step_scratch.argtypes = [P(MatrixDesc), ctypes.c_int, P(Options), ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_void_p]
    lib.muon_destroy.restype = ctypes.c_int
    lib.muon_destroy.argtypes = [ctypes.c_void_p]
    lib.muon_describe.restype = ctypes.c_int
    lib.muon_describe.argtypes = [P(MatrixDesc), ctypes.c_int, P(Options), P(PlanInfo), ctypes.c_int,
                                  P(ctypes.c_int32), ctypes.c_int, P(ctypes.c_int32)]
    lib.muon_profile_enable.restype = ctypes.c_int
    lib.muon_profile_enable.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.muon_profile_select.restype = ctypes.c_int
    lib.muon_profile_select.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
    lib.muon_profile_read.restype = ctypes.c_int
    lib.muon_profile_read.argtypes = [ctypes.c_void_p, P(ctypes.c_double), P(ctypes.c_int64)]
    lib.muon_check.restype = ctypes.c_int
    lib.muon_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.muon_fused_limits.restype = ctypes.c_int
    lib.muon_fused_limits.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != MUON_OK:
        raise MuonError(code, load().muon_last_error().decode())


def last_error() -> str:
    return load().muon_last_error().decode()
