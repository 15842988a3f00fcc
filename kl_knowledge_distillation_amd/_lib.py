"""ctypes view of the C ABI in include/kd_loss.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint32, c_void_p

# KD_LIBRARY may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("KD_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libkdloss.so")

# Status codes and enums (values fixed by include/kd_loss.h).
KD_OK, KD_ERR_NULL, KD_ERR_SHAPE, KD_ERR_DTYPE, KD_ERR_PARAM = 0, 1, 2, 3, 4
KD_ERR_ALIGN, KD_ERR_WORKSPACE, KD_ERR_UNSUPPORTED, KD_ERR_LABEL_RANGE, KD_ERR_HIP = 5, 6, 7, 8, 9
KD_ERR_SAVED = 10
KD_F32, KD_BF16 = 0, 1
KD_STUDENT_PROJECTION, KD_STUDENT_LOGITS = 0, 1
KD_TEACHER_TIED, KD_TEACHER_SEPARATE, KD_TEACHER_TOPK, KD_TEACHER_LOGITS = 1, 2, 3, 4
KD_REDUCE_MEAN, KD_REDUCE_SUM, KD_REDUCE_NONE = 0, 1, 2
KD_KL_FORWARD, KD_KL_REVERSE, KD_KL_JEFFREYS = 0, 1, 2
KERNELS = ["prep", "fwd", "merge", "finalize", "bwd_dz", "scatter", "gemm_dw", "gemm_dh",
           "gemm_dwdh", "bwd_kept"]
KERNEL_ID = {k: i for i, k in enumerate(KERNELS)}


class KdStudent(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("dtype", c_int32), ("n", c_int64), ("d", c_int64),
                ("v", c_int64), ("hidden", c_void_p), ("weight", c_void_p), ("logits", c_void_p)]


class KdTeacher(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("k", c_int32), ("d_t", c_int64), ("hidden", c_void_p),
                ("weight", c_void_p), ("topk_idx", c_void_p), ("topk_prob", c_void_p),
                ("logits", c_void_p)]


class KdParams(ctypes.Structure):
    _fields_ = [("student_ce_weight", c_float), ("teacher_ce_weight", c_float),
                ("kl_weight", c_float), ("temperature", c_float), ("ignore_index", c_int64),
                ("reduction", c_int32), ("normalizer", c_float), ("vocab_chunk", c_int64),
                ("assume_valid_labels", c_int32), ("kl_divergence", c_int32),
                ("teacher_temperature", c_float), ("compact_valid", c_int32),
                ("keep_last_chunk", c_int32), ("saved_bytes", c_int64),
                ("kl_output_unscaled", c_int32), ("dh_dtype", c_int32), ("dw_dtype", c_int32)]


class KdOutputs(ctypes.Structure):
    _fields_ = [("loss", c_void_p), ("student_ce", c_void_p), ("teacher_ce", c_void_p),
                ("kl", c_void_p)]


class KdTrace(ctypes.Structure):
    _fields_ = [("events", POINTER(c_void_p)), ("kinds", POINTER(c_int32)),
                ("capacity", c_int32), ("count", c_int32), ("mask", c_uint32)]


EXPORTS = {
    "kd_workspace_bytes": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                                     c_int32, POINTER(c_size_t)]),
    "kd_saved_bytes": (c_size_t, [c_int64]),
    "kd_saved_bytes_for": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                                     POINTER(c_size_t)]),
    "kd_loss_fwd": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                              c_void_p, POINTER(KdOutputs), c_void_p, c_void_p, c_size_t,
                              c_void_p, POINTER(KdTrace)]),
    "kd_loss_fwd_noalloc": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                                      c_void_p, POINTER(KdOutputs), c_void_p, c_void_p, c_void_p,
                                      POINTER(KdTrace)]),
    "kd_loss_bwd": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                              c_void_p, c_size_t, c_void_p, POINTER(KdTrace)]),
    "kd_loss_bwd_logits": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                     POINTER(KdTrace)]),
    "kd_loss_bwd_teacher": (c_int32, [POINTER(KdStudent), POINTER(KdTeacher), POINTER(KdParams),
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                      c_void_p, c_size_t, c_void_p, POINTER(KdTrace)]),
    "kd_read_status": (c_int32, [c_void_p, c_void_p, POINTER(c_int32)]),
    "kd_status_string": (c_char_p, [c_int32]),
    "kd_device_supported": (c_int32, [c_int32]),
    "kd_events_create": (c_int32, [POINTER(c_void_p), c_int32]),
    "kd_events_destroy": (c_int32, [POINTER(c_void_p), c_int32]),
    "kd_event_elapsed_ms": (c_int32, [c_void_p, c_void_p, POINTER(c_float)]),
    "kd_version": (c_char_p, []),
}

_lib = None


class KdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().kd_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def load():
    """Load libkdloss.so once. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m kl_knowledge_distillation_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != KD_OK:
        raise KdError(status, where)
