"""ctypes view of libswiglu_mlp.so (declarations in include/swiglu_mlp.h)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libswiglu_mlp.so")

BF16, FP16, FP32 = 0, 1, 2
STATUS = {
    0: "SWIGLU_OK", 1: "SWIGLU_ERR_NULL", 2: "SWIGLU_ERR_SHAPE", 3: "SWIGLU_ERR_DTYPE",
    4: "SWIGLU_ERR_ALIGN", 5: "SWIGLU_ERR_ALIAS", 6: "SWIGLU_ERR_WORKSPACE",
    7: "SWIGLU_ERR_DEVICE", 8: "SWIGLU_ERR_LAUNCH", 9: "SWIGLU_ERR_FLAGS", 10: "SWIGLU_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 << 20
FLAG_TWO_ROUND = 1
FLAG_LINEAR_WEIGHTS = 2
NUM_STAGES = 10
STAGE_NAMES = ("gateup_swiglu", "down_proj", "dgu_inplace", "dwd", "dwgu", "dx",
               "infer_gateup", "infer_down", "dwd+dgu", "dwgu+dx")

_lib = None


class SwiGLUError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().swiglu_mlp_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


def lib():
    """Load the library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m backward_gate_up_amd.build` "
            "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.swiglu_mlp_saved_bytes.argtypes = [i64, i64, i32]
    L.swiglu_mlp_saved_bytes.restype = sz
    L.swiglu_mlp_infer_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.swiglu_mlp_infer_workspace_bytes.restype = sz
    L.swiglu_mlp_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.swiglu_mlp_bwd_workspace_bytes.restype = sz
    L.swiglu_mlp_fwd.argtypes = [vp] * 6 + [i64] * 3 + [i32, vp]
    L.swiglu_mlp_fwd.restype = i32
    L.swiglu_mlp_bwd.argtypes = [vp] * 11 + [sz] + [i64] * 3 + [i32, vp]
    L.swiglu_mlp_bwd.restype = i32
    L.swiglu_mlp_bwd_ex.argtypes = [vp] * 11 + [sz] + [i64] * 3 + [i32, ctypes.c_uint, vp]
    L.swiglu_mlp_bwd_ex.restype = i32
    L.swiglu_mlp_infer.argtypes = [vp] * 6 + [sz] + [i64] * 3 + [i32, vp]
    L.swiglu_mlp_infer.restype = i32
    u32 = ctypes.c_uint
    L.swiglu_mlp_fwd_ex.argtypes = [vp] * 6 + [i64] * 3 + [i32, u32, vp]
    L.swiglu_mlp_fwd_ex.restype = i32
    L.swiglu_mlp_infer_ex.argtypes = [vp] * 6 + [sz] + [i64] * 3 + [i32, u32, vp]
    L.swiglu_mlp_infer_ex.restype = i32
    L.swiglu_mlp_infer_noalloc.argtypes = [vp] * 5 + [i64] * 3 + [i32, u32, vp]
    L.swiglu_mlp_infer_noalloc.restype = i32
    L.swiglu_mlp_status_string.argtypes = [i32]
    L.swiglu_mlp_status_string.restype = ctypes.c_char_p
    L.swiglu_mlp_timer_start.argtypes = [i32]
    L.swiglu_mlp_timer_start.restype = i32
    L.swiglu_mlp_timer_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), i32]
    L.swiglu_mlp_timer_stop.restype = i32
    _lib = L
    return L
