"""ctypes declarations of the C ABI in include/wts.h (argument marshalling only).

Every computation happens in libwts.so (HIP, gfx950).  Importing this module
loads the library and raises ImportError if it has not been built; there is
no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwts.so")

WTS_OK = 0
STATUS_NAMES = {0: "WTS_OK", 1: "WTS_ERR_INVALID_ARG", 2: "WTS_ERR_UNSUPPORTED", 3: "WTS_ERR_NO_MEMORY",
                4: "WTS_ERR_DEVICE", 5: "WTS_ERR_TIMEOUT", 6: "WTS_ERR_TOKEN_RANGE"}
HEAD = {"markov": 0, "recurrent": 1}
WTYPE = {"int8": 0, "bf16": 1}
EXEC = {"resident": 0, "stream": 1, "stepwise": 2}
WALK_FIXED_LATENT = 1
WALK_STRESS = 2

EXPORTS = ["wts_create", "wts_walk", "wts_destroy", "wts_get_error", "wts_get_plan", "wts_status_string",
           "wts_check_log_ratio", "wts_walk_noalloc"]
NOALLOC_LSE_BYTES = 1 << 20
# include/wts_roofline.h (measured roofline denominators)
ROOFLINE_EXPORTS = ["wts_roofline"]

c_int32, c_uint64, c_void_p = ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p


class CreateParams(ctypes.Structure):
    _fields_ = [("V", c_int32), ("r", c_int32), ("head", c_int32), ("wtype", c_int32),
                ("W", c_void_p), ("w_scale", c_void_p), ("E", c_void_p), ("A", c_void_p), ("c", c_void_p),
                ("max_batch", c_int32), ("max_steps", c_int32), ("resident_tiles", c_int32),
                ("lds_tiles", c_int32), ("device", c_int32), ("cooperative", c_int32),
                ("watchdog_us", c_int32), ("grid", c_int32), ("exchange", c_int32)]


class WalkParams(ctypes.Structure):
    _fields_ = [("B", c_int32), ("gamma", c_int32), ("step_offset", c_int32), ("temperature", c_int32),
                ("seed", c_uint64), ("base", c_void_p), ("x0", c_void_p), ("h0", c_void_p),
                ("tokens_out", c_void_p), ("logits_out", c_void_p), ("state_out", c_void_p),
                ("exec", c_int32), ("flags", c_int32), ("stream", c_void_p), ("trace_out", c_void_p),
                ("lse_out", c_void_p), ("winners_out", c_void_p)]


class Plan(ctypes.Structure):
    _fields_ = [("grid", c_int32), ("waves", c_int32), ("tiles", c_int32), ("tiles_per_wave", c_int32),
                ("reg_tiles", c_int32), ("lds_tiles", c_int32), ("stream_tiles", c_int32),
                ("resident_bytes", ctypes.c_int64), ("streamed_bytes", ctypes.c_int64),
                ("w_bytes", ctypes.c_int64), ("exchange", c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class RooflineResult(ctypes.Structure):
    _fields_ = [("grid", c_int32), ("pad", c_int32), ("lds_read_GBps", ctypes.c_double),
                ("mfma_i8_TOPs", ctypes.c_double), ("mfma_bf16_TFLOPs", ctypes.c_double),
                ("clock_MHz", ctypes.c_double), ("hbm_read_GBps", ctypes.c_double),
                ("mall_read_GBps", ctypes.c_double), ("exchange_us", ctypes.c_double * 6),
                ("exchange_bad", ctypes.c_int64 * 6), ("hop_xcd_us", ctypes.c_double),
                ("hop_device_us", ctypes.c_double), ("valu_dep_cycles", ctypes.c_double),
                ("valu_indep_cycles", ctypes.c_double), ("valu_indep_2w_cycles", ctypes.c_double),
                ("valu_indep_4w_cycles", ctypes.c_double), ("dot4_2w_cycles", ctypes.c_double)]

    def as_dict(self):
        out = {}
        for k, _ in self._fields_:
            v = getattr(self, k)
            out[k] = list(v) if hasattr(v, "__len__") else v
        out.pop("pad")
        return out


class WtsError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        super().__init__(f"{what}: {STATUS_NAMES.get(code, code)}")


def load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run python -m serial_draft_head_persistent_amd.build")
    # torch ships its own HIP runtime, referenced by a different file name but
    # with the same soname as the system one libwts.so links.  Loading torch
    # first makes libwts.so bind to that already-loaded runtime, so the
    # process has one HIP runtime and torch's device pointers and streams are
    # valid in the library.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.wts_create.argtypes = [P(CreateParams), P(c_void_p)]
    lib.wts_create.restype = ctypes.c_int
    lib.wts_walk.argtypes = [c_void_p, P(WalkParams)]
    lib.wts_walk.restype = ctypes.c_int
    lib.wts_walk_noalloc.argtypes = [c_void_p, P(WalkParams)]
    lib.wts_walk_noalloc.restype = ctypes.c_int
    lib.wts_destroy.argtypes = [c_void_p]
    lib.wts_destroy.restype = None
    lib.wts_get_error.argtypes = [c_void_p, ctypes.c_int]
    lib.wts_get_error.restype = ctypes.c_int
    lib.wts_get_plan.argtypes = [c_void_p, c_int32, c_int32, c_int32, P(Plan)]
    lib.wts_get_plan.restype = ctypes.c_int
    lib.wts_status_string.argtypes = [ctypes.c_int]
    lib.wts_status_string.restype = ctypes.c_char_p
    lib.wts_check_log_ratio.argtypes = [c_int32, P(ctypes.c_int64)]
    lib.wts_check_log_ratio.restype = ctypes.c_int
    lib.wts_roofline.argtypes = [c_int32, P(RooflineResult)]
    lib.wts_roofline.restype = ctypes.c_int
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib
