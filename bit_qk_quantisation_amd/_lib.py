"""ctypes view of libbinattn.so: declarations only, no compute."""

from __future__ import annotations

import ctypes
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libbinattn.so"

# Every symbol that include/binattn.h declares.
EXPORTS = (
    "ba_version", "ba_status_string", "ba_last_error", "ba_pack_words",
    "ba_pack_signs", "ba_workspace_bytes", "ba_attention_fwd", "ba_attention_fwd_strided",
    "ba_attention_fwd_dense_bias", "ba_attention_fwd_dense_bias_prepared", "ba_attention_prepare",
    "ba_workspace_bytes_int8pv", "ba_attention_fwd_int8pv", "ba_workspace_bytes_bwd", "ba_attention_bwd",
    "ba_attention_fwd_prepared", "ba_qk_int_dot", "ba_attention_fwd_train", "ba_attention_bwd_saved",
    "ba_attention_fwd_static",
)

STATUS = {0: "BA_OK", 1: "BA_ERR_NULL", 2: "BA_ERR_SHAPE", 3: "BA_ERR_UNSUPPORTED",
          4: "BA_ERR_ALIGN", 5: "BA_ERR_WORKSPACE", 6: "BA_ERR_HIP"}

ROUTE_MFMA_FP4 = 0
ROUTE_VALU_POPCOUNT = 1
ROUTE_MFMA_INT8 = 2
QK_ROWSUM = 0x100

_lib = None


class BinAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load(path=None) -> ctypes.CDLL:
    """Load (once) and declare the C ABI.  Raises if the library is missing:
    there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = pathlib.Path(path) if path else LIB_PATH
    if not p.exists():
        raise ImportError(
            f"{p} is missing: build it with `python -m bit_qk_quantisation_amd.build`")
    lib = ctypes.CDLL(str(p))
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.ba_version.restype = i32
    lib.ba_version.argtypes = []
    lib.ba_status_string.restype = ctypes.c_char_p
    lib.ba_status_string.argtypes = [i32]
    lib.ba_last_error.restype = ctypes.c_char_p
    lib.ba_last_error.argtypes = []
    lib.ba_pack_words.restype = i32
    lib.ba_pack_words.argtypes = [i32]
    lib.ba_pack_signs.restype = i32
    lib.ba_pack_signs.argtypes = [vp, i64, i64, i64, i32, vp, vp, vp]
    lib.ba_workspace_bytes.restype = sz
    lib.ba_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.ba_attention_fwd.restype = i32
    lib.ba_attention_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32,
                                     ctypes.c_float, vp, vp, sz, vp]
    lib.ba_attention_fwd_strided.restype = i32
    lib.ba_attention_fwd_strided.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32,
                                             ctypes.c_float, vp, ctypes.POINTER(ctypes.c_int64),
                                             vp, sz, vp]
    lib.ba_attention_fwd_dense_bias.restype = i32
    lib.ba_attention_fwd_dense_bias.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32,
                                                ctypes.c_float, vp, ctypes.POINTER(ctypes.c_int64),
                                                vp, sz, vp]
    lib.ba_attention_fwd_dense_bias_prepared.restype = i32
    lib.ba_attention_fwd_dense_bias_prepared.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i32,
                                                         ctypes.c_float, vp, vp, sz, vp]
    lib.ba_workspace_bytes_int8pv.restype = sz
    lib.ba_workspace_bytes_int8pv.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.ba_attention_fwd_int8pv.restype = i32
    lib.ba_attention_fwd_int8pv.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32,
                                            ctypes.c_float, vp, vp, sz, vp]
    lib.ba_workspace_bytes_bwd.restype = sz
    lib.ba_workspace_bytes_bwd.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.ba_attention_bwd.restype = i32
    lib.ba_attention_bwd.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, ctypes.c_float, vp,
                                     vp, vp, vp, vp, vp, sz, vp]
    lib.ba_attention_fwd_train.restype = i32
    lib.ba_attention_fwd_train.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, ctypes.c_float,
                                           vp, vp, vp, sz, vp]
    lib.ba_attention_bwd_saved.restype = i32
    lib.ba_attention_bwd_saved.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, ctypes.c_float,
                                           vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ba_attention_prepare.restype = i32
    lib.ba_attention_prepare.argtypes = [vp, vp, vp, i32, i32, i64, i64, i64, i32, vp, sz, vp]
    lib.ba_attention_fwd_prepared.restype = i32
    lib.ba_attention_fwd_prepared.argtypes = [vp, vp, i32, i32, i64, i64, i64, i32, ctypes.c_float,
                                              vp, vp, sz, vp]
    lib.ba_attention_fwd_static.restype = i32
    lib.ba_attention_fwd_static.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, ctypes.c_float, vp, vp]
    lib.ba_qk_int_dot.restype = i32
    lib.ba_qk_int_dot.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp, vp]
    if path is None:
        _lib = lib
    return lib


def check(lib: ctypes.CDLL, status: int) -> None:
    if status != 0:
        raise BinAttnError(status, lib.ba_last_error().decode(errors="replace"))
