"""ctypes loader for libfa355.so (the C ABI declared in include/fa.h).

The library must have been built in-tree (``python -m exact_io_aware_19_amd.build``);
there is no fallback of any kind: a missing library raises.
"""

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfa355.so")

FA_OK = 0
# include/fa.h: bytes of the library-owned scratch array of fa_backward_noalloc, per GPU
NOALLOC_SCRATCH_BYTES = 16 << 20
STATUS_NAMES = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_SHAPE",
    -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_SCALE",
    -5: "FA_ERR_WORKSPACE",
    -6: "FA_ERR_LAUNCH",
    -7: "FA_ERR_ALIGN",
    -8: "FA_ERR_KVHEADS",
}

EXPORTED = (
    "fa_forward",
    "fa_forward_kvlen",
    "fa_backward_workspace_size",
    "fa_backward",
    "fa_backward_kvlen",
    "fa_backward_dq_pass",
    "fa_backward_dkdv_pass",
    "fa_backward_noalloc",
    "fa_forward_gqa",
    "fa_forward_offset",
    "fa_backward_gqa",
    "fa_backward_gqa_workspace_size",
    "fa_fp8_quantize_qk",
    "fa_fp8_quantize_v",
    "fa_forward_fp8",
    "fa_status_string",
)

_lib = None


def load():
    """Load libfa355.so once and declare the argument types of every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_19_amd.build` (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_kvlen.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.fa_forward_kvlen.restype = i
    lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_kvlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.fa_backward_kvlen.restype = i
    for name in ("fa_backward_dq_pass", "fa_backward_dkdv_pass"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp]
        fn.restype = i
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_forward_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp]
    lib.fa_forward_gqa.restype = i
    lib.fa_forward_offset.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp]
    lib.fa_forward_offset.restype = i
    lib.fa_backward_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, sz, vp]
    lib.fa_backward_gqa.restype = i
    lib.fa_backward_gqa_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_backward_gqa_workspace_size.restype = sz
    lib.fa_fp8_quantize_qk.argtypes = [vp, vp, vp, vp, f, i, i, i, i, vp]
    lib.fa_fp8_quantize_qk.restype = i
    lib.fa_fp8_quantize_v.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.fa_fp8_quantize_v.restype = i
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
    lib.fa_forward_fp8.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


class FAError(RuntimeError):
    def __init__(self, status, where):
        msg = load().fa_status_string(status).decode()
        super().__init__(f"{where} returned {status} ({msg})")
        self.status = status


def check(status, where):
    if status != FA_OK:
        raise FAError(status, where)
