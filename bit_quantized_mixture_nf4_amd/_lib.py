"""ctypes view of ``libe4b.so`` (the C ABI declared in include/e4b.h).

Only argument marshalling lives here: every step of the path runs in the HIP
library. Loading fails loudly when the library has not been built.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libe4b.so")

# status codes (e4b_status)
E4B_OK = 0
E4B_ERR_NULL = 1
E4B_ERR_SHAPE = 2
E4B_ERR_BLOCKSIZE = 3
E4B_ERR_CODEBOOK = 4
E4B_ERR_DTYPE = 5
E4B_ERR_WORKSPACE = 6
E4B_ERR_ALIGN = 7
E4B_ERR_PATH = 8
E4B_ERR_HIP = 9

E4B_CB_NF4, E4B_CB_FP4, E4B_CB_BF16, E4B_CB_MXFP4, E4B_CB_INT8, E4B_CB_FP8 = 0, 1, 2, 3, 4, 5
E4B_F32, E4B_BF16 = 0, 1
E4B_PATH_AUTO, E4B_PATH_GROUPED, E4B_PATH_DECODE, E4B_PATH_MX8 = 0, 1, 2, 3

# every function declared in include/e4b.h
EXPORTS = (
    "e4b_quantize_nf4",
    "e4b_quantize_mxfp4",
    "e4b_mx8_rows",
    "e4b_dequantize_nf4",
    "e4b_moe_forward",
    "e4b_moe_dgrad",
    "e4b_moe_workspace_bytes",
    "e4b_moe_saved_bytes",
    "e4b_moe_lora_forward",
    "e4b_moe_lora_backward",
    "e4b_moe_lora_workspace_bytes",
    "e4b_stack_copy_async",
    "e4b_status_string",
    "e4b_moe_forward_timed",
    "e4b_moe_dgrad_timed",
    "e4b_moe_perm_layout",
    "e4b_moe_forward_noalloc",
)

# bytes of the per-GPU array that e4b_moe_forward_noalloc uses as its workspace
NOALLOC_SCRATCH_BYTES = 32 << 20

# e4b_kernel ids (the slots of e4b_kernel_events)
KERNELS = {
    "gate_up_fwd": 0,
    "down_fwd": 1,
    "down_dgrad": 2,
    "gate_up_dgrad": 3,
    "decode_gate_up": 4,
    "decode_down": 5,
    "route": 6,
    "permute": 7,
    "combine": 8,
    "combine_dgrad": 9,
}
E4B_K_COUNT = 10


class E4bStack(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("E", ctypes.c_int64),
        ("out", ctypes.c_int64),
        ("in_", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("codebook", ctypes.c_int32),
        ("scales", ctypes.c_void_p),
    ]


class E4bLayer(ctypes.Structure):
    _fields_ = [("gate_up", E4bStack), ("down", E4bStack)]


class E4bLora(ctypes.Structure):
    _fields_ = [
        ("A_gu", ctypes.c_void_p),
        ("B_gu", ctypes.c_void_p),
        ("A_dn", ctypes.c_void_p),
        ("B_dn", ctypes.c_void_p),
        ("r", ctypes.c_int32),
        ("alpha", ctypes.c_float),
    ]


class E4bKernelEvents(ctypes.Structure):
    """e4b_kernel_events: start / stop hipEvent_t per kernel id (NULL: not timed)."""

    _fields_ = [("start", ctypes.c_void_p * E4B_K_COUNT), ("stop", ctypes.c_void_p * E4B_K_COUNT)]


class E4bPermLayout(ctypes.Structure):
    _fields_ = [
        ("counts", ctypes.c_size_t),
        ("offsets", ctypes.c_size_t),
        ("tile_offsets", ctypes.c_size_t),
        ("sorted_pair", ctypes.c_size_t),
        ("pos_of_pair", ctypes.c_size_t),
        ("tile_map", ctypes.c_size_t),
        ("m_tiles_bound", ctypes.c_int64),
    ]


_lib = None


def load():
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bit_quantized_mixture_nf4_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    st, lay, lo = ctypes.POINTER(E4bStack), ctypes.POINTER(E4bLayer), ctypes.POINTER(E4bLora)
    sigs = {
        "e4b_quantize_nf4": (i32, [vp, i64, i64, i64, i32, i32, vp, vp, vp]),
        "e4b_quantize_mxfp4": (i32, [vp, i64, i64, i64, vp, vp, vp]),
        "e4b_mx8_rows": (i32, [vp, i64, i64, vp, vp, vp]),
        "e4b_dequantize_nf4": (i32, [st, i32, vp, vp]),
        "e4b_moe_forward": (i32, [lay, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, i32, vp]),
        "e4b_moe_dgrad": (i32, [lay, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "e4b_moe_workspace_bytes": (sz, [lay, i64, i32]),
        "e4b_moe_saved_bytes": (sz, [lay, i64, i32]),
        "e4b_moe_lora_forward": (i32, [lay, lo, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "e4b_moe_lora_backward": (
            i32, [lay, lo, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "e4b_moe_lora_workspace_bytes": (sz, [lay, i64, i32]),
        "e4b_stack_copy_async": (i32, [st, st, vp]),
        "e4b_status_string": (ctypes.c_char_p, [i32]),
        "e4b_moe_forward_timed": (
            i32, [lay, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, i32, vp, ctypes.POINTER(E4bKernelEvents)]),
        "e4b_moe_dgrad_timed": (
            i32, [lay, i64, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(E4bKernelEvents)]),
        "e4b_moe_perm_layout": (i32, [lay, i64, i32, ctypes.POINTER(E4bPermLayout)]),
        "e4b_moe_forward_noalloc": (i32, [lay, i64, i32, vp, vp, vp, vp, vp, vp, i32, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code):
    return load().e4b_status_string(code).decode()


class E4bError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed with status {code}: {status_string(code)}")


def check(fn, code):
    if code != E4B_OK:
        if code == E4B_ERR_HIP:
            raise E4bError(fn, code)
        raise ValueError(f"{fn}: status {code}: {status_string(code)}")
