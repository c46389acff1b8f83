"""ctypes binding of libfp8bl.so: argument marshalling only.

Tensors are torch tensors on a HIP device; only their data pointers, sizes
and the current stream cross into the library. No arithmetic of the method
happens here. If the shared library has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfp8bl.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG_DIR), "include", "fp8bl.h")

FP8BL_OK = 0
FP8BL_INVALID_ARG = 1
FP8BL_ALIGNMENT = 2
FP8BL_WORKSPACE = 3
FP8BL_UNSUPPORTED_DEVICE = 4
FP8BL_HIP_ERROR = 5

PATH_AUTO = 0
PATH_TILED = 1
PATH_SKINNY = 2
PATH_LARGE = 3

_lib = None


class Fp8blError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libfp8bl.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m block_scaled_fp8_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.fp8_block_abi_version.restype = c_int
    lib.fp8_block_abi_version.argtypes = []
    lib.fp8_block_status_string.restype = ctypes.c_char_p
    lib.fp8_block_status_string.argtypes = [c_int]
    lib.fp8_block_device_supported.restype = c_int
    lib.fp8_block_device_supported.argtypes = [c_int]
    lib.fp8_block_dequant.restype = c_int
    lib.fp8_block_dequant.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fp8_block_linear_workspace_size.restype = sz
    lib.fp8_block_linear_workspace_size.argtypes = [i64, i64, i64]
    lib.fp8_block_linear.restype = c_int
    lib.fp8_block_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    lib.fp8_block_linear_ex.restype = c_int
    lib.fp8_block_linear_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, c_int, vp]
    lib.fp8_block_linear_noalloc.restype = c_int
    lib.fp8_block_linear_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_block_mlp_gate_up.restype = c_int
    lib.fp8_block_mlp_gate_up.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.fp8_block_mlp_gate_up_ex.restype = c_int
    lib.fp8_block_mlp_gate_up_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, c_int, vp]
    lib.fp8_act_quantize.restype = c_int
    lib.fp8_act_quantize.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fp8_block_linear_w8a8_workspace_size.restype = sz
    lib.fp8_block_linear_w8a8_workspace_size.argtypes = [i64, i64, i64]
    lib.fp8_block_linear_w8a8.restype = c_int
    lib.fp8_block_linear_w8a8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    lib.fp8_block_linear_w8a8_ex.restype = c_int
    lib.fp8_block_linear_w8a8_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, c_int, vp]
    lib.fp8_block_linear_w8a8_bf16.restype = c_int
    lib.fp8_block_linear_w8a8_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    lib.fp8_block_quantize.restype = c_int
    lib.fp8_block_quantize.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fp8_block_quantize_bf16.restype = c_int
    lib.fp8_block_quantize_bf16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.fp8_block_stream_read.restype = c_int
    lib.fp8_block_stream_read.argtypes = [vp, sz, vp, c_int, vp]
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/fp8bl.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fp8_\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return load().fp8_block_status_string(int(status)).decode()


def abi_version() -> int:
    return load().fp8_block_abi_version()


def device_supported(device: int = 0) -> bool:
    return bool(load().fp8_block_device_supported(int(device)))


def workspace_size(m: int, n: int, k: int) -> int:
    return int(load().fp8_block_linear_workspace_size(int(m), int(n), int(k)))


# Raw pointer-level calls (ints are device addresses); used by the tensor API
# below and by tests that exercise argument checking without a device.

def dequant_raw(q: int, s: int, w: int, n: int, k: int, stream: int = 0) -> int:
    return load().fp8_block_dequant(q, s, w, n, k, stream)


def linear_raw(x: int, q: int, s: int, y: int, m: int, n: int, k: int,
               ws: int, ws_bytes: int, path: int = PATH_AUTO, stream: int = 0) -> int:
    return load().fp8_block_linear_ex(x, q, s, y, m, n, k, ws, ws_bytes, path, stream)


def linear_noalloc_raw(x: int, q: int, s: int, y: int, m: int, n: int, k: int,
                       stream: int = 0) -> int:
    return load().fp8_block_linear_noalloc(x, q, s, y, m, n, k, stream)


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def mlp_gate_up_raw(x: int, qg: int, sg: int, qu: int, su: int, h: int,
                    m: int, n: int, k: int, stream: int = 0) -> int:
    return load().fp8_block_mlp_gate_up(x, qg, sg, qu, su, h, m, n, k, stream)


def mlp_gate_up_ex_raw(x: int, qg: int, sg: int, qu: int, su: int, h: int,
                       m: int, n: int, k: int, path: int, stream: int = 0) -> int:
    return load().fp8_block_mlp_gate_up_ex(x, qg, sg, qu, su, h, m, n, k, path, stream)


def act_quantize_raw(x: int, xq: int, xs: int, m: int, k: int, stream: int = 0) -> int:
    return load().fp8_act_quantize(x, xq, xs, m, k, stream)


def w8a8_workspace_size(m: int, n: int, k: int) -> int:
    return int(load().fp8_block_linear_w8a8_workspace_size(int(m), int(n), int(k)))


def linear_w8a8_raw(xq: int, xs: int, q: int, s: int, y: int, m: int, n: int, k: int,
                    ws: int, ws_bytes: int, stream: int = 0) -> int:
    return load().fp8_block_linear_w8a8(xq, xs, q, s, y, m, n, k, ws, ws_bytes, stream)


def linear_w8a8_ex_raw(xq: int, xs: int, q: int, s: int, y: int, m: int, n: int, k: int,
                       ws: int, ws_bytes: int, path: int, stream: int = 0) -> int:
    return load().fp8_block_linear_w8a8_ex(xq, xs, q, s, y, m, n, k, ws, ws_bytes, path, stream)


def linear_w8a8_bf16_raw(x: int, q: int, s: int, y: int, m: int, n: int, k: int,
                         ws: int, ws_bytes: int, stream: int = 0) -> int:
    return load().fp8_block_linear_w8a8_bf16(x, q, s, y, m, n, k, ws, ws_bytes, stream)


def quantize_raw(w: int, q: int, s: int, n: int, k: int, stream: int = 0) -> int:
    return load().fp8_block_quantize(w, q, s, n, k, stream)


def quantize_bf16_raw(w: int, q: int, s: int, n: int, k: int, stream: int = 0) -> int:
    return load().fp8_block_quantize_bf16(w, q, s, n, k, stream)


def stream_read_raw(buf: int, nbytes: int, sink: int, blocks: int, stream: int = 0) -> int:
    return load().fp8_block_stream_read(buf, nbytes, sink, blocks, stream)
