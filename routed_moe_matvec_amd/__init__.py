"""Python binding of libqgemv -- argument marshalling only.

Every function has the name and argument order of the C entry point declared
in ``include/qgemv.h``; device buffers are passed as torch tensors in the
pointer positions (their ``data_ptr()`` is handed to the library) and the
stream defaults to torch's current stream on the tensors' device.  All
arithmetic happens in the HIP kernels of ``libqgemv.so``: if the library is
missing this module raises at import time; nothing falls back to another path.

A negative status from the library raises :class:`QGError`.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QGError", "FMT_Q8_0", "FMT_Q4K", "library_path", "quantize_act_q8", "qgemv_q8_0", "qgemv_q4k",
    "qgemv_paired", "moe_routed_workspace_bytes", "moe_routed_workspace_layout", "moe_routed_qgemv",
    "qgemm_prefill", "qg_status_string", "qgemv_debug_block_isums", "pointer_table", "WS_REGIONS",
    "qgemv_q8_0_f32", "qgemv_q4k_f32", "qgemv_paired_f32", "qgemm_prefill_workspace_bytes", "qgemm_prefill_ws",
    "qgemv_grouped", "qgemv_q8_0_quality", "FMT_FP8_E4M3_B128", "FMT_FP4_E2M1_MX", "qg_matrix_bytes", "qgemv_mx",
    "moe_routed_qgemv_fmt", "qgemm_q8_0", "qg_stream_read_bursts", "qg_stream_read", "moe_routed_qgemv_noalloc",
    "MOE_SCRATCH_BYTES",
]

FMT_Q8_0 = 0
FMT_Q4K = 1
FMT_FP8_E4M3_B128 = 2
FMT_FP4_E2M1_MX = 3
DEV_OK, DEV_BAD_EXPERT, DEV_NULL_EXPERT = 0, 1, 2
MAX_K, MAX_M, MAX_MOE_PAIRS, MAX_EXPERTS = 16384, 32, 8192, 4096
WS_REGIONS = ["NUNIQ", "UNIQ", "SLOT", "PAIR_OFF", "PAIRS", "G", "V", "H", "HQ", "HD", "HS", "O", "HOT"]
MOE_MM_PAIRS = 9  # QG_MOE_MM_PAIRS
MOE_SCRATCH_BYTES = 8 << 20  # QG_MOE_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqgemv.so")


def library_path() -> str:
    return _LIB_PATH


if not os.path.exists(_LIB_PATH):
    raise ImportError("libqgemv.so is not built (run __graft_entry__.build()); there is no fallback path")

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7).  It is
# loaded first, so that the library binds to it: with the system runtime loaded
# first, torch and the library would not share streams.
try:
    import torch  # noqa: F401
except ImportError:  # the library alone, on the system HIP runtime
    pass

_lib = ctypes.CDLL(_LIB_PATH)
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


def _sig(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_c_quantize = _sig("quantize_act_q8", _i, [_vp, _i, _i, _vp, _vp, _vp, _vp])
_c_q8_0 = _sig("qgemv_q8_0", _i, [_vp, _i, _i, _vp, _vp, _i, _vp, _vp])
_c_q4k = _sig("qgemv_q4k", _i, [_vp, _i, _i, _vp, _vp, _vp, _i, _vp, _vp])
_c_paired = _sig("qgemv_paired", _i, [_i, _vp, _i, _vp, _i, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp])
_c_grouped = _sig("qgemv_grouped", _i, [_i, _vp, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp])
_c_quality = _sig("qgemv_q8_0_quality", _i, [_vp, _i, _i, _vp, _i, _vp, _vp])
_c_isums = _sig("qgemv_debug_block_isums", _i, [_i, _vp, _i, _i, _vp, _i, _vp, _vp])
_c_q8_0_f32 = _sig("qgemv_q8_0_f32", _i, [_vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp])
_c_q4k_f32 = _sig("qgemv_q4k_f32", _i, [_vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp])
_c_paired_f32 = _sig("qgemv_paired_f32", _i, [_i, _vp, _i, _vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp])
_c_status = _sig("qg_status_string", ctypes.c_char_p, [_i])
_c_ws_bytes = _sig("moe_routed_workspace_bytes", _sz, [_i, _i, _i, _i, _i])
_c_ws_layout = _sig("moe_routed_workspace_layout", _i, [_i, _i, _i, _i, _i, _vp])
_c_moe = _sig("moe_routed_qgemv", _i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _sz, _vp, _vp])
_c_moe_fmt = _sig("moe_routed_qgemv_fmt", _i, [_i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _sz, _vp, _vp])
_c_matrix_bytes = _sig("qg_matrix_bytes", _sz, [_i, _i, _i])
_c_mx = _sig("qgemv_mx", _i, [_i, _vp, _i, _i, _vp, _vp, _i, _vp, _vp])
_c_qgemm_q8_0 = _sig("qgemm_q8_0", _i, [_vp, _i, _i, _vp, _vp, _i, _vp, _vp])
_c_prefill = _sig("qgemm_prefill", _i, [_i, _vp, _i, _i, _vp, _i, _vp, _vp])
_c_prefill_ws_bytes = _sig("qgemm_prefill_workspace_bytes", _sz, [_i, _i])
_c_prefill_ws = _sig("qgemm_prefill_ws", _i, [_i, _vp, _i, _i, _vp, _i, _vp, _vp, _sz, _vp])
_c_read_bursts = _sig("qg_stream_read_bursts", _sz, [_sz, _i])
_c_read = _sig("qg_stream_read", _i, [_vp, _sz, _i, _i, _vp, _sz, _vp])
_c_moe_noalloc = _sig("moe_routed_qgemv_noalloc", _i, [_i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                                      _vp, _vp, _vp, _vp])


class QGError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (what, qg_status_string(status), status))


def qg_status_string(status: int) -> str:
    return _c_status(int(status)).decode()


def _ptr(t):
    """Device pointer of a torch tensor (or None -> NULL)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        if not t.is_cuda:
            raise TypeError("libqgemv takes device tensors; got a tensor on %s" % t.device)
        if not t.is_contiguous():
            raise TypeError("libqgemv takes contiguous tensors")
        return t.data_ptr()
    return int(t)


def _stream(stream, *tensors):
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    for t in tensors:
        if t is not None and hasattr(t, "device"):
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _ok(rc: int, what: str):
    if rc != 0:
        raise QGError(rc, what)


def quantize_act_q8(x, M: int, K: int, qx, dx, sx, stream=None) -> None:
    _ok(_c_quantize(_ptr(x), M, K, _ptr(qx), _ptr(dx), _ptr(sx), _stream(stream, x)), "quantize_act_q8")


def qgemv_q8_0(W, N: int, K: int, qx, dx, M: int, y, stream=None) -> None:
    _ok(_c_q8_0(_ptr(W), N, K, _ptr(qx), _ptr(dx), M, _ptr(y), _stream(stream, W)), "qgemv_q8_0")


def qgemv_q4k(W, N: int, K: int, qx, dx, sx, M: int, y, stream=None) -> None:
    _ok(_c_q4k(_ptr(W), N, K, _ptr(qx), _ptr(dx), _ptr(sx), M, _ptr(y), _stream(stream, W)), "qgemv_q4k")


def qgemv_paired(fmt: int, W1, N1: int, W2, N2: int, K: int, qx, dx, sx, M: int, y1, y2, stream=None) -> None:
    _ok(_c_paired(fmt, _ptr(W1), N1, _ptr(W2), N2, K, _ptr(qx), _ptr(dx), _ptr(sx), M, _ptr(y1), _ptr(y2),
                  _stream(stream, W1)), "qgemv_paired")


def qgemv_grouped(fmt: int, W, G: int, N: int, K: int, qx, dx, sx, M: int, y, stream=None) -> None:
    _ok(_c_grouped(fmt, _ptr(W), G, N, K, _ptr(qx), _ptr(dx), _ptr(sx), M, _ptr(y), _stream(stream, W)),
        "qgemv_grouped")


def qgemv_q8_0_quality(W, N: int, K: int, x, M: int, y, stream=None) -> None:
    _ok(_c_quality(_ptr(W), N, K, _ptr(x), M, _ptr(y), _stream(stream, W)), "qgemv_q8_0_quality")


def qgemv_q8_0_f32(W, N: int, K: int, x, M: int, y, qx=None, dx=None, sx=None, stream=None) -> None:
    _ok(_c_q8_0_f32(_ptr(W), N, K, _ptr(x), M, _ptr(y), _ptr(qx), _ptr(dx), _ptr(sx), _stream(stream, W)),
        "qgemv_q8_0_f32")


def qgemv_q4k_f32(W, N: int, K: int, x, M: int, y, qx=None, dx=None, sx=None, stream=None) -> None:
    _ok(_c_q4k_f32(_ptr(W), N, K, _ptr(x), M, _ptr(y), _ptr(qx), _ptr(dx), _ptr(sx), _stream(stream, W)),
        "qgemv_q4k_f32")


def qgemv_paired_f32(fmt: int, W1, N1: int, W2, N2: int, K: int, x, M: int, y1, y2, qx=None, dx=None, sx=None,
                     stream=None) -> None:
    _ok(_c_paired_f32(fmt, _ptr(W1), N1, _ptr(W2), N2, K, _ptr(x), M, _ptr(y1), _ptr(y2), _ptr(qx), _ptr(dx),
                      _ptr(sx), _stream(stream, W1)), "qgemv_paired_f32")


def qgemv_debug_block_isums(fmt: int, W, N: int, K: int, qx, M: int, isum, stream=None) -> None:
    _ok(_c_isums(fmt, _ptr(W), N, K, _ptr(qx), M, _ptr(isum), _stream(stream, W)), "qgemv_debug_block_isums")


def moe_routed_workspace_bytes(T: int, topk: int, E: int, D: int, F: int) -> int:
    return int(_c_ws_bytes(T, topk, E, D, F))


def moe_routed_workspace_layout(T: int, topk: int, E: int, D: int, F: int) -> dict:
    offs = (ctypes.c_size_t * len(WS_REGIONS))()
    _ok(_c_ws_layout(T, topk, E, D, F, ctypes.cast(offs, ctypes.c_void_p)), "moe_routed_workspace_layout")
    return {name: int(offs[i]) for i, name in enumerate(WS_REGIONS)}


def pointer_table(tensors, device):
    """int64 device tensor holding the device addresses of `tensors` (None -> NULL)."""
    import torch
    addrs = [0 if t is None else _ptr(t) for t in tensors]
    return torch.tensor(addrs, dtype=torch.int64, device=device)


def moe_routed_qgemv(qx, dx, sx, T: int, D: int, F: int, E: int, topk: int, ids, rw, gate, up, down, y, ws,
                     ws_bytes: int, d_status, stream=None) -> None:
    _ok(_c_moe(_ptr(qx), _ptr(dx), _ptr(sx), T, D, F, E, topk, _ptr(ids), _ptr(rw), _ptr(gate), _ptr(up),
               _ptr(down), _ptr(y), _ptr(ws), ws_bytes, _ptr(d_status), _stream(stream, qx)), "moe_routed_qgemv")


def moe_routed_qgemv_fmt(fmt: int, qx, dx, sx, T: int, D: int, F: int, E: int, topk: int, ids, rw, gate, up, down,
                         y, ws, ws_bytes: int, d_status, stream=None) -> None:
    _ok(_c_moe_fmt(fmt, _ptr(qx), _ptr(dx), _ptr(sx), T, D, F, E, topk, _ptr(ids), _ptr(rw), _ptr(gate), _ptr(up),
                   _ptr(down), _ptr(y), _ptr(ws), ws_bytes, _ptr(d_status), _stream(stream, qx)),
        "moe_routed_qgemv_fmt")


def qg_matrix_bytes(fmt: int, N: int, K: int) -> int:
    return int(_c_matrix_bytes(fmt, N, K))


def qgemm_q8_0(W, N: int, K: int, qx, dx, M: int, y, stream=None) -> None:
    _ok(_c_qgemm_q8_0(_ptr(W), N, K, _ptr(qx), _ptr(dx), M, _ptr(y), _stream(stream, W)), "qgemm_q8_0")


def qgemv_mx(fmt: int, W, N: int, K: int, qx, dx, M: int, y, stream=None) -> None:
    _ok(_c_mx(fmt, _ptr(W), N, K, _ptr(qx), _ptr(dx), M, _ptr(y), _stream(stream, W)), "qgemv_mx")


def qgemm_prefill(fmt: int, W, N: int, K: int, x_bf16, M: int, y, stream=None) -> None:
    _ok(_c_prefill(fmt, _ptr(W), N, K, _ptr(x_bf16), M, _ptr(y), _stream(stream, W)), "qgemm_prefill")


def qgemm_prefill_workspace_bytes(M: int, K: int) -> int:
    return int(_c_prefill_ws_bytes(M, K))


def qgemm_prefill_ws(fmt: int, W, N: int, K: int, x_bf16, M: int, y, ws, ws_bytes: int, stream=None) -> None:
    _ok(_c_prefill_ws(fmt, _ptr(W), N, K, _ptr(x_bf16), M, _ptr(y), _ptr(ws), ws_bytes, _stream(stream, W)),
        "qgemm_prefill_ws")


def qg_stream_read_bursts(nbytes: int, chunk_kib: int) -> int:
    return int(_c_read_bursts(nbytes, chunk_kib))


def qg_stream_read(buf, nbytes: int, chunk_kib: int, waves: int, burst_xor, burst_xor_len: int, stream=None) -> None:
    _ok(_c_read(_ptr(buf), nbytes, chunk_kib, waves, _ptr(burst_xor), burst_xor_len, _stream(stream, buf)),
        "qg_stream_read")


def moe_routed_qgemv_noalloc(fmt: int, qx, dx, sx, T: int, D: int, F: int, E: int, topk: int, ids, rw, gate, up,
                             down, y, d_status, stream=None) -> None:
    _ok(_c_moe_noalloc(fmt, _ptr(qx), _ptr(dx), _ptr(sx), T, D, F, E, topk, _ptr(ids), _ptr(rw), _ptr(gate),
                       _ptr(up), _ptr(down), _ptr(y), _ptr(d_status), _stream(stream, qx)), "moe_routed_qgemv_noalloc")
