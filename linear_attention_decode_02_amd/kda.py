"""Python binding of the C-ABI library ``libkda_decode.so``.

Argument marshalling only: shapes, dtypes and device placement of torch
tensors are checked, pointers and sizes are handed to ``kda_decode`` (see
include/kda_decode.h for the operation), and the step runs in the HIP
kernel on the given (default: torch's current) stream.  There is no other
implementation behind this module: if the library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda_decode.so")

KDA_OK = 0
KDA_OUTPUT_NORM = 0x1
HEAD_DIM = 128
CONV_WIDTH = 4

_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_MISALIGNED", 4: "KDA_ERR_DEVICE", 5: "KDA_ERR_LAUNCH"}


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("norm_eps", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libkda_decode.so`` (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.kda_decode.restype = ctypes.c_int
        L.kda_decode.argtypes = [ctypes.POINTER(Dims)] + [P] * 11
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_decode_bytes.restype = ctypes.c_uint64
        L.kda_decode_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
        L.kda_state_stream_probe.restype = ctypes.c_int
        L.kda_state_stream_probe.argtypes = [P, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_float, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def decode_raw(dims: Dims, qkv, conv_w, conv_state, rec_state, g, beta, gate,
               norm_w, state_idx, out, stream) -> int:
    """Call ``kda_decode`` with raw integer pointers; returns the status."""
    return lib().kda_decode(ctypes.byref(dims), qkv, conv_w, conv_state,
                            rec_state, g, beta, gate, norm_w, state_idx, out,
                            stream)


def _check(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def kda_decode(qkv, conv_w, conv_state, rec_state, g, beta, gate, norm_w,
               state_idx, out, *, norm: bool = True, eps: float = 1e-5,
               stream=None) -> None:
    """One fused KDA decode step (in place on ``conv_state``/``rec_state``).

    qkv bf16 [B, 3C]; conv_w fp32 [3, 4, C]; conv_state bf16 [S, 3C, 3];
    rec_state fp32 [S, H, 128, 128]; g fp32 [B, H, 128]; beta fp32 [B, H];
    gate bf16 [B, C]; norm_w fp32 [128]; state_idx int32 [B]; out bf16
    [B, C]; C = 128 H.  ``gate``/``norm_w`` may be None when ``norm`` is
    False.  Queued on ``stream`` (a torch.cuda.Stream, a raw handle, or
    None for torch's current stream); nothing is synchronised.
    """
    if rec_state.dim() != 4:
        raise ValueError("rec_state must be [num_slots, H, 128, 128]")
    S, H, D, D2 = rec_state.shape
    B = qkv.shape[0]
    C = H * D
    _check(rec_state, "rec_state", torch.float32, (S, H, D, D2))
    _check(qkv, "qkv", torch.bfloat16, (B, 3 * C))
    _check(conv_w, "conv_w", torch.float32, (3, CONV_WIDTH, C))
    _check(conv_state, "conv_state", torch.bfloat16, (S, 3 * C, CONV_WIDTH - 1))
    _check(g, "g", torch.float32, (B, H, D))
    _check(beta, "beta", torch.float32, (B, H))
    _check(state_idx, "state_idx", torch.int32, (B,))
    _check(out, "out", torch.bfloat16, (B, C))
    if norm:
        _check(gate, "gate", torch.bfloat16, (B, C))
        _check(norm_w, "norm_w", torch.float32, (D,))
    if stream is None:
        stream = torch.cuda.current_stream(qkv.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    dims = Dims(B, H, D, CONV_WIDTH, S, KDA_OUTPUT_NORM if norm else 0,
                float(eps))

    def ptr(t):
        return None if t is None else t.data_ptr()

    with torch.cuda.device(qkv.device):
        rc = decode_raw(dims, ptr(qkv), ptr(conv_w), ptr(conv_state),
                        ptr(rec_state), ptr(g), ptr(beta),
                        ptr(gate) if norm else None,
                        ptr(norm_w) if norm else None, ptr(state_idx),
                        ptr(out), stream)
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def decode_bytes(batch: int, heads: int, live_rows: int, norm: bool = True) -> int:
    """Algorithmic HBM bytes of one call (the library's byte model)."""
    d = Dims(batch, heads, HEAD_DIM, CONV_WIDTH, 1,
             KDA_OUTPUT_NORM if norm else 0, 1e-5)
    return int(lib().kda_decode_bytes(ctypes.byref(d), int(live_rows)))


def state_stream_probe(tiles: torch.Tensor, waves: int = 8,
                       scale: float = 1.0, stream=None) -> None:
    """Read and rewrite (times ``scale``) every [128, 128] fp32 tile of
    ``tiles`` in place with the decode kernel's access pattern: the
    bandwidth ceiling of the state stream (include/kda_probe.h)."""
    _check(tiles, "tiles", torch.float32, tuple(tiles.shape))
    if tiles.dim() < 2 or tuple(tiles.shape[-2:]) != (HEAD_DIM, HEAD_DIM):
        raise ValueError("tiles must be [..., 128, 128]")
    n = tiles.numel() // (HEAD_DIM * HEAD_DIM)
    if stream is None:
        stream = torch.cuda.current_stream(tiles.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    with torch.cuda.device(tiles.device):
        rc = lib().kda_state_stream_probe(tiles.data_ptr(), n, int(waves),
                                          float(scale), stream)
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))
