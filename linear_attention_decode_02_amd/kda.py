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
KDA_OUTPUT_NORM = 0x01
KDA_NO_CONV_UPDATE = 0x02
KDA_CONV_TAP_MAJOR = 0x04
KDA_QK_L2NORM = 0x08
KDA_GATE_SILU = 0x10
KDA_BOUNDED_GATE = 0x20
HEAD_DIM = 128
CONV_WIDTH = 4

_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_MISALIGNED", 4: "KDA_ERR_DEVICE", 5: "KDA_ERR_LAUNCH",
           6: "KDA_ERR_TOO_LARGE"}
KDA_ERR_TOO_LARGE = 6
# bytes of the library's static record array (KDA_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 256 << 20


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


class GateInputs(ctypes.Structure):
    """``kda_gate_inputs``: raw gate operands of the prefill entry points."""
    _fields_ = [("conv_bias", ctypes.c_void_p), ("raw_g", ctypes.c_void_p),
                ("raw_beta", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("lower_bound", ctypes.c_float)]


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
        L.kda_decode_raw_gates.restype = ctypes.c_int
        L.kda_decode_raw_gates.argtypes = (
            [ctypes.POINTER(Dims)] + [P] * 9 + [ctypes.c_float] + [P] * 5)
        L.kda_decode_tokens.restype = ctypes.c_int
        L.kda_decode_tokens.argtypes = ([ctypes.POINTER(Dims), ctypes.c_int32]
                                        + [P] * 11)
        L.kda_decode_tokens_bytes.restype = ctypes.c_uint64
        L.kda_decode_tokens_bytes.argtypes = [ctypes.POINTER(Dims),
                                              ctypes.c_int32, ctypes.c_int32]
        L.kda_prefill.restype = ctypes.c_int
        L.kda_prefill.argtypes = [ctypes.POINTER(Dims)] + [P] * 12
        L.kda_prefill_chunked.restype = ctypes.c_int
        L.kda_prefill_chunked.argtypes = [ctypes.POINTER(Dims)] + [P] * 12
        L.kda_prefill_chunks_workspace_bytes.restype = ctypes.c_uint64
        L.kda_prefill_chunks_workspace_bytes.argtypes = [
            ctypes.POINTER(Dims), ctypes.c_int64]
        L.kda_prefill_chunks.restype = ctypes.c_int
        L.kda_prefill_chunks.argtypes = (
            [ctypes.POINTER(Dims), P, P, P, ctypes.c_int64] + [P] * 10 +
            [P, ctypes.c_uint64, P])
        L.kda_prefill_chunks_static.restype = ctypes.c_int
        L.kda_prefill_chunks_static.argtypes = (
            [ctypes.POINTER(Dims), P, P, P, ctypes.c_int64] + [P] * 10 + [P])
        L.kda_prefill_chunked_raw_gates.restype = ctypes.c_int
        L.kda_prefill_chunked_raw_gates.argtypes = (
            [ctypes.POINTER(Dims)] + [P] * 5 + [ctypes.POINTER(GateInputs)]
            + [P] * 5)
        L.kda_prefill_chunks_raw_gates.restype = ctypes.c_int
        L.kda_prefill_chunks_raw_gates.argtypes = (
            [ctypes.POINTER(Dims), P, P, P, ctypes.c_int64] + [P] * 4 +
            [ctypes.POINTER(GateInputs)] + [P] * 5 + [ctypes.c_uint64, P])
        L.kda_chunk_metadata.restype = ctypes.c_int
        L.kda_chunk_metadata.argtypes = [P, ctypes.c_int32, ctypes.c_int32,
                                         P, P, P]
        L.kda_chunk_count.restype = ctypes.c_int64
        L.kda_chunk_count.argtypes = [P, ctypes.c_int32, ctypes.c_int32]
        L.kda_decode_bytes.restype = ctypes.c_uint64
        L.kda_decode_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
        L.kda_decode_raw_gates_bytes.restype = ctypes.c_uint64
        L.kda_decode_raw_gates_bytes.argtypes = [ctypes.POINTER(Dims),
                                                 ctypes.c_int32, ctypes.c_int32]
        L.kda_state_stream_probe.restype = ctypes.c_int
        L.kda_state_stream_probe.argtypes = [P, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_float, P]
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


def _stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _common(qkv, conv_w, conv_state, rec_state, gate, norm_w, state_idx, out,
            norm, variants):
    if rec_state.dim() != 4:
        raise ValueError("rec_state must be [num_slots, H, 128, 128]")
    S, H, D, D2 = rec_state.shape
    B = qkv.shape[0]
    C = H * D
    _check(rec_state, "rec_state", torch.float32, (S, H, D, D2))
    _check(qkv, "qkv", torch.bfloat16, (B, 3 * C))
    _check(conv_w, "conv_w", torch.float32, (3, CONV_WIDTH, C))
    cs_shape = ((S, CONV_WIDTH - 1, 3 * C) if variants & KDA_CONV_TAP_MAJOR
                else (S, 3 * C, CONV_WIDTH - 1))
    _check(conv_state, "conv_state", torch.bfloat16, cs_shape)
    _check(state_idx, "state_idx", torch.int32, (B,))
    _check(out, "out", torch.bfloat16, (B, C))
    if norm:
        _check(gate, "gate", torch.bfloat16, (B, C))
        _check(norm_w, "norm_w", torch.float32, (D,))
    return B, H, D, S


def kda_decode(qkv, conv_w, conv_state, rec_state, g, beta, gate, norm_w,
               state_idx, out, *, norm: bool = True, eps: float = 1e-5,
               variants: int = 0, stream=None) -> None:
    """One fused KDA decode step (in place on ``conv_state``/``rec_state``).

    qkv bf16 [B, 3C]; conv_w fp32 [3, 4, C]; conv_state bf16 [S, 3C, 3]
    ([S, 3, 3C] with KDA_CONV_TAP_MAJOR); rec_state fp32 [S, H, 128, 128];
    g fp32 [B, H, 128]; beta fp32 [B, H]; gate bf16 [B, C]; norm_w fp32
    [128]; state_idx int32 [B]; out bf16 [B, C]; C = 128 H.  ``gate`` and
    ``norm_w`` may be None when ``norm`` is False.  ``variants``: OR of
    KDA_NO_CONV_UPDATE, KDA_CONV_TAP_MAJOR, KDA_QK_L2NORM, KDA_GATE_SILU.
    Queued on ``stream`` (a torch.cuda.Stream, a raw handle, or None for
    torch's current stream); nothing is synchronised.
    """
    B, H, D, S = _common(qkv, conv_w, conv_state, rec_state, gate, norm_w,
                         state_idx, out, norm, variants)
    _check(g, "g", torch.float32, (B, H, D))
    _check(beta, "beta", torch.float32, (B, H))
    dims = Dims(B, H, D, CONV_WIDTH, S,
                (KDA_OUTPUT_NORM if norm else 0) | int(variants), float(eps))
    with torch.cuda.device(qkv.device):
        rc = decode_raw(dims, _ptr(qkv), _ptr(conv_w), _ptr(conv_state),
                        _ptr(rec_state), _ptr(g), _ptr(beta),
                        _ptr(gate) if norm else None,
                        _ptr(norm_w) if norm else None, _ptr(state_idx),
                        _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def kda_decode_raw_gates(qkv, conv_w, conv_bias, conv_state, rec_state, raw_g,
                         raw_beta, A_log, dt_bias, gate, norm_w, state_idx,
                         out, *, norm: bool = True, eps: float = 1e-5,
                         lower_bound: float | None = None, variants: int = 0,
                         stream=None) -> None:
    """The fused step with raw gate inputs and an optional conv bias.

    raw_g bf16 [B, H, 128]; raw_beta bf16 [B, H]; A_log fp32 [H]; dt_bias
    fp32 [C]; conv_bias fp32 [3C] or None.  ``lower_bound`` (< 0) selects
    the bounded gate.  Other arguments as ``kda_decode``.
    """
    B, H, D, S = _common(qkv, conv_w, conv_state, rec_state, gate, norm_w,
                         state_idx, out, norm, variants)
    C = H * D
    _check(raw_g, "raw_g", torch.bfloat16, (B, H, D))
    _check(raw_beta, "raw_beta", torch.bfloat16, (B, H))
    _check(A_log, "A_log", torch.float32, (H,))
    _check(dt_bias, "dt_bias", torch.float32, (C,))
    if conv_bias is not None:
        _check(conv_bias, "conv_bias", torch.float32, (3 * C,))
    flags = (KDA_OUTPUT_NORM if norm else 0) | int(variants)
    if lower_bound is not None:
        flags |= KDA_BOUNDED_GATE
    dims = Dims(B, H, D, CONV_WIDTH, S, flags, float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_decode_raw_gates(
            ctypes.byref(dims), _ptr(qkv), _ptr(conv_w), _ptr(conv_bias),
            _ptr(conv_state), _ptr(rec_state), _ptr(raw_g), _ptr(raw_beta),
            _ptr(A_log), _ptr(dt_bias),
            float(lower_bound if lower_bound is not None else 0.0),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def kda_decode_tokens(qkv, conv_w, conv_state, rec_state, g, beta, gate,
                      norm_w, state_idx, out, *, norm: bool = True,
                      eps: float = 1e-5, variants: int = 0,
                      stream=None) -> None:
    """T decode tokens per row in one call (= T successive kda_decode).

    qkv bf16 [B, T, 3C]; g fp32 [B, T, H, 128]; beta fp32 [B, T, H]; gate
    bf16 [B, T, C]; out bf16 [B, T, C]; other arguments as kda_decode.
    """
    if qkv.dim() != 3:
        raise ValueError("qkv must be [B, T, 3C]")
    B, T = qkv.shape[0], qkv.shape[1]
    if rec_state.dim() != 4:
        raise ValueError("rec_state must be [num_slots, H, 128, 128]")
    S, H, D, D2 = rec_state.shape
    C = H * D
    _check(rec_state, "rec_state", torch.float32, (S, H, D, D2))
    _check(qkv, "qkv", torch.bfloat16, (B, T, 3 * C))
    _check(conv_w, "conv_w", torch.float32, (3, CONV_WIDTH, C))
    cs_shape = ((S, CONV_WIDTH - 1, 3 * C) if variants & KDA_CONV_TAP_MAJOR
                else (S, 3 * C, CONV_WIDTH - 1))
    _check(conv_state, "conv_state", torch.bfloat16, cs_shape)
    _check(state_idx, "state_idx", torch.int32, (B,))
    _check(out, "out", torch.bfloat16, (B, T, C))
    _check(g, "g", torch.float32, (B, T, H, D))
    _check(beta, "beta", torch.float32, (B, T, H))
    if norm:
        _check(gate, "gate", torch.bfloat16, (B, T, C))
        _check(norm_w, "norm_w", torch.float32, (D,))
    dims = Dims(B, H, D, CONV_WIDTH, S,
                (KDA_OUTPUT_NORM if norm else 0) | int(variants), float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_decode_tokens(
            ctypes.byref(dims), int(T), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), _ptr(g), _ptr(beta),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def _prefill_common(cu_seqlens, qkv, conv_w, conv_state, rec_state, gate,
                    norm_w, state_idx, out, norm, variants):
    """Checks the operands every prefill entry point shares; returns
    (N, tokens, H, D, S)."""
    if rec_state.dim() != 4 or qkv.dim() != 2:
        raise ValueError("rec_state [S, H, 128, 128], qkv [tokens, 3C]")
    S, H, D, D2 = rec_state.shape
    C = H * D
    N = state_idx.shape[0]
    tokens = qkv.shape[0]
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _check(rec_state, "rec_state", torch.float32, (S, H, D, D2))
    _check(qkv, "qkv", torch.bfloat16, (tokens, 3 * C))
    _check(conv_w, "conv_w", torch.float32, (3, CONV_WIDTH, C))
    cs_shape = ((S, CONV_WIDTH - 1, 3 * C) if variants & KDA_CONV_TAP_MAJOR
                else (S, 3 * C, CONV_WIDTH - 1))
    _check(conv_state, "conv_state", torch.bfloat16, cs_shape)
    _check(state_idx, "state_idx", torch.int32, (N,))
    _check(out, "out", torch.bfloat16, (tokens, C))
    if norm:
        _check(gate, "gate", torch.bfloat16, (tokens, C))
        _check(norm_w, "norm_w", torch.float32, (D,))
    return N, tokens, H, D, S


def _gate_inputs(tokens, H, D, conv_bias, raw_g, raw_beta, A_log, dt_bias,
                 lower_bound) -> GateInputs:
    C = H * D
    _check(raw_g, "raw_g", torch.bfloat16, (tokens, H, D))
    _check(raw_beta, "raw_beta", torch.bfloat16, (tokens, H))
    _check(A_log, "A_log", torch.float32, (H,))
    _check(dt_bias, "dt_bias", torch.float32, (C,))
    if conv_bias is not None:
        _check(conv_bias, "conv_bias", torch.float32, (3 * C,))
    return GateInputs(_ptr(conv_bias), _ptr(raw_g), _ptr(raw_beta),
                      _ptr(A_log), _ptr(dt_bias),
                      float(lower_bound if lower_bound is not None else 0.0))


def kda_prefill(cu_seqlens, qkv, conv_w, conv_state, rec_state, g, beta,
                gate, norm_w, state_idx, out, *, norm: bool = True,
                eps: float = 1e-5, variants: int = 0, chunked: bool = False,
                stream=None) -> None:
    """Variable-length prefill: sequence n covers tokens cu_seqlens[n] ..
    cu_seqlens[n+1]-1 of token-major qkv [tokens, 3C], g [tokens, H, 128],
    beta [tokens, H], gate/out [tokens, C]; slot state_idx[n].  ``chunked``
    selects kda_prefill_chunked (16-token chunks on the matrix cores)
    instead of the token-by-token kda_prefill."""
    N, tokens, H, D, S = _prefill_common(cu_seqlens, qkv, conv_w, conv_state,
                                         rec_state, gate, norm_w, state_idx,
                                         out, norm, variants)
    _check(g, "g", torch.float32, (tokens, H, D))
    _check(beta, "beta", torch.float32, (tokens, H))
    dims = Dims(N, H, D, CONV_WIDTH, S,
                (KDA_OUTPUT_NORM if norm else 0) | int(variants), float(eps))
    with torch.cuda.device(qkv.device):
        fn = lib().kda_prefill_chunked if chunked else lib().kda_prefill
        rc = fn(
            ctypes.byref(dims), _ptr(cu_seqlens), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), _ptr(g), _ptr(beta),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


PREFILL_CHUNK = 16   # chunk size of the chunked prefill paths


def prefill_chunks_workspace_bytes(heads: int, max_chunks: int) -> int:
    """Bytes of workspace kda_prefill_chunks needs for up to max_chunks
    chunks of 16 tokens."""
    d = Dims(1, heads, HEAD_DIM, CONV_WIDTH, 1, 0, 1e-5)
    return int(lib().kda_prefill_chunks_workspace_bytes(ctypes.byref(d),
                                                        int(max_chunks)))


def kda_prefill_chunks(cu_seqlens, chunk_indices, chunk_offsets,
                       max_chunks: int, qkv, conv_w, conv_state, rec_state, g,
                       beta, gate, norm_w, state_idx, out, workspace, *,
                       norm: bool = True, eps: float = 1e-5,
                       variants: int = 0, stream=None) -> None:
    """Variable-length prefill in two passes over the device chunk table
    (chunk_metadata(cu_seqlens, 16)): per-chunk operands of all chunks in
    parallel into ``workspace`` (a uint8 device tensor of at least
    prefill_chunks_workspace_bytes bytes), then each sequence's state
    through its chunks.  Other arguments as kda_prefill."""
    N, tokens, H, D, S = _prefill_common(cu_seqlens, qkv, conv_w, conv_state,
                                         rec_state, gate, norm_w, state_idx,
                                         out, norm, variants)
    _check_chunk_table(N, chunk_indices, chunk_offsets, workspace)
    _check(g, "g", torch.float32, (tokens, H, D))
    _check(beta, "beta", torch.float32, (tokens, H))
    dims = Dims(N, H, D, CONV_WIDTH, S,
                (KDA_OUTPUT_NORM if norm else 0) | int(variants), float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_prefill_chunks(
            ctypes.byref(dims), _ptr(cu_seqlens), _ptr(chunk_indices),
            _ptr(chunk_offsets), int(max_chunks), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), _ptr(g), _ptr(beta),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _ptr(workspace),
            int(workspace.numel()), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def kda_prefill_chunks_static(cu_seqlens, chunk_indices, chunk_offsets,
                              max_chunks: int, qkv, conv_w, conv_state,
                              rec_state, g, beta, gate, norm_w, state_idx,
                              out, *, norm: bool = True, eps: float = 1e-5,
                              variants: int = 0, stream=None) -> None:
    """kda_prefill_chunks without a workspace, for callers that cannot
    allocate: the records go to the library's static per-GPU array
    (max_chunks * H * record bytes <= STATIC_SCRATCH_BYTES, else
    KdaError KDA_ERR_TOO_LARGE).  Calls that overlap on one GPU race on
    that array.  Other arguments as kda_prefill_chunks."""
    N, tokens, H, D, S = _prefill_common(cu_seqlens, qkv, conv_w, conv_state,
                                         rec_state, gate, norm_w, state_idx,
                                         out, norm, variants)
    _check(chunk_offsets, "chunk_offsets", torch.int64, (N + 1,))
    _check(chunk_indices, "chunk_indices", torch.int32,
           (chunk_indices.shape[0], 2))
    _check(g, "g", torch.float32, (tokens, H, D))
    _check(beta, "beta", torch.float32, (tokens, H))
    dims = Dims(N, H, D, CONV_WIDTH, S,
                (KDA_OUTPUT_NORM if norm else 0) | int(variants), float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_prefill_chunks_static(
            ctypes.byref(dims), _ptr(cu_seqlens), _ptr(chunk_indices),
            _ptr(chunk_offsets), int(max_chunks), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), _ptr(g), _ptr(beta),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def _check_chunk_table(N, chunk_indices, chunk_offsets, workspace):
    _check(chunk_offsets, "chunk_offsets", torch.int64, (N + 1,))
    _check(chunk_indices, "chunk_indices", torch.int32,
           (chunk_indices.shape[0], 2))
    _check(workspace, "workspace", torch.uint8, (workspace.numel(),))


def kda_prefill_chunked_raw_gates(cu_seqlens, qkv, conv_w, conv_bias,
                                  conv_state, rec_state, raw_g, raw_beta,
                                  A_log, dt_bias, gate, norm_w, state_idx,
                                  out, *, norm: bool = True,
                                  eps: float = 1e-5,
                                  lower_bound: float | None = None,
                                  variants: int = 0, stream=None) -> None:
    """kda_prefill_chunked with the gate activation fused: raw_g bf16
    [tokens, H, 128], raw_beta bf16 [tokens, H], A_log fp32 [H], dt_bias
    fp32 [C], conv_bias fp32 [3C] or None; ``lower_bound`` (< 0) selects
    the bounded gate.  Other arguments as kda_prefill."""
    N, tokens, H, D, S = _prefill_common(cu_seqlens, qkv, conv_w, conv_state,
                                         rec_state, gate, norm_w, state_idx,
                                         out, norm, variants)
    gi = _gate_inputs(tokens, H, D, conv_bias, raw_g, raw_beta, A_log,
                      dt_bias, lower_bound)
    flags = (KDA_OUTPUT_NORM if norm else 0) | int(variants)
    if lower_bound is not None:
        flags |= KDA_BOUNDED_GATE
    dims = Dims(N, H, D, CONV_WIDTH, S, flags, float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_prefill_chunked_raw_gates(
            ctypes.byref(dims), _ptr(cu_seqlens), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), ctypes.byref(gi),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def kda_prefill_chunks_raw_gates(cu_seqlens, chunk_indices, chunk_offsets,
                                 max_chunks: int, qkv, conv_w, conv_bias,
                                 conv_state, rec_state, raw_g, raw_beta,
                                 A_log, dt_bias, gate, norm_w, state_idx, out,
                                 workspace, *, norm: bool = True,
                                 eps: float = 1e-5,
                                 lower_bound: float | None = None,
                                 variants: int = 0, stream=None) -> None:
    """kda_prefill_chunks with the gate activation fused (raw gate operands
    as kda_prefill_chunked_raw_gates)."""
    N, tokens, H, D, S = _prefill_common(cu_seqlens, qkv, conv_w, conv_state,
                                         rec_state, gate, norm_w, state_idx,
                                         out, norm, variants)
    _check_chunk_table(N, chunk_indices, chunk_offsets, workspace)
    gi = _gate_inputs(tokens, H, D, conv_bias, raw_g, raw_beta, A_log,
                      dt_bias, lower_bound)
    flags = (KDA_OUTPUT_NORM if norm else 0) | int(variants)
    if lower_bound is not None:
        flags |= KDA_BOUNDED_GATE
    dims = Dims(N, H, D, CONV_WIDTH, S, flags, float(eps))
    with torch.cuda.device(qkv.device):
        rc = lib().kda_prefill_chunks_raw_gates(
            ctypes.byref(dims), _ptr(cu_seqlens), _ptr(chunk_indices),
            _ptr(chunk_offsets), int(max_chunks), _ptr(qkv), _ptr(conv_w),
            _ptr(conv_state), _ptr(rec_state), ctypes.byref(gi),
            _ptr(gate) if norm else None, _ptr(norm_w) if norm else None,
            _ptr(state_idx), _ptr(out), _ptr(workspace),
            int(workspace.numel()), _stream(stream, qkv.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))


def chunk_metadata(cu_seqlens, chunk_size: int, cu_seqlens_host=None,
                   stream=None):
    """(chunk_indices int32 [total, 2], chunk_offsets int64 [N + 1]) of a
    device cu_seqlens (int32 [N + 1]).  The total is computed on the host
    from ``cu_seqlens_host`` (a CPU tensor; copied from the device if
    omitted, which synchronises)."""
    _check(cu_seqlens, "cu_seqlens", torch.int32, tuple(cu_seqlens.shape))
    N = cu_seqlens.shape[0] - 1
    host = (cu_seqlens.cpu() if cu_seqlens_host is None
            else cu_seqlens_host).to(torch.int32).contiguous()
    total = int(lib().kda_chunk_count(host.data_ptr(), N, int(chunk_size)))
    if total < 0:
        raise ValueError("bad cu_seqlens or chunk_size")
    dev = cu_seqlens.device
    indices = torch.empty(max(total, 1), 2, dtype=torch.int32, device=dev)
    offsets = torch.empty(N + 1, dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        rc = lib().kda_chunk_metadata(_ptr(cu_seqlens), N, int(chunk_size),
                                      _ptr(indices), _ptr(offsets),
                                      _stream(stream, dev))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))
    return indices[:total], offsets


def decode_tokens_bytes(batch: int, heads: int, tokens: int, live_rows: int,
                        norm: bool = True, variants: int = 0) -> int:
    """Algorithmic HBM bytes of one kda_decode_tokens call."""
    d = Dims(batch, heads, HEAD_DIM, CONV_WIDTH, 1,
             (KDA_OUTPUT_NORM if norm else 0) | int(variants), 1e-5)
    return int(lib().kda_decode_tokens_bytes(ctypes.byref(d), int(tokens),
                                             int(live_rows)))


def decode_bytes(batch: int, heads: int, live_rows: int, norm: bool = True,
                 variants: int = 0, raw_gates: bool = False,
                 conv_bias: bool = False) -> int:
    """Algorithmic HBM bytes of one call (the library's byte model)."""
    d = Dims(batch, heads, HEAD_DIM, CONV_WIDTH, 1,
             (KDA_OUTPUT_NORM if norm else 0) | int(variants), 1e-5)
    if raw_gates:
        return int(lib().kda_decode_raw_gates_bytes(ctypes.byref(d),
                                                    int(live_rows),
                                                    int(conv_bias)))
    return int(lib().kda_decode_bytes(ctypes.byref(d), int(live_rows)))


PROBE_RMW, PROBE_READ, PROBE_WRITE = 0, 1, 2


def state_stream_probe(tiles: torch.Tensor, waves: int = 16,
                       scale: float = 1.0, mode: int = PROBE_RMW,
                       stream=None) -> None:
    """Stream every [128, 128] fp32 tile of ``tiles`` with the decode
    kernel's access pattern (include/kda_probe.h): read and rewrite times
    ``scale`` (PROBE_RMW), read only (PROBE_READ) or write ``scale``
    everywhere (PROBE_WRITE)."""
    _check(tiles, "tiles", torch.float32, tuple(tiles.shape))
    if tiles.dim() < 2 or tuple(tiles.shape[-2:]) != (HEAD_DIM, HEAD_DIM):
        raise ValueError("tiles must be [..., 128, 128]")
    n = tiles.numel() // (HEAD_DIM * HEAD_DIM)
    with torch.cuda.device(tiles.device):
        rc = lib().kda_state_stream_probe(tiles.data_ptr(), n, int(waves),
                                          int(mode), float(scale),
                                          _stream(stream, tiles.device))
    if rc != KDA_OK:
        raise KdaError(rc, status_string(rc))
