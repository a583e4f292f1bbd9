"""CPU oracle of the fused KDA decode step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``kda_oracle.cpp`` (fp32 and fp64 instances of one
literal, unfused implementation); this module only marshals numpy arrays.
Every exported function is pinned by the CPU tests (closed forms, special
cases that reduce to torch library routines, brute force on tiny shapes).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("KDA_ORACLE_LIB") or os.path.join(
    _HERE, "libkda_oracle.so")
_lib = None


# flag bits of the extended step (see kda_oracle.cpp)
NORM, NO_CONV_UPDATE, CONV_TAP_MAJOR, QK_L2NORM, GATE_SILU, BOUNDED_GATE = (
    0x01, 0x02, 0x04, 0x08, 0x10, 0x20)


class _Extras(ctypes.Structure):
    _fields_ = [("conv_bias", ctypes.c_void_p), ("raw_g", ctypes.c_void_p),
                ("raw_beta", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("lower_bound", ctypes.c_float)]


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("norm_eps", ctypes.c_float)]


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it with g++ if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        for name in ("kda_oracle_decode_f32", "kda_oracle_decode_f64"):
            f = getattr(_lib, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.POINTER(_Dims)] + [P] * 11 + [ctypes.c_int]
        for name in ("kda_oracle_decode_ext_f32", "kda_oracle_decode_ext_f64"):
            f = getattr(_lib, name)
            f.restype = ctypes.c_int
            f.argtypes = ([ctypes.POINTER(_Dims)] + [P] * 11 + [ctypes.c_int]
                          + [ctypes.POINTER(_Extras)])
        I, SS = ctypes.c_int, ctypes.c_ssize_t
        for suf, flt in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
            f = getattr(_lib, "kda_oracle_conv_" + suf)
            f.restype = None
            f.argtypes = [I, I, P, P, SS, P, SS, SS, P, I, P]
            f = getattr(_lib, "kda_oracle_recurrence_" + suf)
            f.restype = None
            f.argtypes = [I, P, P, P, P, P, flt, P]
            f = getattr(_lib, "kda_oracle_gated_norm_" + suf)
            f.restype = None
            f.argtypes = [I, P, P, P, flt, I, I, P]
        _lib.kda_oracle_l2norm_f64.restype = None
        _lib.kda_oracle_l2norm_f64.argtypes = [I, P, ctypes.c_double]
        _lib.kda_oracle_raw_gates_f64.restype = None
        _lib.kda_oracle_raw_gates_f64.argtypes = [
            I, P, ctypes.c_float, P, I, ctypes.c_float, ctypes.c_uint16, P, P]
        for name in ("kda_oracle_bf16_from_f32", "kda_oracle_f32_from_bf16"):
            f = getattr(_lib, name)
            f.restype = None
            f.argtypes = [P, P, ctypes.c_size_t]
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _f(dtype):
    return np.float64 if dtype == "f64" else np.float32


# ---------------------------------------------------------------- bf16 ----

def bf16_from_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().kda_oracle_bf16_from_f32(_ptr(x), _ptr(y), x.size)
    return y


def f32_from_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.empty(x.shape, dtype=np.float32)
    lib().kda_oracle_f32_from_bf16(_ptr(x), _ptr(y), x.size)
    return y


# -------------------------------------------------------------- stages ----

def conv_stage(x_bits, w, cs_bits, dtype="f64", bias=None, update=True,
               tap_major=False):
    """Causal conv update of ``nch`` channels.

    x_bits: uint16 [nch] current inputs; w: float32 [W, nch] taps (tap W-1
    multiplies the current input); cs_bits: uint16 stored inputs, oldest
    first, [nch, W-1] (or [W-1, nch] with ``tap_major``); bias: optional
    float32 [nch].  Returns (y [nch], new cs_bits); inputs are not modified.
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    cs = np.array(cs_bits, dtype=np.uint16, order="C", copy=True)
    W, nch = w.shape
    assert x_bits.shape == (nch,)
    if tap_major:
        assert cs.shape == (W - 1, nch)
        chan, tap = 1, nch
    else:
        assert cs.shape == (nch, W - 1)
        chan, tap = W - 1, 1
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    y = np.empty(nch, dtype=_f(dtype))
    getattr(lib(), "kda_oracle_conv_" + dtype)(
        nch, W, _ptr(x_bits), _ptr(w), nch, _ptr(cs), chan, tap, _ptr(b),
        int(update), _ptr(y))
    return y, cs


def recurrence_stage(S, q, k, v, g, beta, dtype="f64"):
    """Gated delta-rule step of one unit.  Returns (S' [D, D], o [D])."""
    F = _f(dtype)
    S2 = np.array(S, dtype=F, order="C", copy=True)
    D = S2.shape[0]
    arrs = [np.ascontiguousarray(a, dtype=F) for a in (q, k, v, g)]
    for a in arrs:
        assert a.shape == (D,)
    o = np.empty(D, dtype=F)
    getattr(lib(), "kda_oracle_recurrence_" + dtype)(
        D, _ptr(S2), *[_ptr(a) for a in arrs], float(beta), _ptr(o))
    return S2, o


def gated_norm_stage(o, gate_bits, norm_w, eps, norm=True, dtype="f64",
                     gate_silu=False):
    """Gated RMSNorm of one unit's D outputs (or identity when norm off)."""
    F = _f(dtype)
    o = np.ascontiguousarray(o, dtype=F)
    D = o.shape[0]
    gate_bits = np.ascontiguousarray(gate_bits, dtype=np.uint16)
    norm_w = np.ascontiguousarray(norm_w, dtype=np.float32)
    y = np.empty(D, dtype=F)
    getattr(lib(), "kda_oracle_gated_norm_" + dtype)(
        D, _ptr(o), _ptr(gate_bits), _ptr(norm_w), float(eps), int(norm),
        int(gate_silu), _ptr(y))
    return y


def l2norm_stage(x, scale=1.0):
    """x / sqrt(sum x^2 + 1e-6) * scale (float64)."""
    x = np.array(x, dtype=np.float64, order="C", copy=True)
    lib().kda_oracle_l2norm_f64(x.shape[0], _ptr(x), float(scale))
    return x


def raw_gates_stage(raw_g_bits, a_log, dt_bias, raw_beta_bits, bounded=False,
                    lower_bound=0.0):
    """Gates of one (row, head) from raw inputs: (g [D], beta) in float64."""
    raw = np.ascontiguousarray(raw_g_bits, dtype=np.uint16)
    bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    D = raw.shape[0]
    g = np.empty(D, np.float64)
    beta = np.empty(1, np.float64)
    lib().kda_oracle_raw_gates_f64(D, _ptr(raw), float(a_log), _ptr(bias),
                                   int(bounded), float(lower_bound),
                                   int(raw_beta_bits), _ptr(g), _ptr(beta))
    return g, float(beta[0])


# ----------------------------------------------------------- full step ----

def decode(inp: dict, *, heads: int, head_dim: int = 128, conv_width: int = 4,
           norm: bool = True, eps: float = 1e-5, dtype: str = "f32",
           nthreads: int | None = None, inplace: bool = False,
           flags: int = 0) -> dict:
    """One fused decode call on host arrays (see ``synth`` for layouts).

    Returns a dict with ``out`` (uint16 bf16 bits [B, C]), ``y`` (the output
    before bf16 rounding), ``conv_state`` and ``rec_state`` after the call.
    Unless ``inplace`` the input pools are copied first.  ``dtype="f64"``
    carries the recurrent state in double.  ``flags`` adds variant bits
    (NO_CONV_UPDATE, CONV_TAP_MAJOR -- conv_state then [S, W-1, 3C] --,
    QK_L2NORM, GATE_SILU, BOUNDED_GATE); optional ``inp`` entries
    "conv_bias", and "raw_g"/"raw_beta"/"A_log"/"dt_bias"/"lower_bound"
    (raw gates: then "g" and "beta" are not read).
    """
    F = _f(dtype)
    qkv = np.ascontiguousarray(inp["qkv"], dtype=np.uint16)
    B = qkv.shape[0]
    C = heads * head_dim
    assert qkv.shape == (B, 3 * C)
    cs = inp["conv_state"]
    rs = inp["rec_state"]
    if inplace:
        assert cs.dtype == np.uint16 and cs.flags["C_CONTIGUOUS"]
        assert rs.dtype == F and rs.flags["C_CONTIGUOUS"]
    else:
        cs = np.array(cs, dtype=np.uint16, order="C", copy=True)
        rs = np.array(rs, dtype=F, order="C", copy=True)
    S = cs.shape[0]
    if flags & CONV_TAP_MAJOR:
        assert cs.shape == (S, conv_width - 1, 3 * C)
    else:
        assert cs.shape == (S, 3 * C, conv_width - 1)
    assert rs.shape == (S, heads, head_dim, head_dim)
    conv_w = np.ascontiguousarray(inp["conv_w"], dtype=np.float32)
    raw = inp.get("raw_g") is not None
    g = None if raw else np.ascontiguousarray(inp["g"], dtype=np.float32)
    beta = None if raw else np.ascontiguousarray(inp["beta"], dtype=np.float32)
    gate = np.ascontiguousarray(inp["gate"], dtype=np.uint16)
    norm_w = np.ascontiguousarray(inp["norm_w"], dtype=np.float32)
    idx = np.ascontiguousarray(inp["state_idx"], dtype=np.int32)
    assert conv_w.shape == (3, conv_width, C)
    if not raw:
        assert g.shape == (B, heads, head_dim) and beta.shape == (B, heads)
    keep = []

    def opt(key, dt, shape):
        a = inp.get(key)
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt)
        assert a.shape == shape, (key, a.shape, shape)
        keep.append(a)
        return a.ctypes.data

    ex = _Extras(opt("conv_bias", np.float32, (3 * C,)),
                 opt("raw_g", np.uint16, (B, heads, head_dim)),
                 opt("raw_beta", np.uint16, (B, heads)),
                 opt("A_log", np.float32, (heads,)),
                 opt("dt_bias", np.float32, (C,)),
                 float(inp.get("lower_bound", 0.0)))
    assert idx.shape == (B,)
    out = np.empty((B, C), dtype=np.uint16)
    y = np.empty((B, C), dtype=F)
    d = _Dims(B, heads, head_dim, conv_width, S,
              (NORM if norm else 0) | (flags & ~NORM), eps)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = getattr(lib(), "kda_oracle_decode_ext_" + dtype)(
        ctypes.byref(d), _ptr(qkv), _ptr(conv_w), _ptr(cs), _ptr(rs), _ptr(g),
        _ptr(beta), _ptr(gate), _ptr(norm_w), _ptr(idx), _ptr(out), _ptr(y),
        int(nthreads), ctypes.byref(ex))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (status {rc})")
    return {"out": out, "y": y, "conv_state": cs, "rec_state": rs}


def decode_tokens(inp: dict, *, heads: int, tokens: int, head_dim: int = 128,
                  conv_width: int = 4, norm: bool = True, eps: float = 1e-5,
                  dtype: str = "f32", nthreads: int | None = None,
                  flags: int = 0, inplace: bool = False) -> dict:
    """T tokens per row: by definition T successive single-token calls on
    the same slots.  Token-major inputs: qkv [B, T, 3C], g [B, T, H, D],
    beta [B, T, H], gate [B, T, C]; returns out/y [B, T, C] and the pools
    after the last token (updated in place with ``inplace``, else copied)."""
    F = _f(dtype)
    if inplace:
        cs, rs = inp["conv_state"], inp["rec_state"]
    else:
        cs = np.array(inp["conv_state"], dtype=np.uint16, order="C", copy=True)
        rs = np.array(inp["rec_state"], dtype=F, order="C", copy=True)
    B = inp["qkv"].shape[0]
    C = heads * head_dim
    assert inp["qkv"].shape == (B, tokens, 3 * C)
    out = np.empty((B, tokens, C), np.uint16)
    y = np.empty((B, tokens, C), F)
    for t in range(tokens):
        step = dict(inp, conv_state=cs, rec_state=rs,
                    qkv=np.ascontiguousarray(inp["qkv"][:, t]),
                    g=np.ascontiguousarray(inp["g"][:, t]),
                    beta=np.ascontiguousarray(inp["beta"][:, t]),
                    gate=np.ascontiguousarray(inp["gate"][:, t]))
        r = decode(step, heads=heads, head_dim=head_dim,
                   conv_width=conv_width, norm=norm, eps=eps, dtype=dtype,
                   nthreads=nthreads, inplace=True, flags=flags)
        out[:, t], y[:, t] = r["out"], r["y"]
    return {"out": out, "y": y, "conv_state": cs, "rec_state": rs}


def chunk_metadata(cu_seqlens, chunk_size: int):
    """Chunk bookkeeping of a variable-length batch (plain numpy).

    Sequence i spans cu_seqlens[i] .. cu_seqlens[i+1]; its chunk count is
    ceil(len / chunk_size) (a negative length counts as empty).  Returns
    (chunk_indices int32 [total, 2] holding (sequence, chunk within the
    sequence) in sequence order, chunk_offsets int64 [N + 1] with the first
    chunk row of each sequence and the total last).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.maximum(cu[1:] - cu[:-1], 0)
    nt = (lens + chunk_size - 1) // chunk_size
    offsets = np.concatenate([[0], np.cumsum(nt)]).astype(np.int64)
    seq = np.repeat(np.arange(nt.size, dtype=np.int64), nt)
    within = np.arange(int(offsets[-1]), dtype=np.int64) - np.repeat(
        offsets[:-1], nt)
    indices = np.stack([seq, within], axis=1).astype(np.int32)
    return indices.reshape(-1, 2), offsets


def prefill(inp: dict, cu_seqlens, *, heads: int, head_dim: int = 128,
            conv_width: int = 4, norm: bool = True, eps: float = 1e-5,
            nthreads: int | None = None, flags: int = 0) -> dict:
    """Variable-length prefill on host arrays: the tokens of sequence n
    (cu_seqlens[n] .. cu_seqlens[n+1]-1 of the token-major qkv [tokens, 3C],
    g [tokens, H, D], beta [tokens, H], gate [tokens, C]) run through the
    single-token step in order on slot state_idx[n] (a pair with
    cu_seqlens[n+1] < cu_seqlens[n] is an empty sequence).  fp32.  Optional
    ``inp`` entries as in ``decode``, token-major: "conv_bias" [3C], and the
    raw gates "raw_g" [tokens, H, D] / "raw_beta" [tokens, H] / "A_log" /
    "dt_bias" / "lower_bound" (then "g" and "beta" are not read)."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.size - 1
    C = heads * head_dim
    qkv = np.ascontiguousarray(inp["qkv"], dtype=np.uint16)
    tokens = qkv.shape[0]
    assert qkv.shape == (tokens, 3 * C)
    # a decreasing pair is an empty sequence; every other one lies in range
    live = cu[1:] > cu[:-1]
    assert np.all(cu[:-1][live] >= 0) and np.all(cu[1:][live] <= tokens)
    cs = np.array(inp["conv_state"], dtype=np.uint16, order="C", copy=True)
    rs = np.array(inp["rec_state"], dtype=np.float32, order="C", copy=True)
    S = cs.shape[0]
    conv_w = np.ascontiguousarray(inp["conv_w"], dtype=np.float32)
    raw = inp.get("raw_g") is not None
    g = None if raw else np.ascontiguousarray(inp["g"], dtype=np.float32)
    beta = None if raw else np.ascontiguousarray(inp["beta"], dtype=np.float32)
    gate = np.ascontiguousarray(inp["gate"], dtype=np.uint16)
    norm_w = np.ascontiguousarray(inp["norm_w"], dtype=np.float32)
    idx = np.ascontiguousarray(inp["state_idx"], dtype=np.int32)
    if not raw:
        assert g.shape == (tokens, heads, head_dim) and beta.shape == (
            tokens, heads)
    assert idx.shape == (N,)
    keep = []

    def opt(key, dt, shape):
        a = inp.get(key)
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dt)
        assert a.shape == shape, (key, a.shape, shape)
        keep.append(a)
        return a.ctypes.data

    ex = _Extras(opt("conv_bias", np.float32, (3 * C,)),
                 opt("raw_g", np.uint16, (tokens, heads, head_dim)),
                 opt("raw_beta", np.uint16, (tokens, heads)),
                 opt("A_log", np.float32, (heads,)),
                 opt("dt_bias", np.float32, (C,)),
                 float(inp.get("lower_bound", 0.0)))
    out = np.zeros((tokens, C), np.uint16)
    y = np.zeros((tokens, C), np.float32)
    L = lib()
    if not hasattr(L.kda_oracle_prefill_ext_f32, "_typed"):
        P = ctypes.c_void_p
        L.kda_oracle_prefill_ext_f32.restype = ctypes.c_int
        L.kda_oracle_prefill_ext_f32.argtypes = (
            [ctypes.POINTER(_Dims)] + [P] * 12 + [ctypes.c_int,
                                                  ctypes.POINTER(_Extras)])
        L.kda_oracle_prefill_ext_f32._typed = True
    assert not flags & CONV_TAP_MAJOR, "channel-major conv state only"
    d = _Dims(N, heads, head_dim, conv_width, S,
              (NORM if norm else 0) | (flags & ~NORM), eps)
    rc = L.kda_oracle_prefill_ext_f32(
        ctypes.byref(d), _ptr(cu), _ptr(qkv), _ptr(conv_w), _ptr(cs), _ptr(rs),
        _ptr(g), _ptr(beta), _ptr(gate), _ptr(norm_w), _ptr(idx), _ptr(out),
        _ptr(y), int(nthreads or os.cpu_count() or 1), ctypes.byref(ex))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (status {rc})")
    return {"out": out, "y": y, "conv_state": cs, "rec_state": rs}
