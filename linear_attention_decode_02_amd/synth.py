"""Seeded synthetic inputs for the fused KDA decode step.

This module only draws random numbers and lays them out in the step's
buffer shapes.  It holds none of the step's arithmetic (no conv, no
recurrence, no norm), so both the CPU oracle (in the tests) and the HIP
path (tests, smoke, bench) can take their inputs from it.

The workloads follow the decode setting of the page "PR #50654 完整报告 --
[ROCm][Perf] Kimi-K3 Fused kernel for KDA decode": one token per sequence,
value-head dimension 128, conv width 4, head counts 12/24/48/96 (the 96
Kimi-K3 KDA heads split over TP 8/4/2/1; "Key source excerpts", the
kda_decode.py gate), bf16 activations and conv state, fp32 recurrent state
(section "Implementation breakdown", item 1), a slot-indexed state pool in
which slot 0 is the null padding slot.

Buffers (all contiguous, row-major; C = H*D channels per q/k/v part):
    qkv        bf16 [B, 3C]          part-major q|k|v, head-major inside a part
    conv_w     fp32 [3, W, C]        width-major depthwise conv weight
    conv_state bf16 [S, 3C, W-1]     oldest tap first
    rec_state  fp32 [S, H, D, D]     [slot, head, key i, value j]
    g          fp32 [B, H, D]        log-decay per key channel (<= 0)
    beta       fp32 [B, H]           in (0, 1)
    gate       bf16 [B, C]
    norm_w     fp32 [D]
    state_idx  int32 [B]             slot per row; <= 0 marks a null row

bf16 tensors are returned as numpy uint16 arrays of raw bits.  The float32
to bf16 rounding of the drawn samples is done by torch's CPU cast.

Streams and draw order (fixed): the per-call tensors come from
default_rng([seed, layer, 0]) in the order qkv, conv_w, g, beta, gate,
norm_w, state_idx; the two state pools come from default_rng([seed, layer,
1]) in the order conv_state (every slot), rec_state (every slot).  Further
tokens (make_token) continue the first stream.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HEAD_DIM = 128
CONV_WIDTH = 4
SUPPORTED_HEADS = (12, 24, 48, 96)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one decode batch."""

    name: str
    batch: int
    heads: int
    num_slots: int
    seed: int
    head_dim: int = HEAD_DIM
    conv_width: int = CONV_WIDTH
    norm: bool = True
    eps: float = 1e-5
    null_tail: int = 0          # last rows mapped to slot 0
    null_every: int = 0         # additionally every k-th row null (0: none)
    g_mode: str = "softplus"    # "softplus" or "stress"
    idx_mode: str = "subset"    # "subset": distinct random slots of 1..S-1
                                # "fixed": use fixed_idx
    fixed_idx: tuple = ()
    rec_sigma: float = 0.02
    conv_w_sigma: float = 0.5
    layers: int = 1             # > 1: independent per-layer pools (sweep)

    @property
    def channels(self) -> int:
        return self.heads * self.head_dim

    def units(self, state_idx: np.ndarray) -> int:
        """Non-null (row, head) pairs: the count of state updates."""
        valid = (state_idx > 0) & (state_idx < self.num_slots)
        return int(valid.sum()) * self.heads


# The five reference workloads of the decode step (seed = index).
TINY = Workload("tiny_b1_h12", batch=1, heads=12, num_slots=4, seed=0,
                idx_mode="fixed", fixed_idx=(2,))
B64_H24 = Workload("b64_h24_pool128", batch=64, heads=24, num_slots=128, seed=1)
B256_H48 = Workload("b256_h48_pool512_null32", batch=256, heads=48,
                    num_slots=512, seed=2, null_tail=32)
B512_H96 = Workload("b512_h96_pool640_nonorm", batch=512, heads=96,
                    num_slots=640, seed=3, norm=False, g_mode="stress")
SWEEP69 = Workload("sweep69_b128_h48_pool129", batch=128, heads=48,
                   num_slots=129, seed=4, layers=69)

WORKLOADS = {w.name: w for w in (TINY, B64_H24, B256_H48, B512_H96, SWEEP69)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 with torch's CPU cast; return raw bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _normal(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _softplus(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return np.logaddexp(0.0, x64)


def make_state_idx(w: Workload, rng: np.random.Generator) -> np.ndarray:
    B, S = w.batch, w.num_slots
    if w.idx_mode == "fixed":
        idx = np.asarray(w.fixed_idx, dtype=np.int32)
        assert idx.shape == (B,)
        return idx
    n_live = B - w.null_tail
    if n_live > S - 1:
        raise ValueError(f"{w.name}: {n_live} live rows need > {S - 1} slots")
    idx = np.zeros(B, dtype=np.int32)
    idx[:n_live] = rng.choice(np.arange(1, S, dtype=np.int32), size=n_live,
                              replace=False)
    if w.null_every:
        idx[::w.null_every] = 0
    return idx


def draw_g(w: Workload, rng: np.random.Generator, shape) -> np.ndarray:
    if w.g_mode == "softplus":
        return (-_softplus(_normal(rng, shape))).astype(np.float32)
    if w.g_mode == "stress":
        # One uniform per element: < 0.1 gives a near-zero log-decay, < 0.2 a
        # strongly negative one, otherwise -softplus(N(0, 1)).
        u = rng.random(size=shape)
        base = -_softplus(_normal(rng, shape))
        g = np.where(u < 0.1, -1e-4, np.where(u < 0.2, -8.0, base))
        return g.astype(np.float32)
    raise ValueError(w.g_mode)


def make_token(w: Workload, rng: np.random.Generator) -> dict:
    """Per-token inputs (qkv, g, beta, gate) for one more decode call."""
    B, H, D, C = w.batch, w.heads, w.head_dim, w.channels
    qkv = to_bf16_bits(_normal(rng, (B, 3 * C)))
    g = draw_g(w, rng, (B, H, D))
    beta = (1.0 / (1.0 + np.exp(-_normal(rng, (B, H)).astype(np.float64))))
    gate = to_bf16_bits(_normal(rng, (B, C)))
    return {"qkv": qkv, "g": g, "beta": beta.astype(np.float32), "gate": gate}


def make_inputs(w: Workload, layer: int = 0, pools: bool = True) -> dict:
    """All buffers of one decode call of workload ``w`` (numpy, host).

    ``layer`` selects the per-layer streams of a multi-layer sweep.  With
    ``pools=False`` the state pools are not drawn (None); the other tensors
    are unchanged.  The returned dict also holds the generator of the
    per-call stream under "rng" (for further tokens).
    """
    rng = np.random.default_rng([w.seed, layer, 0])
    B, H, D, W, S, C = (w.batch, w.heads, w.head_dim, w.conv_width,
                        w.num_slots, w.channels)
    qkv = to_bf16_bits(_normal(rng, (B, 3 * C)))
    conv_w = _normal(rng, (3, W, C), w.conv_w_sigma)
    g = draw_g(w, rng, (B, H, D))
    beta = (1.0 / (1.0 + np.exp(-_normal(rng, (B, H)).astype(np.float64))))
    gate = to_bf16_bits(_normal(rng, (B, C)))
    norm_w = (1.0 + _normal(rng, (D,), 0.1)).astype(np.float32)
    state_idx = make_state_idx(w, rng)
    conv_state = rec_state = None
    if pools:
        prng = np.random.default_rng([w.seed, layer, 1])
        conv_state = to_bf16_bits(_normal(prng, (S, 3 * C, W - 1)))
        rec_state = _normal(prng, (S, H, D, D), w.rec_sigma)
    return {
        "qkv": qkv, "conv_w": conv_w, "conv_state": conv_state,
        "rec_state": rec_state, "g": g, "beta": beta.astype(np.float32),
        "gate": gate, "norm_w": norm_w, "state_idx": state_idx,
        "rng": rng,
    }


def make_tokens(w: Workload, tokens: int, layer: int = 0) -> dict:
    """Inputs of a T-token call: the pools and weights of make_inputs plus
    per-token qkv [B, T, 3C], g [B, T, H, D], beta [B, T, H], gate
    [B, T, C] (token 0 is make_inputs' token, then make_token draws)."""
    inp = make_inputs(w, layer)
    rng = inp.pop("rng")
    toks = [{k: inp[k] for k in ("qkv", "g", "beta", "gate")}]
    for _ in range(tokens - 1):
        toks.append(make_token(w, rng))
    for k in ("qkv", "g", "beta", "gate"):
        inp[k] = np.ascontiguousarray(np.stack([t[k] for t in toks], axis=1))
    return inp


def small(name: str, batch: int, heads: int, num_slots: int, seed: int,
          **kw) -> Workload:
    """A test-sized workload with the reference distributions."""
    return Workload(name, batch=batch, heads=heads, num_slots=num_slots,
                    seed=seed, **kw)


_BF16_KEYS = ("qkv", "conv_state", "gate", "raw_g", "raw_beta")


def to_torch(inp: dict, device="cuda") -> dict:
    """Copy the numpy buffers of ``inp`` to torch tensors on ``device``.

    bf16 buffers (uint16 raw bits) become torch.bfloat16 tensors with the
    same bits; everything else keeps its dtype.  Non-array entries are
    dropped.
    """
    out = {}
    for key, a in inp.items():
        if not isinstance(a, np.ndarray):
            continue
        if key in _BF16_KEYS:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
            t = t.view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out[key] = t.to(device)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16 torch tensor as a host uint16 array."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
