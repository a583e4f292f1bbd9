"""Pins of the oracle's chunk metadata and variable-length prefill.

Chunk metadata follows the page "PR #51862 完整报告 -- Remove prefill
pipeline stall in chunk KDA" (implementation items 2-3 and the
kda_metadata.py excerpt): from the cumulative sequence offsets, each
sequence gets ceil(length / chunk size) chunks; chunk_offsets holds the
first chunk row of every sequence (and the total); chunk_indices lists
(sequence, chunk) pairs in order.  The prefill that consumes them is, by
definition here, the single-token step applied to each sequence's tokens
in order.
"""
import numpy as np
import pytest

import oracle as O
from linear_attention_decode_02_amd import synth


def brute_metadata(cu, bt):
    rows, offs = [], [0]
    for i in range(len(cu) - 1):
        length = max(cu[i + 1] - cu[i], 0)
        n = 0
        while n * bt < length:
            rows.append((i, n))
            n += 1
        offs.append(offs[-1] + n)
    return rows, offs


@pytest.mark.parametrize("lens,bt", [
    ([5, 0, 65, 130], 64), ([0, 0, 0], 64), ([1], 1), ([64, 64, 63, 129], 64),
    ([7] * 33, 16), ([1000, 3, 0, 4097], 64),
])
def test_chunk_metadata_matches_brute_force(lens, bt):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx, off = O.chunk_metadata(cu, bt)
    rows, offs = brute_metadata(cu.tolist(), bt)
    assert idx.tolist() == [list(r) for r in rows]
    assert off.tolist() == offs
    assert idx.dtype == np.int32 and off.dtype == np.int64


def test_chunks_cover_every_token_once():
    rng = np.random.default_rng(0)
    lens = rng.integers(0, 300, 50)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    bt = 64
    idx, off = O.chunk_metadata(cu, bt)
    cover = np.zeros(int(cu[-1]), np.int32)
    for s, c in idx:
        lo = cu[s] + c * bt
        hi = min(cu[s] + (c + 1) * bt, cu[s + 1])
        assert lo < hi
        cover[lo:hi] += 1
    assert np.all(cover == 1)
    assert off[-1] == idx.shape[0]
    assert np.all(np.diff(off) == (lens + bt - 1) // bt)


def _tokens_case(seed, lens, H=12, extra_slots=3):
    """Token-major inputs for sequences of the given lengths."""
    w = synth.small("pf", batch=1, heads=H, num_slots=len(lens) + extra_slots,
                    seed=seed)
    base = synth.make_inputs(w)
    rng = base.pop("rng")
    total = int(np.sum(lens))
    toks = [synth.make_token(synth.small("t", batch=1, heads=H, num_slots=2,
                                         seed=seed), rng)
            for _ in range(total)]
    inp = dict(base)
    for k in ("qkv", "g", "beta", "gate"):
        inp[k] = np.ascontiguousarray(np.concatenate([t[k] for t in toks], 0))
    inp["state_idx"] = np.arange(1, len(lens) + 1, dtype=np.int32)[::-1].copy()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return w, inp, cu


def test_prefill_equals_tokens_for_equal_lengths():
    T, N, H = 5, 3, 12
    w, inp, cu = _tokens_case(1, [T] * N, H)
    got = O.prefill(inp, cu, heads=H)
    # the same tokens as a [N, T] multi-token batch
    tok = dict(inp)
    for k in ("qkv", "g", "beta", "gate"):
        a = inp[k]
        tok[k] = np.ascontiguousarray(a.reshape((N, T) + a.shape[1:]))
    ref = O.decode_tokens(tok, heads=H, tokens=T)
    assert np.array_equal(got["out"].reshape(N, T, -1), ref["out"])
    assert np.array_equal(got["rec_state"], ref["rec_state"])
    assert np.array_equal(got["conv_state"], ref["conv_state"])


def test_prefill_split_in_two_calls_equals_one_call():
    H = 12
    w, inp, cu = _tokens_case(2, [9, 0, 4], H)
    one = O.prefill(inp, cu, heads=H)           # tokens 0..8 | - | 9..12
    # first call: tokens 0..4 of sequence 0, none of 1, 9..10 of 2
    sel1 = np.r_[0:5, 9:11]
    first_inp = dict(inp)
    for k in ("qkv", "g", "beta", "gate"):
        first_inp[k] = np.ascontiguousarray(inp[k][sel1])
    first = O.prefill(first_inp, np.array([0, 5, 5, 7], np.int32), heads=H)
    second_inp = dict(inp, conv_state=first["conv_state"],
                      rec_state=first["rec_state"])
    # second call: tokens 5..8 of sequence 0, none of 1, 11..12 of 2
    sel = np.r_[5:9, 11:13]
    for k in ("qkv", "g", "beta", "gate"):
        second_inp[k] = np.ascontiguousarray(inp[k][sel])
    second = O.prefill(second_inp, np.array([0, 4, 4, 6], np.int32), heads=H)
    assert np.array_equal(second["rec_state"], one["rec_state"])
    assert np.array_equal(second["conv_state"], one["conv_state"])
    assert np.array_equal(second["out"], one["out"][sel])


def test_prefill_empty_sequence_and_null_slot_leave_state():
    H = 12
    w, inp, cu = _tokens_case(3, [0, 3], H)
    inp["state_idx"] = np.array([2, 0], np.int32)     # empty seq; null slot
    got = O.prefill(inp, cu, heads=H)
    assert np.array_equal(got["rec_state"], inp["rec_state"])
    assert np.array_equal(got["conv_state"], inp["conv_state"])
    assert np.all(got["out"] == 0)
