"""The C-ABI library loads, exports what include/*.h declares, and rejects
bad arguments on the host (no device calls: run without a GPU).

Argument checks use fake, never-dereferenced pointer values, so this module
is skipped whenever a HIP device is visible: a check that wrongly passed
must never reach a kernel launch.
"""
import ctypes
import glob
import os
import re

import pytest
import torch

from linear_attention_decode_02_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(kda_\w+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = ctypes.CDLL(kda.LIB_PATH)
    names = declared_functions()
    assert "kda_decode" in names and "kda_status_string" in names
    for name in names:
        assert hasattr(L, name), f"{name} declared but not exported"


def test_static_scratch_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "kda_decode.h")).read()
    m = re.search(r"#define KDA_STATIC_SCRATCH_BYTES \((\d+)ull << (\d+)\)",
                  text)
    assert m and int(m.group(1)) << int(m.group(2)) == kda.STATIC_SCRATCH_BYTES


def test_status_strings():
    for code in range(7):
        s = kda.status_string(code)
        assert s and s != "unknown status"
    assert kda.status_string(99) == "unknown status"


def test_byte_model_matches_per_unit_table():
    # Per (row, head) with a valid slot: 64 KiB state in + out, 3 x 128 x 3
    # bf16 conv state in + out, 384 bf16 inputs, 128 fp32 log-decays and one
    # beta, 128 bf16 gate and 128 bf16 outputs; null rows only write output.
    per_unit = 2 * 65536 + 2 * 2304 + 768 + 512 + 4 + 256 + 256
    assert per_unit == 137476
    B, H, live = 256, 48, 224
    expect = (live * H * per_unit + (B - live) * H * 256 + 4 * B
              + 3 * 4 * H * 128 * 4 + 128 * 4)
    assert kda.decode_bytes(B, H, live, norm=True) == expect
    assert abs(expect / 1e6 - 1478.8) < 0.05
    assert kda.decode_bytes(512, 96, 512, norm=False) == (
        512 * 96 * (per_unit - 256) + 4 * 512 + 3 * 4 * 96 * 128 * 4)


no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-pointer checks run only without a GPU")

FAKE = 0x10000          # 16-byte aligned, never dereferenced


def call(dims, ptrs=None):
    p = [FAKE] * 10 if ptrs is None else ptrs
    return kda.decode_raw(dims, *p, None)


def dims(**kw):
    base = dict(batch=4, num_heads=12, head_dim=128, conv_width=4,
                num_slots=8, flags=1, norm_eps=1e-5)
    base.update(kw)
    return kda.Dims(**base)


@no_gpu
def test_null_dims_rejected():
    assert kda.lib().kda_decode(None, *([FAKE] * 10), None) == 1


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), 1), (dict(num_slots=0), 1), (dict(num_heads=0), 1),
    (dict(flags=0x40), 1), (dict(flags=0x21), 1), (dict(norm_eps=0.0), 1),
    (dict(norm_eps=float("nan")), 1), (dict(norm_eps=float("inf")), 1),
    (dict(num_heads=16), 2), (dict(num_heads=8), 2), (dict(head_dim=64), 2),
    (dict(conv_width=3), 2),
])
def test_bad_dims(kw, code):
    assert call(dims(**kw)) == code


@no_gpu
def test_eps_unchecked_when_norm_off_and_batch_zero_is_noop():
    # batch 0: nothing is queued, pointers are not looked at
    assert call(dims(batch=0), [None] * 10) == 0
    # norm off: eps and the gate/norm pointers are not used; the request
    # then fails only at the device check (no GPU here)
    p = [FAKE] * 10
    p[6] = p[7] = None
    assert call(dims(flags=0, norm_eps=0.0), p) == 4


@no_gpu
@pytest.mark.parametrize("which", range(10))
def test_null_pointer_rejected(which):
    p = [FAKE] * 10
    p[which] = None
    assert call(dims(), p) == 1


@no_gpu
@pytest.mark.parametrize("which", range(10))
def test_misaligned_pointer_rejected(which):
    p = [FAKE] * 10
    p[which] = FAKE + 4
    assert call(dims(), p) == 3


@no_gpu
def test_no_device_reported():
    assert call(dims()) == 4


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        kda.lib()


@no_gpu
def test_probe_argument_checks():
    L = kda.lib()
    assert L.kda_state_stream_probe(None, 4, 8, 0, 1.0, None) == 1
    assert L.kda_state_stream_probe(FAKE, -1, 8, 0, 1.0, None) == 1
    assert L.kda_state_stream_probe(FAKE, 4, 5, 0, 1.0, None) == 1
    assert L.kda_state_stream_probe(FAKE, 4, 8, 3, 1.0, None) == 1
    assert L.kda_state_stream_probe(FAKE, 4, 8, 0, float("nan"), None) == 1
    assert L.kda_state_stream_probe(FAKE + 4, 4, 8, 0, 1.0, None) == 3
    assert L.kda_state_stream_probe(FAKE, 0, 8, 0, 1.0, None) == 0
    assert L.kda_state_stream_probe(FAKE, 4, 8, 2, 1.0, None) == 4



def call_raw(dims, ptrs=None, lower_bound=0.0):
    # qkv, conv_w, conv_bias, conv_state, rec_state, raw_g, raw_beta, A_log,
    # dt_bias | lower_bound | gate, norm_w, state_idx, out, stream
    p = [FAKE] * 14 if ptrs is None else ptrs
    return kda.lib().kda_decode_raw_gates(ctypes.byref(dims), *p[:9],
                                          lower_bound, *p[9:], None)


@no_gpu
def test_raw_gates_entry_checks():
    assert call_raw(dims()) == 4                       # valid up to device
    assert call_raw(dims(flags=0x21), lower_bound=-2.0) == 4
    assert call_raw(dims(flags=0x21), lower_bound=0.0) == 1
    assert call_raw(dims(flags=0x21), lower_bound=float("-inf")) == 1
    assert call_raw(dims(flags=0x41)) == 1
    assert call_raw(dims(batch=0), [None] * 14) == 0
    p = [FAKE] * 14
    p[2] = None                                        # no conv bias: fine
    assert call_raw(dims(), p) == 4
    p[2] = FAKE + 8                                    # misaligned conv bias
    assert call_raw(dims(), p) == 3
    for which in (5, 6, 7, 8):                         # raw gate inputs
        p = [FAKE] * 14
        p[which] = None
        assert call_raw(dims(), p) == 1
        p[which] = FAKE + 2
        assert call_raw(dims(), p) == 3


def test_byte_model_variants():
    per_unit = 137476
    B, H = 8, 12
    base = kda.decode_bytes(B, H, B)
    assert base == B * H * per_unit + 4 * B + 3 * 4 * H * 128 * 4 + 512
    assert kda.decode_bytes(B, H, B, variants=kda.KDA_NO_CONV_UPDATE) == \
        base - B * H * 2304
    raw = kda.decode_bytes(B, H, B, raw_gates=True)
    assert raw == base - B * H * (256 + 2) + H * 4 + H * 128 * 4
    assert kda.decode_bytes(B, H, B, raw_gates=True, conv_bias=True) == \
        raw + 3 * H * 128 * 4


def test_chunk_count_host_helper():
    import numpy as np
    import oracle
    for lens, bt in (([5, 0, 65, 130], 64), ([], 64), ([0, 0], 1),
                     ([1000, 3, 4097], 16)):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        got = kda.lib().kda_chunk_count(cu.ctypes.data, len(lens), bt)
        idx, off = oracle.chunk_metadata(cu, bt)
        assert got == idx.shape[0] == off[-1]
    cu = np.array([0, 10], np.int32)
    assert kda.lib().kda_chunk_count(cu.ctypes.data, 1, 0) == -1
    assert kda.lib().kda_chunk_count(None, 1, 64) == -1


@no_gpu
def test_prefill_and_metadata_argument_checks():
    L = kda.lib()
    d = dims()
    p = [FAKE] * 12   # cu, qkv, conv_w, cs, rs, g, beta, gate, norm_w, idx, out
    for fn in (L.kda_prefill, L.kda_prefill_chunked):
        assert fn(ctypes.byref(d), *p[:11], None) == 4
        q = list(p)
        q[0] = None
        assert fn(ctypes.byref(d), *q[:11], None) == 1
        q[0] = FAKE + 4
        assert fn(ctypes.byref(d), *q[:11], None) == 3
        q[0] = FAKE
        q[5] = None                                   # g
        assert fn(ctypes.byref(d), *q[:11], None) == 1
        assert fn(ctypes.byref(dims(flags=0x21)), *p[:11], None) == 1
        assert fn(ctypes.byref(dims(batch=0)), *p[:11], None) == 0
    # kda_prefill_chunks: cu, indices, offsets, max, 10 tensors, ws, bytes
    need = L.kda_prefill_chunks_workspace_bytes(ctypes.byref(d), 5)
    assert need == 5 * 12 * 45120
    assert L.kda_prefill_chunks_workspace_bytes(ctypes.byref(d), -1) == 0
    args = [FAKE, FAKE, FAKE, 5] + [FAKE] * 10 + [FAKE, need, None]
    assert L.kda_prefill_chunks(ctypes.byref(d), *args) == 4
    bad = list(args); bad[-2] = need - 1                  # workspace short
    assert L.kda_prefill_chunks(ctypes.byref(d), *bad) == 1
    bad = list(args); bad[3] = -1                         # max_chunks
    assert L.kda_prefill_chunks(ctypes.byref(d), *bad) == 1
    bad = list(args); bad[2] = None                       # chunk_offsets
    assert L.kda_prefill_chunks(ctypes.byref(d), *bad) == 1
    bad = list(args); bad[-3] = FAKE + 8                  # workspace align
    assert L.kda_prefill_chunks(ctypes.byref(d), *bad) == 3
    assert L.kda_prefill_chunks(ctypes.byref(dims(batch=0)), *args) == 0
    # the static-scratch variant: no workspace arguments; a request past
    # KDA_STATIC_SCRATCH_BYTES is refused before anything else is checked
    sargs = [FAKE, FAKE, FAKE, 5] + [FAKE] * 10 + [None]
    fs = L.kda_prefill_chunks_static
    assert fs(ctypes.byref(d), *sargs) == 4
    fit = kda.STATIC_SCRATCH_BYTES // (12 * 45120)
    big = list(sargs); big[3] = fit
    assert fs(ctypes.byref(d), *big) == 4
    big[3] = fit + 1
    assert fs(ctypes.byref(d), *big) == kda.KDA_ERR_TOO_LARGE
    assert fs(ctypes.byref(dims(batch=0)), *big) == kda.KDA_ERR_TOO_LARGE
    assert fs(ctypes.byref(dims(batch=0)), *sargs) == 0
    bad = list(sargs); bad[3] = -1
    assert fs(ctypes.byref(d), *bad) == 1
    bad = list(sargs); bad[1] = None                      # chunk_indices
    assert fs(ctypes.byref(d), *bad) == 1
    bad = list(sargs); bad[2] = FAKE + 8                  # offsets align
    assert fs(ctypes.byref(d), *bad) == 3
    assert L.kda_chunk_metadata(FAKE, 3, 64, FAKE, FAKE, None) == 4
    assert L.kda_chunk_metadata(FAKE, -1, 64, FAKE, FAKE, None) == 1
    assert L.kda_chunk_metadata(FAKE, 3, 0, FAKE, FAKE, None) == 1
    assert L.kda_chunk_metadata(None, 3, 64, FAKE, FAKE, None) == 1
    assert L.kda_chunk_metadata(FAKE, 3, 64, None, FAKE, None) == 1
    assert L.kda_chunk_metadata(FAKE, 0, 64, None, FAKE, None) == 4
    assert L.kda_chunk_metadata(FAKE, 3, 64, FAKE + 8, FAKE, None) == 3


@no_gpu
def test_prefill_raw_gates_argument_checks():
    L = kda.lib()
    d = dims()
    gi = kda.GateInputs(FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
    gp = ctypes.byref(gi)
    # cu, qkv, conv_w, cs, rs | gates | gate, norm_w, idx, out, stream
    head, tail = [FAKE] * 5, [FAKE] * 4 + [None]
    fn = L.kda_prefill_chunked_raw_gates
    assert fn(ctypes.byref(d), *head, gp, *tail) == 4
    assert fn(ctypes.byref(d), *head, None, *tail) == 1       # no gates
    assert fn(ctypes.byref(dims(batch=0)), *head, gp, *tail) == 0
    bounded = dims(flags=0x21)
    assert fn(ctypes.byref(bounded), *head, gp, *tail) == 1   # bound 0.0
    gb = kda.GateInputs(FAKE, FAKE, FAKE, FAKE, FAKE, -2.0)
    assert fn(ctypes.byref(bounded), *head, ctypes.byref(gb), *tail) == 4
    gn = kda.GateInputs(None, FAKE, FAKE, FAKE, FAKE, 0.0)    # no conv bias
    assert fn(ctypes.byref(d), *head, ctypes.byref(gn), *tail) == 4
    for field in ("raw_g", "raw_beta", "A_log", "dt_bias"):
        g2 = kda.GateInputs(FAKE, FAKE, FAKE, FAKE, FAKE, 0.0)
        setattr(g2, field, None)
        assert fn(ctypes.byref(d), *head, ctypes.byref(g2), *tail) == 1
        setattr(g2, field, FAKE + 2)
        assert fn(ctypes.byref(d), *head, ctypes.byref(g2), *tail) == 3
    ga = kda.GateInputs(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 0.0)
    assert fn(ctypes.byref(d), *head, ctypes.byref(ga), *tail) == 3
    # two-pass: cu, indices, offsets, max | qkv, conv_w, cs, rs | gates |
    # gate, norm_w, idx, out, ws | bytes, stream
    need = L.kda_prefill_chunks_workspace_bytes(ctypes.byref(d), 5)
    fc = L.kda_prefill_chunks_raw_gates
    pre, mid = [FAKE, FAKE, FAKE, 5], [FAKE] * 4
    post = [FAKE] * 5 + [need, None]
    assert fc(ctypes.byref(d), *pre, *mid, gp, *post) == 4
    assert fc(ctypes.byref(d), *pre, *mid, None, *post) == 1
    assert fc(ctypes.byref(bounded), *pre, *mid, gp, *post) == 1
    short = post[:5] + [need - 1, None]
    assert fc(ctypes.byref(d), *pre, *mid, gp, *short) == 1
    g2 = kda.GateInputs(FAKE, None, FAKE, FAKE, FAKE, 0.0)
    assert fc(ctypes.byref(d), *pre, *mid, ctypes.byref(g2), *post) == 1
    assert fc(ctypes.byref(dims(batch=0)), *pre, *mid, gp, *post) == 0
    # the plain entry points still reject the bounded-gate flag
    p = [FAKE] * 12
    assert L.kda_prefill_chunked(ctypes.byref(bounded), *p[:11], None) == 1
