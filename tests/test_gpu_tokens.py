"""GPU parity of kda_decode_tokens (T decode tokens per row in one call).

The page "PR #50654 完整报告 -- [ROCm][Perf] Kimi-K3 Fused kernel for KDA
decode" fuses one token per sequence and gates out speculative decoding
(kda_decode.py excerpt: num_spec must be 0).  The multi-token call is
defined as T successive single-token steps on the same slots; the oracle is
that composition.
"""
import numpy as np
import pytest
import torch

import oracle as O
from linear_attention_decode_02_amd import kda, synth

import _parity as P

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]
DEV = "cuda:0"


def run_tokens(w, inp, T, variants=0, t=None):
    t = synth.to_torch(inp, DEV) if t is None else t
    out = torch.full((w.batch, T, w.channels), float("nan"),
                     dtype=torch.bfloat16, device=DEV)
    kda.kda_decode_tokens(t["qkv"], t["conv_w"], t["conv_state"],
                          t["rec_state"], t["g"], t["beta"],
                          t["gate"] if w.norm else None,
                          t["norm_w"] if w.norm else None, t["state_idx"],
                          out, norm=w.norm, eps=w.eps, variants=variants)
    torch.cuda.synchronize()
    return {"out": synth.bf16_bits(out),
            "conv_state": synth.bf16_bits(t["conv_state"]),
            "rec_state": t["rec_state"].cpu().numpy()}


def run_single_calls(w, inp, T, variants=0):
    """The same tokens through T kda_decode calls."""
    t = synth.to_torch(inp, DEV)
    outs = []
    for i in range(T):
        out = torch.empty(w.batch, w.channels, dtype=torch.bfloat16,
                          device=DEV)
        kda.kda_decode(t["qkv"][:, i].contiguous(), t["conv_w"],
                       t["conv_state"], t["rec_state"],
                       t["g"][:, i].contiguous(), t["beta"][:, i].contiguous(),
                       t["gate"][:, i].contiguous() if w.norm else None,
                       t["norm_w"] if w.norm else None, t["state_idx"], out,
                       norm=w.norm, eps=w.eps, variants=variants)
        outs.append(out)
    torch.cuda.synchronize()
    return {"out": synth.bf16_bits(torch.stack(outs, 1)),
            "conv_state": synth.bf16_bits(t["conv_state"]),
            "rec_state": t["rec_state"].cpu().numpy()}


def check_tokens(w, inp, got, ref, T, flags=0, scaled=False):
    """Parity of a multi-token call.  The state bar is the absolute 1e-3;
    ``scaled`` makes it 1e-3 relative to each unit's largest state
    magnitude, for the expansive regime only (beta |k|^2 > 2: raw keys from
    the reference conv weights, where each token multiplies the state, and
    its fp32 rounding, by up to |1 - beta |k|^2| ~ 20)."""
    cs_got, cs_ref, cs_in = got["conv_state"], ref["conv_state"], \
        inp["conv_state"]
    if flags & O.CONV_TAP_MAJOR:
        cs_got, cs_ref, cs_in = (np.ascontiguousarray(a.transpose(0, 2, 1))
                                 for a in (cs_got, cs_ref, cs_in))
    st = P.check_states(cs_got, got["rec_state"], cs_ref, ref["rec_state"],
                        cs_in, inp["rec_state"], inp["state_idx"],
                        w.num_slots, scaled=scaled)
    for t in range(T):
        st_t = P.check_output(got["out"][:, t], ref["y"][:, t],
                              inp["state_idx"], w.num_slots, w.heads)
        st["out_max_rel"] = max(st.get("out_max_rel", 0), st_t["out_max_rel"])
    return st


def test_one_token_equals_single_step_kernel():
    w = synth.small("t1", batch=33, heads=48, num_slots=40, seed=31,
                    null_every=5)
    inp = synth.make_tokens(w, 1)
    a = run_tokens(w, inp, 1)
    b = run_single_calls(w, inp, 1)
    assert np.array_equal(a["conv_state"], b["conv_state"])
    d_rs = np.abs(a["rec_state"] - b["rec_state"]).max()
    d_out = np.abs(P.bf16_to_f32(a["out"]) - P.bf16_to_f32(b["out"])).max()
    print(f"[t1] bitwise state {d_rs == 0} out {d_out == 0}", flush=True)
    assert d_rs <= 1e-6


@pytest.mark.parametrize("T", [2, 4, 5, 7, 8])
def test_tokens_match_successive_single_calls(T):
    """State kept on chip across T tokens == T calls through HBM."""
    w = synth.small(f"tt{T}", batch=24, heads=24, num_slots=30, seed=40 + T,
                    null_every=6, conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    a = run_tokens(w, inp, T)
    b = run_single_calls(w, inp, T)
    assert np.array_equal(a["conv_state"], b["conv_state"])
    d_rs = np.abs(a["rec_state"] - b["rec_state"]).max()
    print(f"[tokens {T}] vs single calls: state maxdiff {d_rs:.3g}",
          flush=True)
    assert d_rs <= 1e-5
    for t in range(T):
        P.check_output(a["out"][:, t],
                       P.bf16_to_f32(b["out"][:, t]).astype(np.float64),
                       inp["state_idx"], w.num_slots, w.heads)



def test_tokens_decay_extremes():
    """Decays across the whole range within one multi-token call: per
    element -1e-4 (10 %), -8 (20 %), -30 (5 %), -100 (5 %, exp underflows
    to zero or a subnormal) or -softplus(N(0,1)).  Over 12 tokens a key row
    keeps nearly all of its state or forgets it entirely; the result must
    equal the oracle and T single-token calls."""
    T = 12
    w = synth.small("tdecay", batch=9, heads=24, num_slots=14, seed=77,
                    null_every=4, conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    rng = np.random.default_rng(78)
    u = rng.random(inp["g"].shape)
    g = inp["g"].copy()
    g[u < 0.4] = -100.0
    g[u < 0.35] = -30.0
    g[u < 0.30] = -8.0
    g[u < 0.10] = -1e-4
    inp["g"] = np.ascontiguousarray(g.astype(np.float32))
    ref = O.decode_tokens(inp, heads=w.heads, tokens=T, norm=True, eps=w.eps)
    got = run_tokens(w, inp, T)
    st = check_tokens(w, inp, got, ref, T)
    single = run_single_calls(w, inp, T)
    assert np.array_equal(got["conv_state"], single["conv_state"])
    d_rs = np.abs(got["rec_state"] - single["rec_state"]).max()
    print(f"[tokens decay] {st} vs single calls: state maxdiff {d_rs:.3g}",
          flush=True)
    assert d_rs <= 1e-5


CASES = [
    ("plain", 0, True), ("nonorm", 0, False),
    ("tap_major", O.CONV_TAP_MAJOR, True),
    ("l2_silu", O.QK_L2NORM | O.GATE_SILU, True),
    ("no_conv_update", O.NO_CONV_UPDATE, True),
]


@pytest.mark.parametrize("name,flags,norm", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("H,T", [(12, 3), (96, 5)])
def test_tokens_parity_with_oracle(name, flags, norm, H, T):
    w = synth.small(f"to_{name}", batch=9, heads=H, num_slots=14,
                    seed=50 + H + T, null_every=4, norm=norm)
    inp = synth.make_tokens(w, T)
    inp["state_idx"][2] = -3
    if flags & O.CONV_TAP_MAJOR:
        inp["conv_state"] = np.ascontiguousarray(
            inp["conv_state"].transpose(0, 2, 1))
    print(f"[tokens] {name} H={H} T={T}", flush=True)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=norm, eps=w.eps,
                          flags=flags)
    got = run_tokens(w, inp, T, variants=flags)
    # reference conv weights: raw keys are expansive, L2-normalised ones
    # contractive
    st = check_tokens(w, inp, got, ref, T, flags,
                      scaled=not flags & O.QK_L2NORM)
    if flags & O.NO_CONV_UPDATE:
        assert np.array_equal(got["conv_state"], inp["conv_state"])
    print(f"[tokens] {name}: {st}", flush=True)


def test_tokens_b256_h48_full_size():
    """The batch-256, 48-head workload (32 null rows) with 4 tokens per row.
    Raw keys from the reference conv weights: the expansive regime, so the
    state bar is relative to each unit's state magnitude."""
    w = synth.B256_H48
    T = 4
    inp = synth.make_tokens(w, T)
    ref = O.decode_tokens(inp, heads=w.heads, tokens=T, norm=True, eps=w.eps)
    got = run_tokens(w, inp, T)
    st = check_tokens(w, inp, got, ref, T, scaled=True)
    assert np.all(got["out"][-32:] == 0)
    print(f"[tokens b256] {st}", flush=True)


SHORT_CASES = [
    ("plain", 0, True, 8), ("nonorm", 0, False, 6),
    ("tap_major", O.CONV_TAP_MAJOR, True, 8),
    ("l2_silu", O.QK_L2NORM | O.GATE_SILU, True, 7),
    ("no_conv_update", O.NO_CONV_UPDATE, True, 5),
    ("tap_major_no_conv_update", O.CONV_TAP_MAJOR | O.NO_CONV_UPDATE, True,
     6),
]


@pytest.mark.parametrize("name,flags,norm,T", SHORT_CASES,
                         ids=[c[0] for c in SHORT_CASES])
def test_tokens_5_to_8_take_the_short_row_form(name, flags, norm, T):
    """Rows of 5 .. 8 tokens run the short-row kernel (the row's tokens as
    one chunk, one workgroup per (row, head)); every variant must still
    equal T successive single-token steps (the oracle).  Null and
    out-of-range slots inside the batch."""
    H = 24
    w = synth.small(f"ts_{name}", batch=9, heads=H, num_slots=14,
                    seed=130 + T, null_every=4, norm=norm,
                    conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    inp["state_idx"][2] = -3
    inp["state_idx"][5] = w.num_slots
    if flags & O.CONV_TAP_MAJOR:
        inp["conv_state"] = np.ascontiguousarray(
            inp["conv_state"].transpose(0, 2, 1))
    print(f"[tokens short] {name} H={H} T={T}", flush=True)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=norm, eps=w.eps,
                          flags=flags)
    got = run_tokens(w, inp, T, variants=flags)
    st = check_tokens(w, inp, got, ref, T, flags)
    if flags & O.NO_CONV_UPDATE:
        assert np.array_equal(got["conv_state"], inp["conv_state"])
    print(f"[tokens short] {name}: {st}", flush=True)


SHORT_LONG_CASES = [
    ("nonorm", 0, False, 17), ("tap_major", O.CONV_TAP_MAJOR, True, 20),
    ("no_conv_update", O.NO_CONV_UPDATE, True, 33),
    ("l2_silu", O.QK_L2NORM | O.GATE_SILU, True, 64),
]


@pytest.mark.parametrize("name,flags,norm,T", SHORT_LONG_CASES,
                         ids=[c[0] for c in SHORT_LONG_CASES])
def test_tokens_17_to_64_with_many_units_take_the_short_row_form(
        name, flags, norm, T):
    """Rows of 17 .. 64 tokens with at least 4 (row, head) units per compute
    unit (here 48 rows x 24 heads = 1,152) run the short-row kernel in
    chunks of 8 (3 to 8 per row, the last one ragged at 17, 20 and 33);
    every variant against the oracle, null and negative slots inside."""
    H = 24
    w = synth.small(f"tl_{name}", batch=48, heads=H, num_slots=56,
                    seed=230 + T, null_every=6, norm=norm,
                    conv_w_sigma=0.5 if flags & O.QK_L2NORM else 0.05)
    inp = synth.make_tokens(w, T)
    inp["state_idx"][3] = -1
    if flags & O.CONV_TAP_MAJOR:
        inp["conv_state"] = np.ascontiguousarray(
            inp["conv_state"].transpose(0, 2, 1))
    print(f"[tokens short long] {name} H={H} T={T}", flush=True)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=norm, eps=w.eps,
                          flags=flags)
    got = run_tokens(w, inp, T, variants=flags)
    st = check_tokens(w, inp, got, ref, T, flags)
    if flags & O.NO_CONV_UPDATE:
        assert np.array_equal(got["conv_state"], inp["conv_state"])
    print(f"[tokens short long] {name}: {st}", flush=True)


CHUNKED_CASES = [
    ("plain", 0, True, 11), ("nonorm", 0, False, 12),
    ("tap_major", O.CONV_TAP_MAJOR, True, 16),
    ("l2_silu", O.QK_L2NORM | O.GATE_SILU, True, 13),
    ("no_conv_update", O.NO_CONV_UPDATE, True, 15),
    ("plain_two_chunks", 0, True, 29), ("nonorm_two_chunks", 0, False, 30),
    ("tap_major_three_chunks", O.CONV_TAP_MAJOR, True, 33),
    ("no_conv_update_three_chunks", O.NO_CONV_UPDATE, True, 40),
]


@pytest.mark.parametrize("name,flags,norm,T", CHUNKED_CASES,
                         ids=[c[0] for c in CHUNKED_CASES])
def test_tokens_multi_chunk_forms(name, flags, norm, T):
    """Rows longer than one chunk: 11 .. 16 tokens run the short-row kernel
    in two chunks of up to 8; from 17 tokens, with these 216 (row, head)
    units (fewer than 4 per compute unit), the chunked kernel in chunks of
    16 (two or three per row).  Every variant must still equal T successive
    single-token steps (the oracle)."""
    H = 24
    w = synth.small(f"tc_{name}", batch=9, heads=H, num_slots=14,
                    seed=150 + T, null_every=4, norm=norm,
                    conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    inp["state_idx"][2] = -3
    if flags & O.CONV_TAP_MAJOR:
        inp["conv_state"] = np.ascontiguousarray(
            inp["conv_state"].transpose(0, 2, 1))
    print(f"[tokens chunked] {name} H={H} T={T}", flush=True)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=norm, eps=w.eps,
                          flags=flags)
    got = run_tokens(w, inp, T, variants=flags)
    st = check_tokens(w, inp, got, ref, T, flags)
    if flags & O.NO_CONV_UPDATE:
        assert np.array_equal(got["conv_state"], inp["conv_state"])
    print(f"[tokens chunked] {name}: {st}", flush=True)


def test_tokens_agree_with_single_calls_across_the_switches():
    """Either side of each switch of form (token by token up to 4, short
    rows 5 .. 16, and with these 576 (row, head) units the chunked kernel
    from 17), against T single-token kernel calls on the same inputs."""
    for T in (4, 5, 8, 9, 16, 17, 29):
        w = synth.small(f"tsw{T}", batch=12, heads=48, num_slots=20,
                        seed=170 + T, null_every=5, conv_w_sigma=0.05)
        inp = synth.make_tokens(w, T)
        a = run_tokens(w, inp, T)
        b = run_single_calls(w, inp, T)
        assert np.array_equal(a["conv_state"], b["conv_state"])
        d_rs = np.abs(a["rec_state"] - b["rec_state"]).max()
        print(f"[tokens {T}] vs single calls: state maxdiff {d_rs:.3g}",
              flush=True)
        assert d_rs <= 1e-4
        for t in range(T):
            P.check_output(a["out"][:, t],
                           P.bf16_to_f32(b["out"][:, t]).astype(np.float64),
                           inp["state_idx"], w.num_slots, w.heads)


@pytest.mark.parametrize("T", [8, 10, 16, 29])
def test_tokens_b256_h48_full_size(T):
    """The batch-256, 48-head workload (32 null rows) with 8, 10, 16 and 29
    tokens per row at full size (the short-row kernel: one, two and four
    chunks of up to 8, the last ones ragged), every element against the
    oracle.
    q/k are L2-normalised (unit keys, beta < 1: each update contracts the
    state along k).  Without it these inputs give beta |k|^2 near 40, and
    16 or more chained updates amplify fp32 rounding order by that factor
    per token, which no bar meaningful for single steps survives."""
    w = synth.B256_H48
    inp = synth.make_tokens(w, T)
    ref = O.decode_tokens(inp, heads=w.heads, tokens=T, norm=True, eps=w.eps,
                          flags=O.QK_L2NORM)
    got = run_tokens(w, inp, T, variants=O.QK_L2NORM)
    st = check_tokens(w, inp, got, ref, T)
    assert np.all(got["out"][-32:] == 0)
    print(f"[tokens b256 T={T}] {st}", flush=True)


def test_tokens_many_rows_with_null_rows_inside():
    """Rows of 12 tokens at 200 rows x 96 heads: 19,200 (row, head) units,
    the short-row kernel's two chunks each, in many rounds of workgroups
    per compute unit, with a null row every 7; every element against the
    oracle (q/k L2-normalised, the contractive regime: absolute state
    bar)."""
    T, H = 12, 96
    w = synth.small("rows_many", batch=200, heads=H, num_slots=210, seed=410,
                    null_every=7, conv_w_sigma=0.5)
    inp = synth.make_tokens(w, T)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=True, eps=w.eps,
                          flags=O.QK_L2NORM)
    got = run_tokens(w, inp, T, variants=O.QK_L2NORM)
    st = check_tokens(w, inp, got, ref, T)
    null = ~((inp["state_idx"] > 0) & (inp["state_idx"] < w.num_slots))
    assert null.any() and np.all(got["out"][null] == 0)
    print(f"[tokens many rows] {st}", flush=True)


@pytest.mark.parametrize("T,B", [(4, 32), (8, 32), (12, 32), (24, 32),
                                 (24, 2)])
def test_tokens_deterministic_bitwise(T, B):
    """Two identical calls give identical bits in every form: token by
    token (T = 4), short rows in one, two and three chunks (T = 8, 12, and
    24 at 32 rows x 48 heads = 1,536 units) and the chunked kernel (T = 24
    at 2 rows).  No form sums through atomics."""
    w = synth.small(f"tdet{T}_{B}", batch=B, heads=48, num_slots=B + 8,
                    seed=500 + T + B, null_every=5, conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    a = run_tokens(w, inp, T)
    b = run_tokens(w, inp, T)
    for key in ("out", "conv_state"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["rec_state"].view(np.uint32),
                          b["rec_state"].view(np.uint32))


def test_tokens_argument_checks():
    w = synth.small("tc", batch=2, heads=12, num_slots=4, seed=60)
    inp = synth.make_tokens(w, 2)
    t = synth.to_torch(inp, DEV)
    out = torch.empty(2, 2, w.channels, dtype=torch.bfloat16, device=DEV)
    d = kda.Dims(2, 12, 128, 4, 4, 1, 1e-5)
    ptrs = [t[k].data_ptr() for k in ("qkv", "conv_w", "conv_state",
                                      "rec_state", "g", "beta", "gate",
                                      "norm_w", "state_idx")] + [out.data_ptr()]
    L = kda.lib()
    s = torch.cuda.current_stream().cuda_stream
    import ctypes
    assert L.kda_decode_tokens(ctypes.byref(d), 0, *ptrs, s) == 1
    assert L.kda_decode_tokens(ctypes.byref(d), 1025, *ptrs, s) == 1
    d.flags = 0x21
    assert L.kda_decode_tokens(ctypes.byref(d), 2, *ptrs, s) == 1


def test_tokens_maximum_T():
    """T = 1024, the largest count the entry point accepts (64 chunks of
    the matrix-core form), on a small batch with a null row, against 1024
    oracle steps.  q/k L2-normalised, so the long chain stays contractive
    and the single-step bars apply."""
    T = 1024
    w = synth.small("tmax", batch=3, heads=12, num_slots=6, seed=180,
                    null_every=3, conv_w_sigma=0.5)
    inp = synth.make_tokens(w, T)
    ref = O.decode_tokens(inp, heads=w.heads, tokens=T, norm=True, eps=w.eps,
                          flags=O.QK_L2NORM)
    got = run_tokens(w, inp, T, variants=O.QK_L2NORM)
    st = check_tokens(w, inp, got, ref, T)
    print(f"[tokens T=1024] {st}", flush=True)


@pytest.mark.parametrize("T", [4, 8, 12, 30])
def test_tokens_graph_replay_matches_eager(T):
    """kda_decode_tokens captured in a HIP graph (T = 4 token by token,
    T = 8 and 12 short rows in one and two chunks, T = 30 the chunked form)
    and replayed three times with eager work and
    synchronisation in between: each replay equals the same eager call bit
    for bit (pools updated in place, so every replay advances the state)."""
    w = synth.small(f"tgraph{T}", batch=10, heads=24, num_slots=16,
                    seed=190 + T, null_every=4, conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    flags = O.QK_L2NORM if T >= 29 else 0
    te = synth.to_torch(inp, DEV)        # eager copy
    tg = synth.to_torch(inp, DEV)        # graph copy
    out_e = torch.empty(w.batch, T, w.channels, dtype=torch.bfloat16,
                        device=DEV)
    out_g = torch.empty_like(out_e)

    def call(t, out):
        kda.kda_decode_tokens(t["qkv"], t["conv_w"], t["conv_state"],
                              t["rec_state"], t["g"], t["beta"], t["gate"],
                              t["norm_w"], t["state_idx"], out, norm=True,
                              eps=w.eps, variants=flags)

    warm = synth.to_torch(inp, DEV)
    call(warm, torch.empty_like(out_e))   # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cs0, rs0 = tg["conv_state"].clone(), tg["rec_state"].clone()
    with torch.cuda.graph(graph):
        call(tg, out_g)
    tg["conv_state"].copy_(cs0)
    tg["rec_state"].copy_(rs0)
    torch.cuda.synchronize()
    for r in range(3):
        call(te, out_e)
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 20, device=DEV).sum()   # eager work
        graph.replay()
        torch.cuda.synchronize()
        assert scratch.isfinite()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), r
        assert torch.equal(tg["conv_state"].view(torch.int16),
                           te["conv_state"].view(torch.int16)), r
        assert torch.equal(tg["rec_state"].view(torch.int32),
                           te["rec_state"].view(torch.int32)), r
        print(f"[tokens graph T={T}] replay {r} matches eager", flush=True)


@pytest.mark.parametrize("T", [4, 5, 8, 10, 16, 29])
def test_tokens_decay_contract_independent_of_T(T):
    """The contract on g is the same in every form (token by token, short
    rows from 5 tokens in one or two chunks, with these 144 (row, head)
    units the chunked kernel from 17): per element -inf (5 %, the key row
    is forgotten), -1e30 (5 %), -100 (5 %, exp underflows), -1e-4 (5 %) or
    an ordinary decay, against the oracle (exp(-inf) = 0 there)."""
    w = synth.small(f"tginf{T}", batch=6, heads=24, num_slots=10,
                    seed=310 + T, null_every=4, conv_w_sigma=0.05)
    inp = synth.make_tokens(w, T)
    u = np.random.default_rng(311).random(inp["g"].shape)
    g = inp["g"].copy()
    g[u < 0.20] = -1e-4
    g[u < 0.15] = -100.0
    g[u < 0.10] = -1e30
    g[u < 0.05] = -np.inf
    inp["g"] = np.ascontiguousarray(g.astype(np.float32))
    ref = O.decode_tokens(inp, heads=w.heads, tokens=T, norm=True, eps=w.eps)
    assert np.isfinite(ref["rec_state"]).all()
    got = run_tokens(w, inp, T)
    st = check_tokens(w, inp, got, ref, T)
    print(f"[tokens decay contract T={T}] {st}", flush=True)


@pytest.mark.parametrize("B,T", [(64, 1024), (1024, 64)])
def test_tokens_offsets_past_int32_products(B, T):
    """64-bit token offsets in kda_decode_tokens at 96 heads, so that
    row x T x 3C passes 2^31 elements in the last rows: 64 rows x 1024
    tokens (the chunked kernel) and 1024 rows x 64 tokens (98,304 units:
    the short-row kernel, eight chunks per row).  All rows but the last
    four are null (they read no input and write zeros); the last four carry
    seeded inputs and are compared with the oracle.  q/k L2-normalised
    (contractive)."""
    H = 96
    C = H * 128
    live = 4
    assert (B - 1) * T * 3 * C > 2**31
    small = synth.small("tbig", batch=live, heads=H, num_slots=live + 1,
                        seed=320 + T, conv_w_sigma=0.5)
    inp = synth.make_tokens(small, T)
    inp["state_idx"] = np.arange(1, live + 1, dtype=np.int32)
    ref = O.decode_tokens(inp, heads=H, tokens=T, norm=True, eps=small.eps,
                          flags=O.QK_L2NORM)
    t = synth.to_torch(inp, DEV)
    big = {"qkv": torch.empty(B, T, 3 * C, dtype=torch.bfloat16, device=DEV),
           "g": torch.empty(B, T, H, 128, dtype=torch.float32, device=DEV),
           "beta": torch.empty(B, T, H, dtype=torch.float32, device=DEV),
           "gate": torch.empty(B, T, C, dtype=torch.bfloat16, device=DEV)}
    for k, b in big.items():
        b[B - live:].copy_(t[k])
    idx = torch.zeros(B, dtype=torch.int32, device=DEV)
    idx[B - live:] = t["state_idx"]
    out = torch.full((B, T, C), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    kda.kda_decode_tokens(big["qkv"], t["conv_w"], t["conv_state"],
                          t["rec_state"], big["g"], big["beta"], big["gate"],
                          t["norm_w"], idx, out, norm=True, eps=small.eps,
                          variants=O.QK_L2NORM)
    torch.cuda.synchronize()
    assert bool((out[:B - live].view(torch.int16) == 0).all())
    got = {"out": synth.bf16_bits(out[B - live:]),
           "conv_state": synth.bf16_bits(t["conv_state"]),
           "rec_state": t["rec_state"].cpu().numpy()}
    st = check_tokens(small, inp, got, ref, T)
    print(f"[tokens offsets past 2^31] {st}", flush=True)
