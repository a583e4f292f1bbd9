"""Throughput of the fused KDA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one kda_decode call over one batch of the workload (default: the
batch-256, 48-head call with a 512-slot pool and 32 null padding rows),
with every input resident in HBM; for the 69-layer sweep workload a step
is 69 independent single-layer calls, each with its own weights and pools.  The timed region is K calls between two
device synchronisations; each call is also bracketed by HIP events on the
stream it runs on, which give the kernel's average launch duration for the
roofline.  Prints one JSON line.

The metric counts (sequence, head) state updates per second (rows of the
null slot count zero) and the achieved HBM bandwidth from the algorithmic
byte model (state read + write, conv state read + write, inputs, outputs)
against MI355X's 8 TB/s.  The CPU oracle timed on the host cores of the
same machine is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA decode (seq*head) updates/sec + achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
# kda_decode_tokens runs the token-by-token kernel for rows of up to 4
# tokens, the short-row kernel from 5 to 16 tokens (and up to 64 with at
# least 4 (row, head) units per compute unit), else the chunked kernel
SHORT_ROW_MIN_TOKENS = 5
SHORT_ROW_ANY_UNITS_MAX_TOKENS = 16
SHORT_ROW_MAX_TOKENS = 64
SHORT_ROW_MIN_UNITS_PER_CU = 4
# fp32 matrix flop per (16-token chunk, head) of the chunked form: K~S, Q~S
# and the state update (3 x 2*16*128*128), A, B, the solve and B Delta
# (4 x 2*16*16*128).  The kernel reaches fp32 precision on the bf16 matrix
# cores (three bf16 pieces per operand, six piece products), so this
# fp32-equivalent work is priced against the fp32 matrix peak; the bf16
# instructions it executes per (chunk, head) are counted beside it.
CHUNK_MFMA_FLOP = 3 * 2 * 16 * 128 * 128 + 4 * 2 * 16 * 16 * 128
BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
# executed per (chunk, head): 4 state waves x (48 + 48 + 48) and 4 prep
# waves x 12 v_mfma_f32_16x16x32_bf16 (16384 flop each), 4 x 16
# v_mfma_f32_16x16x4_f32 (2048 flop each)
CHUNK_BF16_MFMA = 4 * 144 + 4 * 12
CHUNK_FP32_MFMA = 4 * 16
KERNEL_SRC = os.path.join(ROOT, "linear_attention_decode_02_amd", "csrc",
                          "kda_decode.hip")
KERNEL_END_MARK = "// Several tokens per row in one launch"
TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                            "kda_decode_b256_h48_traffic.md")


# name -> (flag bits, raw gates + conv bias)
VARIANTS = {
    "plain": (0, False),
    "no_conv_update": (0x02, False),
    "conv_tap_major": (0x04, False),
    "qk_l2norm": (0x08, False),
    "gate_silu": (0x10, False),
    "raw_gates": (0, True),
    # raw gates + conv bias + q/k L2 norm + bounded gate
    "kda_full": (0x08 | 0x20, True),
}


def kernel_hash(text: str = None) -> str:
    """Hash of the device code the single-token kernel is built from: the
    source from the opening of its namespace to the end of kda_decode_kernel
    (host code and the other kernels of the file are not part of it)."""
    if text is None:
        with open(KERNEL_SRC, encoding="utf-8") as f:
            text = f.read()
    start = text.index("namespace {")
    end = text.index(KERNEL_END_MARK, start)
    return hashlib.sha256(text[start:end].encode()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """Counter-measured HBM bytes per launch, if recorded for this exact
    kernel source and workload (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    wl = re.search(r"workload:\s*(\S+)", text)
    if not (m and h and wl) or h.group(1) != kernel_hash() or \
            wl.group(1) != workload:
        return None
    return int(m.group(1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b256_h48_pool512_null32")
    ap.add_argument("--variant", default="plain", choices=sorted(VARIANTS),
                    help="kernel variant (default: the plain step)")
    ap.add_argument("--prefill", action="store_true",
                    help="measure the variable-length prefill instead "
                         "(16 sequences, 48 heads, L2-normalised q/k)")
    ap.add_argument("--serving", action="store_true",
                    help="per-call latency of kda_decode at serving batch "
                         "sizes (1..256 rows, 12 and 48 heads, graph replay)")
    ap.add_argument("--tokens", type=int, default=1,
                    help="decode tokens per row and call (> 1: the "
                         "multi-token entry point, state kept on chip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU-oracle time for the baseline (0: skip)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay measurement")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip the plain-copy reference (1 GiB torch copy)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode step has no "
              f"cross-GPU exchange); --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_decode_02_amd import kda, synth

    if args.prefill:
        return bench_prefill(args, np, torch, kda, synth)
    if args.serving:
        return bench_serving(args, np, torch, kda, synth)

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    T = args.tokens
    inp = synth.make_inputs(w) if T == 1 else synth.make_tokens(w, T)
    vflags, raw = VARIANTS[args.variant]
    if T > 1 and (raw or w.layers > 1):
        sys.exit("--tokens > 1 runs the plain flag variants of one layer")
    if vflags & kda.KDA_CONV_TAP_MAJOR:
        inp["conv_state"] = np.ascontiguousarray(
            inp["conv_state"].transpose(0, 2, 1))
    layers = [synth.to_torch(inp, dev)]
    if w.layers > 1:
        # independent layers: own weights, inputs and slots; the pools are
        # copies of layer 0's (values do not change the work done)
        for layer in range(1, w.layers):
            t = synth.to_torch(synth.make_inputs(w, layer, pools=False), dev)
            t["conv_state"] = layers[0]["conv_state"].clone()
            t["rec_state"] = layers[0]["rec_state"].clone()
            layers.append(t)
    for li, t in enumerate(layers):
        t["out"] = torch.empty((w.batch, T, w.channels) if T > 1 else
                               (w.batch, w.channels), dtype=torch.bfloat16,
                               device=dev)
        if raw:     # raw gate inputs and conv bias, drawn per layer
            rh = raw_inputs(w, li, np, synth)
            if li == 0:
                inp.update(rh)
            for key, a in rh.items():
                if isinstance(a, np.ndarray):
                    t[key] = (torch.from_numpy(a.view(np.int16)).view(
                        torch.bfloat16) if a.dtype == np.uint16
                        else torch.from_numpy(a)).to(dev)
    idx = inp["state_idx"]
    live_rows = int(((idx > 0) & (idx < w.num_slots)).sum())
    units = live_rows * w.heads * T                  # per layer
    if T > 1:
        alg_bytes = kda.decode_tokens_bytes(w.batch, w.heads, T, live_rows,
                                            w.norm, variants=vflags)
    else:
        alg_bytes = kda.decode_bytes(w.batch, w.heads, live_rows, w.norm,
                                     variants=vflags & ~kda.KDA_BOUNDED_GATE,
                                     raw_gates=raw, conv_bias=raw)
    L = len(layers)
    stream = torch.cuda.current_stream(dev)

    def call(t, on):
        if T > 1:
            kda.kda_decode_tokens(t["qkv"], t["conv_w"], t["conv_state"],
                                  t["rec_state"], t["g"], t["beta"],
                                  t["gate"], t["norm_w"], t["state_idx"],
                                  t["out"], norm=w.norm, eps=w.eps,
                                  variants=vflags, stream=on)
        elif raw:
            kda.kda_decode_raw_gates(
                t["qkv"], t["conv_w"], t["conv_bias"], t["conv_state"],
                t["rec_state"], t["raw_g"], t["raw_beta"], t["A_log"],
                t["dt_bias"], t["gate"], t["norm_w"], t["state_idx"],
                t["out"], norm=w.norm, eps=w.eps,
                lower_bound=-5.0 if vflags & kda.KDA_BOUNDED_GATE else None,
                variants=vflags & ~kda.KDA_BOUNDED_GATE, stream=on)
        else:
            kda.kda_decode(t["qkv"], t["conv_w"], t["conv_state"],
                           t["rec_state"], t["g"], t["beta"], t["gate"],
                           t["norm_w"], t["state_idx"], t["out"],
                           norm=w.norm, eps=w.eps, variants=vflags,
                           stream=on)

    def step(on=stream):
        # on=None: torch's current stream (the capture stream in a graph)
        for t in layers:
            call(t, on)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K * L)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K * L)]
    print(f"[bench] timing {K} steps of {L} call(s)", file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for li, t in enumerate(layers):
            ev0[i * L + li].record(stream)
            call(t, stream)
            ev1[i * L + li].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in zip(ev0, ev1)]
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    ms_per_step = wall / K * 1e3
    value = units * L * K / wall
    achieved = alg_bytes / kern_avg_s / 1e9

    extra = {
        "kernel_us": {"mean": round(kern_avg_s * 1e6, 2),
                      "p10": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(kern_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 2)},
        "alg_bytes_per_launch": alg_bytes,
        "units_per_launch": units,
        "launches_per_step": L,
        "wall_GBs": round(alg_bytes * L * K / wall / 1e9, 1),
    }
    path = None
    if T > 1:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        path = tokens_path(T, w.batch * w.heads, cus)
        extra["tokens_path"] = path

    if not args.no_graph:
        R = max(1, (max(10, K // 4) + L - 1) // L)      # steps per replay
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(R):
                step(None)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        gstep = e0.elapsed_time(e1) * 1e-3 / R
        extra["graph"] = {"steps": R, "calls": R * L,
                          "us_per_step": round(gstep * 1e6, 2),
                          "us_per_call": round(gstep / L * 1e6, 2),
                          "updates_per_s": units * L / gstep,
                          "GBs": round(alg_bytes * L / gstep / 1e9, 1)}
        del g

    if not args.no_copy_probe:
        extra["copy_probe"] = copy_probe(torch, stream)
        if args.variant == "plain" and T == 1:
            extra["stream_ceiling"] = stream_ceiling(
                torch, kda, stream, w, live_rows, alg_bytes, kern_avg_s)
        if L == 1:
            extra["rotated_pools"] = rotated_pools(
                torch, np, stream, layers[0], call, alg_bytes, K)

    traffic = (recorded_traffic(w.name)
               if args.variant == "plain" and T == 1 else None)
    if traffic is not None:
        extra["traffic_source"] = (
            "recorded: calibrated FETCH_SIZE + WRITE_SIZE counters of this "
            "kernel source on this workload (" +
            os.path.relpath(TRAFFIC_FILE, ROOT) + "), not read in this run")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic}
    if path is not None and path.startswith("chunked"):
        # the chunked matrix-core form: priced in its fp32 MFMA work per
        # (16-token chunk, live row, head)
        chunks = -(-T // 16) * live_rows * w.heads      # per launch
        tflops = chunks * CHUNK_MFMA_FLOP / kern_avg_s / 1e12
        extra["hbm_GBs"] = round(achieved, 1)
        roofline = {"bound": "mfma", "achieved": round(tflops, 2),
                    "peak": FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / FP32_MFMA_TFLOPS, 4),
                    "traffic": None}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_seconds, alg_bytes, units,
                           vflags, T)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "updates/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": args.variant,
                   "tokens_per_row": T, "layers": L,
                   "batch": w.batch,
                   "heads": w.heads,
                   "head_dim": w.head_dim, "conv_width": w.conv_width,
                   "num_slots": w.num_slots, "null_rows": w.batch - live_rows,
                   "output_norm": w.norm, "io": "bf16 qkv/conv_state/gate/out",
                   "state": "fp32", "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def tokens_path(T, units, cus):
    """The kernel kda_decode_tokens runs for rows of T tokens and `units`
    (row, head) pairs on a device of `cus` compute units."""
    if T < SHORT_ROW_MIN_TOKENS:
        return "token by token"
    if T <= SHORT_ROW_ANY_UNITS_MAX_TOKENS or (
            T <= SHORT_ROW_MAX_TOKENS and
            units >= SHORT_ROW_MIN_UNITS_PER_CU * cus):
        return "short rows: chunks of 8 tokens, one workgroup per (row, head)"
    return "chunked: chunks of 16 tokens, one workgroup per (row, head)"


def bench_serving(args, np, torch, kda, synth, copies=8, calls=64):
    """Per-call latency of kda_decode at the batch sizes of serving: 1..256
    rows at 12 heads (the TP8 share of 96), 24 and 48 heads, norm on, every
    row live.  Each point is a graph of ``calls`` calls rotating ``copies``
    copies of the state pools (no reuse through the last-level cache),
    replayed 5 times; the median replay divided by ``calls``."""
    dev = torch.device("cuda:0")
    points = []
    for H in (12, 24, 48):
        for B in (1, 8, 16, 24, 32, 64, 128, 256):
            w = synth.small(f"serving_b{B}_h{H}", batch=B, heads=H,
                            num_slots=B + 1, seed=5)
            t = synth.to_torch(synth.make_inputs(w), dev)
            out = torch.empty(B, w.channels, dtype=torch.bfloat16,
                              device=dev)
            pools = [(t["conv_state"].clone(), t["rec_state"].clone())
                     for _ in range(copies)]

            null_idx = torch.zeros_like(t["state_idx"])
            tiles = [torch.ones(B * H, 128, 128, dtype=torch.float32,
                                device=dev) for _ in range(copies)]

            def call(i):
                cs, rs = pools[i % copies]
                kda.kda_decode(t["qkv"], t["conv_w"], cs, rs, t["g"],
                               t["beta"], t["gate"], t["norm_w"],
                               t["state_idx"], out, norm=True, eps=w.eps)

            def null_call(i):
                # every row on the null slot: the launch and the zero
                # outputs, no state traffic
                cs, rs = pools[i % copies]
                kda.kda_decode(t["qkv"], t["conv_w"], cs, rs, t["g"],
                               t["beta"], t["gate"], t["norm_w"], null_idx,
                               out, norm=True, eps=w.eps)

            def rmw_call(i):
                # the same state bytes read and rewritten with the kernel's
                # tile mapping and nothing else (one 64 KiB tile per
                # 1024-thread workgroup)
                kda.state_stream_probe(tiles[i % copies], 16,
                                       mode=kda.PROBE_RMW)

            def graph_us(fn):
                side = torch.cuda.Stream(dev)
                side.wait_stream(torch.cuda.current_stream(dev))
                with torch.cuda.stream(side):
                    for i in range(copies):
                        fn(i)
                torch.cuda.current_stream(dev).wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(calls):
                        fn(i)
                g.replay()
                torch.cuda.synchronize()
                ts = []
                for _ in range(5):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3 / calls)
                del g
                return float(np.median(ts))

            us = graph_us(call)
            us_null = graph_us(null_call)
            us_rmw = graph_us(rmw_call)
            nbytes = kda.decode_bytes(B, H, B, True)
            points.append({"batch": B, "heads": H, "us_per_call": round(us, 2),
                           "GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                           "null_rows_us": round(us_null, 2),
                           "state_rmw_us": round(us_rmw, 2)})
            print(f"[serving] H={H} B={B}: {us:.2f} us (all rows null "
                  f"{us_null:.2f}, bare state read-modify-write {us_rmw:.2f})",
                  file=sys.stderr, flush=True)
            del pools, t, tiles
    c16 = next(p for p in points if p["batch"] == 16 and p["heads"] == 12)
    line = {
        "metric": "KDA decode latency per call at serving batch sizes",
        "value": c16["us_per_call"], "unit": "us", "n_gpus": 1,
        "steps": calls, "warmup": copies, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "serving_b16_h12 (value); sweep in extra",
                   "head_dim": 128, "conv_width": 4, "output_norm": True,
                   "parallelism": "single-gpu"},
        "roofline": None, "cpu_baseline": None,
        "extra": {"points": points, "pool_copies": copies,
                  "calls_per_graph": calls,
                  "null_rows_us": "the same call with every row on the null "
                                  "slot (launch + zero outputs)",
                  "state_rmw_us": "kda_state_stream_probe read-modify-write "
                                  "of the call's B*H state tiles, 16 waves"},
    }
    print(json.dumps(line), flush=True)


def bench_prefill(args, np, torch, kda, synth):
    """Variable-length prefill: 16 sequences with seeded lengths (1..4096,
    log-uniform), 48 heads, q/k L2-normalised, fresh states.  A step is one
    kda_prefill_chunked call over the batch (16-token chunks on the matrix
    cores); the token-by-token kda_prefill, the two-pass kda_prefill_chunks
    (with its chunk metadata), the raw-gate entry point and the chunk
    metadata kernel are timed beside it."""
    import oracle

    H, N = 48, 16
    rng = np.random.default_rng(7)
    lens = np.exp(rng.uniform(0, np.log(4096), N)).astype(np.int64) + 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    w = synth.small("prefill_16seq_h48", batch=total, heads=H,
                    num_slots=N + 1, seed=7)
    base = synth.make_inputs(synth.small("pf", batch=1, heads=H,
                                         num_slots=N + 1, seed=7))
    rng_t = base.pop("rng")
    tok = synth.make_token(w, rng_t)
    inp = dict(base, **tok)
    inp["state_idx"] = np.arange(1, N + 1, dtype=np.int32)
    inp["rec_state"][:] = 0
    dev = torch.device("cuda:0")
    t = synth.to_torch(inp, dev)
    cu_d = torch.from_numpy(cu).to(dev)
    out = torch.empty(total, w.channels, dtype=torch.bfloat16, device=dev)
    flags = kda.KDA_QK_L2NORM
    stream = torch.cuda.current_stream(dev)

    def step(chunked=True):
        kda.kda_prefill(cu_d, t["qkv"], t["conv_w"], t["conv_state"],
                        t["rec_state"], t["g"], t["beta"], t["gate"],
                        t["norm_w"], t["state_idx"], out, eps=w.eps,
                        variants=flags, chunked=chunked, stream=stream)

    def timed(k, chunked):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(k):
            step(chunked)
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3 / k

    for _ in range(args.warmup):
        step()
    K = args.steps
    wall, kern = timed(K, True)
    step(False)
    _, kern_seq = timed(max(K // 4, 1), False)

    def event_time(fn, k):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / k

    host = torch.from_numpy(cu)
    max_chunks = int(((lens + 15) // 16).sum())
    ws = torch.empty(kda.prefill_chunks_workspace_bytes(H, max_chunks),
                     dtype=torch.uint8, device=dev)

    def two_pass():
        idx, off = kda.chunk_metadata(cu_d, kda.PREFILL_CHUNK,
                                      cu_seqlens_host=host, stream=stream)
        kda.kda_prefill_chunks(cu_d, idx, off, max_chunks, t["qkv"],
                               t["conv_w"], t["conv_state"], t["rec_state"],
                               t["g"], t["beta"], t["gate"], t["norm_w"],
                               t["state_idx"], out, ws, eps=w.eps,
                               variants=flags, stream=stream)

    # raw gates (the activation fused into the chunk kernel): raw_g ~
    # N(-3, 1) (per-token decays of a few hundredths to a few tenths),
    # raw_beta ~ N(0, 1), A_log, dt_bias ~ N(0, 0.5), conv bias ~ N(0, 0.3)
    rr = np.random.default_rng([7, 3])
    rg = synth.to_torch({
        "raw_g": synth.to_bf16_bits(
            rr.normal(-3, 1, (total, H, 128)).astype(np.float32)),
        "raw_beta": synth.to_bf16_bits(
            rr.normal(0, 1, (total, H)).astype(np.float32)),
        "A_log": rr.normal(0, 0.5, H).astype(np.float32),
        "dt_bias": rr.normal(0, 0.5, H * 128).astype(np.float32),
        "conv_bias": rr.normal(0, 0.3, 3 * H * 128).astype(np.float32)}, dev)

    def raw_gates():
        kda.kda_prefill_chunked_raw_gates(
            cu_d, t["qkv"], t["conv_w"], rg["conv_bias"], t["conv_state"],
            t["rec_state"], rg["raw_g"], rg["raw_beta"], rg["A_log"],
            rg["dt_bias"], t["gate"], t["norm_w"], t["state_idx"], out,
            eps=w.eps, variants=flags, stream=stream)

    # the same lengths shortest first (the longest last in the batch; the
    # token rows are reused in place, so each sequence reads other rows):
    # the launch order a caller's batch may come in
    cu_asc = torch.from_numpy(np.concatenate(
        [[0], np.cumsum(np.sort(lens))]).astype(np.int32)).to(dev)

    def ascending():
        kda.kda_prefill(cu_asc, t["qkv"], t["conv_w"], t["conv_state"],
                        t["rec_state"], t["g"], t["beta"], t["gate"],
                        t["norm_w"], t["state_idx"], out, eps=w.eps,
                        variants=flags, chunked=True, stream=stream)

    kern_two = event_time(two_pass, max(K // 2, 1))
    kern_raw = event_time(raw_gates, max(K // 2, 1))
    kern_asc = event_time(ascending, max(K // 2, 1))
    updates = total * H
    # matrix-core work of the chunked form per (16-token chunk, head): K~S,
    # Q~S and the state update (3 x 2*16*128*128), the A and B products and
    # the solve / B Delta products (4 x 2*16*16*128); a ragged last chunk
    # counts as a full one
    chunks = int(((lens + 15) // 16).sum())
    flop_chunk = CHUNK_MFMA_FLOP
    tflops = chunks * H * flop_chunk / kern / 1e12
    # bytes: state once per (sequence, head) in + out, conv state, and per
    # token the inputs and outputs
    per_tok = (3 * 128 * 2 + 128 * 4 + 4 + 128 * 2 + 128 * 2) * H
    nbytes = N * H * (2 * 128 * 128 * 4 + 2 * 2304) + total * per_tok
    # chunk metadata beside it
    kda.chunk_metadata(cu_d, 64, cu_seqlens_host=host)
    torch.cuda.synchronize()
    m0 = torch.cuda.Event(enable_timing=True)
    m1 = torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for _ in range(100):
        kda.chunk_metadata(cu_d, 64, cu_seqlens_host=host, stream=stream)
    m1.record(stream)
    torch.cuda.synchronize()
    meta_us = m0.elapsed_time(m1) * 1e3 / 100
    cpu = None
    if args.cpu_seconds > 0:
        cores, info = cpu_threads()
        # a bounded sample: the 4 shortest sequences, repeated
        order = np.argsort(lens)[:4]
        sub_lens = lens[order]
        sub_cu = np.concatenate([[0], np.cumsum(sub_lens)]).astype(np.int32)
        sel = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
        sub = dict(inp, state_idx=inp["state_idx"][order].copy())
        for k in ("qkv", "g", "beta", "gate"):
            sub[k] = np.ascontiguousarray(inp[k][sel])
        sub_updates = int(sub_lens.sum()) * H
        runs = timed_runs(lambda: oracle.prefill(
            sub, sub_cu, heads=H, eps=w.eps, nthreads=cores, flags=0x08),
            args.cpu_seconds)
        rates = sorted(sub_updates * r / el for r, el in runs)
        cpu = {"value": round(float(np.median(rates)), 1),
               "unit": "token-head updates/s", "cores": cores,
               "kind": "oracle",
               "sample": f"4 shortest sequences ({int(sub_lens.sum())} "
                         f"tokens), median of 3 runs of "
                         f"{args.cpu_seconds / 3:.1f} s, {cores} threads, "
                         f"{info['model']}",
               "runs_updates_per_s": [round(r, 1) for r in rates],
               "host": info}
    line = {
        "metric": "KDA prefill token-head updates/sec (variable length)",
        "value": round(updates * K / wall, 1), "unit": "updates/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill_16seq_h48", "sequences": N,
                   "tokens": total, "lengths": lens.tolist(), "heads": H,
                   "qk_l2norm": True, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP32_MFMA_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
        "extra": {"kernel_us": round(kern * 1e6, 2),
                  "path": "kda_prefill_chunked (16-token chunks; fp32 "
                          "products as 3-piece bf16 on the matrix cores)",
                  "bf16_mfma_tflops_executed": round(
                      chunks * H * CHUNK_BF16_MFMA * 16384 / kern / 1e12, 1),
                  "bf16_mfma_frac_executed": round(
                      chunks * H * CHUNK_BF16_MFMA * 16384 / kern / 1e12
                      / BF16_MFMA_TFLOPS, 4),
                  "chunk_heads": chunks * H,
                  "mfma_flop_per_chunk_head": flop_chunk,
                  "longest_sequence_chunks": int((lens.max() + 15) // 16),
                  "us_per_chunk_on_longest": round(
                      kern * 1e6 / int((lens.max() + 15) // 16), 3),
                  "hbm_GBs": round(nbytes / kern / 1e9, 1),
                  "sequential_kernel_us": round(kern_seq * 1e6, 2),
                  "speedup_vs_sequential": round(kern_seq / kern, 2),
                  "two_pass_us": round(kern_two * 1e6, 2),
                  "raw_gates_us": round(kern_raw * 1e6, 2),
                  "ascending_order_us": round(kern_asc * 1e6, 2),
                  "chunk_metadata_us": round(meta_us, 2)},
    }
    print(json.dumps(line), flush=True)


def raw_inputs(w, layer, np, synth):
    """Seeded raw gate inputs and conv bias of one layer (host arrays)."""
    rng = np.random.default_rng([w.seed, layer, 2])
    B, H, C = w.batch, w.heads, w.channels
    return {
        "raw_g": synth.to_bf16_bits(
            rng.normal(0, 2, (B, H, 128)).astype(np.float32)),
        "raw_beta": synth.to_bf16_bits(
            rng.normal(0, 1, (B, H)).astype(np.float32)),
        "A_log": rng.normal(0, 0.5, H).astype(np.float32),
        "dt_bias": rng.normal(0, 0.5, C).astype(np.float32),
        "conv_bias": rng.normal(0, 0.3, 3 * C).astype(np.float32),
        "lower_bound": -5.0,
    }


def rotated_pools(torch, np, stream, t, call, alg_bytes, steps,
                  copies=4):
    """The same call timed over ``copies`` copies of the state pools in
    turn (call i on copy i mod copies), so that a pool is re-read only after
    the other copies' state has streamed through the 256 MB last-level
    (Infinity) cache: the uncached figure for workloads whose touched state
    fits in that cache (the b64/h24 call touches ~100 MB).  The headline
    timing reuses one pool back to back."""
    pools = [(t["conv_state"], t["rec_state"])]
    for _ in range(copies - 1):
        pools.append((t["conv_state"].clone(), t["rec_state"].clone()))
    views = [dict(t, conv_state=cs, rec_state=rs) for cs, rs in pools]
    for v in views:
        call(v, stream)
    torch.cuda.synchronize()
    n = max(copies * 10, steps)
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        call(views[i % copies], stream)
        e1.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    del views, pools
    return {"copies": copies, "calls": n,
            "kernel_us": {"mean": round(float(us.mean()), 2),
                          "p50": round(float(np.percentile(us, 50)), 2)},
            "GBs": round(alg_bytes / (float(us.mean()) * 1e-6) / 1e9, 1)}


def copy_probe(torch, stream, nbytes=1 << 30, reps=10):
    """A plain device copy of known size (torch's elementwise copy kernel
    reading and writing ``nbytes`` each): a measured bandwidth reference
    on the same GPU, and the calibration launch for the HBM byte counters
    (its FETCH_SIZE / WRITE_SIZE per dispatch correspond to ``nbytes``)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return {"bytes_read": nbytes, "bytes_written": nbytes,
            "us_per_copy": round(sec * 1e6, 2),
            "GBs": round(2 * nbytes / sec / 1e9, 1)}


def stream_ceiling(torch, kda, stream, w, live_rows, alg_bytes, kern_s,
                   reps=10):
    """What HBM delivers to this access pattern when reads and writes run
    alone: the state-tile probe in read-only and in write-only mode over as
    many [128, 128] fp32 tiles as the call has live units, and the time the
    call's own reads and writes would take one after the other at those
    rates (small reads priced at the read rate, conv-state and output
    writes at the write rate).  A kernel that overlaps its reads with its
    writes can beat that serial time; the ratio says how far it does."""
    D = 128
    live_units = live_rows * w.heads
    null_units = (w.batch - live_rows) * w.heads
    conv_state = 3 * D * (w.conv_width - 1) * 2
    wbytes = live_units * (D * D * 4 + conv_state + D * 2) + null_units * D * 2
    rbytes = alg_bytes - wbytes
    tiles = torch.randn(live_units, D, D, dtype=torch.float32, device="cuda:0")
    rates = {}
    for name, mode in (("read", kda.PROBE_READ), ("write", kda.PROBE_WRITE)):
        for _ in range(3):
            kda.state_stream_probe(tiles, 16, mode=mode, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            kda.state_stream_probe(tiles, 16, mode=mode, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / reps
        rates[name] = tiles.numel() * 4 / sec / 1e9
    del tiles
    bound = rbytes / (rates["read"] * 1e9) + wbytes / (rates["write"] * 1e9)
    return {"read_GBs": round(rates["read"], 1),
            "write_GBs": round(rates["write"], 1),
            "call_bytes_read": int(rbytes), "call_bytes_written": int(wbytes),
            "serial_us": round(bound * 1e6, 2),
            "serial_over_kernel": round(bound / kern_s, 4)}


def cpu_threads():
    """Threads for the CPU oracle: every CPU this process may run on
    (its affinity mask), capped by OMP_NUM_THREADS when that is set (the
    GPU host allots each GPU's jobs a CPU share through it).  Returns the
    count and the facts it came from."""
    nproc = os.cpu_count() or 1
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = nproc
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = max(1, min(allowed, omp) if omp > 0 else allowed)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, {"nproc": nproc, "affinity_cpus": allowed,
                     "omp_num_threads": omp or None, "model": model}


def timed_runs(fn, seconds, runs=3):
    """``runs`` timed runs of ``fn`` (each repeated until seconds / runs
    have passed); returns [(calls, elapsed)] per run."""
    res = []
    for _ in range(runs):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds / runs:
                break
        res.append((reps, el))
    return res


def cpu_baseline(w, inp, seconds, alg_bytes, units, flags=0, tokens=1):
    """The CPU oracle (fp32, OpenMP over units) on the same batch, in
    place: the median rate of three runs of about seconds / 3 each on every
    allotted core, and one run of about seconds / 5 on one thread."""
    import numpy as np

    import oracle

    cores, info = cpu_threads()
    oracle.lib()
    print(f"[bench] cpu oracle on {cores} threads ({info})", file=sys.stderr,
          flush=True)

    def one_call(work, nthreads):
        def fn():
            if tokens > 1:
                oracle.decode_tokens(work, heads=w.heads, tokens=tokens,
                                     norm=w.norm, eps=w.eps, dtype="f32",
                                     nthreads=nthreads, flags=flags,
                                     inplace=True)
            else:
                oracle.decode(work, heads=w.heads, norm=w.norm, eps=w.eps,
                              dtype="f32", nthreads=nthreads, inplace=True,
                              flags=flags)
        return fn

    work = dict(inp, conv_state=inp["conv_state"].copy(),
                rec_state=inp["rec_state"].copy())
    runs = timed_runs(one_call(work, cores), seconds)
    rates = sorted(units * r / el for r, el in runs)
    rate = float(np.median(rates))
    (reps1, el1), = timed_runs(one_call(work, 1), seconds / 5, runs=1)
    del work
    return {"value": round(rate, 1), "unit": "updates/s",
            "cores": cores, "kind": "oracle",
            "sample": (f"{'one layer of the ' if w.layers > 1 else ''}"
                       f"full {w.name} batch ({units} updates) in place, "
                       f"median of 3 runs of {seconds / 3:.1f} s "
                       f"({', '.join(str(r) for r, _ in runs)} calls), fp32, "
                       f"{cores} threads, {info['model']}"),
            "runs_updates_per_s": [round(r, 1) for r in rates],
            "host": info,
            "GBs": round(alg_bytes * rate / units / 1e9, 2),
            "single_thread": {"value": round(units * reps1 / el1, 1),
                              "unit": "updates/s", "calls": reps1,
                              "seconds": round(el1, 1)}}


if __name__ == "__main__":
    main()
