"""Benchmark of the TurboQuant KV hot path on one MI355X.

Workload (default): the 32-layer Llama-3.1-8B-shaped stack, batch 4, 32 q / 8 kv heads,
head_dim 128, 32768-token context quantised from bf16 (3-bit keys + QJL, 2-bit values), then
one decode step over all 32 layers.

One step = one pass of the whole path over one batch of synthetic input:
  1. tq_quantize_kv   -- compress the prefill history (Q1-Q6) of every (layer, batch, kv head)
  2. tq_decode_step   -- per layer: one decode-time token per slice into the exact ring (R1,
                         inside the decode kernel) and hybrid attention over packed history +
                         ring (D1-D5)
  3. tq_flush         -- compress the ring contents into the packed store (R2)

Reported:
  * value = decode KV-tokens/s: batch * layers * (packed + ring) context tokens per second of
    decode time (all layers' decode calls), timed back to back over stores that were not
    written or read within the last 512 MB of traffic (the Infinity Cache holds 256 MB);
  * quantize tokens/s (the history's batch * layers * tokens per second of tq_quantize_kv),
    over inputs cycled the same way;
  * ms_per_step: the whole step (quantize + decode + flush) back to back;
  * roofline objects for the dominant kernel of the step and for the decode kernel set,
    achieved = algorithmic bytes per launch / average launch time (HIP events on the stream the
    kernels run on), with measured HBM traffic from the committed rocprofv3 counter summary;
  * cpu_baseline: the oracle on a bounded sample, on the host's cores (threads over slices).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
HBM_PEAK_GBPS = 8000.0
METRIC = "packed-KV decode attention KV-tokens/s + HBM GB/s; quantize tokens/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=5,
                   help="workload id (1..5); 5 = 32 layers x batch 4 x 32K context (the default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--key-bits", type=int, default=0,
                   help="codebook bits per key coordinate (1..4) instead of the workload's 3; the workload "
                        "name gets a _kb<N> suffix")
    p.add_argument("--head-dim", type=int, default=0,
                   help="head_dim (64 or 128) instead of the workload's; the workload name gets a _d<N> suffix")
    p.add_argument("--paged", type=int, default=0, metavar="PAGE_TOKENS",
                   help="keep the packed cache in pages of this many tokens (a multiple of 32), in a "
                        "seeded random page order per slice")
    p.add_argument("--ragged", action="store_true",
                   help="time only the decode, over a ragged batch: sequence b attends to its own seeded "
                        "lengths (packed uniform in [1, packed tokens], ring uniform in [0, ring tokens])")
    p.add_argument("--prefill", type=int, default=0, metavar="QUERY_TOKENS",
                   help="time only prefill attention over the packed cache (layer 0): the last QUERY_TOKENS "
                        "tokens of every sequence's history as causal queries")
    p.add_argument("--kivi", action="store_true",
                   help="time the KIVI 2-bit variant instead (quantize every layer's history into a KIVI "
                        "store, decode attention of every layer over it): its own JSON line")
    p.add_argument("--cpu-sample-tokens", type=int, default=32768)
    p.add_argument("--probe-copy-mib", type=int, default=0,
                   help="only time a plain device-to-device copy of this many MiB (achievable HBM "
                        "bandwidth; also the known-size kernel that calibrates the traffic counters)")
    return p.parse_args()


def probe_copy(mib: int, steps: int):
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    moved = 2 * n * 4
    print(json.dumps({"probe": "device copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": round(ms, 4), "GBps": round(moved / ms / 1e6, 1),
                      "frac_of_8TBps": round(moved / ms / 1e6 / HBM_PEAK_GBPS, 4)}), flush=True)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this workload,
    or None when there is none or the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic__{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if not rec:
        return None
    h = hashlib.sha1()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, "compressed_decode_attention_02_amd", "csrc", f), "rb").read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha1"] else None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    if args.probe_copy_mib:
        probe_copy(args.probe_copy_mib, args.steps)
        return
    import numpy as np
    import torch

    import tq_workloads as W
    import compressed_decode_attention_02_amd as tq

    w = W.WORKLOADS[args.config]
    if args.head_dim and args.head_dim != w.d:
        w = dataclasses.replace(w, d=args.head_dim, name=f"{w.name}_d{args.head_dim}")
    if args.key_bits and args.key_bits != w.key_bits:
        w = dataclasses.replace(w, key_bits=args.key_bits, name=f"{w.name}_kb{args.key_bits}")
    dev = torch.device("cuda:0")
    if args.kivi:
        kivi(args, w, dev)
        return
    d, L, B, hq, hkv = w.d, w.layers, w.batch, w.hq, w.hkv
    n_sl_layer = B * hkv
    n_sl = L * n_sl_layer
    Tp = w.n_packed
    ring_fill = max(w.n_ring - 1, 0)  # the step's append brings the ring to n_ring tokens
    cfg = tq.make_config(d, w.key_bits, w.value_bits, 32, w.buffer_size)
    tables = tq.Tables(cfg, W.TABLE_SEED, device=dev)
    rec = tq.tq_packed_bytes_per_token(cfg)
    in_bytes = 2 if w.in_dtype == "bf16" else 4

    # Working sets: the quantize leg cycles n_in copies of the history K/V and the decode leg
    # n_dec copies of the packed store (with its ring, queries and outputs), enough that each
    # leg streams at least 512 MB (twice the 256 MB Infinity Cache) before it touches the same
    # bytes again.  The large workloads need a single copy.
    mall2 = 2 * 256 * 10**6
    in_bytes_all = n_sl * Tp * 2 * d * in_bytes
    dec_bytes_all = n_sl * ((Tp + w.n_ring) * rec)
    n_in = max(1, math.ceil(mall2 / in_bytes_all))
    n_dec = max(1, math.ceil(mall2 / max(dec_bytes_all, 1)))
    inputs = []
    for c in range(n_in):
        ks, vs = [], []
        for layer in range(L):
            k, v = W.device_kv(w, layer + 1000 * c, Tp, dev)
            ks.append(k.reshape(n_sl_layer, Tp, d))
            vs.append(v.reshape(n_sl_layer, Tp, d))
        K = torch.cat(ks).contiguous() if L > 1 else ks[0]
        V = torch.cat(vs).contiguous() if L > 1 else vs[0]
        del ks, vs
        inputs.append((K, V))
    kn, vn = W.device_kv(w, 7777, 1, dev, tensor_ids=(3, 4))
    kn = kn.reshape(n_sl_layer, d).repeat(L, 1).contiguous()
    vn = vn.reshape(n_sl_layer, d).repeat(L, 1).contiguous()
    copies = []
    for c in range(n_dec):
        if args.paged:
            pps = -(-(Tp + w.buffer_size) // args.paged)
            store = tq.PagedStore(cfg, n_sl, args.paged, pps, n_sl * pps, seed=c, device=dev)
        else:
            store = tq.PackedStore(cfg, n_sl, Tp + w.buffer_size, device=dev)
        ring = tq.Ring(cfg, n_sl, device=dev)
        qs = [W.device_queries(w, layer + 1000 * c, dev) for layer in range(L)]
        outs = [torch.zeros((B, hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
        ws = tq.new_workspace(cfg, B, hq, hkv, Tp + w.buffer_size, device=dev)
        # each layer's decode step, its arguments checked and marshalled once (as a model would
        # hold its layers' cache views), so that the timed loop only launches
        steps = []
        if w.n_ring > 0:
            for layer in range(L):
                off = layer * n_sl_layer
                steps.append(tq.PreparedDecodeStep(cfg, tables, qs[layer], B, hq, hkv, store.struct(off),
                                                   ring.struct(off), kn[off:off + n_sl_layer], vn[off:off + n_sl_layer],
                                                   1.0 / math.sqrt(d), outs[layer], ws))
        # pre-fill ring slots [0, ring_fill) so that the step's append brings it to n_ring tokens
        for t in range(ring_fill):
            tq.tq_append_ring(cfg, ring.struct(), kn, vn, n_sl, t)
        # the history of every store copy, compressed once (the decode leg reads it)
        K, V = inputs[c % n_in]
        tq.tq_quantize_kv(cfg, tables, K, V, n_sl, Tp, store.struct(), 0)
        copies.append(dict(store=store, ring=ring, qs=qs, outs=outs, ws=ws, steps=steps))
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    def quantize(i):
        K, V = inputs[i % n_in]
        tq.tq_quantize_kv(cfg, tables, K, V, n_sl, Tp, copies[i % n_dec]["store"].struct(), 0)

    def decode_all_layers(i):
        cp = copies[i % n_dec]
        st, rg = cp["store"], cp["ring"]
        for layer in range(L):
            off = layer * n_sl_layer
            if w.n_ring > 0:
                # the decode step: the layer's new token into ring slot ring_fill (inside the
                # decode kernel), then attention over packed + ring
                cp["steps"][layer](Tp, ring_fill)
            else:
                tq.tq_decode_attention(cfg, tables, cp["qs"][layer], B, hq, hkv, st.struct(off), Tp,
                                       None, 0, scale, cp["outs"][layer], cp["ws"])

    def flush(i):
        if w.n_ring > 0:
            cp = copies[i % n_dec]
            tq.tq_flush(cfg, tables, cp["ring"].struct(), n_sl, w.n_ring, cp["store"].struct(), Tp)

    def step(i):
        quantize(i)
        decode_all_layers(i)
        flush(i)

    def back_to_back(fn, k):
        """Mean ms of fn(i), k calls back to back with no events between them."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(k):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / k

    def per_call(fn, k):
        """Per-call ms from HIP events recorded around each call on the kernels' stream (an
        event between two launches adds a few microseconds of idle time)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        torch.cuda.synchronize()
        for i in range(k):
            evs[i][0].record(stream)
            fn(i)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.ragged:
        ragged(args, w, cfg, tables, copies, n_dec, scale, rec, in_bytes, kn, vn)
        return
    if args.prefill:
        prefill(args, w, cfg, tables, copies, n_dec, scale, rec, in_bytes)
        return

    K_ = args.steps
    ms_step = back_to_back(step, K_)
    ms_dec = back_to_back(decode_all_layers, K_)
    ms_q = back_to_back(quantize, K_)
    dec_calls = per_call(decode_all_layers, K_)
    q_calls = per_call(quantize, K_)
    f_calls = per_call(flush, K_) if w.n_ring > 0 else [0.0]

    def pct(xs, p):
        xs = sorted(xs)
        return xs[min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))]

    ctx = Tp + w.n_ring
    kv_tokens = B * L * ctx
    q_bytes = n_sl * Tp * (2 * d * in_bytes + rec)
    # per layer: packed records, ring tokens (fp16 K and V; the step's new token is read from its
    # input instead and written to the ring once), queries in, outputs out
    dec_bytes = L * (n_sl_layer * (Tp * rec + w.n_ring * 4 * d + (2 * d * in_bytes if w.n_ring else 0))
                     + B * hq * d * (in_bytes + 4))
    q_gbps = q_bytes / (ms_q * 1e-3) / 1e9
    d_gbps = dec_bytes / (ms_dec * 1e-3) / 1e9
    q_kernels = "k_quant_kv"
    # decode kernel set: a prep launch only at head_dim 256 (at 128 the main kernel prepares
    # the queries itself); the merge launch only when a slice has several splits; the other key
    # widths and head_dim 64: prep, the fp32 decode kernel, merge
    if w.key_bits != 3 or d == 64:
        d_kernels = "k_decode_prep+k_decode_any+k_decode_merge"
    else:
        d_kernels = ("k_decode_prep+" if d == 256 else "") + "k_decode_main+k_decode_merge"
    roof_q = {"kernel": q_kernels, "bound": "hbm", "achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS,
              "unit": "GB/s", "frac": round(q_gbps / HBM_PEAK_GBPS, 4),
              "traffic": measured_traffic(w.name, q_kernels), "algorithmic_bytes_per_launch": q_bytes,
              "launch_ms_mean": round(ms_q, 4)}
    roof_d = {"kernel": d_kernels, "bound": "hbm", "achieved": round(d_gbps, 1), "peak": HBM_PEAK_GBPS,
              "unit": "GB/s", "frac": round(d_gbps / HBM_PEAK_GBPS, 4),
              "traffic": measured_traffic(w.name, d_kernels), "algorithmic_bytes_per_launch": dec_bytes // L,
              "launch_ms_mean": round(ms_dec / L, 5)}
    dominant = roof_q if ms_q >= ms_dec else roof_d

    res = {
        "metric": METRIC,
        "value": round(kv_tokens / (ms_dec * 1e-3), 1),
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic (seeded device draws of the workload's laws)",
        "config": {"workload": w.name, "layers": L, "batch": B, "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "packed_tokens": Tp, "ring_tokens": w.n_ring, "key_bits": w.key_bits, "qjl_bits": 1,
                   "value_bits": w.value_bits, "group": 32, "parallelism": "none (1 GPU)",
                   "input_copies": n_in, "store_copies": n_dec, "paged": args.paged or None},
        "value_is": "decode KV-tokens/s: batch * layers * (packed + ring) per second of all layers' decode calls",
        "decode_ms_per_step": {"mean": round(ms_dec, 4), "p10": round(pct(dec_calls, 10), 4),
                               "p50": round(pct(dec_calls, 50), 4), "p90": round(pct(dec_calls, 90), 4)},
        "quantize_ms": {"mean": round(ms_q, 4), "p10": round(pct(q_calls, 10), 4),
                        "p50": round(pct(q_calls, 50), 4), "p90": round(pct(q_calls, 90), 4)},
        "flush_ms_median": round(statistics.median(f_calls), 4),
        "step_kv_tokens_per_s": round(kv_tokens / (ms_step * 1e-3), 1),
        "quantize_tokens_per_s": round(B * L * Tp / (ms_q * 1e-3), 1),
        "quantize_GBps": round(q_gbps, 1),
        "decode_GBps": round(d_gbps, 1),
        "roofline": dominant,
        "roofline_quantize": roof_q,
        "roofline_decode": roof_d,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)


def ragged(args, w, cfg, tables, copies, n_copies, scale, rec, in_bytes, kn=None, vn=None):
    """Decode-only timing over a ragged batch (per-sequence lengths on the device), against the
    uniform decode of the same stores at the maxima, HIP events around K back-to-back calls."""
    import numpy as np
    import torch
    import compressed_decode_attention_02_amd as tq
    d, L, B, hq, hkv, Tp = w.d, w.layers, w.batch, w.hq, w.hkv, w.n_packed
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cid, 0, 9])))
    lp = r.integers(1, Tp + 1, size=B)
    lr = r.integers(0, w.n_ring + 1, size=B)
    sp = torch.tensor(lp, dtype=torch.int64, device="cuda")
    sr = torch.tensor(lr, dtype=torch.int32, device="cuda")
    n_sl_layer = B * hkv

    def run(rag: bool):
        for i in range(args.warmup):
            call(i % n_copies, rag)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            call(i % n_copies, rag)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def call(c, rag):
        cp = copies[c]
        for layer in range(L):
            off = layer * n_sl_layer
            if rag:
                tq.tq_decode_attention_ragged(cfg, tables, cp["qs"][layer], B, hq, hkv, cp["store"].struct(off), sp,
                                              Tp, cp["ring"].struct(off), sr, w.n_ring, scale, cp["outs"][layer],
                                              cp["ws"])
            else:
                tq.tq_decode_attention(cfg, tables, cp["qs"][layer], B, hq, hkv, cp["store"].struct(off), Tp,
                                       cp["ring"].struct(off), w.n_ring, scale, cp["outs"][layer], cp["ws"])

    ms_r = run(True)
    ms_u = run(False)
    kv_r = int(L * (lp.sum() + lr.sum()))
    bytes_r = L * (hkv * int((lp * rec + lr * 4 * d).sum()) + B * hq * d * (in_bytes + 4))
    print(json.dumps({
        "metric": "ragged-batch decode attention KV-tokens/s + HBM GB/s",
        "value": round(kv_r / (ms_r * 1e-3), 1), "unit": "KV-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_r, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.in_dtype, "data": "synthetic (seeded device draws of the workload's laws)",
        "config": {"workload": w.name + "_ragged", "layers": L, "batch": B, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "packed_tokens_max": Tp, "ring_tokens_max": w.n_ring,
                   "packed_lengths": "uniform [1, %d], seeded" % Tp, "ring_lengths": "uniform [0, %d], seeded" % w.n_ring,
                   "mean_packed": round(float(lp.mean()), 1), "mean_ring": round(float(lr.mean()), 1)},
        "decode_GBps": round(bytes_r / (ms_r * 1e-3) / 1e9, 1),
        "roofline_decode": {"kernel": ("k_decode_prep+" if d == 256 else "") + "k_decode_main+k_decode_merge",
                            "bound": "hbm", "achieved": round(bytes_r / (ms_r * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(bytes_r / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "traffic": None, "algorithmic_bytes_per_launch": bytes_r // L},
        "uniform_at_maxima_ms": round(ms_u, 4),
    }), flush=True)


def prefill(args, w, cfg, tables, copies, n_copies, scale, rec, in_bytes):
    """Prefill attention over the packed cache of layer 0: the last T tokens of every
    sequence's history as causal query tokens (query token i at position n_packed - T + i),
    HIP events around K back-to-back calls."""
    import torch
    import compressed_decode_attention_02_amd as tq
    d, B, hq, hkv, Tp = w.d, w.batch, w.hq, w.hkv, w.n_packed
    T = min(args.prefill, Tp)
    pos0 = Tp - T
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.cid * 1000 + 17)
    dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    q = torch.randn((B, T, hq, d), generator=gen, device="cuda", dtype=torch.float32).to(dt)
    out = torch.empty((B, T, hq, d), dtype=torch.float32, device="cuda")
    ws = tq.new_prefill_workspace(cfg, B, T, hq, hkv, Tp)

    def call(c):
        tq.tq_prefill_attention(cfg, tables, q, B, T, hq, hkv, copies[c]["store"].struct(0), Tp, pos0, True, scale,
                                out, ws)
    for i in range(args.warmup):
        call(i % n_copies)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        call(i % n_copies)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the tiled kernel is bound by its matrix-core products: per (query row, visible packed
    # token) the estimate takes two d-long dot products (centroids, signs) and the value sum one
    # more, 6 d flops; the kernel issues 14 d (fp16 hi + lo operands: four score products and
    # three value products of 2 d each).  Bytes: every sequence's records once, queries in,
    # outputs out.
    pairs = B * hq * sum(min(Tp, pos0 + i + 1) for i in range(T))
    alg_flops = 6 * d * pairs
    issued_flops = 14 * d * pairs
    alg = B * hkv * Tp * rec + B * T * hq * d * (in_bytes + 4)
    tflops = alg_flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "prefill attention over the packed cache: query tokens/s",
        "value": round(B * T / (ms * 1e-3), 1), "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.in_dtype, "data": "synthetic (seeded device draws of the workload's laws)",
        "config": {"workload": w.name + "_prefill%d" % T, "layers": 1, "batch": B, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "packed_tokens": Tp, "query_tokens": T, "causal": True, "first_position": pos0,
                   "key_bits": w.key_bits, "value_bits": w.value_bits},
        "roofline": {"kernel": "k_prefill_prep + k_prefill_tile (+ k_decode_merge), per call", "bound": "mfma",
                     "achieved": round(tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_call": alg_flops, "issued_mfma_flops_per_call": issued_flops,
                     "issued_frac": round(issued_flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                     "hbm_GBps": round(alg / (ms * 1e-3) / 1e9, 1)},
    }), flush=True)


def kivi(args, w, dev):
    """The KIVI 2-bit variant on the workload's shapes: one quantize call over every layer's
    history (whole 32-token groups), then every layer's decode attention over its store; HBM-cold
    copies as in the main leg; HIP events around K back-to-back repetitions of each leg."""
    import torch
    import tq_workloads as W
    import compressed_decode_attention_02_amd as tq
    d, L, B, hq, hkv = w.d, w.layers, w.batch, w.hq, w.hkv
    Tp = w.n_packed // 32 * 32
    n_sl_layer = B * hkv
    n_sl = L * n_sl_layer
    rec = tq.tq_kivi_bytes_per_token(d)
    in_bytes = 2 if w.in_dtype == "bf16" else 4
    mall2 = 2 * 256 * 10**6
    n_cp = max(1, math.ceil(mall2 / (n_sl * Tp * rec)))
    ks, vs = [], []
    for layer in range(L):
        k, v = W.device_kv(w, layer, w.n_packed, dev)
        ks.append(k.reshape(n_sl_layer, w.n_packed, d)[:, :Tp].contiguous())
        vs.append(v.reshape(n_sl_layer, w.n_packed, d)[:, :Tp].contiguous())
    K = torch.cat(ks).contiguous() if L > 1 else ks[0]
    V = torch.cat(vs).contiguous() if L > 1 else vs[0]
    del ks, vs
    stores = [tq.KiviStore(d, n_sl, Tp, device=dev) for _ in range(n_cp)]
    qs = [W.device_queries(w, layer, dev) for layer in range(L)]
    out = torch.empty((B, hq, d), dtype=torch.float32, device=dev)
    ws = tq.new_kivi_workspace(d, B, hq, hkv, Tp, device=dev)
    scale = 1.0 / math.sqrt(d)

    def quant(i):
        tq.tq_kivi_quantize(d, K, V, n_sl, Tp, stores[i % n_cp].struct(), 0)

    def dec(i):
        st = stores[i % n_cp]
        for layer in range(L):
            tq.tq_kivi_decode_attention(d, qs[layer], B, hq, hkv, st.struct(layer * n_sl_layer), Tp, scale, out, ws)

    for i in range(max(args.warmup, n_cp)):
        quant(i)
        dec(i)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    ms_q, ms_d = timed(quant), timed(dec)
    q_bytes = n_sl * Tp * (2 * d * in_bytes + rec)
    d_bytes = n_sl * Tp * rec + L * B * hq * d * (in_bytes + 4)
    dg = d_bytes / (ms_d * 1e-3) / 1e9
    qg = q_bytes / (ms_q * 1e-3) / 1e9
    print(json.dumps({
        "metric": "KIVI 2-bit decode attention KV-tokens/s + HBM GB/s; quantize tokens/s",
        "value": round(B * L * Tp / (ms_d * 1e-3), 1), "unit": "KV-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_d + ms_q, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.in_dtype, "data": "synthetic (seeded device draws of the workload's laws)",
        "config": {"workload": w.name + "_kivi2", "layers": L, "batch": B, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "packed_tokens": Tp, "bits": 2, "key_group": 32, "store_copies": n_cp},
        "decode_ms_per_step": round(ms_d, 4), "quantize_ms": round(ms_q, 4),
        "quantize_tokens_per_s": round(B * L * Tp / (ms_q * 1e-3), 1), "record_bytes": rec,
        "roofline_decode": {"kernel": "k_kivi_decode+k_decode_merge", "bound": "hbm", "achieved": round(dg, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(dg / HBM_PEAK_GBPS, 4),
                            "traffic": None, "algorithmic_bytes_per_launch": d_bytes // L},
        "roofline_quantize": {"kernel": "k_kivi_quant", "bound": "hbm", "achieved": round(qg, 1),
                              "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(qg / HBM_PEAK_GBPS, 4),
                              "traffic": None, "algorithmic_bytes_per_launch": q_bytes},
    }), flush=True)


def host_cpu():
    """(threads to use, logical CPUs seen, CPU model): the pool is sized to the CPUs this
    process may run on, at most 16 (a one-GPU share of the host)."""
    n_aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return max(1, min(16, n_aff)), os.cpu_count() or 1, model


def cpu_baseline(w, sample_tokens: int):
    """The oracle (plain C, fp64, unchanged) timed on a bounded sample of the same step, with
    host threads over independent slices (the oracle's C calls release the interpreter lock):
    quantize `sample_tokens` tokens of every kv head of one layer and one batch element (in
    chunks of rows), then decode all q heads of that batch element over those tokens (one
    kv head's query group per task).  value = decode KV-tokens/s of the sample."""
    import concurrent.futures

    import numpy as np

    import oracle as O
    import tq_workloads as W

    d = w.d
    T = min(sample_tokens, w.n_packed)
    ws = W.custom(w.cid, batch=1)
    (k, v), _ = W.host_kv(ws, 0, T)
    k = k.reshape(ws.hkv * T, d).astype(np.float64)
    v = v.reshape(ws.hkv * T, d).astype(np.float64)
    q, _ = W.host_queries(ws, 0)
    q = q.astype(np.float64)
    c32, b32 = O.stored_codebook(d, w.key_bits)
    sigma, S = O.tables(d, W.TABLE_SEED)
    O.lib()
    threads, ncpu, model = host_cpu()
    chunk = 1024
    spans = [(r, min(r + chunk, k.shape[0])) for r in range(0, k.shape[0], chunk)]

    def quant(span):
        a, b = span
        kq = O.quantize_keys(k[a:b], c32, b32, sigma, S, kb=w.key_bits)
        vq = O.quantize_values(v[a:b], w.value_bits)
        return (O.pack_keys(kq["idx"], kq["z"], w.key_bits), np.stack([kq["norm"], kq["rnorm"]], 1).astype(np.float32),
                O.pack_values(vq["code"], w.value_bits), vq["scale"])

    G = ws.hq // ws.hkv
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        parts = list(ex.map(quant, spans))
        t1 = time.perf_counter()
        kw = np.concatenate([p_[0] for p_ in parts]).reshape(ws.hkv, T, -1)
        kn = np.concatenate([p_[1] for p_ in parts]).reshape(ws.hkv, T, 2)
        vw = np.concatenate([p_[2] for p_ in parts]).reshape(ws.hkv, T, -1)
        vs = np.concatenate([p_[3] for p_ in parts]).reshape(ws.hkv, T, -1)

        def dec(h):
            return O.decode(d=d, kb=w.key_bits, vb=w.value_bits, c32=c32, sigma=sigma, S_bits=S, B=1, Hq=G, Hkv=1,
                            kw=kw[h:h + 1], kn=kn[h:h + 1], vw=vw[h:h + 1], vs=vs[h:h + 1], cap=T, n_packed=T,
                            rk=None, rv=None, buf=0, n_ring=0, q=q[:, h * G:(h + 1) * G], scale=1 / math.sqrt(d))

        t2 = time.perf_counter()
        list(ex.map(dec, range(ws.hkv)))
        t3 = time.perf_counter()
    return {"value": round(T / (t3 - t2), 1), "unit": "KV-tokens/s", "cores": threads, "kind": "oracle",
            "quantize_tokens_per_s": round(T / (t1 - t0), 1),
            "host": {"logical_cpus": ncpu, "threads_used": threads, "cpu_model": model},
            "sample": f"1 layer, batch 1: {ws.hkv} kv heads x {T} tokens quantized ({t1 - t0:.2f} s), then decode "
                      f"of {ws.hq} q heads over them ({t3 - t2:.2f} s); fp64 C oracle on {threads} threads over "
                      f"slices (row chunks of {chunk} for the quantize, one kv head's query group per decode task)"}


if __name__ == "__main__":
    main()
