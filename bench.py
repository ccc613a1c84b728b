"""Benchmark of the relative-attention hot path on one MI355X.

A step is one prefill call (the whole forward: scores, relative bias, mask,
online softmax, PV, epilogue) of the sliding-window layer (B=1, T=8192,
Hq=16, Hkv=2, D=128, d_r=128, rel_extent=1024, window=1024, bf16) on inputs
already resident in HBM.  The line also reports the split-KV decode of 64
sequences x 8192 keys (KV GB/s), each against its roofline, and the fp64 CPU
oracle timed on a bounded sample of the prefill workload; the paged decode,
the extend (chunked prefill) and the attention prologue of an 8192-token
prefill (K/V ShortConv, Q/K RMSNorm, cache write; HBM GB/s) ride along.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibration   (a plain 1 GiB device copy, for
       scaling the HBM byte counters FETCH_SIZE / WRITE_SIZE under rocprofv3)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
PREFILL_WORKLOAD = "swa_prefill_8k"
DECODE_WORKLOAD = "decode_64x8k"
EXTEND_WORKLOAD = "extend_4x1k_8k_paged"
PAGED_DECODE_WORKLOAD = "decode_paged_64x8k"
PROLOGUE_WORKLOAD = "prologue_8k"
BACKWARD_WORKLOAD = "swa_backward_8k"
PREFILL_KERNEL = "prefill_dma_kernel"  # the bf16 path for eight or more query heads per kv head
DECODE_KERNEL = "decode_split_kernel"


def prefill_work(T: int, Hq: int, D: int, d_r: int, E: int, W: int, rows=None):
    """Algorithmic flops of a prefill: 4*D per visible (i, j, h) pair (q.k and
    p.v) plus 2*d_r per needed relative-logit entry (r.P for distances
    0..min(i, E-1) that the mask leaves visible).  Masked pairs, skipped tiles
    and softmax arithmetic are not counted."""
    if rows is None:
        rows = range(T)
    pairs = 0
    rel = 0
    for i in rows:
        vis = i + 1 if W == 0 else min(i + 1, W)
        pairs += vis
        rel += min(vis, E)
    return Hq * (pairs * 4 * D + rel * 2 * d_r), Hq * pairs, Hq * rel


def backward_work(T: int, Hq: int, D: int, d_r: int, E: int, W: int):
    """Algorithmic flops of a backward: 10*D per visible (i, j, h) pair (q.k
    recomputed, dout.v, and the dq, dk and dv products) plus 4*d_r per needed
    relative-logit entry (r.P recomputed, and dr).  The forward's convention
    otherwise: masked pairs, skipped tiles and the softmax are not counted."""
    _, pairs, rel = prefill_work(T, Hq, D, d_r, E, W)
    return pairs * 10 * D + rel * 4 * d_r


def decode_bytes(B: int, L: int, Hq: int, Hkv: int, D: int, d_r: int, E: int, W: int, elem: int = 2):
    """Algorithmic HBM bytes of a decode: K and V of every visible key, plus
    q, r and out of every sequence and P once."""
    vis = L if W == 0 else min(L, W)
    kv = B * vis * Hkv * D * 2 * elem
    per_seq = B * Hq * (D + d_r + D) * elem
    return kv + per_seq + E * d_r * elem, kv


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "transformer_attention_query_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, src_hash: str):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("src_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def _time_launches(fn, steps: int, warmup: int, stream, before=None):
    """Run fn() warmup times, then `steps` times between synchronisations.
    Returns (total ms over the steps, list of per-launch ms from event pairs)."""
    import torch
    for i in range(warmup):
        if before:
            before(i)
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        if before:
            before(i)
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), [a.elapsed_time(b) for a, b in ev]


def _time_batch(fn, steps: int, warmup: int, stream):
    """Run fn() warmup times, then `steps` times back to back between one pair
    of events (no event between launches, so a short kernel is not separated
    by host time).  Returns ms per launch."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bench_prefill(steps: int, warmup: int):
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[PREFILL_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    out = torch.empty_like(x["q"])
    lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(_i):
        ra.prefill(x["q"], x["k"], x["v"], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale, out=out, lse=lse)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    flops, pairs, rel = prefill_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W)
    flops *= w.B
    ms_step = total_ms / steps
    kernel_ms = sum(per) / len(per)
    return w, flops, ms_step, kernel_ms, per


def bench_decode(steps: int, warmup: int):
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[DECODE_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    # Two copies of the cache, used alternately: each launch reads 512 MiB, so
    # the copy it reads was last touched two launches ago, far beyond the 256 MB
    # MALL and the L2s.
    k2 = [x["k"], x["k"].clone()]
    v2 = [x["v"], x["v"].clone()]
    ns, ws_bytes = ra.decode_plan(w.B, w.T, w.Hq, w.Hkv, w.D, w.num_splits, w.W, w.E)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        ra.decode(x["q"], k2[i % 2], v2[i % 2], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale,
                  num_splits=ns, workspace=ws)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    nbytes, kv = decode_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    return w, nbytes, kv, total_ms / steps, sum(per) / len(per), ns


def decode_bytes_mx(B: int, L: int, Hq: int, Hkv: int, D: int, d_r: int, E: int, W: int) -> int:
    """Algorithmic bytes of one decode call over MXFP8 caches: per visible key
    and kv head the K and V codes (D bytes each) and scales (D/32 bytes
    each); q, r and out per sequence (bf16) and P once, as for bf16."""
    vis = min(L, W) if W > 0 else L
    kv = B * vis * Hkv * 2 * (D + D // 32)
    per_seq = B * (Hq * D * 2 + Hq * d_r * 2 + Hq * D * 2)
    return kv + per_seq + E * d_r * 2


def bench_decode_mx(steps: int, warmup: int):
    """decode_64x8k over MXFP8 caches (quantised once from the bf16 ones)."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[DECODE_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    kc, ks = ra.mx_quantize(x["k"])
    vc, vs = ra.mx_quantize(x["v"])
    del x["k"], x["v"]
    # two copies, used alternately: a launch reads ~277 MB, past the 256 MB MALL
    caches = [(kc, ks, vc, vs), (kc.clone(), ks.clone(), vc.clone(), vs.clone())]
    ns, ws_bytes = ra.decode_plan(w.B, w.T, w.Hq, w.Hkv, w.D, 0, w.W, w.E)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        c = caches[i % 2]
        ra.decode_mx(x["q"], c[0], c[1], c[2], c[3], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale,
                     num_splits=ns, workspace=ws)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    nbytes = decode_bytes_mx(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    return w, nbytes, total_ms / steps, sum(per) / len(per), ns


def bench_extend(steps: int, warmup: int):
    """Chunked prefill over a paged cache: the new rows of every sequence."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[EXTEND_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    paged = w.page_size > 0
    k = x["k_pages"] if paged else x["k"]
    v = x["v_pages"] if paged else x["v"]
    bt = x["block_table"] if paged else None
    out = torch.empty_like(x["q"])
    lse = torch.empty(w.Hq, x["q"].shape[0], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(_i):
        ra.extend(x["q"], k, v, x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale, x["q_start"], x["kv_len"],
                  w.n_new, block_table=bt, out=out, lse=lse)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    flops, _, _ = prefill_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W, rows=range(w.T - w.n_new, w.T))
    return w, flops * w.B, total_ms / steps, sum(per) / len(per)


def bench_decode_paged(steps: int, warmup: int):
    """decode_64x8k over a paged cache: the same bytes through a block table."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[PAGED_DECODE_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    # two copies of the page pool, used alternately (each launch reads 512 MiB)
    kp = [x["k_pages"], x["k_pages"].clone()]
    vp = [x["v_pages"], x["v_pages"].clone()]
    ns, ws_bytes = ra.decode_plan(w.B, w.T, w.Hq, w.Hkv, w.D, 0, w.W, w.E)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        ra.decode_paged(x["q"], kp[i % 2], vp[i % 2], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale,
                        x["kv_len"], x["block_table"], w.T, num_splits=ns, workspace=ws)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    nbytes, _ = decode_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.W)
    return w, nbytes, total_ms / steps, sum(per) / len(per), ns


def prologue_bytes(N: int, B: int, Hq: int, Hkv: int, D: int, W: int, state: bool, elem: int = 2) -> int:
    """Algorithmic bytes of one prologue call: every q, k and v row read once
    and written once (q_out, the two caches), the filter and norm weights, and
    the states (read if given, always written)."""
    rows = 2 * N * (Hq + 2 * Hkv) * D * elem
    weights = (2 * Hkv * D * W + 2 * D) * elem
    st = B * 2 * 3 * Hkv * D * elem
    return rows + weights + st * (2 if state else 1)


def bench_prologue(steps: int, warmup: int):
    """The attention prologue of an 8192-token prefill, caches written in place."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[PROLOGUE_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    st_in = x.get("state_in")
    st_out = torch.empty(w.B, 2, 3, w.Hkv * w.D, dtype=x["q"].dtype, device="cuda")
    q_out = torch.empty_like(x["q"])
    stream = torch.cuda.current_stream()

    def step(_i):
        ra.prologue(x["q"], x["k"], x["v"], x["conv_k"], x["conv_v"], x["q_norm_w"], x["k_norm_w"], 1e-6,
                    x["q_start"], x["kv_len"], x["k_cache"], x["v_cache"], state_in=st_in, state_out=st_out,
                    q_out=q_out)

    total_ms, _ = _time_launches(step, steps, warmup, stream)
    # The kernel is short: time it as a batch of launches straight through the
    # C ABI (arguments marshalled once), with no events between them.
    lib = ra.load_library()
    N = w.B * w.n_new
    args = (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["conv_k"].data_ptr(), x["conv_v"].data_ptr(),
            x["q_norm_w"].data_ptr(), x["k_norm_w"].data_ptr(), 1e-6, None if st_in is None else st_in.data_ptr(),
            st_out.data_ptr(), q_out.data_ptr(), x["k_cache"].data_ptr(), x["v_cache"].data_ptr(), 1, w.B, N,
            x["q_start"].data_ptr(), x["kv_len"].data_ptr(), x["k_cache"].shape[1], None, 0, 0, 0, w.Hq, w.Hkv, w.D,
            4, stream.cuda_stream)
    fn = lib.rel_attn_prologue

    def raw(_i):
        fn(*args)

    kernel_ms = _time_batch(raw, max(steps, 100), warmup, stream)
    if fn(*args) != 0:
        raise RuntimeError("prologue call failed: " + lib.rel_attn_last_error().decode())
    nbytes = prologue_bytes(N, w.B, w.Hq, w.Hkv, w.D, 4, st_in is not None)
    return w, nbytes, total_ms / steps, kernel_ms


def bench_backward(steps: int, warmup: int):
    """The backward of the 8K sliding-window layer: dq, dk, dv and dr from the
    forward's out and lse (computed once, outside the timed region)."""
    import torch
    import transformer_attention_query_amd as ra
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[BACKWARD_WORKLOAD]
    x = {n: t.cuda() for n, t in tinputs.make_inputs(w, seed=0).items()}
    out, lse = ra.prefill(x["q"], x["k"], x["v"], x["r"], x["P_cols"], w.alpha, w.E, w.W, w.log_scale)
    ns, ws_bytes = ra.backward_plan(w.B, w.T, w.Hq, w.Hkv, w.D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    dr = torch.empty_like(x["r"])
    stream = torch.cuda.current_stream()
    lib = ra.load_library()
    args = (x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["r"].data_ptr(), x["P_cols"].data_ptr(),
            out.data_ptr(), x["dout"].data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            dr.data_ptr(), 1, w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.alpha, w.E, w.W, 1 if w.log_scale else 0, ns,
            ws.data_ptr(), ws_bytes, stream.cuda_stream)
    fn = lib.rel_attn_backward

    def step(_i):
        fn(*args)

    total_ms, per = _time_launches(step, steps, warmup, stream)
    if fn(*args) != 0:
        raise RuntimeError("backward call failed: " + lib.rel_attn_last_error().decode())
    flops = backward_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W) * w.B
    return w, flops, total_ms / steps, sum(per) / len(per), ns


def cpu_baseline(target_s: float = 15.0):
    """The fp64 oracle, as it stands, on query rows of the prefill workload."""
    import torch
    import oracle
    from transformer_attention_query_amd import inputs as tinputs

    w = tinputs.WORKLOADS[PREFILL_WORKLOAD]
    x = tinputs.make_inputs(w, seed=0)
    threads = torch.get_num_threads()
    stride_rows = lambda n: list(range(w.T - 1, -1, -max(1, w.T // n)))[:n]  # noqa: E731
    run = lambda rows: oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W,  # noqa: E731
                                      w.log_scale, rows=rows)
    # warm up, calibrate on 64 rows, then run a sample sized for about target_s
    run(stride_rows(8))
    t = time.perf_counter()
    run(stride_rows(64))
    per_row = (time.perf_counter() - t) / 64
    n = int(max(64, min(w.T, target_s / max(per_row, 1e-6))))
    rows = stride_rows(n)
    t = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t
    flops, _, _ = prefill_work(w.T, w.Hq, w.D, w.d_r, w.E, w.W, rows=rows)
    return {"value": flops * w.B / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {w.T} query rows (all {w.Hq} heads, evenly spaced) of {w.name}, "
                      f"fp64 torch-CPU oracle, {dt:.1f} s wall"}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device-to-device copy of known size: it reads and writes
    nbytes each, so the counters it produces give the factor between counter
    readings and bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extend", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the relative-attention kernels run on a single MI355X "
              "and this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_query_amd as ra
    ra.load_library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return

    w, flops, ms_step, kernel_ms, per = bench_prefill(args.steps, args.warmup)
    print(f"# prefill {w.name}: {ms_step * 1e3:.1f} us/step, kernel {kernel_ms * 1e3:.1f} us "
          f"(min {min(per) * 1e3:.1f}, max {max(per) * 1e3:.1f})", file=sys.stderr, flush=True)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    line = {
        "metric": "relative-attention prefill TFLOP/s + decode KV GB/s (% of MI355X peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "d_r": w.d_r,
                   "rel_extent": w.E, "window": w.W, "log_scale": w.log_scale, "alpha": "1/sqrt(128)",
                   "algorithmic_flops": flops},
        "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(PREFILL_KERNEL, _src_hash("prefill.hip", "device_common.hpp")),
                     "avg_launch_us": round(kernel_ms * 1e3, 2)},
    }
    if not args.no_decode:
        dw, nbytes, kv, d_ms, d_kernel_ms, ns = bench_decode(args.steps, args.warmup)
        gbps = nbytes / (d_ms * 1e-3) / 1e9
        kgbps = nbytes / (d_kernel_ms * 1e-3) / 1e9
        print(f"# decode {dw.name}: {d_ms * 1e3:.1f} us/step ({ns} splits)", file=sys.stderr, flush=True)
        line["decode"] = {"workload": dw.name, "value": round(gbps, 1), "unit": "GB/s", "ms_per_step": round(d_ms, 5),
                          "num_splits": ns, "algorithmic_bytes": nbytes,
                          "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL + "+merge", "achieved": round(kgbps, 1),
                                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                       "frac": round(kgbps / PEAK_HBM_GBPS, 4),
                                       "traffic": _traffic(DECODE_KERNEL, _src_hash("decode.hip", "device_common.hpp", "mx_common.hpp")),
                                       "avg_launch_us": round(d_kernel_ms * 1e3, 2)}}
    if not args.no_decode:
        pw, p_bytes, p_ms, p_kernel_ms, p_ns = bench_decode_paged(args.steps, args.warmup)
        print(f"# decode {pw.name}: {p_ms * 1e3:.1f} us/step ({p_ns} splits)", file=sys.stderr, flush=True)
        pk = p_bytes / (p_kernel_ms * 1e-3) / 1e9
        line["decode_paged"] = {"workload": pw.name, "value": round(p_bytes / (p_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                "ms_per_step": round(p_ms, 5), "num_splits": p_ns, "algorithmic_bytes": p_bytes,
                                "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL + " (paged)+merge",
                                             "achieved": round(pk, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                             "frac": round(pk / PEAK_HBM_GBPS, 4),
                                             "traffic": _traffic(DECODE_KERNEL + "_paged",
                                                                 _src_hash("decode.hip", "device_common.hpp", "mx_common.hpp")),
                                             "avg_launch_us": round(p_kernel_ms * 1e3, 2)}}
    if not args.no_decode:
        mw, m_bytes, m_ms, m_kernel_ms, m_ns = bench_decode_mx(args.steps, args.warmup)
        print(f"# decode {mw.name} (MXFP8 K/V): {m_ms * 1e3:.1f} us/step ({m_ns} splits)", file=sys.stderr, flush=True)
        mk = m_bytes / (m_kernel_ms * 1e-3) / 1e9
        line["decode_mx"] = {"workload": mw.name + " (MXFP8 K/V)", "value": round(m_bytes / (m_ms * 1e-3) / 1e9, 1),
                             "unit": "GB/s", "ms_per_step": round(m_ms, 5), "num_splits": m_ns,
                             "algorithmic_bytes": m_bytes, "dtype": "mxfp8 K/V, bf16 q/out",
                             "roofline": {"bound": "hbm", "kernel": DECODE_KERNEL + " (MXFP8)+merge",
                                          "achieved": round(mk, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                          "frac": round(mk / PEAK_HBM_GBPS, 4),
                                          "traffic": _traffic(DECODE_KERNEL + "_mx",
                                                              _src_hash("decode.hip", "device_common.hpp", "mx_common.hpp")),
                                          "avg_launch_us": round(m_kernel_ms * 1e3, 2)}}
    if not args.no_extend:
        ew, e_flops, e_ms, e_kernel_ms = bench_extend(args.steps, args.warmup)
        print(f"# extend {ew.name}: {e_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        e_ach = e_flops / (e_kernel_ms * 1e-3) / 1e12
        line["extend"] = {"workload": ew.name, "value": round(e_flops / (e_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                          "ms_per_step": round(e_ms, 5), "algorithmic_flops": e_flops,
                          "config": {"B": ew.B, "kv_len": ew.T, "new_rows": ew.n_new, "page_size": ew.page_size,
                                     "Hq": ew.Hq, "Hkv": ew.Hkv, "d_r": ew.d_r, "rel_extent": ew.E, "window": ew.W},
                          "roofline": {"bound": "mfma", "kernel": "prefill_kernel (extend)",
                                       "achieved": round(e_ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(e_ach / PEAK_BF16_TFLOPS, 4),
                                       "traffic": _traffic("prefill_kernel_extend",
                                                           _src_hash("prefill.hip", "device_common.hpp")),
                                       "avg_launch_us": round(e_kernel_ms * 1e3, 2)}}
    if not args.no_prologue:
        gw, g_bytes, g_ms, g_kernel_ms = bench_prologue(args.steps, args.warmup)
        print(f"# prologue {gw.name}: {g_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        gk = g_bytes / (g_kernel_ms * 1e-3) / 1e9
        line["prologue"] = {"workload": gw.name, "value": round(g_bytes / (g_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                            "ms_per_step": round(g_ms, 5), "algorithmic_bytes": g_bytes,
                            "config": {"B": gw.B, "tokens": gw.B * gw.n_new, "Hq": gw.Hq, "Hkv": gw.Hkv, "D": gw.D,
                                       "conv_width": 4, "page_size": gw.page_size},
                            "roofline": {"bound": "hbm", "kernel": "prologue_kernel", "achieved": round(gk, 1),
                                         "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gk / PEAK_HBM_GBPS, 4),
                                         "traffic": _traffic("prologue_kernel",
                                                             _src_hash("prologue.hip", "device_common.hpp", "mx_common.hpp")),
                                         "avg_launch_us": round(g_kernel_ms * 1e3, 2)}}
    if not args.no_backward:
        bw, b_flops, b_ms, b_kernel_ms, b_ns = bench_backward(args.steps, args.warmup)
        print(f"# backward {bw.name}: {b_ms * 1e3:.1f} us/step ({b_ns} head splits)", file=sys.stderr, flush=True)
        b_ach = b_flops / (b_kernel_ms * 1e-3) / 1e12
        line["backward"] = {"workload": bw.name, "value": round(b_flops / (b_ms * 1e-3) / 1e12, 2),
                            "unit": "TFLOP/s", "ms_per_step": round(b_ms, 5), "algorithmic_flops": b_flops,
                            "head_splits": b_ns,
                            "config": {"B": bw.B, "T": bw.T, "Hq": bw.Hq, "Hkv": bw.Hkv, "D": bw.D, "d_r": bw.d_r,
                                       "rel_extent": bw.E, "window": bw.W, "log_scale": bw.log_scale},
                            "roofline": {"bound": "mfma", "kernel": "bwd_dq_kernel+bwd_dkdv_kernel (+delta, reduce)",
                                         "achieved": round(b_ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(b_ach / PEAK_BF16_TFLOPS, 4),
                                         "traffic": _traffic("backward", _src_hash("backward.hip", "device_common.hpp")),
                                         "avg_launch_us": round(b_kernel_ms * 1e3, 2)}}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
